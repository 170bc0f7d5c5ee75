"""Planted-mistake check of the oracle's pins (CPU only).

Each case copies the oracle's C source, plants one plausible mistake (eps outside the square root, a
dropped residual, a transposed operand, gate and up swapped, r applied twice, gamma dropped, a wrong
mean denominator, a wrong gamma index, a sign flip in silu, a wrong subnormal exponent or exponent bias in the fp8
decoder, one significant bit too few in the fp8 and bf16 roundings, ties rounded away from zero, a wrong
scale index in either dequantiser, the partial sums read transposed, either storage rounding of the
round-points form left out, seven mistakes in the backward, four in the rotary embedding, five in the cross-entropy, three in the block-scaled quantiser and three in the SwiGLU backward), rebuilds it in a temporary directory and runs the pin tests
against it.  Every mutant must fail at least one pin; the unmodified oracle is never touched.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = [
    ("eps_outside_sqrt", "return 1.0 / sqrt(ss / (double)D + eps);", "return 1.0 / (sqrt(ss / (double)D) + eps);"),
    ("dropped_residual", "for (int64_t j = 0; j < D; ++j) hrow[j] += c->R[i * D + j];", ";"),
    ("transposed_w1", "const double* w = c->W1 + k * D;\n    for (int64_t j = 0; j < D; ++j) hrow[j] += x * w[j];",
     "const double* w = c->W1 + k;\n    for (int64_t j = 0; j < D; ++j) hrow[j] += x * w[j * K1];"),
    ("gate_up_swapped", "double v = oracle_silu(z[n]) * z[half + n];", "double v = oracle_silu(z[half + n]) * z[n];"),
    ("row_scale_twice", "z[n] *= r;", "z[n] *= r * r;"),
    ("gamma_dropped", "arow[j] = hrow[j] * r * c->gamma[j];", "arow[j] = hrow[j] * r;"),
    ("mean_denominator", "return 1.0 / sqrt(ss / (double)D + eps);", "return 1.0 / sqrt(ss / (double)(D - 1) + eps);"),
    ("gamma_wrong_index", "W2g[j * N2 + n] = gamma[j] * W2[j * N2 + n];", "W2g[j * N2 + n] = gamma[n % D] * W2[j * N2 + n];"),
    ("silu_sign", "return x / (1.0 + exp(-x));", "return x / (1.0 + exp(x));"),
    ("e4m3_subnormal", "v = ldexp((double)mant, -9);", "v = ldexp((double)mant, -10);"),
    ("e4m3_exponent_bias", "v = ldexp(1.0 + mant / 8.0, exp_bits - 7);", "v = ldexp(1.0 + mant / 8.0, exp_bits - 8);"),
    ("e4m3_encode_three_bits", "round_to_grid(a, 4, -6);", "round_to_grid(a, 3, -6);"),
    ("bf16_seven_bits", "round_to_grid(x, 8, -126);", "round_to_grid(x, 7, -126);"),
    ("ties_away_from_zero", "return nearbyint(x / ulp) * ulp;", "return round(x / ulp) * ulp;"),
    ("dequant_rows_scale_index", "oracle_e4m3_decode(q[i * cols + k]) * (double)s[i];",
     "oracle_e4m3_decode(q[i * cols + k]) * (double)s[0];"),
    ("dequant_cols_scale_index", "oracle_e4m3_decode(q[k * cols + n]) * (double)s[n];",
     "oracle_e4m3_decode(q[k * cols + n]) * (double)s[k % cols];"),
    ("partials_transposed", "ss += part[t * M + i];", "ss += part[i * T + t];"),
    ("roundpts_operand_unrounded", "arow[j] = oracle_bf16_round(hrow[j] * c->gamma[j]);",
     "arow[j] = hrow[j] * c->gamma[j];"),
    ("roundpts_output_unrounded", "c->y[i * half + n] = c->form == FORM_ROUNDPTS ? oracle_bf16_round(v) : v;",
     "c->y[i * half + n] = v;"),
]


# mistakes in the backward: the RMS correction term dropped, its sign flipped, r applied twice, dh_out
# dropped, W1 untransposed in dX, u replaced by n in dW2, gamma dropped from dgamma's product
MUTANTS_BWD = [
    ("bwd_no_correction", "double v = r * (du[j] * c->gamma[j] - n[j] * mean);", "double v = r * (du[j] * c->gamma[j]);"),
    ("bwd_correction_sign", "double v = r * (du[j] * c->gamma[j] - n[j] * mean);",
     "double v = r * (du[j] * c->gamma[j] + n[j] * mean);"),
    ("bwd_r_twice", "double v = r * (du[j] * c->gamma[j] - n[j] * mean);",
     "double v = r * r * (du[j] * c->gamma[j] - n[j] * mean);"),
    ("bwd_dh_out_dropped", "if (c->dh_out) v += c->dh_out[i * D + j];", ";"),
    ("bwd_dx_w1_index", "for (int64_t j = 0; j < D; ++j) s += dh[j] * w[j];",
     "for (int64_t j = 0; j < D; ++j) s += dh[j] * c->W1[(j % K1) * D + k % D];"),
    ("bwd_dw2_uses_n", "const double a = c->u[i * D + j];", "const double a = c->n[i * D + j];"),
    ("bwd_dgamma_uses_u", "g += c->du[i * D + j] * c->n[i * D + j];", "g += c->du[i * D + j] * c->u[i * D + j];"),
]


# mistakes in the rotary embedding: a sign of the rotation flipped, the exponent's factor 2 dropped, the
# position not wrapped at the sequence length, neighbours paired instead of halves
MUTANTS_ROPE = [
    ("rope_sin_sign", "row[h0 + i] = a * c - b * s;", "row[h0 + i] = a * c + b * s;"),
    ("rope_exponent", "pow(base, -2.0 * (double)i / (double)head_dim)", "pow(base, -1.0 * (double)i / (double)head_dim)"),
    ("rope_no_wrap", "const double pos = (double)(m % seq_len);", "const double pos = (double)m;"),
    ("rope_pairing", "const double a = row[h0 + i], b = row[h0 + i + half];",
     "const double a = row[h0 + i], b = row[h0 + (i ^ 1) + half];"),
]


# mistakes in the cross-entropy: the label's neighbour picked, the log dropped, the first logit left out of
# the sum, an ignored row given the full lse as its loss, the max shift not added back
MUTANTS_CE = [
    ("ce_label_neighbour", "c->loss[i] = label < 0 ? 0.0 : l - z[label];",
     "c->loss[i] = label < 0 ? 0.0 : l - z[(label + 1) % c->V];"),
    ("ce_no_log", "const double l = m + log(s);", "const double l = m + s;"),
    ("ce_sum_skips_first", "for (int64_t j = 0; j < c->V; ++j) s += exp(z[j] - m);",
     "for (int64_t j = 1; j < c->V; ++j) s += exp(z[j] - m);"),
    ("ce_ignored_row_loss", "c->loss[i] = label < 0 ? 0.0 : l - z[label];",
     "c->loss[i] = label < 0 ? l : l - z[label];"),
    ("ce_shift_not_restored", "const double l = m + log(s);", "const double l = log(s);"),
]


# mistakes in the block-scaled quantiser: the scale exponent taken one binade low (values above 448 would
# saturate), the block boundary shifted, the scale multiplied instead of divided
MUTANTS_MX = [
    ("mx_exponent_low", "int e = (2.0 * m <= 1.75) ? e2 - 9 : e2 - 8;", "int e = e2 - 9;"),
    ("mx_block_shift", "const double* v = x + i * cols + b * block;", "const double* v = x + i * cols + b * block + (b > 0);"),
    ("mx_scale_multiplied", "oracle_e4m3_encode(ldexp(v[j], -e));", "oracle_e4m3_encode(ldexp(v[j], e));"),
]


# mistakes in the SwiGLU backward: silu' without its correction term, Wd not transposed, gate and up swapped
# in the up-gradient
MUTANTS_SWIGLU_BWD = [
    ("swiglu_bwd_no_correction", "c->dz[i * 2 * F + f] = dy * u * s * (1.0 + g * (1.0 - s));",
     "c->dz[i * 2 * F + f] = dy * u * s;"),
    ("swiglu_bwd_wd_untransposed", "for (int64_t d = 0; d < D; ++d) dy += c->dout[i * D + d] * c->Wd[f * D + d];",
     "for (int64_t d = 0; d < D; ++d) dy += c->dout[i * D + d] * c->Wd[(d % F) * D + f % D];"),
    ("swiglu_bwd_up_uses_u", "c->dz[i * 2 * F + F + f] = dy * g * s;", "c->dz[i * 2 * F + F + f] = dy * u * s;"),
]


def _run_pins(tmp_path, name, before, after, pins):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert before in src, f"mutation site for {name} no longer exists"
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), tmp_path / "tests",
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutants.py"))
    (tmp_path / "oracle" / "oracle.c").write_text(src.replace(before, after, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", pins, "-q", "-x", "-p", "no:cacheprovider"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, f"mutant {name} was not caught:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout


@pytest.mark.parametrize("name,before,after", MUTANTS_SWIGLU_BWD, ids=[m[0] for m in MUTANTS_SWIGLU_BWD])
def test_swiglu_bwd_pins_catch_planted_mistake(tmp_path, name, before, after):
    _run_pins(tmp_path, name, before, after, "tests/test_oracle_swiglu_bwd_pins.py")


@pytest.mark.parametrize("name,before,after", MUTANTS_MX, ids=[m[0] for m in MUTANTS_MX])
def test_mx_pins_catch_planted_mistake(tmp_path, name, before, after):
    _run_pins(tmp_path, name, before, after, "tests/test_oracle_mx_pins.py")


@pytest.mark.parametrize("name,before,after", MUTANTS_CE, ids=[m[0] for m in MUTANTS_CE])
def test_ce_pins_catch_planted_mistake(tmp_path, name, before, after):
    _run_pins(tmp_path, name, before, after, "tests/test_oracle_ce_pins.py")


@pytest.mark.parametrize("name,before,after", MUTANTS_ROPE, ids=[m[0] for m in MUTANTS_ROPE])
def test_rope_pins_catch_planted_mistake(tmp_path, name, before, after):
    _run_pins(tmp_path, name, before, after, "tests/test_oracle_rope_pins.py")


@pytest.mark.parametrize("name,before,after", MUTANTS_BWD, ids=[m[0] for m in MUTANTS_BWD])
def test_backward_pins_catch_planted_mistake(tmp_path, name, before, after):
    _run_pins(tmp_path, name, before, after, "tests/test_oracle_bwd_pins.py")


@pytest.mark.parametrize("name,before,after", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, before, after):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert before in src, f"mutation site for {name} no longer exists"
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), tmp_path / "tests",
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutants.py"))
    (tmp_path / "oracle" / "oracle.c").write_text(src.replace(before, after, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, f"mutant {name} was not caught:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout
