// mfma_ceiling.hip -- the MFMA rate this device sustains with no memory traffic: a measurement aid for the
// roofline of the block's GEMMs (it is not part of the library).
//
// Every wave runs the GEMMs' matrix instruction back to back on eight independent accumulators, two waves per SIMD
// as in the GEMM kernels, with random operands (four fragment sets per lane, rotated from one instruction to the
// next so the operands keep changing, as they do in a GEMM: the matrix cores' power, and so the clock the device
// holds, depends on the data): v_mfma_f32_32x32x16_bf16 on bf16, and v_mfma_scale_f32_32x32x64_f8f6f4 on e4m3 bytes
// with unit block scales (the e4m3 kernels' instruction).  The shader clock comes from the shader-clock counter
// (s_memtime) against the 100 MHz constant counter (s_memrealtime), read inside the kernel.  Prints one JSON line.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define CK(x)                                                                                   \
  do {                                                                                          \
    hipError_t e_ = (x);                                                                        \
    if (e_ != hipSuccess) {                                                                     \
      std::printf("{\"error\": \"%s at line %d\"}\n", hipGetErrorString(e_), __LINE__);       \
      return 1;                                                                                 \
    }                                                                                           \
  } while (0)

__device__ unsigned next_u32(unsigned& s) {
  s = s * 1664525u + 1013904223u;
  return s;
}

// a random bf16 in (-1, 1): random sign, exponent 2^-7 .. 2^-1, random mantissa
__device__ short random_bf16(unsigned& s) {
  const unsigned r = next_u32(s);
  return (short)(((r >> 31) << 15) | ((120 + (r >> 8) % 7) << 7) | (r & 0x7f));
}

// a random e4m3 byte that is neither NaN (S.1111.111) nor tiny: exponent field 4..11
__device__ int random_e4m3x4(unsigned& s) {
  int w = 0;
  for (int b = 0; b < 4; ++b) {
    const unsigned r = next_u32(s);
    w |= (int)((((r >> 31) << 7) | ((4 + (r >> 8) % 8) << 3) | (r & 7)) << (8 * b));
  }
  return w;
}

template <bool FP8>
__global__ __launch_bounds__(256) void mfma_loop(float* out, long long* clk, int iters) {
  unsigned s = 0x9e3779b9u * (blockIdx.x * 256 + threadIdx.x + 1);
  s16x8 a[4], b[4];
  i32x8 qa[4], qb[4];
  for (int j = 0; j < 4; ++j)
    for (int e = 0; e < 8; ++e) {
      if (FP8) {
        qa[j][e] = random_e4m3x4(s);
        qb[j][e] = random_e4m3x4(s);
      } else {
        a[j][e] = random_bf16(s);
        b[j][e] = random_bf16(s);
      }
    }
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  f32x16 acc[8] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (FP8)
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qb[i & 3], qa[(i + (i >> 2)) & 3], acc[i], 0, 0, 0, 127,
                                                                 0, 127);
      else
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b[i & 3]),
                                                        __builtin_bit_cast(bf16x8, a[(i + (i >> 2)) & 3]), acc[i], 0, 0,
                                                        0);
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  float sum = 0.0f;
  for (int i = 0; i < 8; ++i) sum += acc[i][0] + acc[i][15];
  out[blockIdx.x * 256 + threadIdx.x] = sum;  // keeps the loop's results alive
  if (threadIdx.x == 0) {
    clk[blockIdx.x * 2] = t1 - t0;
    clk[blockIdx.x * 2 + 1] = r1 - r0;
  }
}

// Best of three timed launches after three untimed ones: (TFLOP/s, mean shader clock in MHz).
template <bool FP8>
static int measure(float* out, long long* clk, int wgs, int iters, double& tflops_out, double& mhz_out) {
  for (int w = 0; w < 3; ++w) hipLaunchKernelGGL(mfma_loop<FP8>, dim3(wgs), dim3(256), 0, 0, out, clk, iters);
  CK(hipGetLastError());
  CK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  std::vector<long long> h((size_t)wgs * 2);
  tflops_out = 0.0;
  for (int rep = 0; rep < 3; ++rep) {
    CK(hipEventRecord(e0));
    hipLaunchKernelGGL(mfma_loop<FP8>, dim3(wgs), dim3(256), 0, 0, out, clk, iters);
    CK(hipEventRecord(e1));
    CK(hipEventSynchronize(e1));
    float ms = 0.0f;
    CK(hipEventElapsedTime(&ms, e0, e1));
    CK(hipMemcpy(h.data(), clk, h.size() * sizeof(long long), hipMemcpyDeviceToHost));
    double mhz = 0.0;
    for (int i = 0; i < wgs; ++i) mhz += (double)h[2 * i] / ((double)h[2 * i + 1] / 100.0);
    mhz /= wgs;
    const double flops_per_mfma = FP8 ? 131072.0 : 32768.0;
    const double tflops = (double)wgs * 4 * iters * 8 * flops_per_mfma / (ms * 1e-3) / 1e12;
    if (tflops > tflops_out) {
      tflops_out = tflops;
      mhz_out = mhz;
    }
  }
  CK(hipEventDestroy(e0));
  CK(hipEventDestroy(e1));
  return 0;
}

int main() {
  int cus = 0;
  CK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  const int wgs = 2 * cus;  // 8 waves per CU: two per SIMD
  float* out = nullptr;
  long long* clk = nullptr;
  CK(hipMalloc(&out, (size_t)wgs * 256 * sizeof(float)));
  CK(hipMalloc(&clk, (size_t)wgs * 2 * sizeof(long long)));
  double tf16 = 0.0, mhz16 = 0.0, tf8 = 0.0, mhz8 = 0.0;
  if (measure<false>(out, clk, wgs, 40000, tf16, mhz16)) return 1;
  if (measure<true>(out, clk, wgs, 10000, tf8, mhz8)) return 1;
  std::printf("{\"tflops\": %.1f, \"sclk_mhz\": %.0f, \"mfma\": \"v_mfma_f32_32x32x16_bf16\", \"operands\": \"random bf16\", "
              "\"fp8\": {\"tflops\": %.1f, \"sclk_mhz\": %.0f, \"mfma\": \"v_mfma_scale_f32_32x32x64_f8f6f4\", "
              "\"operands\": \"random e4m3\"}, \"workgroups\": %d}\n",
              tf16, mhz16, tf8, mhz8, wgs);
  return 0;
}
