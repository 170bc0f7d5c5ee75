// mfma_ceiling.hip -- the MFMA rate this device sustains with no memory traffic: a measurement aid for the
// roofline of the block's GEMMs (it is not part of the library).
//
// Every wave runs v_mfma_f32_32x32x16_bf16 back to back on eight independent accumulators, two waves per SIMD as
// in the GEMM kernels, with random bf16 operands (four fragment sets per lane, rotated from one instruction to the
// next so the operands keep changing, as they do in a GEMM: the matrix cores' power, and so the clock the device
// holds, depends on the data).  The shader clock comes from the shader-clock counter (s_memtime) against the
// 100 MHz constant counter (s_memrealtime), read inside the kernel.  Prints one JSON line.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

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

__global__ __launch_bounds__(256) void mfma_loop(float* out, long long* clk, int iters) {
  unsigned s = 0x9e3779b9u * (blockIdx.x * 256 + threadIdx.x + 1);
  s16x8 a[4], b[4];
  for (int j = 0; j < 4; ++j)
    for (int e = 0; e < 8; ++e) {
      a[j][e] = random_bf16(s);
      b[j][e] = random_bf16(s);
    }
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  f32x16 acc[8] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b[i & 3]),
                                                      __builtin_bit_cast(bf16x8, a[(i + (i >> 2)) & 3]), acc[i], 0, 0,
                                                      0);
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

int main() {
  int cus = 0;
  CK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  const int wgs = 2 * cus;  // 8 waves per CU: two per SIMD
  const int iters = 40000;
  float* out = nullptr;
  long long* clk = nullptr;
  CK(hipMalloc(&out, (size_t)wgs * 256 * sizeof(float)));
  CK(hipMalloc(&clk, (size_t)wgs * 2 * sizeof(long long)));
  for (int w = 0; w < 3; ++w) hipLaunchKernelGGL(mfma_loop, dim3(wgs), dim3(256), 0, 0, out, clk, iters);
  CK(hipGetLastError());
  CK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  const int reps = 3;
  double best_tflops = 0.0, mhz_at_best = 0.0;
  std::vector<long long> h((size_t)wgs * 2);
  for (int rep = 0; rep < reps; ++rep) {
    CK(hipEventRecord(e0));
    hipLaunchKernelGGL(mfma_loop, dim3(wgs), dim3(256), 0, 0, out, clk, iters);
    CK(hipEventRecord(e1));
    CK(hipEventSynchronize(e1));
    float ms = 0.0f;
    CK(hipEventElapsedTime(&ms, e0, e1));
    CK(hipMemcpy(h.data(), clk, h.size() * sizeof(long long), hipMemcpyDeviceToHost));
    double mhz = 0.0;
    for (int i = 0; i < wgs; ++i) mhz += (double)h[2 * i] / ((double)h[2 * i + 1] / 100.0);
    mhz /= wgs;
    const double tflops = (double)wgs * 4 * iters * 8 * 32768.0 / (ms * 1e-3) / 1e12;
    if (tflops > best_tflops) {
      best_tflops = tflops;
      mhz_at_best = mhz;
    }
  }
  std::printf("{\"tflops\": %.1f, \"sclk_mhz\": %.0f, \"workgroups\": %d, \"mfma\": \"v_mfma_f32_32x32x16_bf16\", "
              "\"operands\": \"random bf16\"}\n",
              best_tflops, mhz_at_best, wgs);
  return 0;
}
