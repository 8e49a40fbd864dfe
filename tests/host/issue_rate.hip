// Issue-rate probe: the cost of v_exp_f32, v_fma_f32 and a 16x16x32 BF16 MFMA on this GPU, alone
// and interleaved, as wall time per wave instruction per SIMD.  Every workgroup has 256 threads
// (one wavefront per SIMD); the grid puts 4 workgroups on each CU, so each SIMD interleaves 4
// wavefronts.  Each wavefront runs 8 independent dependency chains per instruction kind, so the
// figures are throughput, not latency.  3 launches warm the clocks; the 4th is timed with events.
//
// Usage: pkv_issue_rate        (one JSON line per mix)
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#define CHECK(x)                                                                          \
  do {                                                                                    \
    hipError_t e_ = (x);                                                                  \
    if (e_ != hipSuccess) {                                                               \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                                       \
    }                                                                                     \
  } while (0)

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

#define EXP(x) asm volatile("v_exp_f32 %0, %0" : "+v"(x))
#define FMA(x) asm volatile("v_fma_f32 %0, %0, %0, %0" : "+v"(x))
#define MFMA(c) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(m, m, c, 0, 0, 0)

enum Mix { kExp, kFma, kExpFma, kMfma, kMfmaExp, kMfmaFma };

template <int kMix>
__global__ __launch_bounds__(256) void probe(float *out, int iters) {
  float a0 = threadIdx.x * 1e-3f, a1 = a0 + 1, a2 = a0 + 2, a3 = a0 + 3;
  float a4 = a0 + 4, a5 = a0 + 5, a6 = a0 + 6, a7 = a0 + 7;
  float b0 = a0 * 0.5f, b1 = b0 + 1, b2 = b0 + 2, b3 = b0 + 3, b4 = b0 + 4, b5 = b0 + 5, b6 = b0 + 6, b7 = b0 + 7;
  f32x4 c0 = {a0, a1, a2, a3}, c1 = c0, c2 = c0, c3 = c0;
  bf16x8 m = {};
  for (int i = 0; i < 8; ++i) m[i] = (__bf16)(a0 + i);
  for (int it = 0; it < iters; ++it) {
    if (kMix == kExp) { EXP(a0); EXP(a1); EXP(a2); EXP(a3); EXP(a4); EXP(a5); EXP(a6); EXP(a7); }
    if (kMix == kFma) { FMA(a0); FMA(a1); FMA(a2); FMA(a3); FMA(a4); FMA(a5); FMA(a6); FMA(a7); }
    if (kMix == kExpFma) {
      EXP(a0); FMA(b0); EXP(a1); FMA(b1); EXP(a2); FMA(b2); EXP(a3); FMA(b3);
      EXP(a4); FMA(b4); EXP(a5); FMA(b5); EXP(a6); FMA(b6); EXP(a7); FMA(b7);
    }
    if (kMix == kMfma) { MFMA(c0); MFMA(c1); MFMA(c2); MFMA(c3); }
    if (kMix == kMfmaExp) {
      MFMA(c0); EXP(a0); EXP(a1); MFMA(c1); EXP(a2); EXP(a3);
      MFMA(c2); EXP(a4); EXP(a5); MFMA(c3); EXP(a6); EXP(a7);
    }
    if (kMix == kMfmaFma) {
      MFMA(c0); FMA(a0); FMA(a1); MFMA(c1); FMA(a2); FMA(a3);
      MFMA(c2); FMA(a4); FMA(a5); MFMA(c3); FMA(a6); FMA(a7);
    }
  }
  out[blockIdx.x * 256 + threadIdx.x] =
      a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7 + b0 + b1 + b2 + b3 + b4 + b5 + b6 + b7 + c0[0] + c1[1] + c2[2] + c3[3];
}

// Prints ns per instruction per SIMD for each instruction kind of the mix (the mix's wall time
// divided by the instructions one SIMD issues of that kind).
template <int kMix>
void run(const char *name, int blocks, int waves_per_simd, float *out, int iters, int n_exp, int n_fma, int n_mfma) {
  for (int i = 0; i < 3; ++i) hipLaunchKernelGGL(probe<kMix>, dim3(blocks), dim3(256), 0, 0, out, iters);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  CHECK(hipEventRecord(e0));
  hipLaunchKernelGGL(probe<kMix>, dim3(blocks), dim3(256), 0, 0, out, iters);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  const double per_simd = (double)iters * waves_per_simd;  // iterations one SIMD runs
  const double ns = ms * 1e6;
  std::printf("{\"mix\": \"%s\", \"waves_per_simd\": %d, \"ms\": %.4f", name, waves_per_simd, ms);
  if (n_exp) std::printf(", \"ns_per_exp\": %.3f", ns / (per_simd * n_exp));
  if (n_fma) std::printf(", \"ns_per_fma\": %.3f", ns / (per_simd * n_fma));
  if (n_mfma) std::printf(", \"ns_per_mfma\": %.3f, \"mfma_tflops\": %.1f", ns / (per_simd * n_mfma),
                          (double)blocks * 4 * iters * n_mfma * 16384.0 / (ms * 1e-3) / 1e12);
  std::printf("}\n");
  std::fflush(stdout);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  const int blocks = cus * 4;  // 4 workgroups of 4 wavefronts per CU: 4 wavefronts per SIMD
  float *out = nullptr;
  CHECK(hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)));
  const int iters = 20000;
  std::printf("{\"cus\": %d, \"peak_clock_mhz\": %d}\n", cus, prop.clockRate / 1000);
  run<kExp>("exp x8", blocks, 4, out, iters, 8, 0, 0);
  run<kFma>("fma x8", blocks, 4, out, iters, 0, 8, 0);
  run<kExpFma>("exp x8 + fma x8", blocks, 4, out, iters, 8, 8, 0);
  run<kMfma>("mfma x4", blocks, 4, out, iters, 0, 0, 4);
  run<kMfmaExp>("mfma x4 + exp x8", blocks, 4, out, iters, 8, 0, 4);
  run<kMfmaFma>("mfma x4 + fma x8", blocks, 4, out, iters, 0, 8, 4);
  CHECK(hipFree(out));
  return 0;
}
