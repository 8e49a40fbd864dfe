// Read rate of a single workgroup (one CU): nwg workgroups of T threads each read their own 512 KiB
// as 256 runs of 2 KiB (one KV head of one 16-token BF16 page) in a random order, every wavefront
// keeping 4 runs (8 sixteen-byte loads per lane) in flight.  It shows how fast one CU can pull
// pages when only a few workgroups are resident, the regime of small decode batches.
//
// Usage: pkv_cu_read_rate      (one JSON line per shape: best of 10 timed launches after 3 warm-ups)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#define CHECK(x)                                                                          \
  do {                                                                                    \
    hipError_t e_ = (x);                                                                  \
    if (e_ != hipSuccess) {                                                               \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                                       \
    }                                                                                     \
  } while (0)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr size_t kBytes = size_t(1) << 30;
constexpr int kRunVecs = 128;       // 2 KiB in 16-byte vectors
constexpr int kRunsPerWg = 256;     // 512 KiB per workgroup
constexpr int kMaxThreadsTotal = 64 * 1024;

template <int kDepth>
__global__ void read_runs(const u32x4 *__restrict__ base, const int32_t *__restrict__ order, uint32_t *__restrict__ sink) {
  const int waves = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = blockIdx.x * kRunsPerWg;
  uint32_t acc = 0;
  for (int r = wave * kDepth; r < kRunsPerWg; r += waves * kDepth) {
    u32x4 v[kDepth][2];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int rr = min(r + d, kRunsPerWg - 1);
      const u32x4 *p = base + (size_t)order[r0 + rr] * kRunVecs;
      v[d][0] = __builtin_nontemporal_load(p + lane);
      v[d][1] = __builtin_nontemporal_load(p + 64 + lane);
    }
#pragma unroll
    for (int d = 0; d < kDepth; ++d) acc ^= v[d][0].x ^ v[d][1].y;
  }
  sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

int main() {
  u32x4 *d = nullptr;
  int32_t *order = nullptr;
  uint32_t *sink = nullptr;
  const int nruns = (int)(kBytes / 2048);
  CHECK(hipMalloc(&d, kBytes));
  CHECK(hipMemset(d, 1, kBytes));
  std::vector<int32_t> h(nruns);
  for (int i = 0; i < nruns; ++i) h[i] = i;
  std::mt19937 rng(3);
  std::shuffle(h.begin(), h.end(), rng);
  CHECK(hipMalloc(&order, nruns * sizeof(int32_t)));
  CHECK(hipMemcpy(order, h.data(), nruns * sizeof(int32_t), hipMemcpyHostToDevice));
  CHECK(hipMalloc(&sink, kMaxThreadsTotal * sizeof(uint32_t)));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  for (int threads : {256, 512, 1024}) {
    for (int nwg : {1, 8, 64}) {
      if (nwg * kRunsPerWg > nruns || nwg * threads > kMaxThreadsTotal) continue;
      for (int rep = 0; rep < 3; ++rep) hipLaunchKernelGGL(read_runs<4>, dim3(nwg), dim3(threads), 0, 0, d, order, sink);
      CHECK(hipGetLastError());
      CHECK(hipDeviceSynchronize());
      float best = 1e30f;
      for (int rep = 0; rep < 10; ++rep) {
        CHECK(hipEventRecord(e0));
        hipLaunchKernelGGL(read_runs<4>, dim3(nwg), dim3(threads), 0, 0, d, order, sink);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float ms = 0;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        best = std::min(best, ms);
      }
      const double bytes = (double)kRunsPerWg * 2048;
      std::printf("{\"threads\": %d, \"workgroups\": %d, \"kib_per_workgroup\": %d, \"best_us\": %.2f, \"gbps_per_workgroup\": %.1f}\n",
                  threads, nwg, kRunsPerWg * 2, best * 1e3, bytes / (best * 1e-3) / 1e9);
      std::fflush(stdout);
    }
  }
  CHECK(hipFree(d));
  CHECK(hipFree(order));
  CHECK(hipFree(sink));
  return 0;
}
