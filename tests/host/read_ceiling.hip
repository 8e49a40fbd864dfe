// Read-bandwidth ceiling of this GPU for the decode kernels' access pattern: a 1 GiB buffer read
// once as 2 KiB runs (one KV head of one 16-token BF16 page) in a random order, with 16-byte
// loads, fully coalesced per wavefront.  No arithmetic beyond an XOR that keeps the loads live.
// It answers one question: what fraction of the 8 TB/s HBM peak can a pure read stream with this
// pattern reach here, so that the attention kernel's roofline fraction can be read against it.
//
// Usage: pkv_read_ceiling            (prints one JSON line per configuration, then the best)
// Each configuration: 4 wavefronts per workgroup; every wavefront reads `units` units of two runs
// each (like one K and one V run), keeping `depth` units in flight; 3 warm-up launches, then 20
// timed launches between HIP events, reported as the mean and the best.
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
constexpr int kRunBytes = 2048;
constexpr int kRunVecs = kRunBytes / 16;           // 128 sixteen-byte vectors: two per lane
constexpr size_t kRuns = kBytes / kRunBytes;        // 524288
constexpr size_t kUnits = kRuns / 2;                // two runs per unit

template <bool kNonTemporal>
__device__ __forceinline__ u32x4 load16(const u32x4 *p) {
  if (kNonTemporal) return __builtin_nontemporal_load(p);
  return *p;
}

// Wavefront w reads units w * units .. + units - 1; unit u is runs order[2u] and order[2u + 1].
template <int kDepth, bool kNonTemporal>
__global__ __launch_bounds__(256) void read_runs(const u32x4 *__restrict__ base, const int32_t *__restrict__ order,
                                                 int units, uint32_t *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int u0 = wave * units;
  u32x4 buf[kDepth][4];
  auto issue = [&](int u, u32x4(&r)[4]) {
    const u32x4 *a = base + (size_t)order[2 * u] * kRunVecs;
    const u32x4 *b = base + (size_t)order[2 * u + 1] * kRunVecs;
    r[0] = load16<kNonTemporal>(a + lane);
    r[1] = load16<kNonTemporal>(a + 64 + lane);
    r[2] = load16<kNonTemporal>(b + lane);
    r[3] = load16<kNonTemporal>(b + 64 + lane);
  };
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < kDepth; ++i) issue(u0 + i, buf[i]);
  for (int k = 0; k < units; k += kDepth) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc ^= buf[i][j].x ^ buf[i][j].y ^ buf[i][j].z ^ buf[i][j].w;
      if (k + kDepth + i < units) issue(u0 + k + kDepth + i, buf[i]);
    }
  }
  sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

struct Result {
  double mean_gbps, best_gbps;
};

template <int kDepth, bool kNonTemporal>
Result run(const u32x4 *d, const int32_t *order, uint32_t *sink, int units, const char *pattern) {
  const int waves = (int)(kUnits / units);  // units divides kUnits and is a multiple of kDepth
  const int blocks = waves / 4;
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  for (int i = 0; i < 3; ++i) hipLaunchKernelGGL((read_runs<kDepth, kNonTemporal>), dim3(blocks), dim3(256), 0, 0, d, order, units, sink);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  const int reps = 20;
  double total = 0, best = 1e30;
  for (int i = 0; i < reps; ++i) {
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL((read_runs<kDepth, kNonTemporal>), dim3(blocks), dim3(256), 0, 0, d, order, units, sink);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    total += ms;
    best = std::min(best, (double)ms);
  }
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  Result r{kBytes / (total / reps * 1e-3) / 1e9, kBytes / (best * 1e-3) / 1e9};
  std::printf("{\"pattern\": \"%s\", \"loads\": \"%s\", \"depth\": %d, \"units_per_wave\": %d, \"workgroups\": %d, "
              "\"mean_us\": %.2f, \"best_us\": %.2f, \"mean_gbps\": %.1f, \"best_gbps\": %.1f}\n",
              pattern, kNonTemporal ? "nt" : "plain", kDepth, units, blocks, total / reps * 1e3, best * 1e3, r.mean_gbps,
              r.best_gbps);
  std::fflush(stdout);
  return r;
}

int main() {
  u32x4 *d = nullptr;
  int32_t *order = nullptr;
  uint32_t *sink = nullptr;
  CHECK(hipMalloc(&d, kBytes));
  CHECK(hipMemset(d, 1, kBytes));
  CHECK(hipMalloc(&order, kRuns * sizeof(int32_t)));
  CHECK(hipMalloc(&sink, (kUnits / 8 / 4 + 1) * 256 * sizeof(uint32_t)));  // largest grid: 8 units per wave
  std::vector<int32_t> h(kRuns);
  for (size_t i = 0; i < kRuns; ++i) h[i] = (int32_t)i;
  std::vector<int32_t> seq = h;
  std::mt19937 rng(7);
  std::shuffle(h.begin(), h.end(), rng);

  double best_mean = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const bool random = pass == 0;
    CHECK(hipMemcpy(order, random ? h.data() : seq.data(), kRuns * sizeof(int32_t), hipMemcpyHostToDevice));
    const char *pat = random ? "random 2 KiB runs" : "sequential 2 KiB runs";
    for (int units : {8, 16, 32, 64}) {
      best_mean = std::max(best_mean, run<2, true>(d, order, sink, units, pat).mean_gbps);
      best_mean = std::max(best_mean, run<4, true>(d, order, sink, units, pat).mean_gbps);
    }
    run<2, false>(d, order, sink, 16, pat);
    run<4, false>(d, order, sink, 16, pat);
  }
  std::printf("{\"best_mean_gbps_nt\": %.1f, \"pct_of_8000\": %.2f}\n", best_mean, best_mean / 80.0);
  CHECK(hipFree(d));
  CHECK(hipFree(order));
  CHECK(hipFree(sink));
  return 0;
}
