// probe_mfma_clock.hip -- measurement probe (a stand-alone program, not part of libcpattn.so).
//
// What it measures: the bf16 MFMA rate the chip sustains when every SIMD issues nothing but
// v_mfma_f32_32x32x16_bf16, and the shader clock it runs at meanwhile. The published dense peak
// assumes the peak engine clock; the clock the power manager grants under MFMA load depends on
// the operands' bit activity, so the probe runs the same loop twice:
//  - "random": per-lane pseudo-random bf16 operands in [-1, 1) (8 A and 4 B register sets, so
//    consecutive MFMAs see different bits), the case of attention on real activations;
//  - "constant": near-constant operands (few bit toggles), which lets the clock stay high.
// Each wave reads s_memtime (shader-clock counter) and s_memrealtime (fixed 100 MHz counter)
// around its loop; their ratio is the average shader clock. Throughput comes from HIP events.
// Two waves per SIMD (2 x CUs workgroups of 4 waves); the accumulators stay in registers and no
// memory is touched inside the loop. Output: one JSON line with the steady-state figures (the
// median of each mode's later launches, after the clock has settled).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define PROBE_CHECK(x)                                                          \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                             \
    }                                                                           \
  } while (0)

namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kMfmaPerIter = 8;

// integer hash (xor-shift-multiply), used only to spread operand bits
__device__ inline unsigned mix(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

template <bool RANDOM>
__global__ __launch_bounds__(kThreads) void mfma_loop(int iters, unsigned long long* stamps, float* sink) {
  bf16x8 a[8], b[4];
  const unsigned lane_id = blockIdx.x * kThreads + threadIdx.x;
  for (int s = 0; s < 8; ++s)
    for (int i = 0; i < 8; ++i)
      a[s][i] = (__bf16)(RANDOM ? (mix(lane_id * 131u + s * 8 + i) & 0xFFFF) / 32768.f - 1.f
                                : 0.001f * (threadIdx.x + i));
  for (int s = 0; s < 4; ++s)
    for (int i = 0; i < 8; ++i)
      b[s][i] = (__bf16)(RANDOM ? (mix(lane_id * 131u + 1000u + s * 8 + i) & 0xFFFF) / 32768.f - 1.f
                                : 0.002f * i);
  f32x16 c[4];
  for (int j = 0; j < 4; ++j)
    for (int v = 0; v < 16; ++v) c[j][v] = 0.f;

  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < kMfmaPerIter; ++s)
      c[s & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[(3 * s) & 3], c[s & 3], 0, 0, 0);
  }
  float sum = 0.f;
  for (int j = 0; j < 4; ++j)
    for (int v = 0; v < 16; ++v) sum += c[j][v];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();

  const int w = blockIdx.x * (kThreads / 64) + threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) {
    stamps[2 * w] = t1 - t0;
    stamps[2 * w + 1] = r1 - r0;
  }
  if (sum == 12345.0f) sink[threadIdx.x] = sum;  // keeps the loop live
}

struct Sample {
  double tflops, ghz;
};

template <bool RANDOM>
std::vector<Sample> run(int blocks, int iters, int reps) {
  const int waves = blocks * (kThreads / 64);
  unsigned long long* stamps;
  float* sink;
  PROBE_CHECK(hipMalloc(&stamps, (size_t)waves * 2 * sizeof(unsigned long long)));
  PROBE_CHECK(hipMalloc(&sink, kThreads * sizeof(float)));
  hipEvent_t e0, e1;
  PROBE_CHECK(hipEventCreate(&e0));
  PROBE_CHECK(hipEventCreate(&e1));
  std::vector<unsigned long long> h((size_t)waves * 2);
  std::vector<Sample> out;
  for (int r = 0; r < reps; ++r) {
    PROBE_CHECK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL(mfma_loop<RANDOM>, dim3(blocks), dim3(kThreads), 0, 0, iters, stamps, sink);
    PROBE_CHECK(hipGetLastError());
    PROBE_CHECK(hipEventRecord(e1, 0));
    PROBE_CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    PROBE_CHECK(hipEventElapsedTime(&ms, e0, e1));
    PROBE_CHECK(hipMemcpy(h.data(), stamps, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
    double ticks = 0, real = 0;
    for (int w = 0; w < waves; ++w) {
      ticks += (double)h[2 * w];
      real += (double)h[2 * w + 1];
    }
    const double flops = (double)waves * iters * kMfmaPerIter * (2.0 * 32 * 32 * 16);
    out.push_back({flops / (ms * 1e-3) / 1e12, ticks / real * 0.1});
  }
  PROBE_CHECK(hipEventDestroy(e0));
  PROBE_CHECK(hipEventDestroy(e1));
  PROBE_CHECK(hipFree(stamps));
  PROBE_CHECK(hipFree(sink));
  return out;
}

// median of the launches after the first `skip` (the clock settles over the first ones)
Sample settled(std::vector<Sample> v, int skip) {
  v.erase(v.begin(), v.begin() + std::min<size_t>(skip, v.size() - 1));
  std::sort(v.begin(), v.end(), [](const Sample& x, const Sample& y) { return x.tflops < y.tflops; });
  return v[v.size() / 2];
}

}  // namespace

int main() {
  int dev = 0;
  PROBE_CHECK(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  PROBE_CHECK(hipGetDeviceProperties(&prop, dev));
  const int blocks = 2 * prop.multiProcessorCount;  // two waves per SIMD
  const int iters = 50000;                           // ~15 ms per launch at 1.8 GHz
  const Sample rnd = settled(run<true>(blocks, iters, 8), 3);
  const Sample cst = settled(run<false>(blocks, iters, 6), 3);
  std::printf("{\"random\": {\"tflops\": %.1f, \"clock_ghz\": %.3f}, "
              "\"constant\": {\"tflops\": %.1f, \"clock_ghz\": %.3f}, "
              "\"blocks\": %d, \"threads\": %d, \"iters\": %d, \"mfma\": \"v_mfma_f32_32x32x16_bf16\"}\n",
              rnd.tflops, rnd.ghz, cst.tflops, cst.ghz, blocks, kThreads, iters);
  return 0;
}
