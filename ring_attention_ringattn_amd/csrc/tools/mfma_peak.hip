// Matrix-core throughput probe used by the benchmark to report a measured bf16
// peak beside the published one.  Every wave issues back-to-back
// v_mfma_f32_32x32x16_bf16 on register operands into eight independent
// accumulators (so no product waits for the previous one), with no memory
// traffic in the loop; the sums are consumed at the end so nothing is
// eliminated.  Not part of the ring-attention C ABI (libringattn); built into
// libringattn_tools.
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int CHAINS = 8;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)(lane + e));
    b[e] = (__bf16)(1e-3f * (float)(lane - e));
  }
  f32x16 acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) acc[c] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = mfma(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// FLOPs of one launch: blocks * (threads / 64) waves * iters * CHAINS * 32 * 32 * 16 * 2.
// sink: device, blocks * threads floats.  threads: a multiple of 64, at most 256.
extern "C" int ra_tool_mfma_peak(int iters, int blocks, int threads, float* sink, void* stream) {
  if (iters < 1 || blocks < 1 || threads < 64 || threads > 256 || threads % 64 || !sink) return -1;
  mfma_peak_kernel<<<blocks, threads, 0, (hipStream_t)stream>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int ra_tool_mfma_chains(void) { return CHAINS; }
