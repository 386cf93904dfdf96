// HBM streaming probes used by the benchmark to report a measured memory ceiling
// beside the published 8 TB/s: a copy and a read-only sweep over a device buffer,
// 16 bytes per lane, nontemporal (every byte is touched once), grid-stride.  Not
// part of the ring-attention C ABI (libringattn); built into libringattn_tools.
#include <hip/hip_runtime.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                          size_t n) {
  const size_t step = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(256) void stream_read_kernel(const f32x4* __restrict__ src, size_t n, float* sink) {
  const size_t step = (size_t)gridDim.x * blockDim.x;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step)
    acc += __builtin_nontemporal_load(src + i);
  // consumed, so the loads stay; sink holds one float per thread
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
}

}  // namespace

// Copies `bytes` (a multiple of 16; src and dst 16-byte aligned, not overlapping) with
// `blocks` workgroups of 256 threads.  Returns 0, or -1 for bad arguments, else a hipError_t.
extern "C" int ra_tool_hbm_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (!src || !dst || bytes % 16 || blocks < 1 || ((size_t)src | (size_t)dst) % 16) return -1;
  stream_copy_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>((const f32x4*)src, (f32x4*)dst, bytes / 16);
  return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 16, 16-byte aligned) with `blocks` workgroups of 256
// threads; sink: device, blocks * 256 floats.
extern "C" int ra_tool_hbm_read(const void* src, size_t bytes, int blocks, float* sink, void* stream) {
  if (!src || !sink || bytes % 16 || blocks < 1 || (size_t)src % 16) return -1;
  stream_read_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>((const f32x4*)src, bytes / 16, sink);
  return (int)hipGetLastError();
}
