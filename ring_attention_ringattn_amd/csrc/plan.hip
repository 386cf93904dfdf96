// Tile plan helpers: per-tile position/document ranges (used to skip fully
// masked tiles) and document ids from cu_seqlens offsets.
#include "ra_internal.h"

namespace ra {

// One wave per tile of TILE tokens: min/max of positions and documents.
__global__ __launch_bounds__(256) void tile_ranges_kernel(const int* __restrict__ pos,
                                                          const int* __restrict__ doc, int n,
                                                          TileRange* __restrict__ out, int tiles) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tile = blockIdx.x * 4 + wave;
  if (tile >= tiles) return;
  const int t = tile * TILE + lane;
  const bool valid = t < n;
  int p = valid ? pos[t] : 0;
  int d = (valid && doc) ? doc[t] : 0;
  int mn_p = valid ? p : 0x7fffffff, mx_p = valid ? p : (int)0x80000000;
  int mn_d = valid ? d : 0x7fffffff, mx_d = valid ? d : (int)0x80000000;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mn_p = min(mn_p, __shfl_xor(mn_p, off));
    mx_p = max(mx_p, __shfl_xor(mx_p, off));
    mn_d = min(mn_d, __shfl_xor(mn_d, off));
    mx_d = max(mx_d, __shfl_xor(mx_d, off));
  }
  if (lane == 0) out[tile] = TileRange{mn_p, mx_p, mn_d, mx_d};
}

// Several tables in one launch: blockIdx.y selects the job.
__global__ __launch_bounds__(256) void tile_ranges_batch_kernel(TableJobs jobs) {
  const TableJob& jb = jobs.job[blockIdx.y];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tiles = n_tiles(jb.n);
  const int tile = blockIdx.x * 4 + wave;
  if (tile >= tiles) return;
  const int t = tile * TILE + lane;
  const bool valid = t < jb.n;
  int p = valid ? jb.pos[t] : 0;
  int d = (valid && jb.doc) ? jb.doc[t] : 0;
  int mn_p = valid ? p : 0x7fffffff, mx_p = valid ? p : (int)0x80000000;
  int mn_d = valid ? d : 0x7fffffff, mx_d = valid ? d : (int)0x80000000;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mn_p = min(mn_p, __shfl_xor(mn_p, off));
    mx_p = max(mx_p, __shfl_xor(mx_p, off));
    mn_d = min(mn_d, __shfl_xor(mn_d, off));
    mx_d = max(mx_d, __shfl_xor(mx_d, off));
  }
  if (lane == 0) jb.out[tile] = TileRange{mn_p, mx_p, mn_d, mx_d};
}

hipError_t launch_tile_ranges_batch(const TableJobs& jobs, hipStream_t st) {
  if (jobs.count <= 0) return hipSuccess;
  if (jobs.count > TABLE_JOBS) return hipErrorInvalidValue;
  int tiles = 0;
  for (int i = 0; i < jobs.count; ++i) tiles = max(tiles, n_tiles(jobs.job[i].n));
  if (tiles == 0) return hipSuccess;
  tile_ranges_batch_kernel<<<dim3((tiles + 3) / 4, jobs.count), 256, 0, st>>>(jobs);
  return hipGetLastError();
}

hipError_t launch_tile_ranges(const int* pos, const int* doc, int n, TileRange* out, hipStream_t st) {
  const int tiles = n_tiles(n);
  if (tiles == 0) return hipSuccess;
  tile_ranges_kernel<<<(tiles + 3) / 4, 256, 0, st>>>(pos, doc, n, out, tiles);
  return hipGetLastError();
}

// doc[t] = k with cu[k] <= first + t < cu[k+1]; -1 outside every document.
__global__ void docs_from_cu_kernel(const int* __restrict__ cu, int n_docs, int first, int n,
                                    int* __restrict__ doc) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const int x = first + t;
  int lo = 0, hi = n_docs;  // search k in [0, n_docs) with cu[k] <= x < cu[k+1]
  if (n_docs <= 0 || x < cu[0] || x >= cu[n_docs]) {
    doc[t] = -1;
    return;
  }
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= x) lo = mid; else hi = mid;
  }
  doc[t] = lo;
}

hipError_t launch_docs_from_cu(const int* cu, int n_docs, int first, int n, int* doc, hipStream_t st) {
  if (n == 0) return hipSuccess;
  docs_from_cu_kernel<<<(n + 255) / 256, 256, 0, st>>>(cu, n_docs, first, n, doc);
  return hipGetLastError();
}

__global__ void fill_nan_kernel(uint32_t* p, size_t words) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0x7fc07fc0u;   // two bf16 quiet NaNs; as fp32 also a quiet NaN
}

hipError_t launch_fill_nan(void* p, size_t bytes, hipStream_t st) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  fill_nan_kernel<<<(unsigned)blocks, 256, 0, st>>>((uint32_t*)p, words);
  return hipGetLastError();
}

}  // namespace ra
