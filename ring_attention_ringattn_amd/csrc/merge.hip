// HBM-bound helpers: the standalone log-sum-exp combine of two normalised
// partial results, and the backward's D = rowsum(dO * O).
#include "ra_internal.h"

namespace ra {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Weights of the combine (o, lse) = (o_a, lse_a) (+) (o_b, lse_b).
__device__ inline void combine_weights(float la, float lb, float& lse, float& wa, float& wb) {
  const float mx = fmaxf(la, lb);
  if (mx == -INFINITY) {
    lse = -INFINITY; wa = 0.f; wb = 0.f;
    return;
  }
  const float ea = __expf(la - mx), eb = __expf(lb - mx);   // exp(-inf) = 0
  const float s = ea + eb;
  lse = mx + __logf(s);
  const float inv = 1.f / s;
  wa = ea * inv;
  wb = eb * inv;
}

// A group of 32 lanes owns one row (so the in-place lse_b update cannot race
// with another row's reads); each lane handles D/32 consecutive floats.  The
// grid covers every row once.  Every byte is touched once, so the loads and
// stores are nontemporal (no reuse to keep in the caches; measured: 5.1 ->
// 6.4 TB/s on MI355X at 16384 rows x 32 heads, D = 128).
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(long rows, const float* __restrict__ o_a,
                                                    const float* __restrict__ lse_a, float* o_b,
                                                    float* lse_b, void* out, Strides os, int hq, int sq,
                                                    int dtype) {
  constexpr int PER = D / 32;   // 4 (D=128) or 2 (D=64)
  typedef float vec __attribute__((ext_vector_type(PER)));
  const int lane = threadIdx.x & 31;
  const long row = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 5;
  if (row >= rows) return;
  const size_t base = (size_t)row * D + lane * PER;
  const vec a = __builtin_nontemporal_load((const vec*)(o_a + base));
  const vec b = __builtin_nontemporal_load((const vec*)(o_b + base));
  float lse, wa, wb;
  combine_weights(lse_a[row], lse_b[row], lse, wa, wb);
  const vec r = wa * a + wb * b;
  __builtin_nontemporal_store(r, (vec*)(o_b + base));
  if (out) {
    const int bi = row / ((long)hq * sq), h = (row / sq) % hq, s = row % sq;
    const size_t ob = bi * os.b + h * os.h + s * os.s + lane * PER;
    if (dtype == BF16) {
      for (int e = 0; e < PER; ++e) ((__bf16*)out)[ob + e] = (__bf16)r[e];
    } else {
      for (int e = 0; e < PER; ++e) ((float*)out)[ob + e] = r[e];
    }
  }
  if (lane == 0) lse_b[row] = lse;
}

hipError_t launch_merge(int64_t rows, int d, const float* o_a, const float* lse_a, float* o_b, float* lse_b,
                        void* out, Strides os, int hq, int sq, int dtype, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const long blocks = (rows * 32 + 255) / 256;   // one 32-lane group per row (the caller checked the grid fits)
  if (d == 128)
    merge_kernel<128><<<(unsigned)blocks, 256, 0, st>>>(rows, o_a, lse_a, o_b, lse_b, out, os, hq, sq, dtype);
  else
    merge_kernel<64><<<(unsigned)blocks, 256, 0, st>>>(rows, o_a, lse_a, o_b, lse_b, out, os, hq, sq, dtype);
  return hipGetLastError();
}

// delta[row] = sum_d dO[row, d] * O[row, d]; D/8 lanes per row, 8 elements per lane.
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_pre_kernel(int B, int hq, int sq, const T* __restrict__ out,
                                                      const T* __restrict__ d_o, Strides qs,
                                                      float* __restrict__ delta) {
  constexpr int G = D / 8;   // lanes per row (16 or 8)
  const long rows = (long)B * hq * sq;
  const int sub = threadIdx.x % G;
  long row = ((long)blockIdx.x * blockDim.x + threadIdx.x) / G;
  const long stride_rows = ((long)gridDim.x * blockDim.x) / G;
  for (; row < rows; row += stride_rows) {   // uniform trip count per G-lane group
    const int b = row / ((long)hq * sq), h = (row / sq) % hq, s = row % sq;
    const size_t off = b * qs.b + h * qs.h + s * qs.s + sub * 8;
    float acc = 0.f;
    if constexpr (sizeof(T) == 2) {
      const bf16x8 x = *(const bf16x8*)(out + off);
      const bf16x8 y = *(const bf16x8*)(d_o + off);
      for (int e = 0; e < 8; ++e) acc += (float)x[e] * (float)y[e];
    } else {
      const f32x4 x0 = *(const f32x4*)(out + off), x1 = *(const f32x4*)(out + off + 4);
      const f32x4 y0 = *(const f32x4*)(d_o + off), y1 = *(const f32x4*)(d_o + off + 4);
      for (int e = 0; e < 4; ++e) acc += x0[e] * y0[e] + x1[e] * y1[e];
    }
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, G);
    if (sub == 0) delta[row] = acc;
  }
}

hipError_t launch_bwd_preprocess(int B, int hq, int sq, int d, const void* out, const void* d_o,
                                 Strides qs, int dtype, float* delta, hipStream_t st) {
  const long rows = (long)B * hq * sq;
  if (rows == 0) return hipSuccess;
  const int G = d / 8;
  long blocks = (rows * G + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (dtype == BF16) {
    if (d == 128) bwd_pre_kernel<128, __bf16><<<(unsigned)blocks, 256, 0, st>>>(B, hq, sq, (const __bf16*)out, (const __bf16*)d_o, qs, delta);
    else bwd_pre_kernel<64, __bf16><<<(unsigned)blocks, 256, 0, st>>>(B, hq, sq, (const __bf16*)out, (const __bf16*)d_o, qs, delta);
  } else {
    if (d == 128) bwd_pre_kernel<128, float><<<(unsigned)blocks, 256, 0, st>>>(B, hq, sq, (const float*)out, (const float*)d_o, qs, delta);
    else bwd_pre_kernel<64, float><<<(unsigned)blocks, 256, 0, st>>>(B, hq, sq, (const float*)out, (const float*)d_o, qs, delta);
  }
  return hipGetLastError();
}

}  // namespace ra
