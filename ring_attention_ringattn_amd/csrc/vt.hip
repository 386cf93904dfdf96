// Transposed copy of a value block for the bf16 forward kernel.
//
// The forward step contracts P with V over the keys (O^T += V^T P^T).  With V
// stored key-major, the MFMA operand (8 consecutive keys of one head
// dimension per lane) is a column of the tile and needs transpose reads from
// LDS; with V^T (dimension-major) it is a plain 16-byte row read, which the
// LDS serves faster.  A block is transposed once, before the steps that use
// it: V [B][Hkv][Sk][D] (any strides) -> VT [B][Hkv][D][SkP] dense bf16 with
// SkP = Sk rounded up to whole 64-key tiles and zeros in the padding.
#include "ra_internal.h"

namespace ra {

namespace {
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
}

// One workgroup per (64-key tile, kv head, batch): the tile goes through LDS
// so that both the reads (16 B of one key) and the writes (16 B of one head
// dimension) are contiguous.
template <int D>
__global__ __launch_bounds__(256) void vt_transpose_kernel(const __bf16* __restrict__ v, Strides s, int hkv, int sk,
                                                           int skp, __bf16* __restrict__ vt) {
  __shared__ __bf16 t[64][D + 8];   // + 16 B per row against bank conflicts
  const int kb = blockIdx.x * 64, h = blockIdx.y, b = blockIdx.z;
  const __bf16* src = v + b * s.b + h * s.h;
  for (int idx = threadIdx.x; idx < 64 * (D / 8); idx += 256) {
    const int k = idx / (D / 8), c = (idx % (D / 8)) * 8;
    bf16x8v x = {};
    if (kb + k < sk) x = *(const bf16x8v*)(src + (size_t)(kb + k) * s.s + c);
    *(bf16x8v*)&t[k][c] = x;
  }
  __syncthreads();
  __bf16* dst = vt + ((size_t)b * hkv + h) * D * skp + kb;
  for (int idx = threadIdx.x; idx < D * 8; idx += 256) {
    const int d = idx / 8, k8 = (idx % 8) * 8;
    bf16x8v y;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = t[k8 + e][d];
    *(bf16x8v*)(dst + (size_t)d * skp + k8) = y;
  }
}

hipError_t launch_vt_transpose(const void* v, Strides s, int B, int hkv, int sk, int d, void* vt, hipStream_t st) {
  const int skp = vt_keys(sk);
  if (skp == 0) return hipSuccess;
  const dim3 grid(skp / 64, hkv, B);
  if (d == 128)
    vt_transpose_kernel<128><<<grid, 256, 0, st>>>((const __bf16*)v, s, hkv, sk, skp, (__bf16*)vt);
  else
    vt_transpose_kernel<64><<<grid, 256, 0, st>>>((const __bf16*)v, s, hkv, sk, skp, (__bf16*)vt);
  return hipGetLastError();
}

}  // namespace ra
