// fp32 ring-step kernels (forward and backward).
//
// The fp32 problems of this library are small (launch-latency bound), so
// these kernels favour plainness: one wave per row and exact expf/logf.  The
// forward spreads the 64 keys of a tile over the lanes for the scores (each
// lane one key's dot product), then the head dimension over the lanes for the
// P V product (each key's probability read from its lane); the backward kernels
// spread the head dimension over the lanes (1 or 2 elements per lane) and reduce
// dot products across the wave.  Key tiles whose whole range the mask hides are
// skipped with the same per-tile ranges as the bf16 kernels.
#include "ra_internal.h"

namespace ra {

namespace {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ bool visible(int mask, int kp, int kd, int qp, int qd) {
  if (mask == MASK_NONE) return true;
  if (kp > qp) return false;
  return mask != MASK_DOC_CAUSAL || kd == qd;
}

__device__ __forceinline__ void combine(float la, float lb, float& lse, float& wa, float& wb) {
  const float mx = fmaxf(la, lb);
  if (mx == -INFINITY) { lse = -INFINITY; wa = 0.f; wb = 0.f; return; }
  const float ea = expf(la - mx), eb = expf(lb - mx);
  lse = mx + logf(ea + eb);
  wa = ea / (ea + eb);
  wb = eb / (ea + eb);
}

}  // namespace

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Forward: one wave per (b, h, query row); online softmax over 64-key tiles.
template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdArgs a) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const long wid = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const long rows = (long)a.B * a.hq * a.sq;
  if (wid >= rows) return;
  const int row = wid % a.sq;
  const int h = (wid / a.sq) % a.hq;
  const int b = wid / ((long)a.sq * a.hq);
  const int kvh = (h * a.hkv) / a.hq;
  const float* q = (const float*)a.q + b * a.qs.b + h * a.qs.h + (size_t)row * a.qs.s;
  const float* kb = (const float*)a.k + b * a.kvs.b + kvh * a.kvs.h;
  const float* vb = (const float*)a.v + b * a.kvs.b + kvh * a.kvs.h;
  float qr[D];   // the query row, in every lane
#pragma unroll
  for (int d = 0; d < D; ++d) qr[d] = q[d];
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  const int qp = a.q_pos[row];
  const int qd = a.mask == MASK_DOC_CAUSAL ? a.q_doc[row] : 0;
  const TileRange me{qp, qp, qd, qd};
  float m = -INFINITY, l = 0.f;
  const int nkt = n_tiles(a.sk);
  for (int t = 0; t < nkt; ++t) {
    if (!(a.flags & FLAG_NO_SKIP) && classify(me, a.kv_tiles[t], true, a.mask) == TILE_EMPTY) continue;
    // A whole tile's V rows (lane (+ 64 e): head dimension lane + 64 e) are loaded here,
    // together with the K rows of the scores: they do not depend on the scores, and loads
    // issued together take one memory round trip instead of one each.
    const int kn = min(TILE, a.sk - t * TILE);
    const float* vr = vb + (size_t)t * TILE * a.kvs.s + lane;
    float vt[TILE][PER];
    if (kn == TILE) {
#pragma unroll
      for (int k = 0; k < TILE; ++k)
#pragma unroll
        for (int e = 0; e < PER; ++e) vt[k][e] = vr[(size_t)k * a.kvs.s + 64 * e];
    }
    // scores: lane k takes key t*TILE + k
    const int key = t * TILE + lane;
    bool vis = key < a.sk;
    float s = -INFINITY;
    if (vis) {
      const int kd = a.mask == MASK_DOC_CAUSAL ? a.kv_doc[key] : 0;
      vis = visible(a.mask, a.kv_pos[key], kd, qp, qd);
    }
    if (vis) {
      const float* kr = kb + (size_t)key * a.kvs.s;
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot += qr[d] * kr[d];
      s = dot * a.scale;
    }
    const float m_new = fmaxf(m, wave_max(s));
    if (m_new == -INFINITY) continue;      // no visible key so far (uniform)
    const float alpha = expf(m - m_new);   // m = -inf -> 0
    const float p = vis ? expf(s - m_new) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] *= alpha;
    // P V: lane (+ 64 e) takes head dimension lane + 64 e; key k's probability from lane k
    // (a whole tile from the rows loaded above; a partial one with a plain loop)
    if (kn == TILE) {
#pragma unroll
      for (int k = 0; k < TILE; ++k) {
        const float pk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), k));
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += pk * vt[k][e];
      }
    } else {
      for (int k = 0; k < kn; ++k) {
        const float pk = __shfl(p, k);
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += pk * vr[(size_t)k * a.kvs.s + 64 * e];
      }
    }
    m = m_new;
  }
  const float lse_t = l > 0.f ? m + logf(l) : -INFINITY;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const size_t orow = ((size_t)b * a.hq + h) * a.sq + row;
  float lse_new = lse_t, w_p = 0.f, w_t = inv;
  if (!(a.flags & FLAG_FIRST)) {
    float wp, wt;
    combine(a.lse[orow], lse_t, lse_new, wp, wt);
    w_p = wp;
    w_t = wt * inv;
  }
  float* op = a.o_acc + orow * D;
  float* outp = (a.flags & FLAG_LAST) && a.out ? (float*)a.out + b * a.qs.b + h * a.qs.h + (size_t)row * a.qs.s : nullptr;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    float o = acc[e] * w_t;
    if (!(a.flags & FLAG_FIRST)) o += w_p * op[lane + 64 * e];
    op[lane + 64 * e] = o;
    if (outp) outp[lane + 64 * e] = o;
  }
  if (lane == 0) a.lse[orow] = lse_new;
}

hipError_t launch_fwd_f32(const FwdArgs& a, int d, hipStream_t st) {
  const long rows = (long)a.B * a.hq * a.sq;
  if (rows == 0) return hipSuccess;
  const long blocks = (rows + 3) / 4;
  if (d == 128) fwd_f32_kernel<128><<<(unsigned)blocks, 256, 0, st>>>(a);
  else fwd_f32_kernel<64><<<(unsigned)blocks, 256, 0, st>>>(a);
  return hipGetLastError();
}

// Backward dQ: one wave per (b, h, query row).
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(BwdArgs a) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const long wid = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const long rows = (long)a.B * a.hq * a.sq;
  if (wid >= rows) return;
  const int row = wid % a.sq;
  const int h = (wid / a.sq) % a.hq;
  const int b = wid / ((long)a.sq * a.hq);
  const int kvh = (h * a.hkv) / a.hq;
  const size_t qoff = b * a.qs.b + h * a.qs.h + row * a.qs.s;
  const float* kb = (const float*)a.k + b * a.kvs.b + kvh * a.kvs.h;
  const float* vb = (const float*)a.v + b * a.kvs.b + kvh * a.kvs.h;
  float qv[PER], dov[PER], dq[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    qv[e] = ((const float*)a.q)[qoff + lane + 64 * e];
    dov[e] = ((const float*)a.d_o)[qoff + lane + 64 * e];
    dq[e] = 0.f;
  }
  const size_t orow = ((size_t)b * a.hq + h) * a.sq + row;
  const float lse = a.lse[orow], delta = a.delta[orow];
  const int qp = a.q_pos[row];
  const int qd = a.mask == MASK_DOC_CAUSAL ? a.q_doc[row] : 0;
  const TileRange me{qp, qp, qd, qd};
  const int nkt = n_tiles(a.sk);
  if (lse != -INFINITY) {
    for (int t = 0; t < nkt; ++t) {
      if (!(a.flags & FLAG_NO_SKIP) && classify(me, a.kv_tiles[t], true, a.mask) == TILE_EMPTY) continue;
      const int kend = min(a.sk, (t + 1) * TILE);
      for (int key = t * TILE; key < kend; ++key) {
        const int kp = a.kv_pos[key];
        const int kd = a.mask == MASK_DOC_CAUSAL ? a.kv_doc[key] : 0;
        if (!visible(a.mask, kp, kd, qp, qd)) continue;
        float ps = 0.f, pd = 0.f, kk[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          kk[e] = kb[key * a.kvs.s + lane + 64 * e];
          ps += qv[e] * kk[e];
          pd += dov[e] * vb[key * a.kvs.s + lane + 64 * e];
        }
        const float s = wave_sum(ps) * a.scale;
        const float dp = wave_sum(pd);
        const float p = expf(s - lse);
        const float ds = p * (dp - delta);
#pragma unroll
        for (int e = 0; e < PER; ++e) dq[e] += ds * a.scale * kk[e];
      }
    }
  }
  float* dqp = a.dq + orow * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) dqp[lane + 64 * e] += dq[e];
}

// Backward dK/dV: one wave per (b, kv head, key); loops over the group's query heads and rows.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(BwdArgs a) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const long wid = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const long keys = (long)a.B * a.hkv * a.sk;
  if (wid >= keys) return;
  const int key = wid % a.sk;
  const int kvh = (wid / a.sk) % a.hkv;
  const int b = wid / ((long)a.sk * a.hkv);
  const size_t koff = b * a.kvs.b + kvh * a.kvs.h + key * a.kvs.s;
  float kv[PER], vv[PER], dk[PER], dv[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    kv[e] = ((const float*)a.k)[koff + lane + 64 * e];
    vv[e] = ((const float*)a.v)[koff + lane + 64 * e];
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  const int kp = a.kv_pos[key];
  const int kd = a.mask == MASK_DOC_CAUSAL ? a.kv_doc[key] : 0;
  const TileRange me{kp, kp, kd, kd};
  const int group = a.hq / a.hkv;
  const int nqt = n_tiles(a.sq);
  for (int hh = 0; hh < group; ++hh) {
    const int h = kvh * group + hh;
    for (int t = 0; t < nqt; ++t) {
      // skip a query tile that cannot see this key
      const TileRange qr = a.q_tiles[t];
      if (!(a.flags & FLAG_NO_SKIP) && classify(qr, me, true, a.mask) == TILE_EMPTY) continue;
      const int qend = min(a.sq, (t + 1) * TILE);
      for (int row = t * TILE; row < qend; ++row) {
        const int qp = a.q_pos[row];
        const int qd = a.mask == MASK_DOC_CAUSAL ? a.q_doc[row] : 0;
        if (!visible(a.mask, kp, kd, qp, qd)) continue;
        const size_t orow = ((size_t)b * a.hq + h) * a.sq + row;
        const float lse = a.lse[orow];
        if (lse == -INFINITY) continue;
        const size_t qoff = b * a.qs.b + h * a.qs.h + row * a.qs.s;
        float ps = 0.f, pd = 0.f, qq[PER], dd[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          qq[e] = ((const float*)a.q)[qoff + lane + 64 * e];
          dd[e] = ((const float*)a.d_o)[qoff + lane + 64 * e];
          ps += qq[e] * kv[e];
          pd += dd[e] * vv[e];
        }
        const float s = wave_sum(ps) * a.scale;
        const float dp = wave_sum(pd);
        const float p = expf(s - lse);
        const float ds = p * (dp - a.delta[orow]);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          dv[e] += p * dd[e];
          dk[e] += ds * a.scale * qq[e];
        }
      }
    }
  }
  const size_t doff = (((size_t)b * a.hkv + kvh) * a.sk + key) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    a.dk[doff + lane + 64 * e] += dk[e];
    a.dv[doff + lane + 64 * e] += dv[e];
  }
}

hipError_t launch_bwd_f32(const BwdArgs& a, int d, hipStream_t st) {
  const long rows = (long)a.B * a.hq * a.sq;
  const long keys = (long)a.B * a.hkv * a.sk;
  if (rows > 0 && a.sk > 0) {
    if (d == 128) bwd_dq_f32_kernel<128><<<(unsigned)((rows + 3) / 4), 256, 0, st>>>(a);
    else bwd_dq_f32_kernel<64><<<(unsigned)((rows + 3) / 4), 256, 0, st>>>(a);
  }
  if (keys > 0 && a.sq > 0) {
    if (d == 128) bwd_dkdv_f32_kernel<128><<<(unsigned)((keys + 3) / 4), 256, 0, st>>>(a);
    else bwd_dkdv_f32_kernel<64><<<(unsigned)((keys + 3) / 4), 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace ra
