// Forward ring step, bf16 inputs, fp32 accumulation, on gfx950 MFMA.
//
// One workgroup = 4 waves = BM = 128*NB query rows of one (batch, query head);
// it walks the key/value block in tiles of BN = 64 keys, skipping tiles that
// the mask hides entirely (per-tile position/document ranges).  Per tile:
//
//   S^T = K Q^T           v_mfma_f32_32x32x16_bf16, K tile from LDS (A),
//                         the wave's Q rows held in registers (B)
//   mask + online softmax each lane owns whole query columns of S^T, so the
//                         running max/sum need one cross-lane exchange
//   O^T += V^T P^T        V^T from LDS (A); P^T straight from the S^T
//                         accumulator registers (B), converted to bf16
//
// Making the S^T accumulator usable as the P^T operand without a shuffle:
// lane l of a 32x32 MFMA result holds rows {8*(v/4) + 4*(l/32) + v%4}, but
// the K-operand of the next MFMA wants 8 consecutive reduction indices per
// lane.  Loading K row swap23(i) (bits 2 and 3 of the row index swapped) into
// MFMA row i makes lane l's 8 values of each half belong to 8 consecutive
// keys, which is exactly the operand layout; the keys of the V^T operand are
// then read in natural order.
//
// Pipeline: the next tile's K/V are loaded from HBM into registers at the top
// of an iteration and stored into the other half of a double-buffered LDS at
// its bottom, so one barrier per tile orders everything.  Two workgroups fit
// on a CU (<= 256 VGPRs per lane), so one workgroup's softmax overlaps the
// other's MFMAs.
//
// Online softmax with a lazily updated maximum: the running maximum m only
// moves when a tile's maximum exceeds it by more than RESCALE_SLACK (log2
// units), so exp2(s - m) <= 2^RESCALE_SLACK and the accumulator is rescaled
// only on those (rare) tiles; the result is the same up to rounding.
//
// The step's normalised partial (O_t = acc / l, LSE_t = m ln2 + ln l) is
// merged into the running (o_acc, lse) in the epilogue with the exact
// log-sum-exp combine; FIRST overwrites, LAST also writes bf16 `out`.
#include "ra_internal.h"

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int BN = 64;      // keys per tile (== TILE)
constexpr int NWAVES = 4;
constexpr int LIST = 256;   // tile-list chunk (one tile per thread when building it)
constexpr float LN2 = 0.69314718055994530942f;
constexpr float RESCALE_SLACK = 8.0f;

template <int D, int NB>
struct Cfg {
  static constexpr int WQ = 32 * NB;       // query rows per wave
  static constexpr int BM = NWAVES * WQ;   // query rows per workgroup
  static constexpr int KS = D + 8;         // K tile row stride in LDS (elements)
  static constexpr int VS = BN + 8;        // V^T tile row stride in LDS (elements)
  static constexpr int KCH = BN * D / 8 / 256;        // 16-byte K chunks per thread per tile
  static constexpr int NVQ = (BN / 4) * (D / 8);        // 4-key x 8-dim V blocks per tile
  static constexpr int VQ = (NVQ + 255) / 256;          // ... per thread (threads past NVQ idle)
};

__device__ __forceinline__ int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge weights of (lse_a) (+) (lse_b): returns lse, weights of a and b.
__device__ __forceinline__ void lse_combine(float la, float lb, float& lse, float& wa, float& wb) {
  const float mx = fmaxf(la, lb);
  if (mx == -INFINITY) { lse = -INFINITY; wa = 0.f; wb = 0.f; return; }
  const float ea = expf(la - mx), eb = expf(lb - mx);
  const float s = ea + eb;
  lse = mx + logf(s);
  wa = ea / s;
  wb = eb / s;
}

// Workgroup -> (batch, query head, query tile).  Hardware hands consecutive
// workgroup ids to the 8 XCDs round-robin; renumber so that each XCD gets a
// contiguous range of logical ids, ordered [batch][kv head][query tile, latest
// first][query head of the GQA group]: the workgroups sharing an XCD's L2 then
// stream the same K/V tiles at about the same time, and the query tiles that
// see the most keys under a causal mask start first.
__device__ __forceinline__ void map_block(int n_qt, int hq, int hkv, int total, int& b, int& h, int& qt) {
  const int i = blockIdx.x;
  const int per = total / 8, rem = total % 8;
  const int xcd = i % 8, local = i / 8;
  const int logical = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int grp = hq / hkv;
  int r = logical;
  const int hh = r % grp; r /= grp;
  qt = n_qt - 1 - (r % n_qt); r /= n_qt;
  const int kvh = r % hkv;
  b = r / hkv;
  h = kvh * grp + hh;
}

}  // namespace

template <int D, int NB>
__global__ __launch_bounds__(256, NB == 1 ? 2 : 1) void fwd_bf16_kernel(FwdArgs a) {
  using C = Cfg<D, NB>;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][BN * C::KS];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[2][D * C::VS];
  __shared__ __attribute__((aligned(16))) int kvp[2][BN];
  __shared__ __attribute__((aligned(16))) int kvd[2][BN];
  __shared__ int list[LIST];
  __shared__ int wave_cnt[NWAVES];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, j = lane & 31;
  const int n_qt = (a.sq + C::BM - 1) / C::BM;
  int b, h, qt;
  map_block(n_qt, a.hq, a.hkv, n_qt * a.hq * a.B, b, h, qt);
  const int kvh = (h * a.hkv) / a.hq;
  const int q0 = qt * C::BM;
  const int mask = a.mask;

  // Position/document range of this query tile (valid rows only).
  TileRange qr{0x7fffffff, (int)0x80000000, 0x7fffffff, (int)0x80000000};
  {
    const int t_end = min(n_tiles(a.sq), (q0 + C::BM) / TILE);
    for (int t = q0 / TILE; t < t_end; ++t) {
      const TileRange r = a.q_tiles[t];
      qr.min_pos = min(qr.min_pos, r.min_pos); qr.max_pos = max(qr.max_pos, r.max_pos);
      qr.min_doc = min(qr.min_doc, r.min_doc); qr.max_doc = max(qr.max_doc, r.max_doc);
    }
  }

  // This wave's query rows: Q fragments (MFMA B operand) and positions.
  const __bf16* qptr = (const __bf16*)a.q + b * a.qs.b + h * a.qs.h;
  bf16x8 qf[NB][D / 16];
  int qpos[NB], qdoc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = q0 + wave * C::WQ + nb * 32 + j;
    const bool valid = row < a.sq;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      bf16x8 z = {};
      qf[nb][ks] = valid ? *(const bf16x8*)(qptr + row * a.qs.s + ks * 16 + g * 8) : z;
    }
    qpos[nb] = valid ? a.q_pos[row] : -1;
    qdoc[nb] = (valid && mask == MASK_DOC_CAUSAL) ? a.q_doc[row] : 0;
  }

  float m_run[NB], l_run[NB];
  f32x16 acc[NB][D / 32];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[nb][db] = f32x16{};
  }

  const __bf16* kptr = (const __bf16*)a.k + b * a.kvs.b + kvh * a.kvs.h;
  const __bf16* vptr = (const __bf16*)a.v + b * a.kvs.b + kvh * a.kvs.h;
  const int nkt = n_tiles(a.sk);
  const bool no_skip = (a.flags & FLAG_NO_SKIP) != 0;
  const float sl2 = a.scale_log2;

  // register staging of one tile on its way from HBM to LDS
  bf16x8 kreg[C::KCH];
  bf16x8 vreg[C::VQ][4];
  int preg = POS_INVALID, dreg = 0;

  auto load_tile = [&](int kbase) {
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) {
      const int c = tid + 256 * i;
      const int key = c / (D / 8), c8 = c % (D / 8);
      bf16x8 z = {};
      kreg[i] = kbase + key < a.sk ? *(const bf16x8*)(kptr + (kbase + key) * a.kvs.s + c8 * 8) : z;
    }
#pragma unroll
    for (int i = 0; i < C::VQ; ++i) {
      const int qd = tid + 256 * i;
      const int kq = qd % (BN / 4), c8 = qd / (BN / 4);
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int key = kbase + kq * 4 + e4;
        bf16x8 z = {};
        vreg[i][e4] = (qd < C::NVQ && key < a.sk) ? *(const bf16x8*)(vptr + key * a.kvs.s + c8 * 8) : z;
      }
    }
    if (tid < BN) {
      const int key = kbase + tid;
      const bool ok = key < a.sk;
      preg = ok ? a.kv_pos[key] : POS_INVALID;
      dreg = (ok && mask == MASK_DOC_CAUSAL) ? a.kv_doc[key] : 0;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) {
      const int c = tid + 256 * i;
      const int key = c / (D / 8), c8 = c % (D / 8);
      *(bf16x8*)(&Ks[buf][key * C::KS + c8 * 8]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < C::VQ; ++i) {
      const int qd = tid + 256 * i;
      const int kq = qd % (BN / 4), c8 = qd / (BN / 4);
      if (qd >= C::NVQ) break;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 col = {vreg[i][0][e], vreg[i][1][e], vreg[i][2][e], vreg[i][3][e]};
        *(bf16x4*)(&Vt[buf][(c8 * 8 + e) * C::VS + kq * 4]) = col;
      }
    }
    if (tid < BN) {
      kvp[buf][tid] = preg;
      kvd[buf][tid] = dreg;
    }
  };

  for (int c0 = 0; c0 < nkt; c0 += LIST) {
    // ---- compact the non-empty tiles of this chunk into `list` ----
    const int t = c0 + tid;
    int cls = TILE_EMPTY;
    if (t < nkt) {
      cls = classify(qr, a.kv_tiles[t], (t + 1) * TILE <= a.sk, mask);
      if (no_skip && cls == TILE_EMPTY) cls = TILE_PARTIAL;
    }
    const unsigned long long bal = __ballot(cls != TILE_EMPTY);
    const int my = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int off = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) {
      const int c = wave_cnt[w];
      off += (w < wave) ? c : 0;
      total += c;
    }
    if (cls != TILE_EMPTY) list[off + my] = t | (cls << 24);
    __syncthreads();
    if (total == 0) continue;

    load_tile((list[0] & 0xffffff) * BN);
    store_tile(0);
    __syncthreads();

    for (int li = 0; li < total; ++li) {
      const int buf = li & 1;
      const int ent = list[li];
      const bool partial = (ent >> 24) == TILE_PARTIAL;
      const bool more = li + 1 < total;
      if (more) load_tile((list[li + 1] & 0xffffff) * BN);

      // ---- S^T = K Q^T (raw scores) ----
      f32x16 s[2][NB];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[mb][nb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 kf = *(const bf16x8*)(&Ks[buf][(mb * 32 + swap23(j)) * C::KS + ks * 16 + g * 8]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            s[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[nb][ks], s[mb][nb], 0, 0, 0);
        }
      }

      // ---- mask, online softmax ----
      // lane (g, j), value v of block mb holds key mb*32 + 16*(v/8) + 8*g + v%8 for query j.
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (partial) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int base = mb * 32 + 16 * hh + 8 * g;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const int kp = kvp[buf][base + e];
                bool ok = kp != POS_INVALID;
                if (mask != MASK_NONE) ok = ok && kp <= qpos[nb];
                if (mask == MASK_DOC_CAUSAL) ok = ok && kvd[buf][base + e] == qdoc[nb];
                if (!ok) s[mb][nb][hh * 8 + e] = -INFINITY;
              }
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[mb][nb][v]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt = mx * sl2;   // tile maximum, scaled log2 units (-inf stays -inf)
        // move the running maximum only when this tile would overflow the slack
        const bool grow = mt > m_run[nb] + RESCALE_SLACK;
        if (__any(grow)) {
          // lanes that do not grow keep their maximum (alpha = 1; their m may still be -inf)
          const float alpha = grow ? fast_exp2(m_run[nb] - mt) : 1.f;   // 0 when growing from -inf
          m_run[nb] = grow ? mt : m_run[nb];
          l_run[nb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) acc[nb][db] *= alpha;
        }
        const float m_use = m_run[nb] == -INFINITY ? 0.f : m_run[nb];
        float rs = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float p = fast_exp2(__builtin_fmaf(s[mb][nb][v], sl2, -m_use));
            s[mb][nb][v] = p;
            rs += p;
          }
        l_run[nb] += rs;
      }

      // ---- O^T += V^T P^T ----
      bf16x8 pf[NB][4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[nb][kk][e] = (__bf16)s[kk >> 1][nb][(kk & 1) * 8 + e];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 vf = *(const bf16x8*)(&Vt[buf][(db * 32 + j) * C::VS + kk * 16 + g * 8]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[nb][kk], acc[nb][db], 0, 0, 0);
        }
      }
      if (more) store_tile(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: normalise, merge into (o_acc, lse), optionally write out ----
  const bool first = (a.flags & FLAG_FIRST) != 0;
  const bool last = (a.flags & FLAG_LAST) != 0 && a.out != nullptr;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float l_tot = l_run[nb] + __shfl_xor(l_run[nb], 32);
    const int row = q0 + wave * C::WQ + nb * 32 + j;
    if (row >= a.sq) continue;
    const float lse_t = l_tot > 0.f ? (m_run[nb] + log2f(l_tot)) * LN2 : -INFINITY;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const size_t orow = ((size_t)b * a.hq + h) * a.sq + row;
    float lse_new = lse_t, w_p = 0.f, w_t = inv;
    if (!first) {
      float wp, wt;
      lse_combine(a.lse[orow], lse_t, lse_new, wp, wt);
      w_p = wp;
      w_t = wt * inv;
    }
    float* op = a.o_acc + orow * D;
    __bf16* outp = last ? (__bf16*)a.out + b * a.qs.b + h * a.qs.h + row * a.qs.s : nullptr;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int vh = 0; vh < 4; ++vh) {
        const int d = db * 32 + vh * 8 + g * 4;
        f32x4 o = {acc[nb][db][vh * 4 + 0] * w_t, acc[nb][db][vh * 4 + 1] * w_t,
                   acc[nb][db][vh * 4 + 2] * w_t, acc[nb][db][vh * 4 + 3] * w_t};
        if (!first) o += w_p * *(const f32x4*)(op + d);
        *(f32x4*)(op + d) = o;
        if (last) {
          bf16x4 ob = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
          *(bf16x4*)(outp + d) = ob;
        }
      }
    }
    if (g == 0) a.lse[orow] = lse_new;
  }
}

#ifndef RA_FWD_NB
#define RA_FWD_NB 1
#endif

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t st) {
  constexpr int NB = RA_FWD_NB;
  const int bm = NWAVES * 32 * NB;
  const long blocks = (long)((a.sq + bm - 1) / bm) * a.hq * a.B;
  if (blocks == 0) return hipSuccess;
  if (d == 128) fwd_bf16_kernel<128, NB><<<(unsigned)blocks, 256, 0, st>>>(a);
  else fwd_bf16_kernel<64, NB><<<(unsigned)blocks, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace ra
