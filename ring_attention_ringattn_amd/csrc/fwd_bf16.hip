// Forward ring step, bf16 inputs, fp32 accumulation, on gfx950 MFMA.
//
// One workgroup = 4 waves = BM = 128 query rows of one (batch, query head);
// it walks the key/value block in tiles of BN = 64 keys, skipping tiles that
// the mask hides entirely (per-tile position/document ranges).  Per tile:
//
//   S^T = K Q^T           v_mfma_f32_32x32x16_bf16, K tile from LDS (A),
//                         the wave's Q rows held in registers (B)
//   mask + online softmax each lane owns whole query columns of S^T, so the
//                         running max/sum need one cross-lane exchange
//   O^T += V^T P^T        V^T read from the row-major V tile with the LDS
//                         transpose read (A); P^T straight from the S^T
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
// Data movement: K and V tiles go from HBM straight into LDS with buffer
// loads (no register staging; the buffer range zero-fills keys past the end
// of the block), double-buffered so the next tile streams in during the
// current one's MFMAs; one barrier per tile.  Tiles are row-major and
// swizzled (mfma_tile.h) so the K operand reads and the V transpose reads
// are free of bank conflicts.
// Two workgroups fit on a CU, so one workgroup's softmax overlaps the other's
// MFMAs.
//
// Online softmax with a lazily updated maximum: the running maximum m only
// moves when a tile's maximum exceeds it by more than RESCALE_SLACK (log2
// units), so exp2(s - m) <= 2^RESCALE_SLACK and the accumulator is rescaled
// only on those (rare) tiles; the result is the same up to rounding.  The
// row sum is accumulated in fp32.
//
// The step's normalised partial (O_t = acc / l, LSE_t = m ln2 + ln l) is
// merged into the running (o_acc, lse) in the epilogue with the exact
// log-sum-exp combine; FIRST overwrites, LAST also writes bf16 `out`.
#include "mfma_tile.h"

namespace ra {

namespace {

constexpr int BN = 64;      // keys per tile (== TILE)
constexpr int NWAVES = 4;
constexpr int BM = NWAVES * 32;   // query rows per workgroup (32 per wave)
constexpr int LIST = 256;   // tile-list chunk (one tile per thread when building it)
constexpr float RESCALE_SLACK = 8.0f;

template <int D>
struct Cfg {
  static constexpr int CHUNKS = BN * D * 2 / 1024;   // 1 KB buffer->LDS chunks per tile
  static constexpr int CPW = CHUNKS / NWAVES;        // ... per wave
};

// Workgroup -> (batch, query head, query tile).  Hardware hands consecutive
// workgroup ids to the 8 XCDs round-robin; renumber so that each XCD gets a
// contiguous range of logical ids, ordered [batch][kv head][query tile, latest
// first][query head of the GQA group]: the workgroups sharing an XCD's L2 then
// stream the same K/V tiles at about the same time, and the query tiles that
// see the most keys under a causal mask start first.
__device__ __forceinline__ void map_block(int n_qt, int hq, int hkv, int total, int& b, int& h, int& qt) {
  const int grp = hq / hkv;
  int r = xcd_logical(blockIdx.x, total);
  const int hh = r % grp; r /= grp;
  qt = n_qt - 1 - (r % n_qt); r /= n_qt;
  const int kvh = r % hkv;
  b = r / hkv;
  h = kvh * grp + hh;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdArgs a) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(1024))) __bf16 Ks[2][BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 Vs[2][BN * D];
  __shared__ __attribute__((aligned(16))) int kvp[2][BN];
  __shared__ __attribute__((aligned(16))) int kvd[2][BN];
  __shared__ int list[LIST + 1];   // + sentinel
  __shared__ int wave_cnt[NWAVES];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, j = lane & 31;
  const int n_qt = (a.sq + BM - 1) / BM;
  int b, h, qt;
  map_block(n_qt, a.hq, a.hkv, n_qt * a.hq * a.B, b, h, qt);
  const int kvh = (h * a.hkv) / a.hq;
  const int q0 = qt * BM;
  const int mask = a.mask;

  // Position/document range of this query tile (valid rows only).
  TileRange qr{0x7fffffff, (int)0x80000000, 0x7fffffff, (int)0x80000000};
  {
    const int t_end = min(n_tiles(a.sq), (q0 + BM) / TILE);
    for (int t = q0 / TILE; t < t_end; ++t) {
      const TileRange r = a.q_tiles[t];
      qr.min_pos = min(qr.min_pos, r.min_pos); qr.max_pos = max(qr.max_pos, r.max_pos);
      qr.min_doc = min(qr.min_doc, r.min_doc); qr.max_doc = max(qr.max_doc, r.max_doc);
    }
  }

  // This wave's 32 query rows: Q fragments (MFMA B operand) and positions.
  const __bf16* qptr = (const __bf16*)a.q + b * a.qs.b + h * a.qs.h;
  const int qrow = q0 + wave * 32 + j;
  const bool qvalid = qrow < a.sq;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    bf16x8 z = {};
    qf[ks] = qvalid ? *(const bf16x8*)(qptr + qrow * a.qs.s + ks * 16 + g * 8) : z;
  }
  const int qpos = qvalid ? a.q_pos[qrow] : -1;
  const int qdoc = (qvalid && mask == MASK_DOC_CAUSAL) ? a.q_doc[qrow] : 0;

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  const __bf16* kptr = (const __bf16*)a.k + b * a.kvs.b + kvh * a.kvs.h;
  const __bf16* vptr = (const __bf16*)a.v + b * a.kvs.b + kvh * a.kvs.h;
  const int rsb = (int)(a.kvs.s * 2);   // bytes between consecutive keys
  const int nkt = n_tiles(a.sk);
  const bool no_skip = (a.flags & FLAG_NO_SKIP) != 0;
  const float sl2 = a.scale_log2;

  // Per-lane byte offsets (within a tile) of this lane's 16-byte unit of each
  // of the wave's CPW buffer->LDS chunks: chunk q = c*4 + wave covers LDS
  // units [64q, 64q+64); unit p holds row p/U, logical column (p%U) ^ swz(row).
  int voff[C::CPW];
#pragma unroll
  for (int c = 0; c < C::CPW; ++c) voff[c] = chunk_voff<D>(c * NWAVES + wave, lane, rsb);
  int preg = POS_INVALID, dreg = 0;

  // Start streaming tile `tile` into LDS buffer `buf`.
  auto issue_tile = [&] __device__(int tile, int buf) {
    const int kbase = tile * BN;
    const int rows = min(BN, a.sk - kbase);
    const __bf16* kb = kptr + (size_t)kbase * a.kvs.s;
    const __bf16* vb = vptr + (size_t)kbase * a.kvs.s;
#pragma unroll
    for (int c = 0; c < C::CPW; ++c) {
      const int q = c * NWAVES + wave;
      dma16(kb, rows * rsb, (RA_LDS void*)&Ks[buf][q * 512], voff[c]);
      dma16(vb, rows * rsb, (RA_LDS void*)&Vs[buf][q * 512], voff[c]);
    }
    if (tid < BN) {
      const int key = kbase + tid;
      const bool ok = key < a.sk;
      preg = ok ? a.kv_pos[key] : POS_INVALID;
      dreg = (ok && mask == MASK_DOC_CAUSAL) ? a.kv_doc[key] : 0;
    }
  };
  auto finish_tile = [&] __device__(int buf) {
    if (tid < BN) {
      kvp[buf][tid] = preg;
      kvd[buf][tid] = dreg;
    }
    wait_vmem();   // this thread's buffer->LDS loads have landed
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
    if (tid == 0) list[total] = 0;   // read (and ignored) by the look-ahead past the last entry
    __syncthreads();
    if (total == 0) continue;

    // list entries are workgroup-uniform: keep them scalar so the branches on them stay branches
    int ent = __builtin_amdgcn_readfirstlane(list[0]);
    issue_tile(ent & 0xffffff, 0);
    finish_tile(0);
    __syncthreads();

    for (int li = 0; li < total; ++li) {
      const int buf = li & 1;
      const bool partial = (ent >> 24) == TILE_PARTIAL;
      const int kvalid = a.sk - (ent & 0xffffff) * BN;   // keys of this tile that exist (>= BN: all)
      const bool more = li + 1 < total;
      const int ent_next = __builtin_amdgcn_readfirstlane(list[li + 1]);
      if (more) issue_tile(ent_next & 0xffffff, buf ^ 1);

      // ---- S^T = K Q^T (raw scores) ----
      f32x16 s[2];
      s[0] = f32x16{};
      s[1] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 kf = *(const bf16x8*)(&Ks[buf][tile_off<D>(mb * 32 + swap23(j), ks * 16 + g * 8)]);
          s[mb] = mfma(kf, qf[ks], s[mb]);
        }
      }

      // ---- mask (partial tiles only), online softmax ----
      // lane (g, j), value v of block mb holds key mb*32 + 16*(v/8) + 8*g + v%8 for query j.
      if (partial) {
        asm volatile("" ::: "memory");   // keep this a real branch: full tiles must not pay for masking
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int base = mb * 32 + 16 * hh + 8 * g;
            const i32x4 p0 = *(const i32x4*)&kvp[buf][base], p1 = *(const i32x4*)&kvp[buf][base + 4];
            const i32x4 d0 = *(const i32x4*)&kvd[buf][base], d1 = *(const i32x4*)&kvd[buf][base + 4];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int kp = e < 4 ? p0[e] : p1[e - 4];
              const int kd = e < 4 ? d0[e] : d1[e - 4];
              bool ok = base + e < kvalid;
              if (mask != MASK_NONE) ok = ok && kp <= qpos;
              if (mask == MASK_DOC_CAUSAL) ok = ok && kd == qdoc;
              s[mb][hh * 8 + e] = ok ? s[mb][hh * 8 + e] : -INFINITY;
            }
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[mb][v]);
      const float mt = pair_max(mx) * sl2;   // tile maximum, scaled log2 units (-inf stays -inf)
      // move the running maximum only when this tile would overflow the slack
      const bool grow = mt > m_run + RESCALE_SLACK;
      if (__any(grow)) {
        // lanes that do not grow keep their maximum (alpha = 1; their m may still be -inf)
        const float alpha = grow ? fast_exp2(m_run - mt) : 1.f;   // 0 when growing from -inf
        m_run = grow ? mt : m_run;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
      }
      const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
      // probabilities: fp32 for the row sum (the LSE needs it; a sum of the bf16-rounded
      // values would be off by up to 2^-9 relative), bf16 for the PV product
      bf16x8 pf[4];
      float rs = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(__builtin_fmaf(s[kk >> 1][(kk & 1) * 8 + e], sl2, neg_m));
          rs += p;
          pf[kk][e] = (__bf16)p;
        }
      l_run += rs;

      // ---- O^T += V^T P^T, V^T from the row-major tile by transpose reads ----
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] = mfma(tr_operand<D>(Vs[buf], kk * 16, db * 32, lane), pf[kk], acc[db]);
      if (more) finish_tile(buf ^ 1);
      ent = ent_next;
      __syncthreads();
    }
  }

  // ---- epilogue: normalise, merge into (o_acc, lse), optionally write out ----
  const bool first = (a.flags & FLAG_FIRST) != 0;
  const bool last = (a.flags & FLAG_LAST) != 0 && a.out != nullptr;
  const float l_tot = pair_sum(l_run);
  if (!qvalid) return;
  const float lse_t = l_tot > 0.f ? (m_run + log2f(l_tot)) * LN2F : -INFINITY;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const size_t orow = ((size_t)b * a.hq + h) * a.sq + qrow;
  float lse_new = lse_t, w_p = 0.f, w_t = inv;
  if (!first) {
    float wp, wt;
    lse_combine(a.lse[orow], lse_t, lse_new, wp, wt);
    w_p = wp;
    w_t = wt * inv;
  }
  float* op = a.o_acc + orow * D;
  __bf16* outp = last ? (__bf16*)a.out + b * a.qs.b + h * a.qs.h + qrow * a.qs.s : nullptr;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int vh = 0; vh < 4; ++vh) {
      const int d = db * 32 + vh * 8 + g * 4;
      f32x4 o = {acc[db][vh * 4 + 0] * w_t, acc[db][vh * 4 + 1] * w_t, acc[db][vh * 4 + 2] * w_t,
                 acc[db][vh * 4 + 3] * w_t};
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

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t st) {
  const long blocks = (long)((a.sq + BM - 1) / BM) * a.hq * a.B;
  if (blocks == 0) return hipSuccess;
  if (d == 128) fwd_bf16_kernel<128><<<(unsigned)blocks, 256, 0, st>>>(a);
  else fwd_bf16_kernel<64><<<(unsigned)blocks, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace ra
