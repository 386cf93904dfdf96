// Backward ring step, bf16 inputs, fp32 accumulation, on gfx950 MFMA.
//
// The attention weights are recomputed from the final LSE (no merge is
// needed in the backward: P = exp(s - LSE) is already the globally
// normalised weight), with the loss L = sum(O * dO):
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - delta),  dQ = scale dS K,
//   dK = scale dS^T Q,          delta = rowsum(dO * O).
// Two kernels, so that every output has one writer (deterministic, no
// atomics):
//
// bwd_dkdv_kernel: a workgroup of 8 waves owns 128 keys of one kv head, whose
//   K and V rows it stages once in LDS, and streams the GQA group's query tiles
//   (64 rows of Q, dO, LSE, delta, positions) through double-buffered swizzled
//   LDS.  Wave w takes keys 32 (w % 4) .. +32 and rows 32 (w / 4) .. +32 of
//   every tile, so two waves share each key group and each SIMD runs two waves.
//   Per wave and tile:
//     S  = Q K^T, dP = dO V^T          (Q, dO rows as A operands, loaded in
//                                        swap23 order; K, V rows as B operands)
//     P  = exp2(S c - LSE log2 e), dS = P (dP - delta)
//     dV += P^T dO, dK += dS^T Q       (P, dS straight from registers as A
//                                        operands; dO, Q by transpose reads)
//   then the two halves of each key group are summed through LDS and dk, dv
//   (fp32, owned by this workgroup) += the sums.
//
// bwd_dq_kernel: a workgroup owns 128 query rows of one query head (32 per
//   wave; Q and dO rows in registers as B operands) -- of two query heads of
//   one GQA group when the group size is even (8 waves: the heads see the
//   same keys under the same mask, so each K/V tile is staged once for both)
//   -- and streams 64-key K/V tiles like the forward kernel.  Per tile:
//     S^T = K Q^T, dP^T = V dO^T, P^T, dS^T (as above, transposed)
//     dQ^T += K^T dS^T                  (K^T by transpose reads, dS^T from
//                                        registers)
//   then dq += scale dQ.
// Fully masked tile pairs are skipped in both kernels.
#include "mfma_tile.h"

namespace ra {

namespace {

constexpr int NWAVES = 4;              // dQ kernel
constexpr int BQ = 64;                 // query rows per staged tile (dK/dV kernel)
constexpr int BK = 128;                // keys per workgroup (dK/dV kernel)
constexpr int BKT = 64;                // keys per staged tile (dQ kernel)
constexpr int BMQ = NWAVES * 32;       // query rows per workgroup (dQ kernel)
constexpr int LIST = 256;

// Compact the indices i in [c0, c0 + NW * 64) with cls(i) != EMPTY into `list`
// (entries i | cls << 24); returns their number.  All NW * 64 threads must call it.
template <int NW, typename F>
__device__ __forceinline__ int build_list(int c0, int n, F cls_of, int* list, int* wave_cnt) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = c0 + tid;
  const int cls = i < n ? cls_of(i) : TILE_EMPTY;
  const unsigned long long bal = __ballot(cls != TILE_EMPTY);
  const int my = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) wave_cnt[wave] = __popcll(bal);
  __syncthreads();
  int off = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = wave_cnt[w];
    off += (w < wave) ? c : 0;
    total += c;
  }
  if (cls != TILE_EMPTY) list[off + my] = i | (cls << 24);
  __syncthreads();
  return total;
}

}  // namespace

// ------------------------------------------------------------------ dK / dV
// A workgroup of 8 waves owns 128 keys of one kv head, held in LDS (K and V
// are read as MFMA B operands from there); wave w takes keys 32 (w % 4) ..
// +32 and, of every streamed 64-row query tile, rows 32 (w / 4) .. +32.  So
// two waves share each key group and every SIMD runs two waves, one of which
// can issue products while the other computes exponentials or waits for LDS.
// The two partial dK, dV of a key group are summed through LDS at the end.
template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NW = 8;
  constexpr int CPW = BQ * D * 2 / 1024 / NW;     // buffer->LDS chunks per wave per streamed operand
  constexpr int KCPW = BK * D * 2 / 1024 / NW;    // ... of the stationary K (and V) tile
  __shared__ __attribute__((aligned(1024))) __bf16 QO[2][2][BQ * D];   // [buffer][Q, dO]
  __shared__ __attribute__((aligned(1024))) __bf16 KV[2][BK * D];      // [K, V] of the workgroup's keys
  __shared__ __attribute__((aligned(16))) float lse2s[2][BQ];          // LSE log2(e); +inf: row sees nothing
  __shared__ __attribute__((aligned(16))) float dels[2][BQ];
  __shared__ __attribute__((aligned(16))) int qps[2][BQ];
  __shared__ __attribute__((aligned(16))) int qds[2][BQ];
  __shared__ int list[LIST];
  __shared__ int wave_cnt[NW];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, j = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave & 3, mb = wave >> 2;   // key group, row half of each query tile
  const int n_kt = (a.sk + BK - 1) / BK;
  int r = xcd_logical(blockIdx.x, n_kt * a.hkv * a.B);
  const int kt = r % n_kt; r /= n_kt;
  const int kvh = r % a.hkv, b = r / a.hkv;
  const int k0 = kt * BK;
  const int mask = a.mask;
  const int grp = a.hq / a.hkv;

  // key range of the workgroup
  TileRange kr{0x7fffffff, (int)0x80000000, 0x7fffffff, (int)0x80000000};
  for (int t = k0 / TILE; t < min(n_tiles(a.sk), (k0 + BK) / TILE); ++t) {
    const TileRange x = a.kv_tiles[t];
    kr.min_pos = min(kr.min_pos, x.min_pos); kr.max_pos = max(kr.max_pos, x.max_pos);
    kr.min_doc = min(kr.min_doc, x.min_doc); kr.max_doc = max(kr.max_doc, x.max_doc);
  }
  const bool kcomplete = k0 + BK <= a.sk;

  // the workgroup's K and V rows into LDS (rows past the end of the block read as zero)
  const int rsk = (int)(a.kvs.s * 2);
  const int krows = min(BK, a.sk - k0);
  {
    const size_t kbase = b * a.kvs.b + kvh * a.kvs.h + (size_t)k0 * a.kvs.s;
#pragma unroll
    for (int c = 0; c < KCPW; ++c) {
      const int q = c * NW + wave;
      const int vo = chunk_voff<D>(q, lane, rsk);
      dma16((const __bf16*)a.k + kbase, krows * rsk, (RA_LDS void*)&KV[0][q * 512], vo);
      dma16((const __bf16*)a.v + kbase, krows * rsk, (RA_LDS void*)&KV[1][q * 512], vo);
    }
  }
  // this lane's key (lane j of the wave's key group)
  const int key = k0 + kw * 32 + j;
  const bool kvalid = key < a.sk;
  const int kpos = kvalid ? a.kv_pos[key] : POS_INVALID;
  const int kdoc = (kvalid && mask == MASK_DOC_CAUSAL) ? a.kv_doc[key] : 0;

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const int n_qt = n_tiles(a.sq);
  const int rsb = (int)(a.qs.s * 2);
  const float sl2 = a.scale_log2;
  int voff[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) voff[c] = chunk_voff<D>(c * NW + wave, lane, rsb);
  unsigned rraw = 0;
  bool rok = false;

  // stage query tile `item` (= query head in group * n_qt + tile) into buffer `buf`
  auto issue_tile = [&] __device__(int item, int buf) {
    const int hh = item / n_qt, qt = item % n_qt;
    const int h = kvh * grp + hh;
    const int q0 = qt * BQ;
    const int rows = min(BQ, a.sq - q0);
    const size_t base = b * a.qs.b + h * a.qs.h + (size_t)q0 * a.qs.s;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int q = c * NW + wave;
      dma16((const __bf16*)a.q + base, rows * rsb, (RA_LDS void*)&QO[buf][0][q * 512], voff[c]);
      dma16((const __bf16*)a.d_o + base, rows * rsb, (RA_LDS void*)&QO[buf][1][q * 512], voff[c]);
    }
    // per-row values (waves 0-3: LSE, delta, position, document): one unconditional raw
    // 4-byte load per thread, converted by finish_tile (rows past the end reread the last row)
    if (tid < 4 * 64) {
      const int row = tid & 63, part = tid >> 6;
      rok = row < rows;
      const int rr = q0 + min(row, rows - 1);
      const size_t lrow = ((size_t)b * a.hq + h) * a.sq + rr;
      const int* doc = mask == MASK_DOC_CAUSAL ? a.q_doc : a.q_pos;
      const unsigned* src = part == 0 ? (const unsigned*)(a.lse + lrow)
                          : part == 1 ? (const unsigned*)(a.delta + lrow)
                          : part == 2 ? (const unsigned*)(a.q_pos + rr) : (const unsigned*)(doc + rr);
      rraw = *src;
    }
  };
  auto finish_tile = [&] __device__(int buf) {
    wait_vmem();
    if (tid < 4 * 64) {
      const int row = tid & 63, part = tid >> 6;
      const float f = __uint_as_float(rraw);
      const int iv = (int)rraw;
      if (part == 0) lse2s[buf][row] = (rok && f != -INFINITY) ? f * LOG2E : INFINITY;
      else if (part == 1) dels[buf][row] = rok ? f : 0.f;
      else if (part == 2) qps[buf][row] = rok ? iv : -1;
      else qds[buf][row] = (rok && mask == MASK_DOC_CAUSAL) ? iv : 0;
    }
  };

  const int n_items = grp * n_qt;
  const bool no_skip = (a.flags & FLAG_NO_SKIP) != 0;
  int seen = 0;   // query tiles this workgroup processed (uniform)
  for (int c0 = 0; c0 < n_items; c0 += LIST) {
    // list of the non-empty items of this chunk (classified by the first LIST threads)
    const int i = c0 + tid;
    int cls = TILE_EMPTY;
    if (tid < LIST && i < n_items) {
      cls = classify(a.q_tiles[i % n_qt], kr, kcomplete, mask);
      if (no_skip && cls == TILE_EMPTY) cls = TILE_PARTIAL;
    }
    const unsigned long long bal = __ballot(cls != TILE_EMPTY);
    const int my = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int off = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int c = wave_cnt[w];
      off += (w < wave) ? c : 0;
      total += c;
    }
    if (cls != TILE_EMPTY) list[off + my] = i | (cls << 24);
    __syncthreads();
    total = __builtin_amdgcn_readfirstlane(total);
    seen += total;
    if (total == 0) continue;
    issue_tile(__builtin_amdgcn_readfirstlane(list[0]) & 0xffffff, 0);
    finish_tile(0);   // also waits for the stationary K, V loads of the first chunk
    __syncthreads();

    for (int li = 0; li < total; ++li) {
      const int buf = li & 1;
      const int ent = __builtin_amdgcn_readfirstlane(list[li]);
      const bool partial = (ent >> 24) == TILE_PARTIAL;
      const bool more = li + 1 < total;
      if (more) issue_tile(__builtin_amdgcn_readfirstlane(list[li + 1]) & 0xffffff, buf ^ 1);

      f32x16 s = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int off = tile_off<D>(mb * 32 + swap23(j), ks * 16 + g * 8);
        const int koff = tile_off<D>(kw * 32 + j, ks * 16 + g * 8);
        s = mfma(*(const bf16x8*)&QO[buf][0][off], *(const bf16x8*)&KV[0][koff], s);
        dp = mfma(*(const bf16x8*)&QO[buf][1][off], *(const bf16x8*)&KV[1][koff], dp);
      }
      // lane (g, j), value v = hh*8 + e: query row mb*32 + 16*hh + 8*g + e, key j
      bf16x8 pb[2], db_[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int rbase = mb * 32 + 16 * hh + 8 * g;
        const f32x4 l0 = *(const f32x4*)&lse2s[buf][rbase], l1 = *(const f32x4*)&lse2s[buf][rbase + 4];
        const f32x4 d0 = *(const f32x4*)&dels[buf][rbase], d1 = *(const f32x4*)&dels[buf][rbase + 4];
        if (partial) {
          asm volatile("" ::: "memory");   // keep this a real branch
          const i32x4 p0 = *(const i32x4*)&qps[buf][rbase], p1 = *(const i32x4*)&qps[buf][rbase + 4];
          const i32x4 q0 = *(const i32x4*)&qds[buf][rbase], q1 = *(const i32x4*)&qds[buf][rbase + 4];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int qp = e < 4 ? p0[e] : p1[e - 4];
            const int qd = e < 4 ? q0[e] : q1[e - 4];
            bool ok = true;
            if (mask != MASK_NONE) ok = kpos <= qp;
            if (mask == MASK_DOC_CAUSAL) ok = ok && kdoc == qd;
            s[hh * 8 + e] = ok ? s[hh * 8 + e] : -INFINITY;
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float l2 = e < 4 ? l0[e] : l1[e - 4];
          const float de = e < 4 ? d0[e] : d1[e - 4];
          const float p = fast_exp2(__builtin_fmaf(s[hh * 8 + e], sl2, -l2));
          pb[hh][e] = (__bf16)p;
          db_[hh][e] = (__bf16)(p * (dp[hh * 8 + e] - de));
        }
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dv[db] = mfma(pb[hh], tr_operand<D>(QO[buf][1], mb * 32 + 16 * hh, db * 32, lane), dv[db]);
          dk[db] = mfma(db_[hh], tr_operand<D>(QO[buf][0], mb * 32 + 16 * hh, db * 32, lane), dk[db]);
        }
      if (more) finish_tile(buf ^ 1);
      __syncthreads();
    }
  }

  wait_vmem();              // the stationary K, V loads, when no chunk had a visible tile
  if (seen == 0) return;   // nothing visible: dk, dv stay as they are (uniform over the workgroup)
  // Sum the two row halves of each key group through LDS: waves 4-7 hand their dK to
  // waves 0-3 (which write dK), waves 0-3 hand their dV to waves 4-7 (which write dV).
  __syncthreads();
  float* xk = (float*)&QO[0][0][0];   // 4 key groups x D/32 x 16 values x 64 lanes floats
  float* xv = (float*)&KV[0][0];
  // the lane's id and output column again, from the lane id (not held across the loop:
  // registers are scarce)
  const int ln_ = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int g_ = ln_ >> 5, j_ = ln_ & 31;
  auto slot = [&] __device__(int db, int v) { return ((kw * (D / 32) + db) * 16 + v) * 64 + ln_; };
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      if (mb == 1) xk[slot(db, v)] = dk[db][v];
      else xv[slot(db, v)] = dv[db][v];
    }
  __syncthreads();
  // C layout: lane (g, j), value v -> key kw*32 + 8*(v/4) + 4*g + v%4, dim db*32 + j.
  // All of the lane's current values are read before any of them is written back, so the
  // reads are in flight together (one read-modify-write at a time costs a memory round trip
  // each).
  const size_t obase = ((size_t)b * a.hkv + kvh) * a.sk;
  float* dst = mb == 0 ? a.dk : a.dv;
  const float sc = mb == 0 ? a.scale : 1.f;
  float old[16][D / 32];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int kr_ = k0 + kw * 32 + 8 * (v / 4) + 4 * g_ + (v % 4);
    const float* p = dst + (obase + min(kr_, a.sk - 1)) * D;   // keys past the end reread the last key
#pragma unroll
    for (int db = 0; db < D / 32; ++db) old[v][db] = p[db * 32 + j_];
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int kr_ = k0 + kw * 32 + 8 * (v / 4) + 4 * g_ + (v % 4);
    if (kr_ >= a.sk) continue;
    float* p = dst + (obase + kr_) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const float tot = mb == 0 ? dk[db][v] + xk[slot(db, v)] : dv[db][v] + xv[slot(db, v)];
      p[db * 32 + j_] = old[v][db] + sc * tot;
    }
  }
}

// ------------------------------------------------------------------ dQ
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void bwd_dq_kernel(BwdArgs a) {
  constexpr int HPW = NW / 4;   // query heads per workgroup (of one GQA group: same keys, same mask)
  constexpr int LISTN = NW * 64;
  constexpr int CPW = BKT * D * 2 / 1024 / NW;
  __shared__ __attribute__((aligned(1024))) __bf16 Ks[2][BKT * D];
  __shared__ __attribute__((aligned(1024))) __bf16 Vs[2][BKT * D];
  __shared__ __attribute__((aligned(16))) int kvp[2][BKT];
  __shared__ __attribute__((aligned(16))) int kvd[2][BKT];
  __shared__ int list[LISTN];
  __shared__ int wave_cnt[NW];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, j = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the head and row bases stay scalar
  const int n_qt = (a.sq + BMQ - 1) / BMQ;
  const int grp = a.hq / a.hkv;
  int r = xcd_logical(blockIdx.x, n_qt * (a.hq / HPW) * a.B);
  const int hp = r % (grp / HPW); r /= grp / HPW;
  const int qt = n_qt - 1 - (r % n_qt); r /= n_qt;
  const int kvh = r % a.hkv, b = r / a.hkv;
  const int h = kvh * grp + hp * HPW + wave / 4;
  const int q0 = qt * BMQ;
  const int mask = a.mask;

  TileRange qr{0x7fffffff, (int)0x80000000, 0x7fffffff, (int)0x80000000};
  for (int t = q0 / TILE; t < min(n_tiles(a.sq), (q0 + BMQ) / TILE); ++t) {
    const TileRange x = a.q_tiles[t];
    qr.min_pos = min(qr.min_pos, x.min_pos); qr.max_pos = max(qr.max_pos, x.max_pos);
    qr.min_doc = min(qr.min_doc, x.min_doc); qr.max_doc = max(qr.max_doc, x.max_doc);
  }

  // this wave's 32 query rows: Q and dO as MFMA B operands (lane j = row)
  const int qrow = q0 + (wave & 3) * 32 + j;
  const bool qvalid = qrow < a.sq;
  // (loaded once the first tile list with a visible tile exists)
  bf16x8 qf[D / 16], of[D / 16];
  bool q_loaded = false;
  const size_t lrow = ((size_t)b * a.hq + h) * a.sq + qrow;
  float lse2 = INFINITY, delta = 0.f;
  if (qvalid) {
    const float l = a.lse[lrow];
    lse2 = l == -INFINITY ? INFINITY : l * LOG2E;
    delta = a.delta[lrow];
  }
  const int qpos = qvalid ? a.q_pos[qrow] : -1;
  const int qdoc = (qvalid && mask == MASK_DOC_CAUSAL) ? a.q_doc[qrow] : 0;

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};

  const __bf16* kptr = (const __bf16*)a.k + b * a.kvs.b + kvh * a.kvs.h;
  const __bf16* vptr = (const __bf16*)a.v + b * a.kvs.b + kvh * a.kvs.h;
  const int rsb = (int)(a.kvs.s * 2);
  const float sl2 = a.scale_log2;
  int voff[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) voff[c] = chunk_voff<D>(c * NW + wave, lane, rsb);
  int preg = POS_INVALID, dreg = 0;

  auto issue_tile = [&] __device__(int tile, int buf) {
    const int kbase = tile * BKT;
    const int rows = min(BKT, a.sk - kbase);
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int q = c * NW + wave;
      dma16(kptr + (size_t)kbase * a.kvs.s, rows * rsb, (RA_LDS void*)&Ks[buf][q * 512], voff[c]);
      dma16(vptr + (size_t)kbase * a.kvs.s, rows * rsb, (RA_LDS void*)&Vs[buf][q * 512], voff[c]);
    }
    // positions and documents of the tile's keys: unconditional raw loads (keys past the
    // end reread the last key; the mask drops them by index).  Nothing here may depend on
    // the loaded values, else the wait for them would also wait for the tile loads above.
    const int key = kbase + min(tid & (BKT - 1), rows - 1);
    preg = a.kv_pos[key];
    dreg = (mask == MASK_DOC_CAUSAL ? a.kv_doc : a.kv_pos)[key];
  };
  auto finish_tile = [&] __device__(int buf) {
    wait_vmem();
    if (tid < BKT) {
      kvp[buf][tid] = preg;
      kvd[buf][tid] = mask == MASK_DOC_CAUSAL ? dreg : 0;
    }
  };

  const int nkt = n_tiles(a.sk);
  const bool no_skip = (a.flags & FLAG_NO_SKIP) != 0;
  int seen = 0;   // key tiles this workgroup processed (uniform)
  for (int c0 = 0; c0 < nkt; c0 += LISTN) {
    const int total = build_list<NW>(c0, nkt, [&] __device__(int t) {
      int c = classify(qr, a.kv_tiles[t], (t + 1) * TILE <= a.sk, mask);
      return (no_skip && c == TILE_EMPTY) ? (int)TILE_PARTIAL : c;
    }, list, wave_cnt);
    seen += total;
    if (total == 0) continue;
    if (!q_loaded) {
      // the row's address is formed here, not held across the loop (registers are scarce)
      int qr_ = qrow, g_ = g;
      asm volatile("" : "+v"(qr_), "+v"(g_));
      const size_t qoff = b * a.qs.b + h * a.qs.h + (size_t)qr_ * a.qs.s + g_ * 8;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        bf16x8 z = {};
        qf[ks] = qvalid ? *(const bf16x8*)((const __bf16*)a.q + qoff + ks * 16) : z;
        of[ks] = qvalid ? *(const bf16x8*)((const __bf16*)a.d_o + qoff + ks * 16) : z;
      }
      q_loaded = true;
    }
    issue_tile(__builtin_amdgcn_readfirstlane(list[0]) & 0xffffff, 0);
    finish_tile(0);
    __syncthreads();

    for (int li = 0; li < total; ++li) {
      const int buf = li & 1;
      const int ent = __builtin_amdgcn_readfirstlane(list[li]);
      const bool partial = (ent >> 24) == TILE_PARTIAL;
      const int kvalid = a.sk - (ent & 0xffffff) * BKT;
      const bool more = li + 1 < total;
      if (more) issue_tile(__builtin_amdgcn_readfirstlane(list[li + 1]) & 0xffffff, buf ^ 1);

      f32x16 s[2], dp[2];
      s[0] = s[1] = dp[0] = dp[1] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int off = tile_off<D>(mb * 32 + swap23(j), ks * 16 + g * 8);
          s[mb] = mfma(*(const bf16x8*)&Ks[buf][off], qf[ks], s[mb]);
          dp[mb] = mfma(*(const bf16x8*)&Vs[buf][off], of[ks], dp[mb]);
        }
      // lane (g, j), value v = hh*8 + e of block mb: key mb*32 + 16*hh + 8*g + e, query j
      if (partial) {
        asm volatile("" ::: "memory");   // keep this a real branch
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
      bf16x8 dsb[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int v = (kk & 1) * 8 + e;
          const float p = fast_exp2(__builtin_fmaf(s[kk >> 1][v], sl2, -lse2));
          dsb[kk][e] = (__bf16)(p * (dp[kk >> 1][v] - delta));
        }
      // consecutive MFMAs update different accumulators (a dependent MFMA waits for the previous one)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) dq[db] = mfma(tr_operand<D>(Ks[buf], kk * 16, db * 32, lane), dsb[kk], dq[db]);
      if (more) finish_tile(buf ^ 1);
      __syncthreads();
    }
  }

  // this lane's row again, from the lane id (not held across the loop: registers are scarce)
  const int ln_ = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int qr_ = q0 + (wave & 3) * 32 + (ln_ & 31);
  if (qr_ >= a.sq || seen == 0) return;   // seen == 0: nothing visible, dq stays as it is
  // dq += scale dQ; C layout of dQ^T: lane (g, j), value v -> dim db*32 + 8*(v/4) + 4*g + v%4, query j
  float* dqp = a.dq + (((size_t)b * a.hq + h) * a.sq + qr_) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int vh = 0; vh < 4; ++vh) {
      const int d = db * 32 + vh * 8 + (ln_ >> 5) * 4;
      f32x4 o = *(const f32x4*)(dqp + d);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] += a.scale * dq[db][vh * 4 + e];
      *(f32x4*)(dqp + d) = o;
    }
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int d, hipStream_t st) {
  // dQ: two query heads of a GQA group per 8-wave workgroup (their K/V tiles and mask are the same)
  const bool pair = (a.hq / a.hkv) % 2 == 0;
  const long dq_blocks = (long)((a.sq + BMQ - 1) / BMQ) * a.hq * a.B / (pair ? 2 : 1);
  const long kv_blocks = (long)((a.sk + BK - 1) / BK) * a.hkv * a.B;
  if (dq_blocks == 0 || kv_blocks == 0) return hipSuccess;
  if (d == 128) {
    if (pair) bwd_dq_kernel<128, 8><<<(unsigned)dq_blocks, 512, 0, st>>>(a);
    else bwd_dq_kernel<128, 4><<<(unsigned)dq_blocks, 256, 0, st>>>(a);
    bwd_dkdv_kernel<128><<<(unsigned)kv_blocks, 512, 0, st>>>(a);
  } else {
    if (pair) bwd_dq_kernel<64, 8><<<(unsigned)dq_blocks, 512, 0, st>>>(a);
    else bwd_dq_kernel<64, 4><<<(unsigned)dq_blocks, 256, 0, st>>>(a);
    bwd_dkdv_kernel<64><<<(unsigned)kv_blocks, 512, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace ra
