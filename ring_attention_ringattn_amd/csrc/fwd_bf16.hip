// Forward ring step, bf16 inputs, fp32 accumulation, on gfx950 MFMA.
//
// One workgroup = 8 waves = BM = 256 query rows of one (batch, query head)
// (32 rows per wave); it walks the key/value block in tiles of BN = 64 keys,
// skipping tiles that the mask hides entirely (per-tile position/document
// ranges).  Per tile and wave:
//
//   S^T = K Q^T           v_mfma_f32_32x32x16_bf16, K tile from LDS (A),
//                         the wave's Q rows held in registers (B)
//   mask + online softmax each lane owns whole query columns of S^T, so the
//                         running max/sum need one cross-lane exchange
//   O^T += V^T P^T        V^T (A) from the transposed value tile (the value
//                         block is staged as V^T, so a plain 16-byte read);
//                         P^T (B) straight from the S^T accumulator
//                         registers, converted to bf16
//
// Making the S^T accumulator usable as the P^T operand without a shuffle:
// lane l of a 32x32 MFMA result holds rows {8*(v/4) + 4*(l/32) + v%4}, but
// the K-operand of the next MFMA wants 8 consecutive reduction indices per
// lane.  Loading K row swap23(i) (bits 2 and 3 of the row index swapped) into
// MFMA row i makes lane l's 8 values of each half belong to 8 consecutive
// keys, which is exactly the operand layout; the keys of the V^T operand are
// then read in natural order.
//
// Ping-pong schedule.  The softmax of a tile costs about as many issue
// cycles as its two products, so the workgroup is split into two groups of
// four waves, one wave of each group per SIMD, running half a period apart
// and separated by workgroup barriers:
//
//   period i, phase X:  leading group   PV(i-1), S(i)      (matrix cores)
//                       trailing group  softmax(i-1)       (vector ALU)
//   period i, phase Y:  leading group   softmax(i)
//                       trailing group  PV(i-1), S(i)
//
// so on every SIMD one wave feeds the matrix core while the other computes
// exponentials (and reads the first key group of V(i) for the next PV: a lone
// wave's LDS read rate is what holds the matrix phase back).  Both phases of
// period i read the same two tiles, K(i) and V(i-1) (and V(i) for that key
// group); later tiles stream from HBM straight into LDS (buffer loads,
// no register staging, zero-fill past the end of the block) into 4-deep
// buffers, K three tiles ahead and V two.  Tiles are swizzled (mfma_tile.h)
// so the K and V^T operand reads are free of bank conflicts.
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
//
// All-gather mode: one launch may take up to MAX_FUSED_BLOCKS resident K/V
// blocks; the tile list then spans every block (entries carry the block
// index) and the softmax state stays in registers across blocks, so there is
// no running output between blocks (the launch is FIRST | LAST).
#include "mfma_tile.h"

namespace ra {

namespace {

constexpr int BN = 64;             // keys per tile (== TILE)
constexpr int NWAVES = 8;          // two groups of four (one wave of each per SIMD)
constexpr int BM = NWAVES * 32;    // query rows per workgroup (32 per wave)
constexpr int LIST = NWAVES * 64;  // tile-list chunk (one tile per thread when building it)
constexpr int NBUF = 4;            // K/V tile buffers: the tiles of periods i .. i+3
constexpr float RESCALE_SLACK = 8.0f;
#ifndef RA_FWD_AHEAD
#define RA_FWD_AHEAD 3      // operand reads issued ahead of the MFMA that uses them
#endif

template <int D>
struct Cfg {
  static constexpr int CHUNKS = BN * D * 2 / 1024;   // 1 KB buffer->LDS chunks per tile and operand
  static constexpr int CPW = CHUNKS / NWAVES;        // ... per wave
  static_assert(CPW * NWAVES == CHUNKS, "tile chunks must divide over the waves");
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

// MULTI: several resident blocks (entries carry a block index); otherwise block 0 only.
// KREL: byte offsets of K rows within a block fit 31 bits (one resource per block).
template <int D, bool MULTI, bool KREL>
__global__ __launch_bounds__(NWAVES * 64, 1) void fwd_bf16_kernel(FwdArgs a) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(1024))) __bf16 Ks[NBUF][BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 Vs[NBUF][BN * D];
  __shared__ __attribute__((aligned(16))) int kvp[NBUF][BN];   // positions of the keys of K buffer i
  __shared__ __attribute__((aligned(16))) int kvd[NBUF][BN];   // ... and their documents
  __shared__ int list[LIST];
  __shared__ int wave_cnt[NWAVES];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, j = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool leading = wave < NWAVES / 2;
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
  // (loaded once the first tile list with a visible tile exists: a workgroup that
  // sees no key of the block never reads its queries)
  bf16x8 qf[D / 16];
  bool q_loaded = false;
  const int qpos = qvalid ? a.q_pos[qrow] : -1;
  const int qdoc = (qvalid && mask == MASK_DOC_CAUSAL) ? a.q_doc[qrow] : 0;

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  const size_t kvoff = b * a.kvs.b + kvh * a.kvs.h;   // this (batch, kv head) within a block
  const int rsb = (int)(a.kvs.s * 2);   // bytes between consecutive keys
  const int nkt = n_tiles(a.sk);        // tiles per block
  const int ntot = nkt * a.n_blocks;    // tiles over all blocks (list index space)
  const bool no_skip = (a.flags & FLAG_NO_SKIP) != 0;
  const float sl2 = a.scale_log2;
  const bool no_causal = mask == MASK_NONE, no_doc = mask != MASK_DOC_CAUSAL;

  // Per-lane byte offsets (within a tile) of this lane's 16-byte unit of each
  // of the wave's CPW buffer->LDS chunks: chunk q = c*NWAVES + wave covers
  // LDS units [64q, 64q+64); unit p holds row p/U, logical column
  // (p%U) ^ swz(row).
  int voff[C::CPW];
#pragma unroll
  for (int c = 0; c < C::CPW; ++c) voff[c] = chunk_voff<D>(c * NWAVES + wave, lane, rsb);
  // The same for the transposed value tiles (D rows of 64 keys, 128 bytes): unit p
  // holds row p/8 (a head dimension), key unit (p%8) ^ vswz(row).
  const int skp = a.skp;
  const size_t vtoff = ((size_t)b * a.hkv + kvh) * D * skp;   // this (batch, kv head) within a V^T block
  int vtoff_lane[C::CPW];
#pragma unroll
  for (int c = 0; c < C::CPW; ++c) {
    const int p = (c * NWAVES + wave) * 64 + lane, r = p >> 3;
    vtoff_lane[c] = r * skp * 2 + (((p & 7) ^ vswz(r)) << 4);
  }

  // Buffer resources of the block being issued, built once per block: the K rows of this
  // (batch, kv head), its V^T rows, the key positions and documents.  A tile is then issued
  // with its byte offset added to each lane's offset, and the range check zero-fills keys
  // past the block's end.  KREL: the K offsets fit 31 bits (else, very wide token-major
  // blocks, each K tile gets a resource of its own).  One block: loop invariant.  Several:
  // the list runs through the blocks in order, so each side (K, V) rebuilds its resources
  // only when the block changes.
  const int kspan = KREL ? a.sk * rsb : 0, pspan = a.sk * 4, vspan = D * skp * 2;
  const __bf16* kblk_p = (const __bf16*)a.kb[0] + kvoff;
  i32x4 k_rsrc = buffer_rsrc(kblk_p, kspan);
  i32x4 kpos_rsrc = buffer_rsrc(a.kposb[0], pspan);
  i32x4 kdoc_rsrc = buffer_rsrc(mask == MASK_DOC_CAUSAL ? a.kdocb[0] : a.kposb[0], pspan);
  i32x4 v_rsrc = buffer_rsrc((const __bf16*)a.vtb[0] + vtoff, vspan);
  int kblk = 0, vblk = 0;

  // Start streaming the K rows (with the key positions and documents, wave 0)
  // / the V rows of the tile of list position li (entry ent: tile | block << 12)
  // into buffer li % NBUF.  Every wave issues its share; keys past the end of
  // the block read as zero.
  auto issue_k = [&] __device__(int li, int ent) {
    const int buf = li % NBUF, tile = ent & 0xfff;
    if (MULTI) {
      const int blk = (ent >> 12) & 0xf;
      if (blk != kblk) {
        kblk = blk;
        kblk_p = (const __bf16*)a.kb[blk] + kvoff;
        if (KREL) k_rsrc = buffer_rsrc(kblk_p, kspan);
        kpos_rsrc = buffer_rsrc(a.kposb[blk], pspan);
        if (mask == MASK_DOC_CAUSAL) kdoc_rsrc = buffer_rsrc(a.kdocb[blk], pspan);
      }
    }
    const int kbase = tile * BN;
    if (wave == 0) {
      dma4r(kpos_rsrc, (RA_LDS void*)&kvp[buf][0], (kbase + lane) * 4);
      if (mask == MASK_DOC_CAUSAL) dma4r(kdoc_rsrc, (RA_LDS void*)&kvd[buf][0], (kbase + lane) * 4);
    }
    if (KREL) {
      const int ko = kbase * rsb;
#pragma unroll
      for (int c = 0; c < C::CPW; ++c) dma16r(k_rsrc, (RA_LDS void*)&Ks[buf][(c * NWAVES + wave) * 512], voff[c] + ko);
    } else {
      const int rows = min(BN, a.sk - kbase);
      const __bf16* kb = kblk_p + (size_t)kbase * a.kvs.s;
#pragma unroll
      for (int c = 0; c < C::CPW; ++c)
        dma16(kb, rows * rsb, (RA_LDS void*)&Ks[buf][(c * NWAVES + wave) * 512], voff[c]);
    }
  };
  // V^T rows of the tile: D rows of 64 keys (the padding past the block end is zero)
  auto issue_v = [&] __device__(int li, int ent) {
    const int buf = li % NBUF, tile = ent & 0xfff;
    if (MULTI) {
      const int blk = (ent >> 12) & 0xf;
      if (blk != vblk) {
        vblk = blk;
        v_rsrc = buffer_rsrc((const __bf16*)a.vtb[blk] + vtoff, vspan);
      }
    }
    const int vo = tile * BN * 2;
#pragma unroll
    for (int c = 0; c < C::CPW; ++c)
      dma16r(v_rsrc, (RA_LDS void*)&Vs[buf][(c * NWAVES + wave) * 512], vtoff_lane[c] + vo);
  };

  // V^T operands (lane j: head dimension db*32 + j, 8 keys) of the transposed tile in V
  // buffer `buf`.  Those of the first key group of the next PV are read in the softmax
  // phase, where the other wave of the SIMD reads its own operands: one wave alone gets
  // about 1 KB of LDS data per 40 cycles, less than a 32-cycle MFMA consumes.  (Reading
  // more groups early lengthens the softmax phase by more than it saves: measured.)
  auto v_operand = [&] __device__(int buf, int kk, int db) {
    const int r = db * 32 + j;
    return *(const bf16x8*)(&Vs[buf][r * BN + (((kk * 2 + g) ^ vswz(r)) << 3)]);
  };
  bf16x8 vpre[D / 32];
  auto prefetch_v = [&] __device__(int buf) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) vpre[db] = v_operand(buf, 0, db);
  };

  // Matrix phase: O^T += V^T P^T (V buffer `vbuf`; P^T straight from registers), then
  // S^T = K Q^T (raw scores) of the tile in K buffer `kbuf`.
  auto matrix = [&] __device__(int vbuf, int kbuf, const bf16x8(&pf)[4], f32x16(&s)[2]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] = mfma(kk == 0 ? vpre[db] : v_operand(vbuf, kk, db), pf[kk], acc[db]);
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 kf = *(const bf16x8*)(&Ks[kbuf][tile_off<D>(mb * 32 + swap23(j), ks * 16 + g * 8)]);
        s[mb] = mfma(kf, qf[ks], s[mb]);
      }
    // issue order: each operand read runs AHEAD products ahead of its MFMA (one wave per
    // SIMD feeds the matrix core in this phase, so nothing else hides the LDS latency);
    // the first D/32 products take their operands from registers
    constexpr int M = D / 4, PRE = D / 32, R = M - PRE, AH = RA_FWD_AHEAD;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int before = m + AH - PRE < 0 ? 0 : (m + AH - PRE > R ? R : m + AH - PRE);
      const int prev = m == 0 ? 0 : (m - 1 + AH - PRE < 0 ? 0 : (m - 1 + AH - PRE > R ? R : m - 1 + AH - PRE));
#pragma unroll
      for (int x = 0; x < before - prev; ++x) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };

  // Mask (partial tiles only) and online softmax of the tile of list entry
  // `ent` (workgroup-uniform, scalar; key positions in buffer `buf`): rescales acc/l_run when the maximum moves,
  // returns the probabilities as bf16 P^T operands.
  // lane (g, j), value v of block mb holds key mb*32 + 16*(v/8) + 8*g + v%8 for query j.
  auto softmax = [&] __device__(int ent, int buf, f32x16(&s)[2], bf16x8(&pf)[4]) {
    const bool partial = (ent >> 24) == TILE_PARTIAL;
    const int kvalid = a.sk - (ent & 0xfff) * BN;   // keys of this tile that exist (>= BN: all)
    if (partial) {
      asm volatile("" ::: "memory");   // keep this a real branch: full tiles must not pay for masking
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int base = mb * 32 + 16 * hh + 8 * g;
          const i32x4 p0 = *(const i32x4*)&kvp[buf][base], p1 = *(const i32x4*)&kvp[buf][base + 4];
          const i32x4 d0 = *(const i32x4*)&kvd[buf][base], d1 = *(const i32x4*)&kvd[buf][base + 4];
          const int lim = kvalid - base;   // e < lim: key base + e exists
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int kp = e < 4 ? p0[e] : p1[e - 4];
            const int kd = e < 4 ? d0[e] : d1[e - 4];
            // bitwise, not short-circuit: one select per score, no branches
            const bool ok = (e < lim) & (no_causal | (kp <= qpos)) & (no_doc | (kd == qdoc));
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
  };

  f32x16 s[2];
  bf16x8 pf[4];
  int seen = 0;   // tiles this workgroup processed (uniform)
  for (int c0 = 0; c0 < ntot; c0 += LIST) {
    // ---- compact the non-empty tiles of this chunk into `list` ----
    const int t = c0 + tid;
    int cls = TILE_EMPTY;
    int tl = 0, blk = 0;
    if (t < ntot) {
      blk = t / nkt;
      tl = t - blk * nkt;
      cls = classify(qr, a.ktilesb[blk][tl], (tl + 1) * TILE <= a.sk, mask);
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
    if (cls != TILE_EMPTY) list[off + my] = tl | (blk << 12) | (cls << 24);
    __syncthreads();
    total = __builtin_amdgcn_readfirstlane(total);
    seen += total;
    if (total == 0) continue;
    if (!q_loaded) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        bf16x8 z = {};
        qf[ks] = qvalid ? *(const bf16x8*)(qptr + qrow * a.qs.s + ks * 16 + g * 8) : z;
      }
      q_loaded = true;
    }
    // list entry li (tile | block << 12 | class << 24), scalar
    auto tile_of = [&] __device__(int li) { return __builtin_amdgcn_readfirstlane(list[li]); };

    // prologue: K(0..2), V(0..1); V(-1) := 0 and P := 0 so that period 0's PV adds nothing
    for (int t = 0; t < min(3, total); ++t) issue_k(t, tile_of(t) & 0xffff);
    for (int t = 0; t < min(2, total); ++t) issue_v(t, tile_of(t) & 0xffff);
    for (int e = tid * 8; e < BN * D; e += NWAVES * 64 * 8) *(bf16x8*)&Vs[NBUF - 1][e] = bf16x8{};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) pf[kk] = bf16x8{};
#pragma unroll
    for (int db = 0; db < D / 32; ++db) vpre[db] = bf16x8{};
    wait_vmem();
    __syncthreads();

    // Both groups run the same sequence, the trailing one shifted by one
    // barrier, so that while one group is in its matrix phase the other is in
    // its softmax phase.  Period i reads K(i) and V(i-1); in its softmax phase
    // each group issues its share of K(i+3) and V(i+2), which period i+3 reads.
    // A wave waits for them at the end of the matrix phase of period i+2, just
    // before that period's first barrier: for the leading group that barrier
    // precedes everyone's period i+3; for the trailing group it is the barrier
    // the leading group's period i+3 starts from.  One read comes earlier: the
    // first key group of V(i+2) is read in the softmax phase of period i+2,
    // which for the leading group starts one barrier before the trailing
    // group's matrix-phase wait; so the trailing group also waits at the end of
    // its softmax phase of period i+1.  Leading loads thus have about two
    // periods to land, trailing ones one and a half, and the waits sit where
    // the loads are normally long done.
    //
    // The periods that issue both tiles (all but the last three) run in a loop
    // with no conditions; the last ones drain.  List entries (workgroup-uniform)
    // rotate through scalar registers: period i reads the entry of tile i+4
    // from LDS and turns it scalar one period later, when it has long arrived.
    int ent0 = tile_of(0), ent1 = tile_of(min(1, LIST - 1)), ent2 = tile_of(min(2, LIST - 1));
    int nxt = list[min(3, LIST - 1)];
    if (!leading) __syncthreads();
    int i = 0;
    // (phase_barrier: the matrix work must not drift past the barrier into the softmax
    // phase, nor the softmax work into the matrix phase: MFMAs touch no memory, so the
    // workgroup barrier alone does not hold them)
    auto phase_barrier = [] __device__() {
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    for (; i + 3 < total; ++i) {
      matrix((i + NBUF - 1) % NBUF, i % NBUF, pf, s);
      wait_vmem_n<2 * C::CPW>();   // period i-1 issued K(i+2) and V(i+1); period i-2's loads have landed
      phase_barrier();
      const int ent3 = __builtin_amdgcn_readfirstlane(nxt);
      nxt = list[min(i + 4, LIST - 1)];
      issue_k(i + 3, ent3 & 0xffff);
      issue_v(i + 2, ent2 & 0xffff);
      prefetch_v(i % NBUF);   // V(i), read by the next period's PV
      softmax(ent0, i % NBUF, s, pf);
      // The leading group's softmax(i+1), which starts at the next barrier, reads V(i+1)
      // early (prefetch_v), and a quarter of that tile arrives through the trailing
      // waves' loads of period i-1: the trailing group waits for them here (what
      // period i issued after them, K(i+3) and V(i+2), may still be in flight).
      if (!leading) wait_vmem_n<2 * C::CPW>();
      phase_barrier();
      ent0 = ent1;
      ent1 = ent2;
      ent2 = ent3;
    }
    for (; i <= total; ++i) {
      matrix((i + NBUF - 1) % NBUF, i % NBUF, pf, s);
      // this wave's loads of period i-2 have landed: vmcnt = what period i-1 issued
      // (K(i+2) if it exists, V(i+1) if it exists; wave 0's position loads only make
      // the wait stricter)
      if (i + 2 < total) wait_vmem_n<2 * C::CPW>();
      else if (i + 1 < total) wait_vmem_n<C::CPW>();
      else wait_vmem();
      phase_barrier();
      if (i + 2 < total) issue_v(i + 2, ent2 & 0xffff);
      if (i < total) {
        prefetch_v(i % NBUF);
        softmax(ent0, i % NBUF, s, pf);
      }
      if (!leading && i + 1 < total) {   // as above; period i issued at most V(i+2)
        if (i + 2 < total) wait_vmem_n<C::CPW>();
        else wait_vmem();
      }
      phase_barrier();
      ent0 = ent1;
      ent1 = ent2;
    }
    if (leading) __syncthreads();
  }

  // ---- epilogue: normalise, merge into (o_acc, lse), optionally write out ----
  const bool first = (a.flags & FLAG_FIRST) != 0;
  const bool last = (a.flags & FLAG_LAST) != 0 && a.out != nullptr;
  // No key of this block is visible to the tile: merging the empty partial (LSE -inf)
  // leaves (o_acc, lse) exactly as they are, so a middle step skips the round trip and
  // the last step only writes the bf16 output.
  const bool unchanged = seen == 0 && !first;
  if (unchanged && !last) return;
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
  float* op = a.o_acc ? a.o_acc + orow * D : nullptr;   // null: fused launch, out and lse only
  __bf16* outp = last ? (__bf16*)a.out + b * a.qs.b + h * a.qs.h + qrow * a.qs.s : nullptr;
  // the running output is read whole before any of it is combined or written, so the reads
  // are in flight together (a read per use would wait a memory round trip each)
  f32x4 prev[D / 32][4];
  if (!first) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int vh = 0; vh < 4; ++vh) prev[db][vh] = *(const f32x4*)(op + db * 32 + vh * 8 + g * 4);
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int vh = 0; vh < 4; ++vh) {
      const int d = db * 32 + vh * 8 + g * 4;
      f32x4 o = {acc[db][vh * 4 + 0] * w_t, acc[db][vh * 4 + 1] * w_t, acc[db][vh * 4 + 2] * w_t,
                 acc[db][vh * 4 + 3] * w_t};
      if (!first) o += w_p * prev[db][vh];
      if (op && !unchanged) *(f32x4*)(op + d) = o;
      if (last) {
        bf16x4 ob = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
        *(bf16x4*)(outp + d) = ob;
      }
    }
  }
  if (g == 0 && !unchanged) a.lse[orow] = lse_new;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t st) {
  const long blocks = (long)((a.sq + BM - 1) / BM) * a.hq * a.B;
  if (blocks == 0) return hipSuccess;
  const bool multi = a.n_blocks > 1;
  // the largest K offset of a tile load is below (tiles * 64) rows of the block
  const bool krel = (int64_t)n_tiles(a.sk) * TILE * a.kvs.s * 2 < ((int64_t)1 << 31);
  const dim3 grid((unsigned)blocks), block(NWAVES * 64);
#define RA_FWD_LAUNCH(DD, MM, KK) fwd_bf16_kernel<DD, MM, KK><<<grid, block, 0, st>>>(a)
  if (d == 128) {
    if (multi) { if (krel) RA_FWD_LAUNCH(128, true, true); else RA_FWD_LAUNCH(128, true, false); }
    else { if (krel) RA_FWD_LAUNCH(128, false, true); else RA_FWD_LAUNCH(128, false, false); }
  } else {
    if (multi) { if (krel) RA_FWD_LAUNCH(64, true, true); else RA_FWD_LAUNCH(64, true, false); }
    else { if (krel) RA_FWD_LAUNCH(64, false, true); else RA_FWD_LAUNCH(64, false, false); }
  }
#undef RA_FWD_LAUNCH
  return hipGetLastError();
}

}  // namespace ra
