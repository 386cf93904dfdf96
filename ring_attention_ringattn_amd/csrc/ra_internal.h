// Internal declarations shared by the host driver and the HIP kernels of
// libringattn.  Not part of the public C ABI (include/ringattn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// Positions/documents are summarised per run of TILE tokens; the step
// kernels' key tile is this many tokens and query tiles are multiples of it.
constexpr int TILE = 64;
constexpr int POS_INVALID = 0x7fffffff;   // sentinel: a key slot past the end of the block

enum Mask { MASK_NONE = 0, MASK_CAUSAL = 1, MASK_DOC_CAUSAL = 2 };
enum DType { F32 = 0, BF16 = 1 };
enum StepFlags { FLAG_FIRST = 1, FLAG_LAST = 2, FLAG_NO_SKIP = 4 };

// Per-tile summary: {min pos, max pos, min doc, max doc} over the tile's tokens.
struct TileRange {
  int min_pos, max_pos, min_doc, max_doc;
};

__host__ __device__ inline int n_tiles(int s) { return (s + TILE - 1) / TILE; }
// keys of a transposed value block row: whole tiles
__host__ __device__ inline int vt_keys(int sk) { return n_tiles(sk) * TILE; }
// bytes of one transposed bf16 value block
inline size_t vt_block_bytes(int B, int hkv, int d, int sk) { return (size_t)B * hkv * d * vt_keys(sk) * 2; }

struct Strides {
  int64_t b, h, s;
};

constexpr int MAX_FUSED_BLOCKS = 16;   // K/V blocks one fused (all-gather) forward launch can take

struct FwdArgs {
  const void* q;
  const void* k;      // block 0 (the only block of a ring step)
  const void* v;
  float* o_acc;       // dense [B][Hq][Sq][D]
  float* lse;         // dense [B][Hq][Sq]
  void* out;          // q strides, problem dtype; written when FLAG_LAST and non-null
  const int* q_pos;
  const int* kv_pos;
  const int* q_doc;
  const int* kv_doc;
  const TileRange* q_tiles;
  const TileRange* kv_tiles;
  Strides qs, kvs;
  int B, hq, hkv, sq, sk;
  float scale;        // softmax scale
  float scale_log2;   // softmax scale * log2(e)
  int mask;
  int flags;
  // Fused (all-gather) forward: n_blocks K/V blocks of sk keys each, same strides;
  // entry 0 repeats k, v, kv_pos, kv_doc, kv_tiles.  A ring step has n_blocks = 1.
  // o_acc may be null for a fused launch (FIRST | LAST: out and lse only).
  int n_blocks;
  const void* kb[MAX_FUSED_BLOCKS];
  const void* vb[MAX_FUSED_BLOCKS];
  // bf16 forward: each block's values transposed, [B][Hkv][D][skp] dense (vt_transpose)
  const void* vtb[MAX_FUSED_BLOCKS];
  int skp;
  const int* kposb[MAX_FUSED_BLOCKS];
  const int* kdocb[MAX_FUSED_BLOCKS];
  const TileRange* ktilesb[MAX_FUSED_BLOCKS];
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* d_o;    // q strides
  const float* lse;   // dense [B][Hq][Sq]
  const float* delta; // dense [B][Hq][Sq]
  float* dq;          // dense [B][Hq][Sq][D]
  float* dk;          // dense [B][Hkv][Sk][D]
  float* dv;
  const int* q_pos;
  const int* kv_pos;
  const int* q_doc;
  const int* kv_doc;
  const TileRange* q_tiles;
  const TileRange* kv_tiles;
  Strides qs, kvs;
  int B, hq, hkv, sq, sk;
  float scale;
  float scale_log2;
  int mask;
  int flags;
};

// Tile classes of a (query tile, key tile) pair.
enum TileClass { TILE_EMPTY = 0, TILE_FULL = 1, TILE_PARTIAL = 2 };

// Classify a query-range/key-tile pair.  `kv_complete` says all TILE key slots
// of the tile hold real keys.
__host__ __device__ inline int classify(const TileRange& qr, const TileRange& kr, bool kv_complete,
                                        int mask) {
  if (mask != MASK_NONE) {
    if (kr.min_pos > qr.max_pos) return TILE_EMPTY;
    if (mask == MASK_DOC_CAUSAL && (kr.max_doc < qr.min_doc || kr.min_doc > qr.max_doc)) return TILE_EMPTY;
  }
  if (!kv_complete) return TILE_PARTIAL;
  if (mask == MASK_NONE) return TILE_FULL;
  if (kr.max_pos > qr.min_pos) return TILE_PARTIAL;
  if (mask == MASK_DOC_CAUSAL &&
      !(kr.min_doc == kr.max_doc && qr.min_doc == qr.max_doc && kr.min_doc == qr.min_doc))
    return TILE_PARTIAL;
  return TILE_FULL;
}

// ---- launchers (each returns hipGetLastError() of its launches) ----
hipError_t launch_tile_ranges(const int* pos, const int* doc, int n, TileRange* out, hipStream_t st);
// Several tile tables in one launch (the ring builds one per emulated rank's queries and per block).
constexpr int TABLE_JOBS = 48;
struct TableJob {
  const int* pos;
  const int* doc;   // null: every token in document 0
  TileRange* out;
  int n;
};
struct TableJobs {
  TableJob job[TABLE_JOBS];
  int count;
};
hipError_t launch_tile_ranges_batch(const TableJobs& jobs, hipStream_t st);
hipError_t launch_docs_from_cu(const int* cu, int n_docs, int first, int n, int* doc, hipStream_t st);
hipError_t launch_merge(int64_t rows, int d, const float* o_a, const float* lse_a, float* o_b, float* lse_b,
                        void* out, Strides os, int hq, int sq, int dtype, hipStream_t st);
hipError_t launch_bwd_preprocess(int B, int hq, int sq, int d, const void* out, const void* d_o,
                                 Strides qs, int dtype, float* delta, hipStream_t st);
hipError_t launch_fill_nan(void* p, size_t bytes, hipStream_t st);
// V [B][Hkv][Sk][D] (strides s) -> VT [B][Hkv][D][vt_keys(Sk)] dense, zero padding
hipError_t launch_vt_transpose(const void* v, Strides s, int B, int hkv, int sk, int d, void* vt, hipStream_t st);
hipError_t launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t st);
hipError_t launch_fwd_f32(const FwdArgs& a, int d, hipStream_t st);
hipError_t launch_bwd_bf16(const BwdArgs& a, int d, hipStream_t st);
hipError_t launch_bwd_f32(const BwdArgs& a, int d, hipStream_t st);

}  // namespace ra
