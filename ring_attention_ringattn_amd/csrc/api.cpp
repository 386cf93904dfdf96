// C ABI of libringattn: argument validation (pure host code, before any HIP
// call), workspace layout, kernel dispatch and the N-step ring driver.
#include "ringattn.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "ra_internal.h"

using namespace ra;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return RA_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t n) { return ((uintptr_t)p % n) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t elem_size(int dtype) { return dtype == RA_BF16 ? 2 : 4; }

// Rows addressed through (batch, head, token) strides must not overlap when
// they are written: sorted by stride, each dimension must start past the
// previous one's extent.
bool non_overlapping(const int64_t st[3], int64_t B, int64_t H, int64_t S, int64_t D) {
  struct Dim { int64_t stride, extent; } dims[3] = {{st[0], B}, {st[1], H}, {st[2], S}};
  for (int i = 0; i < 3; ++i)
    for (int k = i + 1; k < 3; ++k)
      if (dims[k].stride < dims[i].stride) std::swap(dims[i], dims[k]);
  int64_t need = D;
  for (auto& d : dims) {
    if (d.extent <= 1) continue;
    if (d.stride < need) return false;
    need = d.stride * d.extent;
  }
  return true;
}

// A dispatch holds the work-item count of each grid dimension in 32 bits: the blocks of
// one launch times its threads per block must fit.
bool grid_fits(int64_t blocks, int threads) { return blocks <= (int64_t)(0xffffffffu / (unsigned)threads); }

// Workgroups per row of the standalone merge (and the merge-kernel run mode): one
// 32-lane group per (batch, head, token) row in 256-thread blocks.
bool merge_fits(int64_t rows) { return grid_fits((rows * 32 + 255) / 256, 256); }

// Every launch this problem can make (forward, backward, merge) must have a grid that
// fits, and the per-workgroup work lists index their items in 24 bits.
int check_launch_sizes(const ra_problem* p) {
  const int64_t B = p->batch, hq = p->hq, hkv = p->hkv, sq = p->sq, sk = p->sk;
  const int64_t rows = B * hq * sq, keys = B * hkv * sk;
  bool fits = merge_fits(rows) && grid_fits((rows * (p->head_dim / 8) + 255) / 256, 256);
  if (p->dtype == RA_BF16)
    fits = fits && grid_fits((sq + 255) / 256 * hq * B, 512)   // forward step
           && grid_fits((sq + 127) / 128 * hq * B, 256)        // dQ, one query head per workgroup
           && grid_fits((sk + 127) / 128 * hkv * B, 512)       // dK/dV
           && (hq / hkv) * ((sq + 63) / 64) < (1 << 24);       // dK/dV work items (query head, tile)
  else
    fits = fits && grid_fits((rows + 3) / 4, 256) && grid_fits((keys + 3) / 4, 256);
  if (!fits)
    return fail(RA_ERR_UNSUPPORTED, "problem too large for one launch (batch %d x hq %d x sq %d, hkv %d, sk %d)",
                p->batch, p->hq, p->sq, p->hkv, p->sk);
  return RA_OK;
}

int check_problem(const ra_problem* p) {
  if (!p) return fail(RA_ERR_INVALID, "problem descriptor is NULL");
  if (p->batch < 1 || p->hq < 1 || p->hkv < 1)
    return fail(RA_ERR_INVALID, "batch, hq and hkv must be >= 1 (got %d, %d, %d)", p->batch, p->hq, p->hkv);
  if (p->hq % p->hkv)
    return fail(RA_ERR_INVALID, "hq (%d) must be a multiple of hkv (%d)", p->hq, p->hkv);
  if (p->sq < 0 || p->sk < 0) return fail(RA_ERR_INVALID, "sq and sk must be >= 0 (got %d, %d)", p->sq, p->sk);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", p->head_dim);
  if (p->dtype != RA_F32 && p->dtype != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "dtype %d not supported", p->dtype);
  if (p->sk > RA_MAX_SK) return fail(RA_ERR_UNSUPPORTED, "sk %d exceeds RA_MAX_SK (%d)", p->sk, RA_MAX_SK);
  for (int i = 0; i < 3; ++i) {
    if (p->q_stride[i] <= 0 || p->q_stride[i] % 8)
      return fail(RA_ERR_INVALID, "q_stride[%d] = %lld must be a positive multiple of 8", i, (long long)p->q_stride[i]);
    if (p->kv_stride[i] <= 0 || p->kv_stride[i] % 8)
      return fail(RA_ERR_INVALID, "kv_stride[%d] = %lld must be a positive multiple of 8", i, (long long)p->kv_stride[i]);
  }
  // The kernels stage up to 128 consecutive tokens with one 32-bit byte range (and address
  // a token inside a staged tile with a 32-bit byte offset): 128 token strides must stay
  // below 2^31 bytes.
  {
    const int64_t esize = p->dtype == RA_F32 ? 4 : 2, lim = ((int64_t)1 << 31) / (128 * esize);
    if (p->q_stride[2] >= lim || p->kv_stride[2] >= lim)
      return fail(RA_ERR_UNSUPPORTED, "token stride (q %lld, kv %lld elements) must be below %lld elements",
                  (long long)p->q_stride[2], (long long)p->kv_stride[2], (long long)lim);
  }
  if (!non_overlapping(p->q_stride, p->batch, p->hq, p->sq, p->head_dim))
    return fail(RA_ERR_INVALID, "q strides make rows overlap (out is written with them)");
  if (!std::isfinite(p->softmax_scale) || p->softmax_scale < 0.f)
    return fail(RA_ERR_INVALID, "softmax_scale must be finite and >= 0");
  return check_launch_sizes(p);
}

int check_ptr(const void* ptr, const char* name, size_t align = 16) {
  if (!ptr) return fail(RA_ERR_INVALID, "%s is NULL", name);
  if (!aligned(ptr, align)) return fail(RA_ERR_INVALID, "%s is not %zu-byte aligned", name, align);
  return RA_OK;
}

int check_mask(int mask_mode, const int32_t* q_doc, const int32_t* kv_doc, bool need_kv) {
  if (mask_mode < RA_MASK_NONE || mask_mode > RA_MASK_DOC_CAUSAL)
    return fail(RA_ERR_UNSUPPORTED, "mask_mode %d not supported (none, causal, doc-causal)", mask_mode);
  if (mask_mode == RA_MASK_DOC_CAUSAL) {
    if (int rc = check_ptr(q_doc, "q_doc", 4)) return rc;
    if (need_kv)
      if (int rc = check_ptr(kv_doc, "kv_doc", 4)) return rc;
  }
  return RA_OK;
}

float eff_scale(const ra_problem* p) {
  return p->softmax_scale > 0.f ? p->softmax_scale : 1.f / std::sqrt((float)p->head_dim);
}

size_t step_ws(int sq, int sk) {
  return align256((size_t)n_tiles(sq) * sizeof(TileRange)) + align256((size_t)n_tiles(sk) * sizeof(TileRange));
}

// The bf16 forward reads each value block transposed (vt_transpose): room for one.
size_t vt_ws(const ra_problem* p) {
  return p->dtype == RA_BF16 ? align256(vt_block_bytes(p->batch, p->hkv, p->head_dim, p->sk)) : 0;
}

hipError_t transpose_v(const ra_problem* p, const void* v, void* vt, hipStream_t st) {
  if (p->sk == 0) return hipSuccess;
  return launch_vt_transpose(v, Strides{p->kv_stride[0], p->kv_stride[1], p->kv_stride[2]}, p->batch, p->hkv, p->sk,
                             p->head_dim, vt, st);
}

struct StepTables {
  TileRange* q;
  TileRange* kv;
};

StepTables carve_step_ws(void* ws, int sq) {
  char* base = (char*)ws;
  return {(TileRange*)base, (TileRange*)(base + align256((size_t)n_tiles(sq) * sizeof(TileRange)))};
}

Strides strides3(const int64_t s[3]) { return Strides{s[0], s[1], s[2]}; }

FwdArgs make_fwd(const ra_problem* p, const void* q, const void* k, const void* v, float* o_acc, float* lse,
                 void* out, const int32_t* q_pos, const int32_t* kv_pos, const int32_t* q_doc,
                 const int32_t* kv_doc, const TileRange* qt, const TileRange* kt, int mask, int flags) {
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o_acc = o_acc; a.lse = lse; a.out = out;
  a.q_pos = q_pos; a.kv_pos = kv_pos; a.q_doc = q_doc; a.kv_doc = kv_doc;
  a.q_tiles = qt; a.kv_tiles = kt;
  a.qs = strides3(p->q_stride); a.kvs = strides3(p->kv_stride);
  a.B = p->batch; a.hq = p->hq; a.hkv = p->hkv; a.sq = p->sq; a.sk = p->sk;
  a.scale = eff_scale(p);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.mask = mask; a.flags = flags;
  a.n_blocks = 1;
  a.skp = vt_keys(p->sk);
  for (int j = 0; j < MAX_FUSED_BLOCKS; ++j) {
    a.kb[j] = k; a.vb[j] = v; a.vtb[j] = v; a.kposb[j] = kv_pos; a.kdocb[j] = kv_doc; a.ktilesb[j] = kt;
  }
  return a;
}

BwdArgs make_bwd(const ra_problem* p, const void* q, const void* k, const void* v, const void* d_o,
                 const float* lse, const float* delta, float* dq, float* dk, float* dv, const int32_t* q_pos,
                 const int32_t* kv_pos, const int32_t* q_doc, const int32_t* kv_doc, const TileRange* qt,
                 const TileRange* kt, int mask, int flags) {
  BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.d_o = d_o; a.lse = lse; a.delta = delta;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.q_pos = q_pos; a.kv_pos = kv_pos; a.q_doc = q_doc; a.kv_doc = kv_doc;
  a.q_tiles = qt; a.kv_tiles = kt;
  a.qs = strides3(p->q_stride); a.kvs = strides3(p->kv_stride);
  a.B = p->batch; a.hq = p->hq; a.hkv = p->hkv; a.sq = p->sq; a.sk = p->sk;
  a.scale = eff_scale(p);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.mask = mask; a.flags = flags;
  return a;
}

hipError_t enqueue_fwd(const ra_problem* p, const FwdArgs& a, hipStream_t st) {
  return p->dtype == RA_BF16 ? launch_fwd_bf16(a, p->head_dim, st) : launch_fwd_f32(a, p->head_dim, st);
}

hipError_t enqueue_bwd(const ra_problem* p, const BwdArgs& a, hipStream_t st) {
  return p->dtype == RA_BF16 ? launch_bwd_bf16(a, p->head_dim, st) : launch_bwd_f32(a, p->head_dim, st);
}

const int kStepFlags = RA_STEP_FIRST | RA_STEP_LAST | RA_NO_SKIP;

// Host validation of a forward step's arguments, all but the workspace (nothing is
// checked past the descriptor, mask and flags when the query shard is empty).
int check_step_fwd(const ra_problem* p, const void* q, const void* k_blk, const void* v_blk, const float* o_acc,
                   const float* lse, const void* out, const int32_t* q_pos, const int32_t* kv_pos,
                   const int32_t* q_doc, const int32_t* kv_doc, int mask_mode, int flags) {
  if (int rc = check_problem(p)) return rc;
  if (int rc = check_mask(mask_mode, q_doc, kv_doc, p->sk > 0)) return rc;
  if (flags & ~kStepFlags) return fail(RA_ERR_INVALID, "unknown step flags 0x%x", flags);
  if (p->sq == 0) return RA_OK;
  if (int rc = check_ptr(q, "q")) return rc;
  if (int rc = check_ptr(o_acc, "o_acc")) return rc;
  if (int rc = check_ptr(lse, "lse", 4)) return rc;
  if (int rc = check_ptr(q_pos, "q_pos", 4)) return rc;
  if (p->sk > 0) {
    if (int rc = check_ptr(k_blk, "k_blk")) return rc;
    if (int rc = check_ptr(v_blk, "v_blk")) return rc;
    if (int rc = check_ptr(kv_pos, "kv_pos", 4)) return rc;
  }
  if (out && !aligned(out, 16)) return fail(RA_ERR_INVALID, "out is not 16-byte aligned");
  return RA_OK;
}

// Enqueue a validated forward step whose tile tables and transposed value block go
// into `ws` (step_ws + vt_ws bytes, 16-byte aligned; every byte read is written first).
int enqueue_step_fwd(const ra_problem* p, const void* q, const void* k_blk, const void* v_blk, float* o_acc,
                     float* lse, void* out, const int32_t* q_pos, const int32_t* kv_pos, const int32_t* q_doc,
                     const int32_t* kv_doc, int mask_mode, int flags, void* ws, hipStream_t st) {
  const bool doc = mask_mode == RA_MASK_DOC_CAUSAL;
  StepTables t = carve_step_ws(ws, p->sq);
  hipError_t e = launch_tile_ranges(q_pos, doc ? q_doc : nullptr, p->sq, t.q, st);
  if (e == hipSuccess) e = launch_tile_ranges(kv_pos, doc ? kv_doc : nullptr, p->sk, t.kv, st);
  if (e != hipSuccess) return hip_fail(e, "tile-range kernel launch");
  FwdArgs a = make_fwd(p, q, k_blk, v_blk, o_acc, lse, out, q_pos, kv_pos, q_doc, kv_doc, t.q, t.kv, mask_mode, flags);
  if (vt_ws(p)) {
    void* vt = (char*)ws + step_ws(p->sq, p->sk);
    if ((e = transpose_v(p, v_blk, vt, st)) != hipSuccess) return hip_fail(e, "value transpose kernel launch");
    a.vtb[0] = vt;
  }
  e = enqueue_fwd(p, a, st);
  if (e != hipSuccess) return hip_fail(e, "forward step kernel launch");
  return ok();
}

}  // namespace

extern "C" {

int ringattn_version(void) { return RINGATTN_VERSION; }

const char* ringattn_last_error(void) { return g_err.c_str(); }

size_t ringattn_step_workspace_size(const ra_problem* p) {
  if (check_problem(p)) return 0;
  return step_ws(p->sq, p->sk) + vt_ws(p);
}

int ringattn_step_fwd(const ra_problem* p, const void* q, const void* k_blk, const void* v_blk, float* o_acc,
                      float* lse, void* out, const int32_t* q_pos, const int32_t* kv_pos, const int32_t* q_doc,
                      const int32_t* kv_doc, int mask_mode, int flags, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (int rc = check_step_fwd(p, q, k_blk, v_blk, o_acc, lse, out, q_pos, kv_pos, q_doc, kv_doc, mask_mode, flags))
    return rc;
  if (p->sq == 0) return ok();
  const size_t need = step_ws(p->sq, p->sk) + vt_ws(p);
  if (workspace_bytes < need || (need && !workspace))
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!aligned(workspace, 16)) return fail(RA_ERR_INVALID, "workspace is not 16-byte aligned");
  return enqueue_step_fwd(p, q, k_blk, v_blk, o_acc, lse, out, q_pos, kv_pos, q_doc, kv_doc, mask_mode, flags,
                          workspace, (hipStream_t)stream);
}

}  // extern "C"

// ------------------------------------------------------- allocation-free forward step
// The workspace of ringattn_step_fwd_noalloc: a file-scope device array, one copy per GPU
// (each device that loads the library holds its own, until the process ends).  In host
// code its name is only a stand-in: the kernels get the per-device address that
// hipGetSymbolAddress returns, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[RA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of this device's `scratch` (device = the calling thread's current device, which
// must be the one `stream` belongs to).
int scratch_of_current_device(void* stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(RA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  if (stream) {
    hipDevice_t sd = -1;
    if ((e = hipStreamGetDevice((hipStream_t)stream, &sd)) != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    if (sd != dev) return fail(RA_ERR_INVALID, "the stream belongs to device %d but device %d is current", (int)sd, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess)
      return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return RA_OK;
}

}  // namespace

extern "C" {

int ringattn_step_fwd_noalloc(const ra_problem* p, const void* q, const void* k_blk, const void* v_blk, float* o_acc,
                              float* lse, void* out, const int32_t* q_pos, const int32_t* kv_pos,
                              const int32_t* q_doc, const int32_t* kv_doc, int mask_mode, int flags, void* stream) {
  if (int rc = check_step_fwd(p, q, k_blk, v_blk, o_acc, lse, out, q_pos, kv_pos, q_doc, kv_doc, mask_mode, flags))
    return rc;
  if (p->sq == 0) return ok();
  const size_t need = step_ws(p->sq, p->sk) + vt_ws(p);
  if (need > RA_NOALLOC_SCRATCH_BYTES)
    return fail(RA_ERR_UNSUPPORTED,
                "this step needs %zu bytes of scratch (tile tables and the transposed value block); the "
                "allocation-free entry point has %zu: use ringattn_step_fwd with a workspace",
                need, (size_t)RA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (int rc = scratch_of_current_device(stream, &ws)) return rc;
  return enqueue_step_fwd(p, q, k_blk, v_blk, o_acc, lse, out, q_pos, kv_pos, q_doc, kv_doc, mask_mode, flags, ws,
                          (hipStream_t)stream);
}

size_t ringattn_fused_workspace_size(const ra_problem* p, int n_blocks) {
  if (check_problem(p)) return 0;
  if (n_blocks < 1 || n_blocks > RA_FUSED_MAX_BLOCKS) return 0;
  return align256((size_t)n_tiles(p->sq) * sizeof(TileRange)) +
         (size_t)n_blocks * (align256((size_t)n_tiles(p->sk) * sizeof(TileRange)) + vt_ws(p));
}

int ringattn_fused_fwd(const ra_problem* p, int n_blocks, const void* q, const void* const* k_blocks,
                       const void* const* v_blocks, float* lse, void* out, const int32_t* q_pos,
                       const int32_t* const* kv_pos, const int32_t* q_doc, const int32_t* const* kv_doc,
                       int mask_mode, int flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = check_problem(p)) return rc;
  if (n_blocks < 1 || n_blocks > RA_FUSED_MAX_BLOCKS)
    return fail(RA_ERR_INVALID, "n_blocks = %d outside [1, %d]", n_blocks, RA_FUSED_MAX_BLOCKS);
  if (p->dtype != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "the fused forward is bf16 only");
  if (flags & ~RA_NO_SKIP) return fail(RA_ERR_INVALID, "unknown fused flags 0x%x", flags);
  if (!k_blocks || !v_blocks || !kv_pos) return fail(RA_ERR_INVALID, "k_blocks, v_blocks and kv_pos are required");
  const bool doc = mask_mode == RA_MASK_DOC_CAUSAL;
  if (doc && !kv_doc) return fail(RA_ERR_INVALID, "kv_doc is required for DOC_CAUSAL");
  for (int j = 0; j < n_blocks; ++j)
    if (int rc = check_mask(mask_mode, q_doc, doc ? kv_doc[j] : nullptr, p->sk > 0)) return rc;
  if (p->sq == 0) return ok();
  if (int rc = check_ptr(q, "q")) return rc;
  if (int rc = check_ptr(lse, "lse", 4)) return rc;
  if (int rc = check_ptr(out, "out")) return rc;
  if (int rc = check_ptr(q_pos, "q_pos", 4)) return rc;
  if (p->sk > 0) {
    for (int j = 0; j < n_blocks; ++j) {
      if (int rc = check_ptr(k_blocks[j], "k_blocks[j]")) return rc;
      if (int rc = check_ptr(v_blocks[j], "v_blocks[j]")) return rc;
      if (int rc = check_ptr(kv_pos[j], "kv_pos[j]", 4)) return rc;
    }
  }
  const size_t need = ringattn_fused_workspace_size(p, n_blocks);
  if (workspace_bytes < need || (need && !workspace))
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!aligned(workspace, 16)) return fail(RA_ERR_INVALID, "workspace is not 16-byte aligned");

  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)workspace;
  TileRange* tq = (TileRange*)base;
  base += align256((size_t)n_tiles(p->sq) * sizeof(TileRange));
  const size_t kv_bytes = align256((size_t)n_tiles(p->sk) * sizeof(TileRange));
  char* vt_base = base + n_blocks * kv_bytes;
  hipError_t e = launch_tile_ranges(q_pos, doc ? q_doc : nullptr, p->sq, tq, st);
  for (int j = 0; j < n_blocks && e == hipSuccess && p->sk > 0; ++j)
    e = launch_tile_ranges(kv_pos[j], doc ? kv_doc[j] : nullptr, p->sk, (TileRange*)(base + j * kv_bytes), st);
  if (e != hipSuccess) return hip_fail(e, "tile-range kernel launch");
  for (int j = 0; j < n_blocks && e == hipSuccess && p->sk > 0; ++j)
    e = transpose_v(p, v_blocks[j], vt_base + j * vt_ws(p), st);
  if (e != hipSuccess) return hip_fail(e, "value transpose kernel launch");
  FwdArgs a = make_fwd(p, q, p->sk > 0 ? k_blocks[0] : nullptr, p->sk > 0 ? v_blocks[0] : nullptr, nullptr, lse, out,
                       q_pos, p->sk > 0 ? kv_pos[0] : nullptr, q_doc, doc ? kv_doc[0] : nullptr, tq,
                       (TileRange*)base, mask_mode, flags | RA_STEP_FIRST | RA_STEP_LAST);
  a.n_blocks = n_blocks;
  for (int j = 0; j < n_blocks && p->sk > 0; ++j) {
    a.kb[j] = k_blocks[j];
    a.vb[j] = v_blocks[j];
    a.vtb[j] = vt_base + j * vt_ws(p);
    a.kposb[j] = kv_pos[j];
    a.kdocb[j] = doc ? kv_doc[j] : nullptr;
    a.ktilesb[j] = (const TileRange*)(base + j * kv_bytes);
  }
  e = launch_fwd_bf16(a, p->head_dim, st);
  if (e != hipSuccess) return hip_fail(e, "fused forward kernel launch");
  return ok();
}

int ringattn_merge(const ra_problem* p, const float* o_a, const float* lse_a, float* o_b, float* lse_b,
                   void* stream) {
  if (!p) return fail(RA_ERR_INVALID, "problem descriptor is NULL");
  if (p->batch < 1 || p->hq < 1 || p->sq < 0)
    return fail(RA_ERR_INVALID, "batch and hq must be >= 1 and sq >= 0");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", p->head_dim);
  const int64_t rows = (int64_t)p->batch * p->hq * p->sq;
  if (rows == 0) return ok();
  if (!merge_fits(rows))
    return fail(RA_ERR_UNSUPPORTED, "%lld rows exceed one merge launch", (long long)rows);
  if (int rc = check_ptr(o_a, "o_a")) return rc;
  if (int rc = check_ptr(o_b, "o_b")) return rc;
  if (int rc = check_ptr(lse_a, "lse_a", 4)) return rc;
  if (int rc = check_ptr(lse_b, "lse_b", 4)) return rc;
  hipError_t e = launch_merge(rows, p->head_dim, o_a, lse_a, o_b, lse_b, nullptr, Strides{0, 0, 0}, p->hq,
                              p->sq, p->dtype, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  return ok();
}

int ringattn_bwd_preprocess(const ra_problem* p, const void* out, const void* d_o, float* delta, void* stream) {
  if (int rc = check_problem(p)) return rc;
  if (p->sq == 0) return ok();
  if (int rc = check_ptr(out, "out")) return rc;
  if (int rc = check_ptr(d_o, "d_o")) return rc;
  if (int rc = check_ptr(delta, "delta", 4)) return rc;
  hipError_t e = launch_bwd_preprocess(p->batch, p->hq, p->sq, p->head_dim, out, d_o, strides3(p->q_stride),
                                       p->dtype, delta, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "backward preprocess kernel launch");
  return ok();
}

int ringattn_step_bwd(const ra_problem* p, const void* q, const void* k_blk, const void* v_blk, const void* d_o,
                      const float* lse, const float* delta, float* dq_acc, float* dk_acc, float* dv_acc,
                      const int32_t* q_pos, const int32_t* kv_pos, const int32_t* q_doc, const int32_t* kv_doc,
                      int mask_mode, int flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = check_problem(p)) return rc;
  if (int rc = check_mask(mask_mode, q_doc, kv_doc, p->sk > 0)) return rc;
  if (flags & ~kStepFlags) return fail(RA_ERR_INVALID, "unknown step flags 0x%x", flags);
  if (p->sq == 0 || p->sk == 0) return ok();
  if (int rc = check_ptr(q, "q")) return rc;
  if (int rc = check_ptr(k_blk, "k_blk")) return rc;
  if (int rc = check_ptr(v_blk, "v_blk")) return rc;
  if (int rc = check_ptr(d_o, "d_o")) return rc;
  if (int rc = check_ptr(lse, "lse", 4)) return rc;
  if (int rc = check_ptr(delta, "delta", 4)) return rc;
  if (int rc = check_ptr(dq_acc, "dq_acc")) return rc;
  if (int rc = check_ptr(dk_acc, "dk_acc")) return rc;
  if (int rc = check_ptr(dv_acc, "dv_acc")) return rc;
  if (int rc = check_ptr(q_pos, "q_pos", 4)) return rc;
  if (int rc = check_ptr(kv_pos, "kv_pos", 4)) return rc;
  const size_t need = step_ws(p->sq, p->sk);
  if (workspace_bytes < need || !workspace)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (!aligned(workspace, 16)) return fail(RA_ERR_INVALID, "workspace is not 16-byte aligned");

  hipStream_t st = (hipStream_t)stream;
  const bool doc = mask_mode == RA_MASK_DOC_CAUSAL;
  StepTables t = carve_step_ws(workspace, p->sq);
  hipError_t e = launch_tile_ranges(q_pos, doc ? q_doc : nullptr, p->sq, t.q, st);
  if (e == hipSuccess) e = launch_tile_ranges(kv_pos, doc ? kv_doc : nullptr, p->sk, t.kv, st);
  if (e != hipSuccess) return hip_fail(e, "tile-range kernel launch");
  BwdArgs a = make_bwd(p, q, k_blk, v_blk, d_o, lse, delta, dq_acc, dk_acc, dv_acc, q_pos, kv_pos, q_doc, kv_doc,
                       t.q, t.kv, mask_mode, flags);
  e = enqueue_bwd(p, a, st);
  if (e != hipSuccess) return hip_fail(e, "backward step kernel launch");
  return ok();
}

int ringattn_docs_from_cu_seqlens(const int32_t* cu_seqlens, int32_t n_docs, int32_t first_token, int32_t n_tokens,
                                  int32_t* doc, void* stream) {
  if (n_docs < 0 || n_tokens < 0 || first_token < 0)
    return fail(RA_ERR_INVALID, "n_docs, first_token and n_tokens must be >= 0");
  if (n_tokens == 0) return ok();
  if (int rc = check_ptr(cu_seqlens, "cu_seqlens", 4)) return rc;
  if (int rc = check_ptr(doc, "doc", 4)) return rc;
  hipError_t e = launch_docs_from_cu(cu_seqlens, n_docs, first_token, n_tokens, doc, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "docs kernel launch");
  return ok();
}

}  // extern "C"

// ------------------------------------------------------------------ ring driver
namespace {

struct RunLayout {
  size_t blk_elems;     // elements of one K (or V) block
  size_t blk_bytes;
  bool vt;              // bf16 forward: value blocks circulate transposed
  size_t vslot_bytes;   // one staged value block (V, or V^T when vt)
  size_t off_vth;       // all-gather with vt: N transposed home value blocks
  size_t off_slots;     // 2 slots x R ranks x (K, V)
  size_t off_qtab;      // R q tables
  size_t off_kvtab;     // N kv tables
  size_t off_part;      // merge-kernel mode: R partial (o, lse)
  size_t qtab_bytes, kvtab_bytes, part_o_bytes, part_l_bytes;
  size_t total;
};

RunLayout run_layout(const ra_run_desc* d) {
  const ra_problem* p = &d->prob;
  RunLayout L{};
  L.blk_elems = (size_t)p->batch * p->hkv * p->sk * p->head_dim;
  L.blk_bytes = align256(L.blk_elems * elem_size(p->dtype));
  L.qtab_bytes = align256((size_t)n_tiles(p->sq) * sizeof(TileRange));
  L.kvtab_bytes = align256((size_t)n_tiles(p->sk) * sizeof(TileRange));
  L.vt = d->pass == RA_PASS_FWD && p->dtype == RA_BF16 && p->sk > 0;
  L.vslot_bytes = L.vt ? vt_ws(p) : L.blk_bytes;
  size_t off = 0;
  L.off_vth = off;
  if (L.vt && (d->flags & RA_RUN_ALLGATHER)) {
    off += (size_t)d->n_ranks * L.vslot_bytes;   // every block resident: no staging slots
  } else {
    L.off_slots = off;
    off += 2 * (size_t)d->n_emulated * (L.blk_bytes + L.vslot_bytes);
  }
  L.off_qtab = off;
  off += (size_t)d->n_emulated * L.qtab_bytes;
  L.off_kvtab = off;
  off += (size_t)d->n_ranks * L.kvtab_bytes;
  L.off_part = off;
  if (d->pass == RA_PASS_FWD && (d->flags & RA_RUN_MERGE_KERNEL)) {
    L.part_o_bytes = align256((size_t)p->batch * p->hq * p->sq * p->head_dim * 4);
    L.part_l_bytes = align256((size_t)p->batch * p->hq * p->sq * 4);
    off += (size_t)d->n_emulated * (L.part_o_bytes + L.part_l_bytes);
  }
  L.total = off;
  return L;
}

const int kRunFlags = RA_NO_SKIP | RA_RUN_SERIAL_COPY | RA_RUN_POISON | RA_RUN_MERGE_KERNEL | RA_RUN_COPY_ENGINE |
                      RA_RUN_ALLGATHER;

int check_run(const ra_run_desc* d) {
  if (!d) return fail(RA_ERR_INVALID, "run descriptor is NULL");
  if (int rc = check_problem(&d->prob)) return rc;
  if (d->n_ranks < 1) return fail(RA_ERR_INVALID, "n_ranks must be >= 1");
  if (d->n_emulated < 1 || d->n_emulated > d->n_ranks)
    return fail(RA_ERR_INVALID, "n_emulated must be in [1, n_ranks]");
  if (d->first_rank < 0 || d->first_rank >= d->n_ranks) return fail(RA_ERR_INVALID, "first_rank out of range");
  const int stop = d->stop_step == 0 ? d->n_ranks : d->stop_step;
  if (d->start_step < 0 || d->start_step >= d->n_ranks) return fail(RA_ERR_INVALID, "start_step out of range");
  if (stop <= d->start_step || stop > d->n_ranks) return fail(RA_ERR_INVALID, "stop_step out of range");
  if (d->pass != RA_PASS_FWD && d->pass != RA_PASS_BWD) return fail(RA_ERR_INVALID, "pass must be 1 or 2");
  if (d->flags & ~kRunFlags) return fail(RA_ERR_INVALID, "unknown run flags 0x%x", d->flags);
  if (d->flags & RA_RUN_ALLGATHER) {
    if (d->pass != RA_PASS_FWD) return fail(RA_ERR_INVALID, "RA_RUN_ALLGATHER is a forward-pass mode");
    if (d->prob.dtype != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "RA_RUN_ALLGATHER is bf16 only");
    if (d->n_ranks > RA_FUSED_MAX_BLOCKS)
      return fail(RA_ERR_UNSUPPORTED, "RA_RUN_ALLGATHER takes at most %d ranks", RA_FUSED_MAX_BLOCKS);
    if (d->start_step != 0 || (d->stop_step != 0 && d->stop_step != d->n_ranks))
      return fail(RA_ERR_INVALID, "RA_RUN_ALLGATHER runs the whole ring (start_step 0, stop_step n_ranks)");
  }
  const ra_problem* p = &d->prob;
  const int64_t* s = p->kv_stride;
  const int64_t span = (int64_t)(p->batch - 1) * s[0] + (int64_t)(p->hkv - 1) * s[1] + (int64_t)(p->sk - 1) * s[2] +
                       p->head_dim;
  if (p->sk > 0 && span != (int64_t)p->batch * p->hkv * p->sk * p->head_dim)
    return fail(RA_ERR_INVALID, "ringattn_run needs densely packed key/value blocks (strides cover %lld elements)",
                (long long)span);
  return RA_OK;
}

// Flags of the events that order the copy and compute streams of a ring.  They serve
// device-side waits only (the host never inspects them), and the kernels on either side
// carry device-scope fences of their own in their dispatch, so the system-scope fence an event
// performs on completion is left out: a `done` event sits between two step kernels on
// the compute stream, where that fence (a cache write-back and invalidation) would delay
// the next step.
#ifndef RA_RING_EVENT_FLAGS
#define RA_RING_EVENT_FLAGS (hipEventDisableTiming | hipEventDisableSystemFence)
#endif

struct Events {
  std::vector<hipEvent_t> ev;
  ~Events() {
    for (auto e : ev) (void)hipEventDestroy(e);
  }
  hipError_t make(hipEvent_t* out) {
    hipError_t e = hipEventCreateWithFlags(out, RA_RING_EVENT_FLAGS);
    if (e == hipSuccess) ev.push_back(*out);
    return e;
  }
};

}  // namespace

extern "C" size_t ringattn_run_workspace_size(const ra_run_desc* d) {
  if (check_run(d)) return 0;
  return run_layout(d).total;
}

extern "C" int ringattn_run(const ra_run_desc* d, const void* const* q, const void* const* k_home,
                            const void* const* v_home, float* const* o_acc, float* const* lse, void* const* out,
                            const int32_t* const* q_pos, const int32_t* const* kv_pos,
                            const int32_t* const* q_doc, const int32_t* const* kv_doc, const void* const* d_o,
                            float* const* delta, float* const* dq, float* const* dk, float* const* dv,
                            void* workspace, size_t workspace_bytes, void* compute_stream, void* copy_stream) {
  if (int rc = check_run(d)) return rc;
  const ra_problem* p = &d->prob;
  const int N = d->n_ranks, R = d->n_emulated;
  const int start = d->start_step, stop = d->stop_step == 0 ? N : d->stop_step;
  const int mask = d->mask_mode;
  const bool fwd = d->pass == RA_PASS_FWD;
  const bool doc = mask == RA_MASK_DOC_CAUSAL;
  if (mask < RA_MASK_NONE || mask > RA_MASK_DOC_CAUSAL)
    return fail(RA_ERR_UNSUPPORTED, "mask_mode %d not supported (none, causal, doc-causal)", mask);
  if (p->sq == 0) return ok();

  // ---- host-side validation of every pointer the selected pass uses ----
  if (!q || !k_home || !v_home || !q_pos || !kv_pos) return fail(RA_ERR_INVALID, "q, k_home, v_home, q_pos and kv_pos arrays are required");
  if (doc && (!q_doc || !kv_doc)) return fail(RA_ERR_INVALID, "doc-causal mask needs q_doc and kv_doc arrays");
  const bool allgather = (d->flags & RA_RUN_ALLGATHER) != 0;
  if (fwd && !allgather && (!o_acc || !lse)) return fail(RA_ERR_INVALID, "forward needs o_acc and lse arrays");
  if (allgather && (!lse || !out)) return fail(RA_ERR_INVALID, "all-gather mode needs lse and out arrays");
  if (!fwd && (!lse || !out || !d_o || !delta || !dq || !dk || !dv))
    return fail(RA_ERR_INVALID, "backward needs lse, out, d_o, delta, dq, dk and dv arrays");
  char name[64];
  for (int i = 0; i < R; ++i) {
    snprintf(name, sizeof name, "q[%d]", i);
    if (int rc = check_ptr(q[i], name)) return rc;
    snprintf(name, sizeof name, "q_pos[%d]", i);
    if (int rc = check_ptr(q_pos[i], name, 4)) return rc;
    if (doc) {
      snprintf(name, sizeof name, "q_doc[%d]", i);
      if (int rc = check_ptr(q_doc[i], name, 4)) return rc;
    }
    snprintf(name, sizeof name, "lse[%d]", i);
    if (int rc = check_ptr(lse[i], name, 4)) return rc;
    if (fwd && allgather) {
      snprintf(name, sizeof name, "out[%d]", i);
      if (int rc = check_ptr(out[i], name)) return rc;
    } else if (fwd) {
      snprintf(name, sizeof name, "o_acc[%d]", i);
      if (int rc = check_ptr(o_acc[i], name)) return rc;
      if (out && out[i] && !aligned(out[i], 16)) return fail(RA_ERR_INVALID, "out[%d] is not 16-byte aligned", i);
    } else {
      snprintf(name, sizeof name, "out[%d]", i);
      if (int rc = check_ptr(out[i], name)) return rc;
      snprintf(name, sizeof name, "d_o[%d]", i);
      if (int rc = check_ptr(d_o[i], name)) return rc;
      snprintf(name, sizeof name, "delta[%d]", i);
      if (int rc = check_ptr(delta[i], name, 4)) return rc;
      snprintf(name, sizeof name, "dq[%d]", i);
      if (int rc = check_ptr(dq[i], name)) return rc;
    }
  }
  if (p->sk > 0) {
    for (int n = 0; n < N; ++n) {
      snprintf(name, sizeof name, "k_home[%d]", n);
      if (int rc = check_ptr(k_home[n], name)) return rc;
      snprintf(name, sizeof name, "v_home[%d]", n);
      if (int rc = check_ptr(v_home[n], name)) return rc;
      snprintf(name, sizeof name, "kv_pos[%d]", n);
      if (int rc = check_ptr(kv_pos[n], name, 4)) return rc;
      if (doc) {
        snprintf(name, sizeof name, "kv_doc[%d]", n);
        if (int rc = check_ptr(kv_doc[n], name, 4)) return rc;
      }
      if (!fwd) {
        snprintf(name, sizeof name, "dk[%d]", n);
        if (int rc = check_ptr(dk[n], name)) return rc;
        snprintf(name, sizeof name, "dv[%d]", n);
        if (int rc = check_ptr(dv[n], name)) return rc;
      }
    }
  }
  const RunLayout L = run_layout(d);
  if (workspace_bytes < L.total || (L.total && !workspace))
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, workspace_bytes);
  if (!aligned(workspace, 256)) return fail(RA_ERR_INVALID, "workspace is not 256-byte aligned");

  // ---- enqueue ----
  hipStream_t cs = (hipStream_t)compute_stream;
  hipStream_t xs = (hipStream_t)copy_stream;
  const bool serial = (d->flags & RA_RUN_SERIAL_COPY) || xs == nullptr || xs == cs;
  if (serial) xs = cs;
  const bool poison = (d->flags & RA_RUN_POISON) != 0;
  const hipMemcpyKind copy_kind = (d->flags & RA_RUN_COPY_ENGINE) ? hipMemcpyDeviceToDeviceNoCU
                                                                    : hipMemcpyDeviceToDevice;
  const int step_flags_extra = d->flags & RA_NO_SKIP;
  char* ws = (char*)workspace;
  auto slot_k = [&](int slot, int i) {
    return (void*)(ws + L.off_slots + (size_t)(slot * R + i) * (L.blk_bytes + L.vslot_bytes));
  };
  auto slot_v = [&](int slot, int i) { return (void*)((char*)slot_k(slot, i) + L.blk_bytes); };
  auto qtab = [&](int i) { return (TileRange*)(ws + L.off_qtab + (size_t)i * L.qtab_bytes); };
  auto kvtab = [&](int n) { return (TileRange*)(ws + L.off_kvtab + (size_t)n * L.kvtab_bytes); };
  auto rank_of = [&](int i) { return (d->first_rank + i) % N; };
  auto block_of = [&](int i, int t) { return ((rank_of(i) - t) % N + N) % N; };
  const size_t copy_bytes = L.blk_elems * elem_size(p->dtype);

  Events evs;
  hipError_t e;
  std::vector<hipEvent_t> ready(N, nullptr), done(N, nullptr);
  hipEvent_t inputs_ready = nullptr;
  if (!serial) {
    // the copy stream must not read the home blocks before the compute stream's earlier work made them
    if ((e = evs.make(&inputs_ready)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    if ((e = hipEventRecord(inputs_ready, cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipStreamWaitEvent(xs, inputs_ready, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    for (int t = start; t < stop; ++t) {
      if ((e = evs.make(&ready[t])) != hipSuccess) return hip_fail(e, "hipEventCreate");
      if ((e = evs.make(&done[t])) != hipSuccess) return hip_fail(e, "hipEventCreate");
    }
  }

  // tile tables: every emulated rank's queries and every block's keys
  {
    // one launch per TABLE_JOBS tables
    TableJobs jobs{};
    auto add = [&](TableJob jb) -> hipError_t {
      jobs.job[jobs.count++] = jb;
      if (jobs.count < TABLE_JOBS) return hipSuccess;
      const hipError_t err = launch_tile_ranges_batch(jobs, cs);
      jobs.count = 0;
      return err;
    };
    for (int i = 0; i < R; ++i)
      if ((e = add(TableJob{q_pos[i], doc ? q_doc[i] : nullptr, qtab(i), p->sq})) != hipSuccess)
        return hip_fail(e, "tile-range kernel launch");
    for (int n = 0; n < N && p->sk > 0; ++n)
      if ((e = add(TableJob{kv_pos[n], doc ? kv_doc[n] : nullptr, kvtab(n), p->sk})) != hipSuccess)
        return hip_fail(e, "tile-range kernel launch");
    if ((e = launch_tile_ranges_batch(jobs, cs)) != hipSuccess) return hip_fail(e, "tile-range kernel launch");
  }
  if (!fwd)
    for (int i = 0; i < R; ++i)
      if ((e = launch_bwd_preprocess(p->batch, p->hq, p->sq, p->head_dim, out[i], d_o[i], strides3(p->q_stride),
                                     p->dtype, delta[i], cs)) != hipSuccess)
        return hip_fail(e, "backward preprocess kernel launch");
  if (allgather) {
    // every block is resident: one launch per emulated rank over all of them, in ring order.
    // The transposed value blocks are what an all-gather of V^T would deliver (each rank
    // transposes its own block once); emulated here for all N blocks.
    auto vth = [&](int n) { return (void*)(ws + L.off_vth + (size_t)n * L.vslot_bytes); };
    for (int n = 0; n < N && L.vt; ++n)
      if ((e = transpose_v(p, v_home[n], vth(n), cs)) != hipSuccess) return hip_fail(e, "value transpose kernel launch");
    if (d->step_events && d->step_events[0] && (e = hipEventRecord((hipEvent_t)d->step_events[0], cs)) != hipSuccess)
      return hip_fail(e, "hipEventRecord (step_events)");
    for (int i = 0; i < R; ++i) {
      const int n0 = block_of(i, 0);
      FwdArgs a = make_fwd(p, q[i], k_home[n0], v_home[n0], nullptr, lse[i], out[i], q_pos[i], kv_pos[n0],
                           doc ? q_doc[i] : nullptr, doc ? kv_doc[n0] : nullptr, qtab(i), kvtab(n0), mask,
                           step_flags_extra | RA_STEP_FIRST | RA_STEP_LAST);
      a.n_blocks = N;
      for (int t = 0; t < N; ++t) {
        const int n = block_of(i, t);
        a.kb[t] = k_home[n];
        a.vb[t] = v_home[n];
        if (L.vt) a.vtb[t] = vth(n);
        a.kposb[t] = kv_pos[n];
        a.kdocb[t] = doc ? kv_doc[n] : nullptr;
        a.ktilesb[t] = kvtab(n);
      }
      if ((e = launch_fwd_bf16(a, p->head_dim, cs)) != hipSuccess) return hip_fail(e, "fused forward kernel launch");
    }
    if (d->step_events && d->step_events[1] && (e = hipEventRecord((hipEvent_t)d->step_events[1], cs)) != hipSuccess)
      return hip_fail(e, "hipEventRecord (step_events)");
    return ok();
  }

  // Copy block (rank - t) of every emulated rank into slot t & 1.  In the bf16 forward
  // the value block travels transposed: its copy is the transpose kernel (always on
  // the compute units) and step 0 transposes the home block on the compute stream.
  auto issue_copy = [&](int t) -> hipError_t {
    hipError_t err = hipSuccess;
    const int slot = t & 1;
    for (int i = 0; i < R && p->sk > 0; ++i) {
      const int n = block_of(i, t);
      if (poison) {
        if ((err = launch_fill_nan(slot_k(slot, i), copy_bytes, xs)) != hipSuccess) return err;
        if ((err = launch_fill_nan(slot_v(slot, i), L.vt ? vt_block_bytes(p->batch, p->hkv, p->head_dim, p->sk)
                                                           : copy_bytes, xs)) != hipSuccess) return err;
      }
      if ((err = hipMemcpyAsync(slot_k(slot, i), k_home[n], copy_bytes, copy_kind, xs)) != hipSuccess) return err;
      if (L.vt)
        err = transpose_v(p, v_home[n], slot_v(slot, i), xs);
      else
        err = hipMemcpyAsync(slot_v(slot, i), v_home[n], copy_bytes, copy_kind, xs);
      if (err != hipSuccess) return err;
    }
    return err;
  };
  if (L.vt && start == 0)
    for (int i = 0; i < R; ++i)
      if ((e = transpose_v(p, v_home[block_of(i, 0)], slot_v(0, i), cs)) != hipSuccess)
        return hip_fail(e, "value transpose kernel launch");

  // Step `start` needs its block before the loop when it is not the home block.
  if (start >= 1) {
    if ((e = issue_copy(start)) != hipSuccess) return hip_fail(e, "staging copy");
    if (!serial && (e = hipEventRecord(ready[start], xs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  }

  for (int t = start; t < stop; ++t) {
    // prefetch the block of step t+1 while step t computes
    if (t + 1 < stop) {
      if (!serial && t - 1 >= start && (e = hipStreamWaitEvent(xs, done[t - 1], 0)) != hipSuccess)
        return hip_fail(e, "hipStreamWaitEvent");   // slot (t+1)&1 was last read by step t-1
      if (!serial) {
        if ((e = issue_copy(t + 1)) != hipSuccess) return hip_fail(e, "staging copy");
        if ((e = hipEventRecord(ready[t + 1], xs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
      }
    }
    if (!serial && t >= 1 && (e = hipStreamWaitEvent(cs, ready[t], 0)) != hipSuccess)
      return hip_fail(e, "hipStreamWaitEvent");
    if (serial && t >= 1 && t != start) {
      if ((e = issue_copy(t)) != hipSuccess) return hip_fail(e, "staging copy");
    }

    if (d->step_events && d->step_events[2 * t] &&
        (e = hipEventRecord((hipEvent_t)d->step_events[2 * t], cs)) != hipSuccess)
      return hip_fail(e, "hipEventRecord (step_events)");
    int flags = step_flags_extra;
    if (t == 0) flags |= RA_STEP_FIRST;
    if (t == N - 1) flags |= RA_STEP_LAST;
    for (int i = 0; i < R; ++i) {
      const int n = block_of(i, t);
      const void* kb = t == 0 ? k_home[n] : slot_k(t & 1, i);
      const void* vb = t == 0 && !L.vt ? v_home[n] : slot_v(t & 1, i);
      if (fwd) {
        const bool merge_k = (d->flags & RA_RUN_MERGE_KERNEL) != 0 && !(flags & RA_STEP_FIRST);
        if (!merge_k) {
          FwdArgs a = make_fwd(p, q[i], kb, vb, o_acc[i], lse[i], out ? out[i] : nullptr, q_pos[i], kv_pos[n],
                               doc ? q_doc[i] : nullptr, doc ? kv_doc[n] : nullptr, qtab(i), kvtab(n), mask, flags);
          if (L.vt) a.vb[0] = nullptr;   // only the transposed copy is staged
          if ((e = enqueue_fwd(p, a, cs)) != hipSuccess) return hip_fail(e, "forward step kernel launch");
        } else {
          float* po = (float*)(ws + L.off_part + (size_t)i * (L.part_o_bytes + L.part_l_bytes));
          float* pl = (float*)((char*)po + L.part_o_bytes);
          FwdArgs a = make_fwd(p, q[i], kb, vb, po, pl, nullptr, q_pos[i], kv_pos[n], doc ? q_doc[i] : nullptr,
                               doc ? kv_doc[n] : nullptr, qtab(i), kvtab(n), mask,
                               (flags & RA_NO_SKIP) | RA_STEP_FIRST);
          if (L.vt) a.vb[0] = nullptr;
          if ((e = enqueue_fwd(p, a, cs)) != hipSuccess) return hip_fail(e, "forward step kernel launch");
          void* fin = (flags & RA_STEP_LAST) && out ? out[i] : nullptr;
          if ((e = launch_merge((int64_t)p->batch * p->hq * p->sq, p->head_dim, po, pl, o_acc[i], lse[i], fin,
                                strides3(p->q_stride), p->hq, p->sq, p->dtype, cs)) != hipSuccess)
            return hip_fail(e, "merge kernel launch");
        }
      } else if (p->sk > 0) {
        BwdArgs a = make_bwd(p, q[i], kb, vb, d_o[i], lse[i], delta[i], dq[i], dk[n], dv[n], q_pos[i], kv_pos[n],
                             doc ? q_doc[i] : nullptr, doc ? kv_doc[n] : nullptr, qtab(i), kvtab(n), mask, flags);
        if ((e = enqueue_bwd(p, a, cs)) != hipSuccess) return hip_fail(e, "backward step kernel launch");
      }
    }
    if (d->step_events && d->step_events[2 * t + 1] &&
        (e = hipEventRecord((hipEvent_t)d->step_events[2 * t + 1], cs)) != hipSuccess)
      return hip_fail(e, "hipEventRecord (step_events)");
    if (!serial && (e = hipEventRecord(done[t], cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  return ok();
}
