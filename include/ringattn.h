/*
 * ringattn.h -- C ABI of the per-device hot path of ring attention on MI355X.
 *
 * Ring attention (the NVSHMEM page, "Optimización en el entrenamiento de
 * modelos de lenguaje de largo contexto con NVSHMEM en JAX y XLA", section
 * "Paralelismo de contexto y atención en anillo") splits the sequence over N
 * ranks: every rank keeps its
 * query shard Q_i, attends to its own key/value block and then to every other
 * rank's block as the blocks travel around a ring, computing attention
 * incrementally; the combined result equals standard attention.  The
 * Accelerate guide ("Context Parallel no 🤗 accelerate", section "Então, como
 * funciona?" and its pseudocode) describes the same loop as attn(Q_i, K_j, V_j)
 * per block followed by combine().  This library implements, on one GPU:
 *
 *   ringattn_step_fwd        attn(Q_i, K_j, V_j) with the combine fused in
 *   ringattn_fused_fwd       all blocks resident: attention over every block in one launch
 *   ringattn_merge           combine() of two normalised partial results
 *   ringattn_bwd_preprocess  D = rowsum(dO * O), needed by the backward
 *   ringattn_step_bwd        gradient contributions of one block
 *   ringattn_run             the whole ring of N steps, the next block copied
 *                            device-to-device into a staging slot on a side
 *                            stream while the current one is computed
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked "device" are HIP device pointers; every other pointer is a
 *   host pointer.  Streams are hipStream_t handles passed as void* (NULL is
 *   the legacy default stream).
 * - The caller allocates and owns every buffer, the workspace and the streams.
 *   The library never allocates or frees device memory, never synchronises the
 *   device and keeps no pointer after returning.  Work is enqueued
 *   asynchronously; device faults surface at the caller's next synchronise.
 * - Validation is pure host code and runs before any HIP call.  On an error
 *   nothing is enqueued and no output is touched; ringattn_last_error() gives
 *   the reason.  Well-formed but unsupported input (the Accelerate guide,
 *   section "Como usar paralelismo de contexto?", raises an error for
 *   attention it cannot handle: SDPA with no mask or a causal mask only)
 *   returns RA_ERR_UNSUPPORTED.
 * - Layouts.  q, d_o and out (the problem dtype) are [B][Hq][Sq][D] and k, v
 *   are [B][Hkv][Sk][D], addressed through (batch, head, token) strides in
 *   elements with D contiguous; a packed THD tensor [T][H][D] is B = 1 with
 *   head stride D and token stride H*D.  The fp32 buffers o_acc, dq are dense
 *   [B][Hq][Sq][D]; dk, dv are dense [B][Hkv][Sk][D]; lse and delta are dense
 *   [B][Hq][Sq].  Strides must be positive multiples of 8 elements and every
 *   device pointer 16-byte aligned.
 * - Positions q_pos[Sq], kv_pos[Sk] are the tokens' global indices (int32,
 *   device, 0 <= pos < 2^31 - 1), shared by all batches and heads.  Documents
 *   q_doc[Sq], kv_doc[Sk] (int32, device) are needed only for
 *   RA_MASK_DOC_CAUSAL; ringattn_docs_from_cu_seqlens builds them.
 * - Mask (the Accelerate guide, section "Como usar paralelismo de contexto?":
 *   SDPA with no mask or a causal mask; the Dynamic-CP page, section
 *   "Reprogramación dinámica y empaquetado de datos": packed THD sequences
 *   described by cu_seqlens):
 *     RA_MASK_NONE        every key visible
 *     RA_MASK_CAUSAL      key visible iff kv_pos <= q_pos
 *     RA_MASK_DOC_CAUSAL  causal and kv_doc == q_doc
 * - Softmax scale: softmax_scale, or 1/sqrt(D) when it is 0 (SDPA's default).
 * - GQA: query head h reads key/value head floor(h * Hkv / Hq); Hq % Hkv == 0.
 * - Normalised partial results: after any step, (o_acc, lse) hold attention of
 *   Q over the union of the blocks seen so far, o_acc normalised and lse the
 *   natural log of the softmax denominator (-inf and o_acc = 0 for a row that
 *   has seen no visible key).  This makes every step a resumable checkpoint.
 */
#ifndef RINGATTN_H
#define RINGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RINGATTN_VERSION 2

typedef enum {
  RA_OK = 0,
  RA_ERR_INVALID = -1,      /* malformed arguments (null pointer, bad size, alignment, stride) */
  RA_ERR_UNSUPPORTED = -2,  /* well-formed but not handled (head_dim, dtype, mask mode, size cap) */
  RA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than the *_workspace_size query */
  RA_ERR_HIP = -4           /* a HIP call failed while enqueueing */
} ra_status;

typedef enum { RA_MASK_NONE = 0, RA_MASK_CAUSAL = 1, RA_MASK_DOC_CAUSAL = 2 } ra_mask_mode;
typedef enum { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;

/* step flags */
enum {
  RA_STEP_FIRST = 1,   /* first step of a ring: ignore the contents of o_acc/lse and overwrite them */
  RA_STEP_LAST = 2,    /* last step: also write the final output `out` (problem dtype) when non-NULL */
  RA_NO_SKIP = 4       /* debug: do not skip fully masked tiles (results must not change) */
};

/* ringattn_run flags (RA_NO_SKIP applies too) */
enum {
  RA_RUN_SERIAL_COPY = 16,   /* copy each block on the compute stream (no overlap) */
  RA_RUN_POISON = 32,        /* fill a staging slot with NaN right before each copy into it */
  RA_RUN_MERGE_KERNEL = 64,  /* forward: step kernel writes a separate partial, then ringattn_merge */
  RA_RUN_COPY_ENGINE = 128,  /* stage blocks with the DMA-engine copy (hipMemcpyDeviceToDeviceNoCU)
                                instead of a copy kernel that shares the compute units */
  RA_RUN_ALLGATHER = 256     /* forward pass, all blocks resident (the all-gather rotation): each
                                emulated rank does ONE ringattn_fused_fwd launch over all n_ranks
                                home blocks (in ring order) instead of n_ranks steps; no staging
                                copies, o_acc is not written, out[i] is required.  bf16 only,
                                n_ranks <= RA_FUSED_MAX_BLOCKS, the whole ring (start 0, stop n). */
};

enum { RA_PASS_FWD = 1, RA_PASS_BWD = 2 };

/* Largest key/value block (tokens) one step handles; larger is RA_ERR_UNSUPPORTED. */
#define RA_MAX_SK 262144

/* One attention problem: a local query shard against one key/value block. */
typedef struct {
  int32_t batch;        /* B  >= 1 */
  int32_t hq;           /* query heads >= 1 */
  int32_t hkv;          /* key/value heads >= 1, hq % hkv == 0 */
  int32_t head_dim;     /* D: 64 or 128 */
  int32_t sq;           /* tokens of the query shard >= 0 (0 = nothing to do) */
  int32_t sk;           /* tokens of the key/value block >= 0, <= RA_MAX_SK */
  int64_t q_stride[3];  /* (batch, head, token) strides in elements of q, d_o and out */
  int64_t kv_stride[3]; /* (batch, head, token) strides in elements of k and v; every stride a
                           positive multiple of 8, a token stride below 2^31 / (128 x element
                           size) (RA_ERR_UNSUPPORTED otherwise) */
  int32_t dtype;        /* ra_dtype of q, k, v, d_o and out; accumulation is fp32 */
  float softmax_scale;  /* 0 = 1/sqrt(head_dim) */
} ra_problem;

/* Bytes of device workspace the step entry points need for this problem
 * (per-tile position/document ranges used to skip fully masked tiles; for
 * bf16, room for the value block transposed to [B][Hkv][D][Sk rounded up to
 * 64], which the forward step writes there and reads its V^T tiles from). */
size_t ringattn_step_workspace_size(const ra_problem* p);

/*
 * One forward ring step: attention of q against one block (k_blk, v_blk),
 * merged into the running normalised result (o_acc, lse) with the exact
 * log-sum-exp combine (the combine of the Accelerate guide's pseudocode,
 * section "Então, como funciona?", left undefined there, read as the only
 * combine that keeps equality with full attention: the NVSHMEM page, section
 * "Paralelismo de contexto y atención en anillo").
 *   q [B,Hq,Sq,D], k_blk/v_blk [B,Hkv,Sk,D]      (device, problem dtype, in)
 *   o_acc [B,Hq,Sq,D] fp32, lse [B,Hq,Sq] fp32    (device, in/out; out only with RA_STEP_FIRST)
 *   out [B,Hq,Sq,D] problem dtype, q_stride        (device, out, only with RA_STEP_LAST; may be NULL)
 *   q_pos, kv_pos, q_doc, kv_doc                  (device int32, in; docs only for DOC_CAUSAL)
 *   workspace                                     (device, >= ringattn_step_workspace_size bytes)
 * Fully masked (query tile, key tile) pairs are skipped; their result is unchanged by it.
 */
int ringattn_step_fwd(const ra_problem* p, const void* q, const void* k_blk, const void* v_blk,
                      float* o_acc, float* lse, void* out,
                      const int32_t* q_pos, const int32_t* kv_pos,
                      const int32_t* q_doc, const int32_t* kv_doc,
                      int mask_mode, int flags, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Bytes of the device scratch array behind ringattn_step_fwd_noalloc (36 MiB per GPU). */
#define RA_NOALLOC_SCRATCH_BYTES (36u << 20)

/*
 * ringattn_step_fwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and errors as ringattn_step_fwd; the
 * tile tables and the transposed value block go into a file-scope device array of
 * RA_NOALLOC_SCRATCH_BYTES that each GPU holds from the library's first use of it on
 * that device until the process ends.  The call allocates and frees nothing.
 *   Limit: ringattn_step_workspace_size(p) <= RA_NOALLOC_SCRATCH_BYTES, else
 *   RA_ERR_UNSUPPORTED (e.g. 16384-key blocks of 8 kv heads at D = 128 fit: 32 MiB of
 *   transposed values; 32768-key blocks do not).
 *   Device: the calling thread's current device, which must be the stream's
 *   (RA_ERR_INVALID otherwise); its first call on a device looks up the array's
 *   address there.
 *   Concurrency: every call on one GPU shares that GPU's array.  Calls on one stream
 *   are ordered; calls that overlap on one GPU (several streams, several threads)
 *   race on it and give wrong results.  Nothing in the array has to start at zero:
 *   each call writes every byte it reads.
 */
int ringattn_step_fwd_noalloc(const ra_problem* p, const void* q, const void* k_blk, const void* v_blk,
                              float* o_acc, float* lse, void* out,
                              const int32_t* q_pos, const int32_t* kv_pos,
                              const int32_t* q_doc, const int32_t* kv_doc,
                              int mask_mode, int flags, void* stream);

/* Most K/V blocks one ringattn_fused_fwd call takes. */
#define RA_FUSED_MAX_BLOCKS 16

/* Bytes of device workspace ringattn_fused_fwd needs (per-tile ranges of the
 * queries and of each of the n_blocks blocks, and each value block
 * transposed, as for ringattn_step_fwd). */
size_t ringattn_fused_workspace_size(const ra_problem* p, int n_blocks);

/*
 * All-gather forward (the page "Context Parallel no 🤗 accelerate", section
 * "all-to-all vs all-gather": the all-gather variant): once every K,V block is
 * resident, attention of q against all n_blocks blocks in ONE launch.  The
 * tile list of a query tile spans every block and the online-softmax state
 * stays in registers across blocks, so unlike a ring of ringattn_step_fwd
 * calls there is no running fp32 output between blocks; the result is exactly
 * full attention over the union of the blocks (up to rounding order).
 *   p->sk                       keys per block; every block has the same size and kv_stride
 *   k_blocks, v_blocks          host arrays of n_blocks device pointers, [B,Hkv,Sk,D] bf16 (in)
 *   kv_pos, kv_doc              host arrays of n_blocks device int32 pointers (in; docs only
 *                               for DOC_CAUSAL, else kv_doc may be NULL)
 *   lse [B,Hq,Sq] fp32 dense, out [B,Hq,Sq,D] bf16 with q_stride   (device, out)
 *   workspace                   device, >= ringattn_fused_workspace_size(p, n_blocks) bytes
 * 1 <= n_blocks <= RA_FUSED_MAX_BLOCKS.  bf16 only (fp32 problems return
 * RA_ERR_UNSUPPORTED).  flags: 0 or RA_NO_SKIP.  The pointer arrays are read
 * during the call only.
 */
int ringattn_fused_fwd(const ra_problem* p, int n_blocks, const void* q,
                       const void* const* k_blocks, const void* const* v_blocks,
                       float* lse, void* out,
                       const int32_t* q_pos, const int32_t* const* kv_pos,
                       const int32_t* q_doc, const int32_t* const* kv_doc,
                       int mask_mode, int flags, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * combine() of two normalised partials over disjoint key sets, in place into b:
 *   lse_b' = ln(exp(lse_a) + exp(lse_b)),
 *   o_b'   = exp(lse_a - lse_b') o_a + exp(lse_b - lse_b') o_b,
 * with lse = -inf (o = 0) the identity.  o_a, o_b [B,Hq,Sq,D] fp32 dense;
 * lse_a, lse_b [B,Hq,Sq] fp32 (device).  Only p->batch, hq, sq, head_dim are read.
 */
int ringattn_merge(const ra_problem* p, const float* o_a, const float* lse_a,
                   float* o_b, float* lse_b, void* stream);

/*
 * delta[b,h,i] = sum_d d_o[b,h,i,d] * out[b,h,i,d] (fp32), from the final
 * output `out` and its gradient d_o (device, problem dtype, q_stride).
 */
int ringattn_bwd_preprocess(const ra_problem* p, const void* out, const void* d_o, float* delta,
                            void* stream);

/*
 * Gradient contributions of one block, recomputing the attention weights from
 * the final lse (no merge is needed in the backward):
 *   P = exp(s - lse), dV += P^T dO, dP = dO V^T, dS = P (dP - delta),
 *   dQ += scale dS K, dK += scale dS^T Q
 * dq_acc [B,Hq,Sq,D], dk_acc/dv_acc [B,Hkv,Sk,D] fp32 dense (device) are
 * accumulated (+=); zero them before the first step.  dk/dv sum over the query
 * heads of each GQA group.  lse and delta are the final forward LSE and
 * ringattn_bwd_preprocess's output.
 */
int ringattn_step_bwd(const ra_problem* p, const void* q, const void* k_blk, const void* v_blk,
                      const void* d_o, const float* lse, const float* delta,
                      float* dq_acc, float* dk_acc, float* dv_acc,
                      const int32_t* q_pos, const int32_t* kv_pos,
                      const int32_t* q_doc, const int32_t* kv_doc,
                      int mask_mode, int flags, void* workspace, size_t workspace_bytes,
                      void* stream);

/* A ring of N key/value blocks and R emulated ranks on one GPU. */
typedef struct {
  ra_problem prob;      /* per-rank problem: sq = shard tokens, sk = block tokens */
  int32_t n_ranks;      /* N >= 1: ring size = number of key/value blocks */
  int32_t n_emulated;   /* R, 1 <= R <= N: ranks computed here */
  int32_t first_rank;   /* emulated rank i is (first_rank + i) mod N */
  int32_t start_step;   /* first step to run, 0 <= start_step < N (resume point) */
  int32_t stop_step;    /* one past the last step to run; 0 means N */
  int32_t mask_mode;    /* ra_mask_mode */
  int32_t pass;         /* RA_PASS_FWD or RA_PASS_BWD */
  int32_t flags;        /* RA_NO_SKIP | RA_RUN_* */
  /* Optional observability: NULL, or a host array of 2*N hipEvent_t created by
   * the caller; events [2t] and [2t+1] are recorded on compute_stream right
   * before and right after the kernels of step t (after its wait for the
   * staged block), so their elapsed time is the step's compute time. */
  void* const* step_events;
} ra_run_desc;

/* Bytes of device workspace ringattn_run needs: two staging slots of one
 * key/value block per emulated rank (in the bf16 forward the value slot
 * holds the block transposed, see ringattn_step_fwd), plus tile tables; with
 * RA_RUN_ALLGATHER, the N value blocks transposed instead of the slots. */
size_t ringattn_run_workspace_size(const ra_run_desc* d);

/*
 * The ring: at step t emulated rank r attends to block (r - t) mod N, which
 * it holds after t hops of "send to the next rank" (NVSHMEM/XLA page: point
 * to point transfers of KV to the next device, computed on while the next
 * block is fetched).  Step 0 reads the rank's own home block; every later
 * block is copied device-to-device from its home buffer into a staging slot
 * of the workspace, one step ahead, on copy_stream, double-buffered and
 * ordered with events so a slot is not overwritten before the step that
 * reads it has finished.  In the bf16 forward the value block travels
 * transposed: its staging copy is a transpose on copy_stream, and step 0
 * transposes the home block on compute_stream.  All arrays below are host arrays of device
 * pointers, indexed by emulated rank i (length R) or by block owner n
 * (length N).
 *
 * Forward (pass RA_PASS_FWD): q[i], k_home[n], v_home[n], q_pos[i],
 *   kv_pos[n], q_doc[i], kv_doc[n] in; o_acc[i], lse[i] out (running
 *   normalised result, valid after every step); out[i] written at step N-1
 *   when non-NULL.
 * Backward (pass RA_PASS_BWD): q, k_home, v_home, out (the forward output),
 *   lse (the final forward LSE), d_o in; delta[i] written first; dq[i],
 *   dk[n], dv[n] accumulated (+=): rank r's contribution to block n's dK/dV
 *   lands in dk[n]/dv[n], where the real ring would send it back to n.
 * Unused arrays may be NULL.  compute_stream runs the kernels; copy_stream the
 * staging copies (NULL or equal to compute_stream means serial copies).
 * Returns after enqueueing; synchronise compute_stream before reading results.
 * Calls that share a workspace must not overlap.
 */
int ringattn_run(const ra_run_desc* d,
                 const void* const* q, const void* const* k_home, const void* const* v_home,
                 float* const* o_acc, float* const* lse, void* const* out,
                 const int32_t* const* q_pos, const int32_t* const* kv_pos,
                 const int32_t* const* q_doc, const int32_t* const* kv_doc,
                 const void* const* d_o, float* const* delta,
                 float* const* dq, float* const* dk, float* const* dv,
                 void* workspace, size_t workspace_bytes,
                 void* compute_stream, void* copy_stream);

/*
 * doc[t] = k for cu_seqlens[k] <= first_token + t < cu_seqlens[k+1], for
 * t in [0, n_tokens): the document id of each token of a packed THD stream
 * (the Dynamic-CP page, "Optimización del entrenamiento variable con Dynamic
 * Context Parallelism en Megatron Core", section "Reprogramación dinámica y
 * empaquetado de datos": cu_seqlens describes the packed sequences).  cu_seqlens
 * [n_docs+1] int32 ascending with cu_seqlens[0] = 0 (device); doc [n_tokens]
 * int32 (device).  Tokens outside every document get doc = -1.
 */
int ringattn_docs_from_cu_seqlens(const int32_t* cu_seqlens, int32_t n_docs, int32_t first_token,
                                  int32_t n_tokens, int32_t* doc, void* stream);

/* Reason for the last error on this thread ("" if none); valid until the next call. */
const char* ringattn_last_error(void);

/* RINGATTN_VERSION of the loaded library. */
int ringattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RINGATTN_H */
