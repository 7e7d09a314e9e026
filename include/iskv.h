/*
 * iskv.h -- C ABI of the MI355X (gfx950) library for basis-synchronized online
 * low-rank KV-cache compression.
 *
 * Source of the operations (page: "iS-KV -- Basis-synchronized online low-rank
 * KV compression -- What does it mean?", learnaivisually.com explainer of the
 * iS-KV paper, cited below as [iS-KV explainer]):
 *   - recent tokens are kept exact, older tokens as coefficient vectors over a
 *     shared basis, no position is dropped            [TL;DR; window paragraph]
 *   - every 64 tokens that leave the exact window are folded in as one block
 *     by Brand's block-incremental SVD on a small core matrix
 *                                                     [Jargon "Block-incremental
 *                                                      SVD"; drift paragraph]
 *   - the stored coefficients are rewritten whenever the basis changes
 *     (basis synchronization)                         [FAQ "What is basis
 *                                                      synchronization?"]
 *   - keys are compressed before RoPE and RoPE is re-applied on rebuild
 *                                                     [Jargon "Pre-RoPE keys"]
 *   - attention at a new position covers all predecessors, none evicted
 *                                                     [re-attention paragraph]
 *   - persistent-KV bytes = factors + exact rows      [Jargon "Persistent-KV
 *                                                      compression"]
 *   - some prompt positions are protected and kept uncompressed
 *                                                     [window paragraph; the
 *                                                      page does not say which:
 *                                                      here a leading prefix]
 * The page gives no interface; the verbs below follow its statement of the
 * problem: append tokens, fold a block, synchronize, attend.
 *
 * Conventions
 *   - Every pointer named dev_* or documented as "device" is a device pointer on
 *     the GPU current when iskv_init ran; host_* pointers are host memory.
 *   - Tensors are dense, row-major, innermost dimension last.
 *   - All verbs except iskv_status / iskv_export_state / iskv_import_state
 *     enqueue work on the stream given to iskv_init and return without waiting.
 *     Caller buffers must stay valid until the stream reaches the call.
 *   - Return codes are from host-side validation (ISKV_E*); a launch failure
 *     returns ISKV_EDEVICE.  Device-detected numeric trouble (non-finite input
 *     or core, Jacobi sweep cap reached) is reported by iskv_status.
 *   - A context is not thread-safe.  Sequences of a batch advance in lockstep
 *     through the uniform calls, or each at its own pace through the ragged
 *     calls (iskv_append_ragged and iskv_decode_attn_ragged below).
 *   - head_dim must be 128; rank must be 16, 32, 64 or 128 (rank_v equal to it
 *     or twice it); window a multiple of 64; num_q_heads a multiple of
 *     num_kv_heads, at most 16 times it.
 */
#ifndef ISKV_H
#define ISKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct iskv_ctx iskv_ctx; /* opaque; host heap; owned by the library */

typedef enum { ISKV_F32 = 0, ISKV_BF16 = 1 } iskv_dtype;

enum {
  ISKV_OK = 0,
  ISKV_EINVAL = -1,   /* bad argument or unsupported configuration */
  ISKV_ESTATE = -2,   /* verb not allowed in the current state */
  ISKV_ENOMEM = -3,   /* workspace smaller than iskv_workspace_bytes() */
  ISKV_EDEVICE = -4,  /* HIP runtime error */
  ISKV_ENUMERIC = -5, /* device-side numeric flag raised (see iskv_status) */
  ISKV_ESCRATCH = -6  /* iskv_decode_attn_noalloc: the configuration's split
                         records exceed its static array */
};

/* Device numeric flags reported in iskv_status_t.numeric_flags. */
enum {
  ISKV_FLAG_NONFINITE_CORE = 1,  /* NaN/Inf met while folding a block */
  ISKV_FLAG_JACOBI_CAP = 2,      /* core SVD hit its sweep cap unconverged */
  ISKV_FLAG_NONFINITE_INPUT = 4  /* NaN/Inf in appended k or v */
};

typedef struct {
  int32_t batch;          /* sequences (lockstep, or ragged: at most 64) */
  int32_t num_layers;
  int32_t num_kv_heads;
  int32_t num_q_heads;    /* multiple of num_kv_heads (grouped-query attention) */
  int32_t head_dim;       /* 128 */
  int32_t rank;           /* r: 16, 32, 64 or 128 (<= head_dim) */
  int32_t window;         /* W: exact tokens kept after a fold; multiple of 64 */
  int32_t block;          /* tokens per fold; must be 64 */
  int32_t max_tokens;     /* capacity per sequence and layer */
  int32_t storage;        /* iskv_dtype of ring rows and coefficients */
  float rope_base;        /* RoPE base, e.g. 10000 */
  float softmax_scale;    /* <= 0 selects 1/sqrt(head_dim) */
  int32_t protected_prefix; /* P: positions 0..P-1 stay exact and are never
                               folded (protected prompt rows); a multiple of 64,
                               0 <= P <= max_tokens; 0 = none */
  int32_t rank_v;         /* rank of the value factor: 0 (= rank), rank, or
                             2 * rank (<= head_dim); `rank` is then the key
                             rank.  Keys compress better than values
                             [KV-CoRE page, Key Results "Asymmetry of K
                             and V"] */
  int32_t async_maintenance; /* 0, or 1 for copy-on-write maintenance
                             (iskv_maintain / iskv_switch): a second
                             generation of bases, singular values and
                             coefficients, and 64 more ring slots, so that
                             decode goes on over the current generation
                             while the next one is built on the maintenance
                             stream ["ASKV" design report, Design
                             requirements: maintenance off the critical
                             path; copy-on-write, switched at a decode
                             boundary].  At most 64 layers. */
  int32_t joint_heads;    /* 0: one basis per (sequence, layer, KV head), d x r.
                             1: one basis per (sequence, layer) and factor over
                             all KV heads: a token's row is its heads' rows
                             side by side (num_kv_heads * head_dim wide), folded
                             and synchronized as one, with one coefficient row
                             per token for all heads; decode of KV head h
                             rebuilds its keys and values from rows
                             h*head_dim .. of that basis.  Ranks 64-128 over
                             128-dim heads compress 4-7x [iS-KV explainer,
                             the worked example and Table 1], which needs a
                             basis over several heads.  Requires rank and
                             rank_v <= 64 and num_kv_heads <= 32;
                             iskv_prefill is ESTATE. */
} iskv_config;

typedef struct {
  int64_t length;             /* tokens appended to the layer (per sequence) */
  int64_t compressed;         /* tokens held as coefficients (N_c, multiple of 64:
                                 positions P .. P+N_c-1) */
  int32_t blocks_ready;       /* 1: ring is full, a block must be folded before the next append */
  int32_t pending_sync;       /* 1: iskv_block_update ran and iskv_sync has not */
  int64_t folds;              /* iskv_block_update calls that folded this layer */
  int64_t syncs;              /* iskv_sync calls that synchronized this layer */
  uint64_t persistent_bytes;  /* kept bytes of all layers (coefficients, bases,
                                 singular values, exact rows) for the whole batch */
  uint64_t full_bytes;        /* bytes of the same tokens uncompressed (K+V, storage dtype) */
  int32_t numeric_flags;      /* OR of ISKV_FLAG_* raised since init */
  int32_t reserved;
} iskv_status_t;

/* Device workspace bytes needed for cfg (0 if cfg is invalid). */
size_t iskv_workspace_bytes(const iskv_config *cfg);

/* Bytes of one layer's state blob for iskv_export_state / iskv_import_state
 * (0 if cfg is invalid). Layout, all little-endian:
 *   int64 length, int64 compressed, then for b in [0,batch), h in [0,kv_heads),
 *   X in (K, V), with r = rank for K and rank_v (or rank) for V:
 *                 float basis[head_dim][r], float S[r],
 *                 float coeff[max_tokens][r]      (row = position; rows outside
 *                                                  P .. P+compressed-1 are 0),
 *                 float ring[S][head_dim]         (slot = position % S, S = window+64,
 *                                                  window+128 with async_maintenance),
 *                 float prefix[P][head_dim]       (protected rows, P = protected_prefix).
 * With joint_heads, basis is rows h*head_dim .. of the sequence's joint basis,
 * and S and coeff (shared by its heads) are listed under every head: export
 * writes them under each, import reads them from head 0. */
size_t iskv_state_bytes(const iskv_config *cfg);

/* Validate cfg, carve the caller's device workspace (dev_ws, ws_bytes >=
 * iskv_workspace_bytes), and reset every layer to the empty state: basis
 * I[:, :rank], S = 0, no tokens.  hip_stream is a hipStream_t (NULL = default
 * stream); all later work is enqueued on it.  The workspace is owned by the
 * caller and must outlive the context.  Synchronizes the stream once. */
int iskv_init(const iskv_config *cfg, void *dev_ws, size_t ws_bytes, void *hip_stream,
              iskv_ctx **out);

/* Append n_tokens tokens of every sequence to one layer.
 * dev_k, dev_v: [batch][n_tokens][num_kv_heads][head_dim] of dtype in_dtype,
 * keys before RoPE.  Each row is rounded to the storage dtype (round to nearest
 * even) and written to the protected prefix row (position < P) or to ring slot
 * position % (window+64).
 * ESTATE if the ring would hold more than window+64 tokens (the positions from
 * P + compressed on) or if length would pass max_tokens.
 * *blocks_ready (may be NULL) is set to 1 when the ring is full, i.e. the next
 * call must be iskv_block_update. */
int iskv_append(iskv_ctx *c, int layer, const void *dev_k, const void *dev_v, int n_tokens,
                int in_dtype, int *blocks_ready);

/* Fold the oldest 64 exact tokens of every (sequence, KV head, K|V) of the
 * layer (with joint_heads: every (sequence, K|V), the heads' rows side by
 * side) (layer = -1: every layer that has a full ring) into its rank-r basis
 * by Brand's block-incremental SVD: projection, residual CholeskyQR2, core
 * [[diag S, 0], [P, R_r^T]] of size (r+64)^2, one-sided Jacobi SVD, truncation
 * to r.  Writes the new basis, S, the block's coefficients, and the pending
 * synchronization matrix M = B_old^T B_new.  ESTATE if no block is ready (for
 * layer >= 0) or a sync is pending. */
int iskv_block_update(iskv_ctx *c, int layer);

/* Basis synchronization: rewrite every older coefficient row of the layer
 * (layer = -1: every layer with a pending update) as C <- C M.  ESTATE if no
 * update is pending (layer >= 0).  A pending sync blocks further folds of
 * that layer until iskv_sync or iskv_discard_sync. */
int iskv_sync(iskv_ctx *c, int layer);

/* Drop a pending synchronization without applying it: the old coefficients
 * stay in the previous basis (the basis-only update, which drifts). ESTATE if
 * none is pending (layer >= 0). */
int iskv_discard_sync(iskv_ctx *c, int layer);

/* Decode attention of one query per query head over every cached position of
 * the layer: keys rebuilt from coefficients (or read exact from the ring),
 * rotated by RoPE at their position; the query rotated at q_pos; softmax with
 * the configured scale; values accumulated in coefficient space and mapped
 * back by the value basis; protected prefix rows are exact like the ring rows.
 * dev_q: float [batch][num_q_heads][head_dim], before
 * RoPE.  dev_out: float [batch][num_q_heads][head_dim].  Query head h reads KV
 * head h / (num_q_heads / num_kv_heads).  q_pos must lie in [0, max_tokens + 128)
 * (the range of the RoPE tables built at init), else EINVAL.  ESTATE if the
 * layer is empty.  Arithmetic: fp32 accumulation throughout; with bf16
 * storage the key rebuild multiplies the stored coefficients (converted to
 * fp16 exactly; a coefficient beyond +-65504 saturates there) by the key
 * basis rounded to fp16, and the score product takes the rotated key in fp16
 * against the query as fp16 high + low parts; with fp32 storage both products
 * carry ~2^-16 relative error or less. */
int iskv_decode_attn(iskv_ctx *c, int layer, const float *dev_q, int64_t q_pos, float *dev_out);

/* One decode step in one launch: iskv_append of a single token (dev_k, dev_v:
 * [batch][1][num_kv_heads][head_dim], in_dtype ISKV_F32 or ISKV_BF16)
 * followed by iskv_decode_attn, with the same results, ring contents, error
 * codes and *blocks_ready as the two calls (the workgroup that attends over
 * the newest position writes its ring rows first).  A fused convenience of
 * this library, not an operation of the pages: it saves one launch per step
 * of an append-then-attend loop. */
int iskv_append_decode(iskv_ctx *c, int layer, const void *dev_k, const void *dev_v, int in_dtype,
                       const float *dev_q, int64_t q_pos, float *dev_out, int *blocks_ready);

/* iskv_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same kernels, arguments, results (bit for bit), and errors, but the
 * split-K partial records and merge counters live in a file-scope device
 * array of the library (32 MiB per GPU, held until the process ends) instead
 * of the context's workspace.  Nothing is allocated or freed by the call.
 * The array's address is looked up once per device by iskv_init.  Limit:
 * iskv_noalloc_scratch_bytes(cfg) must be <= 32 MiB (else ISKV_ESCRATCH;
 * with 8 KV heads: batch <= 126 at 4 query heads per KV head, <= 63 at 8).
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (other streams, other contexts, other threads) race and must be ordered by
 * the caller. */
int iskv_decode_attn_noalloc(iskv_ctx *c, int layer, const float *dev_q, int64_t q_pos,
                             float *dev_out);

/* Bytes of the static array that iskv_decode_attn_noalloc needs for cfg (0 if
 * cfg is invalid). */
size_t iskv_noalloc_scratch_bytes(const iskv_config *cfg);

/* Synchronizes the stream; fills *st for one layer.  Returns ISKV_ENUMERIC if
 * any numeric flag is set (st is still filled), else ISKV_OK. */
int iskv_status(iskv_ctx *c, int layer, iskv_status_t *st);

/* ---- Ragged batches: sequences of one batch at different lengths ----------
 * The pages fold a single stream; a batch whose sequences advance at their
 * own pace keeps one state per sequence: its own length, compressed count,
 * ring and fold schedule.  The calls below need batch <= 64 (else EINVAL).
 * A layer turns ragged at its first iskv_append_ragged; the uniform calls
 * (iskv_append, iskv_decode_attn, iskv_append_decode, iskv_status,
 * iskv_export_state) return ESTATE while its sequences differ, and work again
 * once they agree.  On a ragged layer iskv_block_update folds every sequence
 * whose ring is full (ESTATE for layer >= 0 if none is), iskv_sync and
 * iskv_discard_sync act on every sequence with a pending fold; a sequence
 * with a pending sync does not fold again until it is synchronized. */

/* Append counts[b] tokens to sequence b (0 <= counts[b] <= n_tokens; counts:
 * host int32 [batch]).  dev_k, dev_v: [batch][n_tokens][num_kv_heads][head_dim]
 * (device, in_dtype ISKV_F32 or ISKV_BF16), sequence b's tokens in its first
 * counts[b] rows; other rows are not read.  Positions continue each
 * sequence's own length.  Checked for every sequence before anything is
 * written: ESTATE if a ring would overflow or max_tokens be passed.
 * *seqs_ready (optional): how many sequences have a full ring. */
int iskv_append_ragged(iskv_ctx *c, int layer, const void *dev_k, const void *dev_v, int n_tokens,
                       int in_dtype, const int32_t *counts, int *seqs_ready);

/* iskv_decode_attn with each sequence at its own length and query position:
 * q_pos host int64 [batch] (each in the range iskv_decode_attn accepts, else
 * EINVAL).  Works on uniform layers too.  ESTATE if a sequence is empty. */
int iskv_decode_attn_ragged(iskv_ctx *c, int layer, const float *dev_q, const int64_t *q_pos,
                            float *dev_out);

/* iskv_status for one sequence (length, compressed, blocks_ready and
 * pending_sync are that sequence's; the rest as iskv_status). */
int iskv_seq_status(iskv_ctx *c, int layer, int seq, iskv_status_t *st);

/* Copy one layer's state to / from a host blob (layout: iskv_state_bytes).
 * Both synchronize the stream.  Import rounds coefficients and ring rows to
 * the storage dtype, clears any pending sync, and rebuilds derived operands. */
int iskv_export_state(iskv_ctx *c, int layer, void *host_buf, size_t bytes);
int iskv_import_state(iskv_ctx *c, int layer, const void *host_buf, size_t bytes);

/* Maintenance off the decode path ([ASKV report, Design requirements]:
 * maintenance must not block token generation).  With a non-NULL hip_stream
 * (a hipStream_t on the same device, distinct from the init stream),
 * iskv_block_update and iskv_sync enqueue their kernels there instead: each
 * call is ordered after everything already enqueued on the init stream, and
 * later init-stream work that touches the same layer (append, decode,
 * export/import) waits for that layer's maintenance; other layers' work does
 * not.  Results are identical to the single-stream order.  NULL (or the init
 * stream) returns to single-stream operation.  Pending maintenance is joined
 * into the init stream before the switch.  The caller keeps ownership of the
 * stream, which must outlive the context or the next switch. */
int iskv_set_maintenance_stream(iskv_ctx *c, void *hip_stream);

/* Make the init stream wait for the pending maintenance of `layer` (-1: all
 * layers).  Enqueued, does not block the host: init-stream work issued after
 * it is ordered after every block update and sync of that layer issued so
 * far.  (Verbs that touch a layer do this themselves; the call lets a caller
 * place the wait, e.g. outside a timed interval.)  EINVAL for a bad layer. */
int iskv_join_maintenance(iskv_ctx *c, int layer);

/* Prefill: append n_tokens prompt tokens (dev_k, dev_v: [batch][n_tokens]
 * [num_kv_heads][head_dim], device, in_dtype ISKV_F32 or ISKV_BF16) to a
 * layer whose ring is empty (length = P + N_c, P positions of protected
 * prefix already appended), folding every block that leaves the window in
 * one pass: m = (n_tokens - window) / 64 blocks (0 if n_tokens < window + 64),
 * the same blocks, in the same order, that appending the tokens and folding
 * + synchronizing each time the ring fills would fold [iS-KV explainer, the
 * trade-off paragraph: the prompt is compressed like the generated tokens].
 * The folds read the blocks straight from the input (rounded to the storage
 * type, as the ring would hold them) and are the same fold; the
 * synchronizations are deferred: each older row is mapped once by the
 * product of every later M instead of once per fold, which reads and writes
 * the history once per pass (a pass covers up to 64 MiB of M matrices)
 * instead of once per block; the results equal block-by-block
 * synchronization up to the rounding order of those products.  The last
 * n_tokens - 64 m tokens (window .. window + 63 of them) go to the ring.
 * ESTATE: ring not empty, pending sync, protected prefix not yet full,
 * max_tokens exceeded, a copy-on-write or a joint_heads context.  Counters: folds += m,
 * syncs += passes. */
int iskv_prefill(iskv_ctx *c, int layer, const void *dev_k, const void *dev_v, int n_tokens,
                 int in_dtype);

/* iskv_prefill of n_layers distinct layers (layers: host int32 array;
 * dev_k, dev_v: host arrays of device pointers, one input per layer) in the
 * same launches: every layer must hold the same length and compressed count.
 * The layers' folds run side by side (one workgroup per layer, unit and
 * factor), up to 16 layers per launch, sharing the M slots of one pass. */
int iskv_prefill_layers(iskv_ctx *c, int n_layers, const int *layers, const void *const *dev_k,
                        const void *const *dev_v, int n_tokens, int in_dtype);

/* Copy-on-write maintenance (contexts with async_maintenance = 1; ESTATE
 * otherwise) ["ASKV" design report, Design requirements: compression must not
 * hold up generation; the new cache version is built aside and switched to
 * at a decode boundary, the current one used until it is ready].
 *
 * iskv_maintain: for `layer` (-1: every layer with a block ready and none in
 * flight) enqueue, on the maintenance stream (the init stream if none is
 * set) and after all init-stream work issued so far, the fold of the oldest
 * ring block (positions P+N_c .. +63) and the synchronization of rows
 * P .. P+N_c-1, both reading the layer's current generation and writing the
 * other one (new basis, S, synchronized coefficients and the block's own
 * rows).  Returns at once.  The current generation is untouched: decode,
 * append and status go on as if the fold had not happened, the block's rows
 * still exact in the ring (which holds window + 128 rows in this mode).
 * ESTATE if the layer (layer >= 0) has no block ready (fewer than window + 64
 * ring rows) or a maintenance in flight.  The layer's folds and syncs
 * counters advance here.
 *
 * iskv_switch: the decode boundary.  If the layer's maintenance has finished
 * (wait = 0: a non-blocking query; wait = 1: the init stream is made to wait
 * for it, the host does not block), the layer switches to the new generation
 * (N_c grows by 64) and 1 is returned; 0 if nothing is in flight or it has
 * not finished (decoding continues on the current generation).
 * iskv_decode_attn, iskv_decode_attn_noalloc, iskv_append_decode and
 * iskv_append make the non-blocking switch themselves on entry; an append
 * that would overflow the ring waits for the switch instead.  Results do not
 * depend on when the switch happens beyond which generation a decode reads:
 * iskv_status after a decode reports the generation it used (compressed,
 * and pending_sync = 1 while a maintenance is in flight).
 *
 * The block update, sync and discard verbs and the ragged verbs return
 * ESTATE in this mode.  iskv_join_maintenance switches with wait = 1.  The
 * second generation is maintenance workspace: persistent_bytes counts the
 * current one only. */
int iskv_maintain(iskv_ctx *c, int layer);
int iskv_switch(iskv_ctx *c, int layer, int wait);

/* Free the context (not the caller's workspace).  Joins pending maintenance,
 * then synchronizes the init stream. */
int iskv_destroy(iskv_ctx *c);

/* Static string for a return code. */
const char *iskv_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ISKV_H */
