/*
 * dsa.h -- C ABI of the MI355X (gfx950) DSA hot path: the fused Lightning
 * Indexer (per-head relevance scores read straight from a paged K cache, a
 * head-weighted sum, a causal mask and Top-K selection) and Sparse Flash
 * Attention over the selected latent KV rows.
 *
 * The operations are the ones the pages describe:
 *   - "Deep Fusion of LI and SFA" (Day0 Inference Optimization on Ascend CANN,
 *     sec. 2; Inference Acceleration for Next-Gen Attention Architectures,
 *     sec. 3.1-3.2): relevance scoring, head weighting and Top-K in one operator
 *     that reads the paged cache directly; SFA then reads the main-attention KV
 *     rows at the selected indices.
 *   - causal index computation (Adapting and Optimizing Inference for a New
 *     Model Architecture on Ascend, sec. 5.2): a query at position t selects
 *     among positions 0..t only.
 *   - quantised index path (same page, sec. 4.2): MXFP8 with one scale shared
 *     by every 32 elements.
 *
 * Conventions shared by every entry point
 *   Ownership: every array argument is a DEVICE pointer owned by the caller;
 *     the structs themselves are host memory read only during the call.  The
 *     library never allocates, frees or synchronises device memory; scratch
 *     memory comes from the caller's workspace `ws` of `ws_bytes` bytes, sized
 *     with dsa_workspace_size().  One workspace must not be used by two calls
 *     that may run concurrently.
 *   Workspace state: a workspace must be zero-filled before its first use
 *     (hipMemsetAsync, or allocate it zeroed).  The decode indexer keeps its
 *     cross-workgroup counters and histograms at the START of the workspace
 *     and every call leaves them zero again when its kernels finish (which
 *     saves a fill launch per call); scratch (index rows, attention partials)
 *     is placed at the END of the workspace and left as it is.  So one
 *     workspace serves later calls of other shapes without being cleared,
 *     provided it holds the largest state and the largest scratch among them
 *     at once: sizing it with dsa_workspace_size() for a call whose batch,
 *     query-token count and topk are each at least those of every call that
 *     shares it is enough.  Its first 256 bytes are a header that calls do
 *     not leave zero: the sticky error bits (dsa_take_device_errors) and a
 *     count of fused decode calls that dates their handoffs (zero-filling the
 *     whole workspace again between calls is always allowed).
 *   Alignment: the workspace and the q, k_cache / kv_cache data and output
 *     arrays are 16-byte aligned (the kernels move them 16 bytes at a time);
 *     scale pools, head weights, lse, index rows, lengths and block tables
 *     4-byte aligned.  A misaligned pointer is DSA_ERR_INVALID_ARG.
 *   Ordering: work is enqueued asynchronously on `stream` (a hipStream_t, NULL
 *     = the default stream); nothing is waited for, except by calls under
 *     DSA_DEBUG=1 and by dsa_take_device_errors, which say so below.
 *   Empty calls: with total_q = 0 (every sequence without a new query token)
 *     a call validates its arguments as usual and returns DSA_OK having
 *     computed nothing; the arrays with one entry per query token (q, head
 *     weights, q scales, outputs, index rows, the prolog's x) may then be
 *     NULL.
 *   Errors: arguments are validated on the host before anything is enqueued;
 *     a failed check returns its status and enqueues nothing.  A failed launch
 *     returns DSA_ERR_HIP.  dsa_last_error() returns a thread-local message for
 *     the last failure.  Contents of device arrays (block-table entries, lengths)
 *     are preconditions: block_table entries < num_pages, seq_lens[b] <=
 *     max_pages_per_seq * page_size, 0 <= q_lens <= seq_lens, values finite,
 *     index rows given to dsa_sparse_attn within [-1, seq_len).  With
 *     DSA_DEBUG=1 in the environment every call first checks the lengths,
 *     query offsets, block-table entries of the pages in use (and those
 *     index rows) on the device, waits for the result and returns
 *     DSA_ERR_INVALID_ARG, having enqueued nothing else, if one is violated.
 *     The decode indexer's workgroups wait for each other with bounded waits
 *     (its grid is sized to be resident as a whole; other work sharing the
 *     device can keep part of it waiting).  If a
 *     wait ever gives up, the affected queries' index rows are overwritten
 *     with -1 (slot 0 included, which no valid row has), and a sticky error
 *     bit is set in the workspace; with DSA_DEBUG=1 in the environment each
 *     call synchronises after the indexer and returns DSA_ERR_HIP for it.
 *   Positions: sequence b has L_b = seq_lens[b] keys in the caches; its
 *     T_b = cu_q[b+1] - cu_q[b] query tokens are the LAST T_b positions, query
 *     i sitting at t = L_b - T_b + i.  Key position s of sequence b lives in
 *     row s % P of physical page block_table[b][s / P] of both caches.
 *   Top-K: a query at t keeps n = min(topk, t + 1) positions with the largest
 *     scores; equal scores go to the smaller position.  Output rows hold the n
 *     LOGICAL positions in any order followed by -1 in slots n..topk-1.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,         /* null pointer, negative size, inconsistent scalars */
  DSA_ERR_UNSUPPORTED = 2,         /* shape / dtype / page size not compiled in        */
  DSA_ERR_WORKSPACE_TOO_SMALL = 3, /* ws_bytes < dsa_workspace_size(...)              */
  DSA_ERR_HIP = 4                  /* a HIP runtime call failed                         */
} dsa_status;

typedef enum {
  DSA_F32 = 0,         /* float32                                                */
  DSA_BF16 = 1,        /* bfloat16                                               */
  DSA_FP8_E4M3 = 2,    /* OCP e4m3fn bytes + one float32 scale per row           */
  DSA_MXFP8_E4M3 = 3,  /* OCP e4m3fn bytes + one e8m0 scale byte per 32 elements */
  DSA_FP8_E4M3_TILE128 = 4  /* OCP e4m3fn bytes + one float32 scale per tile of 128
                               consecutive elements of a row (the last tile of a
                               row may be shorter): the SFA KV cache format      */
} dsa_dtype;

typedef enum {
  DSA_OP_INDEXER_TOPK = 0,
  DSA_OP_SPARSE_ATTN = 1,
  DSA_OP_FUSED_DECODE = 2,
  DSA_OP_FUSED_PREFILL = 3
} dsa_op;

/* A paged pool: data [num_pages][page_size][dim] elements of `dtype`.
 * scale: DSA_FP8_E4M3   -> float32 [num_pages][page_size] (one per token)
 *        DSA_MXFP8_E4M3 -> uint8 e8m0 [num_pages][page_size][dim / 32]
 *        DSA_FP8_E4M3_TILE128 -> float32 [num_pages][page_size][ceil(dim / 128)]
 *                          (element c of a row is byte c times scale c / 128;
 *                          per token, head and tile of 128: "Adapting and
 *                          Optimizing Inference for a New Model Architecture on
 *                          Ascend", sec. 4.3; one head, the latent row, in the
 *                          absorbed MLA form)
 *        otherwise NULL.                                                      */
typedef struct {
  const void* data;
  const void* scale;
  int32_t dtype;
  int32_t num_pages;
  int32_t page_size;           /* tokens per page: a power of two in [1, 4096]    */
  int32_t dim;
} dsa_paged_cache;

/* The batch: B sequences, device arrays plus host-side scalars that bound them. */
typedef struct {
  int32_t batch;               /* B >= 1                                          */
  const int32_t* seq_lens;     /* device [B]: L_b                                 */
  const int32_t* cu_q;         /* device [B+1]: query-token offsets, cu_q[0] = 0  */
  const int32_t* block_table;  /* device [B][max_pages_per_seq]                   */
  int32_t max_pages_per_seq;
  int32_t total_q;             /* == cu_q[B]                                      */
  int32_t max_q_len;           /* >= every T_b                                    */
  int32_t max_seq_len;         /* >= every L_b                                    */
} dsa_batch;

/* Indexer operands.
 * q            device [total_q][n_heads][head_dim] of q_dtype (== k_cache->dtype)
 * q_scale      DSA_FP8_E4M3: float32 [total_q][n_heads];
 *              DSA_MXFP8_E4M3: uint8 e8m0 [total_q][n_heads][head_dim / 32]; else NULL
 * head_weights device float32 [total_q][n_heads] (any sign)
 * k_cache      paged pool with dim == head_dim                                */
typedef struct {
  const void* q;
  int32_t q_dtype;
  const void* q_scale;
  const float* head_weights;
  int32_t n_heads;
  int32_t head_dim;
  int32_t topk;
  const dsa_paged_cache* k_cache;
} dsa_indexer_args;

/* SFA operands (absorbed MLA form: one latent row per position, shared by all heads).
 * q        device [total_q][n_heads][qk_dim] of q_dtype (F32 or BF16)
 * kv_cache paged pool with dim == qk_dim, dtype == q_dtype or
 *          DSA_FP8_E4M3_TILE128 (rows decoded with their tile scales);
 *          V is the first v_dim columns of a row.
 * Logits are softmax_scale * q_h . row over all qk_dim columns.                */
typedef struct {
  const void* q;
  int32_t q_dtype;
  int32_t n_heads;
  int32_t qk_dim;
  int32_t v_dim;
  float softmax_scale;
  const dsa_paged_cache* kv_cache;
} dsa_sfa_args;

/* Indexer prolog operands: the projections of the new tokens' hidden rows
 * that feed the indexer ("Three-Stream Coordination for Indexer Prolog", Day0
 * Inference Optimization on Ascend CANN, sec. 2; Adapting and Optimizing
 * Inference for a New Model Architecture on Ascend, sec. 3.2 and 4.2).
 * x        device bf16 [total_q][d_model], one hidden row per new token
 * w_q      device bf16 [n_heads * head_dim][d_model]  (linear-layer layout)
 * w_k      device bf16 [head_dim][d_model]
 * w_w      device bf16 [n_heads][d_model]
 * ln_gamma, ln_beta  device float32 [head_dim]: the key LayerNorm
 * out_dtype DSA_BF16, DSA_FP8_E4M3 or DSA_MXFP8_E4M3: how q and the appended
 *          keys are stored (the indexer's dtype)                            */
typedef struct {
  const void* x;
  int32_t d_model;             /* a positive multiple of 128                     */
  const void* w_q;
  const void* w_k;
  const void* w_w;
  const float* ln_gamma;
  const float* ln_beta;
  float ln_eps;
  int32_t n_heads;             /* a multiple of 32                                */
  int32_t head_dim;            /* 128                                             */
  int32_t out_dtype;
} dsa_prolog_args;

/* Bytes of workspace the call needs (0 is possible).  Device pointers are not
 * read; the scalars are, and sfa->kv_cache->dtype when sfa->kv_cache is not
 * NULL (an FP8 KV cache changes the work split).  `topk` for
 * DSA_OP_SPARSE_ATTN comes from idx->topk when idx is given, else 2048.
 * Returns 0 for an invalid op.                                                */
size_t dsa_workspace_size(int32_t op, const dsa_batch* batch,
                          const dsa_indexer_args* idx, const dsa_sfa_args* sfa);

/* Fused Lightning Indexer: scores, head weighting, causal mask and Top-K in
 * one pass over the paged K cache; the full score row is never written to
 * device memory.  idx_out: device int32 [total_q][topk] (see Top-K above).
 * Decode-sized batches select with an exact radix select across the
 * workgroups that share a sequence; when few keys share the first pass's
 * boundary bin, the sequence's last workgroup finishes the choice alone.
 * DSA_INDEXER_HANDOFF_CAP=n in the environment caps that bin (0: never; the
 * result is the same index set either way, a test and diagnostic switch). */
dsa_status dsa_indexer_topk(const dsa_batch* batch, const dsa_indexer_args* args,
                            int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/* Sparse Flash Attention over the given index rows.
 * idx: device int32 [total_q][topk] logical positions, -1 entries ignored
 *      (each row must hold at least one valid position <= the query's t).
 * out: device [total_q][n_heads][v_dim] in q_dtype.
 * lse: device float32 [total_q][n_heads] natural-log sum-exp of the scaled
 *      logits, or NULL.
 * Launches that split index rows across workgroups (few query tokens) keep
 * the normalised per-range results in fp16, so bf16 latent values must stay
 * below 65504 in magnitude there (a larger one shows up as a non-finite
 * output).                                                                    */
dsa_status dsa_sparse_attn(const dsa_batch* batch, const dsa_sfa_args* args,
                           const int32_t* idx, int32_t topk, void* out, float* lse,
                           void* ws, size_t ws_bytes, void* stream);

/* Decode step (small T_b): indexer + Top-K, then SFA on the selected rows.
 * idx_out may be NULL (the indices then live in the workspace).
 * The two operators run fused in one kernel where the shapes allow it (bf16
 * SFA over bf16 rows with 128 heads and 576/512 dims; the indexer in bf16,
 * FP8 or MXFP8; at most as many (token, slot range) tasks as the device has
 * compute units): each sequence's attention starts as soon as its own index
 * rows are complete, the deep fusion of LI and SFA of "Day0 Inference
 * Optimization on Ascend CANN", section 2.  Results are those of the two
 * separate operators up to the order of positions within an index row (and
 * the rounding that order brings).  DSA_FUSED_KERNEL=0 in the environment
 * selects the two-kernel path.                                              */
dsa_status dsa_fused_decode(const dsa_batch* batch, const dsa_indexer_args* iargs,
                            const dsa_sfa_args* sargs, void* out, float* lse,
                            int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/* Causal (chunked) prefill (large T_b): query blocks of q_block tokens are
 * paired from the two ends of each sequence (zigzag) so that every workgroup
 * gets one short-history and one long-history block; results are written back
 * to their original rows.  q_block must be 64.  idx_out may be NULL.
 * The zigzag pairing is the load balancing of causal prefill described in
 * "Adapting and Optimizing Inference for a New Model Architecture on Ascend",
 * section 5.2, and in "Day0 Inference Optimization on Ascend CANN: A Deep
 * Dive into Hybrid Architecture Acceleration", section 4 (its zigzag layout),
 * where it balances devices; here it balances workgroups of one GPU.  The
 * indexer scores and selection follow the same pages' section 2 (indexer)
 * and the sparse attention their section 3.1, as for dsa_fused_decode.  The
 * indexer may be bf16, DSA_FP8_E4M3 or DSA_MXFP8_E4M3 here as in decode (the
 * fused indexer serves both phases quantised: the Day0 page, section 2); an
 * MXFP8 k_cache->scale must then be 4-byte aligned (each row's 4 scale bytes
 * are read as one word), else DSA_ERR_INVALID_ARG.                          */
dsa_status dsa_fused_prefill(const dsa_batch* batch, const dsa_indexer_args* iargs,
                             const dsa_sfa_args* sargs, int32_t q_block, void* out,
                             float* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                             void* stream);

/* dsa_fused_decode without a workspace, for callers that cannot allocate
 * device memory (code under graph capture, serving loops that forbid
 * allocation).  Same arguments, results and errors as dsa_fused_decode; the
 * scratch memory is a static array of dsa_noalloc_scratch_bytes() (64 MiB)
 * that every GPU the library runs on holds until the process ends, looked up
 * once per device.  Its first 16 MiB hold the zero state, the rest the
 * scratch, so calls of any shapes may follow each other; a call whose state
 * or scratch (together dsa_workspace_size(DSA_OP_FUSED_DECODE, ...)) exceeds
 * its part returns DSA_ERR_UNSUPPORTED and enqueues nothing.  The first
 * call on a device also enqueues one clear of the array (make that call
 * before capturing a graph, or every replay repeats the clear).  Replays of
 * a captured call are safe: the handoff inside each is dated by a counter
 * on the device, not by a value frozen into the graph.  All calls on one
 * GPU share its array: calls that may overlap on the same GPU (other streams,
 * other host threads) race and must be ordered by the caller.               */
dsa_status dsa_fused_decode_noalloc(const dsa_batch* batch, const dsa_indexer_args* iargs,
                                    const dsa_sfa_args* sargs, void* out, float* lse,
                                    int32_t* idx_out, void* stream);

/* Bytes of the static scratch array behind dsa_fused_decode_noalloc. */
size_t dsa_noalloc_scratch_bytes(void);

/* Indexer prolog for the new tokens of a step (the steps the pages place
 * before the fused indexer: Q projection, K normalisation, dynamic Q
 * quantisation, head-weight projection; index Q/K dynamically quantised, MXFP8
 * in groups of 32 -- same pages as dsa_prolog_args).  For every new token:
 *   q = bf16(x W_q^T) as [n_heads][head_dim]; k = bf16(LayerNorm(x W_k^T))
 *   (biased variance, ln_eps, then gamma and beta); w = x W_w^T (float32).
 *   Quantisation per out_dtype: FP8 scale = amax / 448 (1 for an all-zero
 *   row) in float32, elements x / scale rounded to nearest even and saturated,
 *   per (token, head) for q and per token for k; MXFP8 E = floor(log2 amax) - 8
 *   clamped to [-127, 127] per 32 elements, elements x 2^-E rounded and
 *   saturated (OCP MX v1.0 for e4m3).
 * Outputs (device): q_out [total_q][n_heads][head_dim] (bf16 or e4m3 bytes);
 *   q_scale_out float32 [total_q][n_heads] (FP8) or e8m0 [total_q][n_heads]
 *   [head_dim/32] (MXFP8), NULL for bf16; w_out float32 [total_q][n_heads].
 *   Token i of sequence b (t = L_b - T_b + i) has its key written into
 *   k_cache at row t % P of page block_table[b][t / P], with its scale(s);
 *   no other cache row is touched (k_cache->dtype must equal out_dtype).
 *   q_bf16_out (optional, [total_q][n_heads*head_dim] bf16) receives q before
 *   quantisation (ignored for bf16 output, where q_out holds it), k_bf16_out
 *   (optional, [total_q][head_dim]) k before it.
 * Alignment: x, the weights, q_out, q_bf16_out and w_out 16 bytes.
 * Workspace: dsa_prolog_workspace_size() bytes (no state kept between calls).
 * Errors as for the other entry points.                                     */
dsa_status dsa_indexer_prolog(const dsa_batch* batch, const dsa_prolog_args* args, void* q_out,
                              void* q_scale_out, float* w_out, const dsa_paged_cache* k_cache,
                              void* q_bf16_out, void* k_bf16_out, void* ws, size_t ws_bytes,
                              void* stream);

/* Bytes of workspace dsa_indexer_prolog needs (0 for invalid arguments). */
size_t dsa_prolog_workspace_size(const dsa_batch* batch, const dsa_prolog_args* args);

/* Static text for a status code. */
const char* dsa_status_string(int32_t status);

/* Thread-local description of the last failure in this thread ("" if none). */
const char* dsa_last_error(void);

/*
 * dsa_take_device_errors -- whether a bounded cross-workgroup wait of the
 * decode indexer gave up in any call since the last report, without running
 * every call under DSA_DEBUG.  Such a call has already overwritten the
 * affected index rows with -1 (see "Errors" above); this reports it on the
 * host.
 *   ws:     the workspace those calls used, whose first 4 bytes hold the
 *           sticky error bits (16-byte aligned, device memory), or NULL for
 *           this device's static scratch of dsa_fused_decode_noalloc (DSA_OK
 *           if no such call ran on this device yet).
 *   stream: synchronised first (a hipStream_t; NULL = the default stream).
 * Returns DSA_ERR_HIP if any bit is set, clearing them (each failure is
 * reported once), else DSA_OK.  It blocks: meant as a periodic check between
 * steps, not for code under graph capture.
 */
dsa_status dsa_take_device_errors(void* ws, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
