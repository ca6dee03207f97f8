/*
 * clsa.h - C ABI of the CLSA (Cross-Layer Sparse Attention, "You Only Index Once")
 * decode / prefill hot path on AMD Instinct MI355X (gfx950).
 *
 * What the path computes (picx.dev summary of "You Only Index Once: Cross-Layer Sparse
 * Attention with Shared Routing", section Methodology > Architecture Overview):
 *   eq. 2  I = Q_idx K_idx^T  and  S_t = TopK(I_t, k)   - routing, computed ONCE per step
 *   eq. 3  O_t^(l) = Attn(Q_t^(l), K_{S_t}, V_{S_t})    - every cross-decoder layer l reads
 *          the same selected rows of the one shared (YOCO) KV cache
 * with Attn(Q, K, V) = softmax(Q K^T / sqrt(d)) V (zhichai.net explainer "... (CLSA)
 * Explained", section Background: Attention and Its Limits), and the Selector gathering
 * KV rows by the shared index (same explainer, section CLSA: Sharing the Index Across Layers).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All functions return clsa_status; nothing throws or aborts across the ABI.  On any
 *    error, clsa_last_error_message() (thread-local) describes it.
 *  - Every argument is validated on the host BEFORE any launch; a rejected call launches
 *    nothing and touches no memory.
 *  - Ownership: the caller allocates every device buffer (inputs, outputs, workspace) and
 *    keeps it alive until the stream has passed the call.  The library allocates no device
 *    memory and keeps no pointer after returning.  (clsa_step_no_alloc, at the end, is the one
 *    exception: its workspace is a static array of the library's own device code.)
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *  - Device pointers must be 16-byte aligned; the workspace 256-byte aligned.  bf16 values are
 *    passed as uint16 bit patterns.
 *  - Workspace: its content on entry does not matter (every call clears what it needs); two
 *    calls that share one workspace must not overlap in time on the device.
 *  - Token indices are int32 and LOCAL to their sequence.
 *  - Query rows.  DECODE: row r is sequence r (n_rows == batch) and sees all N_r tokens of
 *    its sequence, N_r = cu_seqlens[r+1] - cu_seqlens[r].  PREFILL: the rows are the query
 *    positions pos0 .. pos0+n_rows-1 of sequence `seq`; row i sees tokens 0 .. pos0+i of
 *    that sequence (causal).
 *  - Readings of the method fixed by this ABI: scores are plain dot products (no scale, no
 *    activation); |S| = min(k, visible tokens); ties at the k-th score go to the LOWER token
 *    index; S is returned in ASCENDING index order, padded with -1; one S per query row is
 *    shared by all layers and all query heads; the softmax scale is 1/sqrt(head_dim) unless
 *    dims.sm_scale > 0; query head h reads KV head floor(h * hkv / hq).
 *  - NaN or Inf scores are not supported (the selection is then unspecified).
 *  - Token indices passed in idx must be tokens the row sees; out-of-range values are clamped
 *    into the row (the output is then unspecified, but no access leaves the cache).
 *  - Device failures (a failed launch) return CLSA_ERR_DEVICE with the HIP error text.
 */
#ifndef CLSA_H_
#define CLSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t clsa_bf16;  /* bf16 bit pattern */
typedef void* clsa_stream;   /* hipStream_t */

typedef enum clsa_status {
  CLSA_OK = 0,
  CLSA_ERR_INVALID_ARGUMENT = 1, /* NULL / misaligned pointer, inconsistent sizes, bad lengths */
  CLSA_ERR_UNSUPPORTED = 2,      /* head_dim != 128, d_idx not 64/128, sizes beyond the limits */
  CLSA_ERR_WORKSPACE = 3,        /* workspace missing or smaller than clsa_workspace_bytes() */
  CLSA_ERR_DEVICE = 4            /* a HIP launch / runtime failure */
} clsa_status;

enum { CLSA_MODE_DECODE = 0, CLSA_MODE_PREFILL = 1 };
enum { CLSA_SCHEDULE_LAYER_BATCHED = 0, CLSA_SCHEDULE_PER_LAYER = 1, CLSA_SCHEDULE_PER_LAYER_ROUTING = 2 };

/* Limits (CLSA_ERR_UNSUPPORTED beyond them). */
#define CLSA_HEAD_DIM 128
#define CLSA_MAX_TOPK 65536
#define CLSA_MAX_ROW_LEN (1 << 24)

typedef struct clsa_dims {
  int32_t batch;    /* B >= 1: sequences in the cache; cu_seqlens has B+1 entries          */
  int32_t d_idx;    /* width of the single-head indexer: 64 or 128                        */
  int32_t topk;     /* k, 1 .. CLSA_MAX_TOPK                                              */
  int32_t n_layers; /* L >= 1: cross-decoder layers sharing the selection                 */
  int32_t hq;       /* query heads per layer, multiple of hkv                             */
  int32_t hkv;      /* KV heads of the shared cache                                       */
  int32_t head_dim; /* must be 128                                                        */
  float sm_scale;   /* softmax scale; <= 0 selects 1/sqrt(head_dim)                       */
} clsa_dims;

typedef struct clsa_rows {
  int32_t mode;        /* CLSA_MODE_DECODE or CLSA_MODE_PREFILL                              */
  int32_t n_rows;      /* R >= 1 query rows; DECODE requires R == batch                      */
  int32_t seq;         /* PREFILL: sequence the rows belong to (0 <= seq < batch)            */
  int32_t pos0;        /* PREFILL: cache position of row 0 (row i sees pos0 + i + 1 tokens)  */
  int32_t max_row_len; /* host bound on tokens a row sees: DECODE >= max N_r,
                          PREFILL == pos0 + n_rows                                          */
  int64_t total_tokens;          /* T = cu_seqlens[batch]: rows of k_idx / k_cache / v_cache   */
  const int32_t* cu_seqlens_host; /* optional host copy of cu_seqlens [B+1]; when given it is
                                     checked (starts at 0, non-decreasing, ends at T, every
                                     N_r <= max_row_len, DECODE N_r >= 1, PREFILL
                                     pos0 + n_rows <= N_seq)                                  */
} clsa_rows;

/* Human-readable name of a status code (static storage). */
const char* clsa_status_string(clsa_status status);

/* Detail of the last error raised on this thread ("" if none); valid until the next call. */
const char* clsa_last_error_message(void);

/* ABI revision of this header; bumped on any incompatible change. */
int32_t clsa_abi_version(void);
#define CLSA_ABI_VERSION 1

/* Device workspace, in bytes, that clsa_topk, clsa_sparse_attn (any n_layers_call) and
 * clsa_step (with this `schedule` and `prefill_chunk_rows`, 0 = default) need for these sizes:
 * the maximum over the three.  Pure host function.  Returns 0 and sets the error message if the
 * arguments are invalid. */
size_t clsa_workspace_bytes(const clsa_dims* dims, const clsa_rows* rows, int32_t schedule,
                            int32_t prefill_chunk_rows);

/*
 * Routing scores, eq. 2 first half (picx.dev summary, Architecture Overview):
 *   scores[r * ld_scores + j] = sum_c q_idx[r, c] * k_idx[cu_seqlens[s_r] + j, c]
 * for every token j the row sees (j < N_r in DECODE, j <= pos0 + r in PREFILL), accumulated
 * in fp32 from bf16 products.  Entries past the row's visible length are not written.
 *   q_idx      [R, d_idx] bf16         k_idx [T, d_idx] bf16 (token-major, packed by cu_seqlens)
 *   cu_seqlens [B+1] int32 (device)    scores [R, ld_scores] fp32, ld_scores >= max_row_len and
 *                                      a multiple of 4
 * DECODE streams k_idx once (bandwidth bound); PREFILL runs the causal Q_idx K_idx^T
 * product on the matrix cores.
 */
clsa_status clsa_index_scores(const clsa_dims* dims, const clsa_rows* rows, const clsa_bf16* q_idx,
                              const clsa_bf16* k_idx, const int32_t* cu_seqlens, float* scores,
                              int64_t ld_scores, clsa_stream stream);

/*
 * Token-level top-k, eq. 2 second half (picx.dev summary, Architecture Overview): for each
 * row, the first m = min(k, visible length) tokens in the order (score descending, token
 * index ascending), written in ascending index order:
 *   idx   [R, k] int32  - idx[r, 0..m) ascending local token ids, idx[r, m..k) = -1
 *   count [R]    int32  - m
 * scores as written by clsa_index_scores (only the visible entries of each row are read;
 * -0.0 and +0.0 are equal).  The result is unique and deterministic.
 * Workspace: >= clsa_workspace_bytes(dims, rows, CLSA_SCHEDULE_LAYER_BATCHED, 0).
 */
clsa_status clsa_topk(const clsa_dims* dims, const clsa_rows* rows, const int32_t* cu_seqlens,
                      const float* scores, int64_t ld_scores, int32_t* idx, int32_t* count,
                      void* workspace, size_t workspace_bytes, clsa_stream stream);

/*
 * The Selector: gather the selected rows of the shared cache (zhichai.net explainer, CLSA:
 * Sharing the Index Across Layers; K_{S_t}, V_{S_t} of eq. 3), bit-exact copies:
 *   k_sel[r, g, i, :] = k_cache[cu_seqlens[s_r] + idx[r, i], g, :]   for i < count[r]
 *   k_sel[r, g, i, :] = 0                                             for count[r] <= i < k
 * (same for v_sel).  k_cache, v_cache [T, hkv, 128] bf16; k_sel, v_sel [R, hkv, k, 128] bf16
 * (head-major, so one KV head's selected rows are contiguous).
 */
clsa_status clsa_gather_kv(const clsa_dims* dims, const clsa_rows* rows, const clsa_bf16* k_cache,
                           const clsa_bf16* v_cache, const int32_t* cu_seqlens, const int32_t* idx,
                           const int32_t* count, clsa_bf16* k_sel, clsa_bf16* v_sel, clsa_stream stream);

/*
 * Sparse attention of n_layers_call layers over each row's selected set, eq. 3 with the
 * softmax attention of the zhichai.net Background section:
 *   out[r, l, h, :] = sum_i softmax_i(q[r, l, h, :] . K_i / sqrt(128)) V_i
 * over the count[r] selected rows i of KV head g = floor(h * hkv / hq).
 *   q   : row r at q + r * q_row_stride, laid out [n_layers_call, hq, 128] bf16
 *   out : row r at out + r * out_row_stride, laid out [n_layers_call, hq, 128] bf16 (RNE)
 *   K/V : either the compact buffers k_sel/v_sel [R, hkv, k, 128] of clsa_gather_kv, or - when
 *         k_sel == v_sel == NULL - read straight from k_cache/v_cache through idx/cu_seqlens.
 *   idx, count as written by clsa_topk.  count[r] >= 1 is required.
 * Softmax and accumulation are fp32 (online softmax, split over the selected rows and
 * recombined); 1 <= n_layers_call <= dims.n_layers.
 */
clsa_status clsa_sparse_attn(const clsa_dims* dims, const clsa_rows* rows, const clsa_bf16* q,
                             int64_t q_row_stride, int32_t n_layers_call, const clsa_bf16* k_sel,
                             const clsa_bf16* v_sel, const clsa_bf16* k_cache, const clsa_bf16* v_cache,
                             const int32_t* cu_seqlens, const int32_t* idx, const int32_t* count,
                             clsa_bf16* out, int64_t out_row_stride, void* workspace,
                             size_t workspace_bytes, clsa_stream stream);

/*
 * The step before the routing (DECODE only): the shared indexer's projections of each
 * sequence's new token, eq. 1 of the picx.dev summary (Architecture Overview):
 * Q_idx = H W_idx^Q, K_idx = H W_idx^K, and the append of that token to the caches.  Sequence
 * b's new token is its LAST cache position t_b = cu_seqlens[b+1] - 1 (the caller has already
 * counted it in cu_seqlens); a following clsa_index_scores / clsa_step sees it like any other
 * token.
 *   h        [B, d_model] bf16       hidden state of each sequence's new token
 *   w_q_idx  [d_idx, d_model] bf16   row j = the weights of indexer channel j (W_idx^Q transposed)
 *   w_k_idx  [d_idx, d_model] bf16   (W_idx^K transposed)
 *   q_idx    [B, d_idx] bf16 (output)   q_idx[b, j] = RNE(sum_c h[b, c] * w_q_idx[j, c])
 *   k_idx    [T, d_idx] bf16            row t_b := RNE(sum_c h[b, c] * w_k_idx[j, c]); no other
 *                                       row is written
 *   k_new, v_new [B, hkv, 128] bf16, optional (both or neither): copied bit for bit into row t_b
 *            of k_cache / v_cache [T, hkv, 128] (both required when k_new is given)
 * Products are accumulated in fp32 in an order fixed by d_model alone (not by timing); when
 * every partial sum is exact in fp32 the result is the bf16 rounding (nearest, ties to even) of
 * the exact sum.  d_model: a multiple of 32, at most CLSA_MAX_D_MODEL.  No workspace.  A
 * sequence of length 0 (possible only when cu_seqlens_host is not given) gets q_idx but no
 * append.  Returns CLSA_ERR_UNSUPPORTED for PREFILL rows or an unsupported d_model.
 */
#define CLSA_MAX_D_MODEL 65536
clsa_status clsa_index_project(const clsa_dims* dims, const clsa_rows* rows, int32_t d_model, const clsa_bf16* h,
                               const clsa_bf16* w_q_idx, const clsa_bf16* w_k_idx, const int32_t* cu_seqlens,
                               clsa_bf16* q_idx, clsa_bf16* k_idx, const clsa_bf16* k_new, const clsa_bf16* v_new,
                               clsa_bf16* k_cache, clsa_bf16* v_cache, clsa_stream stream);

/*
 * The multi-layer distillation target and loss of the shared index (picx.dev summary,
 * Methodology, Multi-Layer Distillation, eq. 4-5), PREFILL rows only.  Row i is position
 * t = pos0 + i of sequence `seq` and sees tokens j = 0..t:
 *   A_t[j] = 1/(L hq) sum_{l < L, h < hq} softmax_j(q[i, l, h, :] . k_cache[cu[seq] + j, g(h), :] * scale)
 *   kl[i]  = KL(A_t || softmax_j(scores[i, j])) = sum_j A_t[j] (ln A_t[j] - ln softmax(scores[i])_j)
 *   *loss  = (1 / n_rows) sum_i kl[i]                                   (when loss != NULL)
 * with scale and g(h) = floor(h * hkv / hq) as in clsa_sparse_attn (the layers' own attention
 * distributions).  L = dims.n_layers.
 *   q       row i at q + i * q_row_stride, laid out [L, hq, 128] bf16 (q_row_stride >= L hq 128,
 *           a multiple of 8)
 *   k_cache [T, hkv, 128] bf16 (only K is read)
 *   scores  [n_rows, ld_scores] fp32: the routing scores I of the same rows, as clsa_index_scores
 *           writes them (ld_scores >= max_row_len, a multiple of 4)
 *   kl      [n_rows] fp32 (output), loss: one fp32 (output, optional)
 * fp32 softmax statistics and sums on bf16 products; every sum runs in an order fixed by the
 * sizes, so the results do not depend on timing.  The stop-gradient of eq. 5 does not change
 * these values.  Workspace: >= clsa_distill_workspace_bytes(dims, rows); its content on entry
 * does not matter.  Returns CLSA_ERR_UNSUPPORTED for DECODE rows.
 */
size_t clsa_distill_workspace_bytes(const clsa_dims* dims, const clsa_rows* rows);
clsa_status clsa_distill_kl(const clsa_dims* dims, const clsa_rows* rows, const clsa_bf16* q, int64_t q_row_stride,
                            const clsa_bf16* k_cache, const int32_t* cu_seqlens, const float* scores,
                            int64_t ld_scores, float* kl, float* loss, void* workspace, size_t workspace_bytes,
                            clsa_stream stream);

/* Everything one step reads and writes (all device pointers). */
typedef struct clsa_step_args {
  const clsa_bf16* q_idx;     /* [R, d_idx]                                               */
  const clsa_bf16* k_idx;     /* [T, d_idx]                                               */
  const clsa_bf16* k_cache;   /* [T, hkv, 128]                                            */
  const clsa_bf16* v_cache;   /* [T, hkv, 128]                                            */
  const int32_t* cu_seqlens;  /* [B+1]                                                    */
  const clsa_bf16* q;         /* [R, L, hq, 128]                                          */
  clsa_bf16* out;             /* [R, L, hq, 128]                                          */
  int32_t* idx;               /* [R, k]   selected set (output)                           */
  int32_t* count;             /* [R]      (output)                                        */
  float* scores;              /* optional [R, ld_scores] routing scores (output); NULL = kept
                                 in the workspace                                          */
  int64_t ld_scores;          /* used when scores != NULL                                 */
  clsa_bf16* k_sel;           /* optional compact buffers [R, hkv, k, 128] for the PER_LAYER */
  clsa_bf16* v_sel;           /*   DECODE schedule; NULL = carved from the workspace       */
  int32_t schedule;           /* CLSA_SCHEDULE_LAYER_BATCHED (all L layers in one pass over
                                 each selected row), CLSA_SCHEDULE_PER_LAYER (one pass per
                                 layer, as when layer l's query waits for layer l-1), or
                                 CLSA_SCHEDULE_PER_LAYER_ROUTING (the ablation without the
                                 shared index, see clsa_step)                               */
  int32_t prefill_chunk_rows; /* PREFILL: rows per chunk (0 = library default)            */
} clsa_step_args;

/*
 * One whole step: routing scores and top-k ONCE, then all L layers over the same selection
 * (eq. 2-3; the indexer cost is paid once rather than once per layer, picx.dev summary,
 * section Complexity Comparison).  Produces idx, count, out (and scores if requested).
 * DECODE: one launch sequence on `stream`.  PREFILL: rows processed in chunks of
 * prefill_chunk_rows.  Workspace: >= clsa_workspace_bytes(dims, rows, schedule,
 * prefill_chunk_rows).
 */
/*
 * CLSA_SCHEDULE_PER_LAYER_ROUTING (DECODE only) is the ablation the method is compared with:
 * routing is NOT shared, every layer l scores the cache with its own indexer query and selects
 * its own set (the per-layer indexer whose cost the picx.dev summary, section Complexity
 * Comparison, puts at eta L N instead of eta N).  The same kernels run once per layer:
 *   q_idx [R, L, d_idx]  (layer l's indexer query of row r at q_idx + (r * L + l) * d_idx)
 *   idx   [L, R, k], count [L, R]  (layer l's selection)
 *   out[r, l] = attention of layer l's query over layer l's selection.
 * scores, k_sel and v_sel must be NULL.  Workspace: clsa_workspace_bytes(..., this schedule, 0).
 */
clsa_status clsa_step(const clsa_dims* dims, const clsa_rows* rows, const clsa_step_args* args,
                      void* workspace, size_t workspace_bytes, clsa_stream stream);

/*
 * clsa_step for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments (minus the workspace), results and
 * errors as clsa_step; the caller still passes every input and output buffer.  The workspace is a
 * static device array of CLSA_NO_ALLOC_SCRATCH_BYTES owned by the library: each GPU holds its own
 * copy from the first call on that GPU until the process ends.  The call allocates nothing and calls
 * nothing that allocates.
 *  - Limit: a call whose step needs more scratch than that (at most clsa_workspace_bytes(dims, rows,
 *    args->schedule, args->prefill_chunk_rows) bytes) launches nothing and returns
 *    CLSA_ERR_UNSUPPORTED; smaller prefill chunks, or caller-owned scores / k_sel / v_sel, need less.
 *  - Concurrency: every call on one GPU shares that GPU's scratch, which keeps the last call's
 *    contents (each call clears what must start at zero).  Calls that overlap in time on one GPU
 *    (on other streams or from other threads) race on it and must not be made.
 */
#define CLSA_NO_ALLOC_SCRATCH_BYTES ((size_t)64 << 20)
clsa_status clsa_step_no_alloc(const clsa_dims* dims, const clsa_rows* rows, const clsa_step_args* args,
                               clsa_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* CLSA_H_ */
