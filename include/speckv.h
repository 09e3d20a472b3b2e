/*
 * speckv.h — C ABI of the MI355X (gfx950) SpecKV / SpecPC scoring library.
 *
 * The operations follow the paper notes "Draft-based Approximate Inference
 * for LLMs" (ICLR 2026 notes page):
 *   - section "Key designs", SpecKV paragraph: per attention head, the
 *     importance of each KV pair is the cross-attention of the observation
 *     queries (the last n_window input tokens plus the n_lookahead draft
 *     tokens) against the remaining input keys; the top C_max pairs are kept
 *     together with the window's pairs;
 *   - section "Key designs", SpecPC paragraph: token importance from the
 *     draft's attention activations over a window of queries with weights
 *     that fall away from the end, skipping the first l_skip layers, mean
 *     first and then max;
 *   - section "Key designs", SpecKV-PC paragraph: SpecPC first cuts the
 *     prompt, then SpecKV cuts the target's cache over the shorter prompt;
 *   - section "Loss / training strategy": local pooling keeps the kept
 *     tokens contiguous;
 *   - section "Background": attention compute and KV-cache memory grow with
 *     the context, which decode attention over the compacted cache saves.
 *
 * Conventions shared by every entry point
 *   - All buffer pointers are DEVICE pointers owned by the caller, including
 *     the workspace.  The library allocates and frees no device memory.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *     null stream) and returns; outputs are valid once the stream has
 *     completed.  Calls that share one workspace must be ordered on one
 *     stream.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is launched and the outputs are untouched.  No C++
 *     exception crosses this interface: every entry point catches them and
 *     returns SKV_ERR_INTERNAL.
 *   - The library keeps no state between calls except the optional
 *     event-timing lists of speckv_profile_* (host memory, process-wide,
 *     empty unless profiling is enabled).
 *   - NaN or Inf inputs give undefined (but memory-safe) results.
 *   - Element types: SKV_F32 (float) or SKV_BF16 (bfloat16 stored as
 *     uint16).  head_dim must be 64 or 128.  Query, key and value buffers
 *     (inputs and compacted or gathered outputs) and the workspace must be
 *     16-byte aligned, and kv_head_stride * element size must be a multiple
 *     of 16; score, pooled, weight, index and decode-output buffers need
 *     4-byte alignment.  A violation returns SKV_ERR_ALIGN.
 */
#ifndef SPECKV_H
#define SPECKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum skv_status {
  SKV_OK = 0,
  SKV_ERR_NULL = 1,      /* a required pointer is NULL                           */
  SKV_ERR_SHAPE = 2,     /* sizes inconsistent, out of range or unsupported      */
  SKV_ERR_DTYPE = 3,     /* unsupported element type                             */
  SKV_ERR_PARAM = 4,     /* C_max, pooling, l_skip or n_keep out of range        */
  SKV_ERR_WORKSPACE = 5, /* workspace NULL or smaller than the query returns     */
  SKV_ERR_ALIGN = 6,     /* a pointer or the head stride is not 16-byte aligned  */
  SKV_ERR_ALIAS = 7,     /* outputs overlap inputs other than the in-place form  */
  SKV_ERR_HIP = 8,       /* a HIP runtime call or kernel launch failed           */
  SKV_ERR_INTERNAL = 9   /* host-side failure inside the library (a C++          */
                         /* exception, e.g. out of host memory) caught at the    */
                         /* interface; outputs are then unspecified              */
} skv_status;

typedef enum skv_dtype { SKV_F32 = 0, SKV_BF16 = 1 } skv_dtype;

typedef enum skv_pool { SKV_POOL_NONE = 0, SKV_POOL_MAX = 1, SKV_POOL_AVG = 2 } skv_pool;

/* Aggregation of the observation rows' probabilities into a key's score. */
typedef enum skv_agg { SKV_AGG_SUM = 0, SKV_AGG_MAX = 1 } skv_agg;

/* Problem shape.  Layouts (row-major, head_dim contiguous):
 *   K, V   : [n_layers][n_kv_heads][kv_head_stride]; head slab h of layer l
 *            holds n_in rows of head_dim elements, rows beyond n_in unused.
 *   SpecKV : Q_obs [n_layers][n_q_heads][n_window + n_lookahead][head_dim],
 *            window rows first, then lookahead rows.
 *   SpecPC : Q_win [n_layers][n_q_heads][n_window][head_dim]; row i is the
 *            query of input position n_in - n_window + i.
 * Query head hq uses KV head hq / G, G = n_q_heads / n_kv_heads.
 * SpecKV scores, selects and compacts per "head" h < H, where H = n_kv_heads
 * (one kept set per KV head, shared by its G query heads; the default) or
 * H = n_q_heads with per_query_head = 1 (the key designs paragraph
 * estimates importance per attention head; query head hq is scored alone
 * against KV head hq / G, and its compacted cache holds rows of that KV
 * head). */
typedef struct skv_shape {
  int32_t n_layers;       /* >= 1                                                   */
  int32_t n_q_heads;      /* multiple of n_kv_heads                                 */
  int32_t n_kv_heads;     /* >= 1                                                   */
  int32_t head_dim;       /* 64 or 128                                              */
  int64_t n_in;           /* input tokens (K/V rows per head), 1 .. 2^31 - 1        */
  int64_t kv_head_stride; /* elements between head slabs; 0 means n_in * head_dim   */
  int32_t n_window;       /* SpecKV: window rows (0 .. n_in); SpecPC: W (1 .. n_in) */
  int32_t n_lookahead;    /* SpecKV: draft rows (>= 0); SpecPC: 1                   */
  float scale;            /* logit scale; 0 means 1 / sqrt(head_dim)                */
  int32_t dtype;          /* skv_dtype of Q, K and V                                */
  int32_t aggregation;    /* SpecKV: skv_agg over the observation rows; SpecPC: 0   */
  int32_t per_query_head; /* SpecKV: 0 (H = n_kv_heads) or 1 (H = n_q_heads); SpecPC: 0 */
} skv_shape;

/* Human-readable name of a status code (static storage). */
const char* speckv_status_string(int32_t status); /* any value; unknown codes get "unknown status" */

/* Workspace bytes that suffice for every entry point below on this shape
 * (SpecKV with the given C_max, or SpecPC when called as such).  The same
 * workspace may be reused by consecutive calls on one stream. */
skv_status speckv_workspace_bytes(const skv_shape* shape, int32_t C_max, size_t* out_bytes);

/* Kept rows per head: min(C_max, n_in - n_window) + n_window (SpecKV, key
 * designs paragraph: the top C_max pairs plus the window pairs). */
skv_status speckv_n_keep(const skv_shape* shape, int32_t C_max, int64_t* out_n_keep);

/* SpecKV importance scores ("Key designs", SpecKV).
 * For every layer l and head h < H, with rows r = (query head g of h's
 * group, or h's query head alone with per_query_head, and observation row
 * i) and the n_pre = n_in - n_window remaining input keys:
 *   P[r][j]  = softmax over j < n_pre of scale * <q_r, k_j>
 *   score[j] = sum over r of P[r][j]        (aggregation SKV_AGG_SUM)
 *            = max over r of P[r][j]        (aggregation SKV_AGG_MAX)
 * Inputs : q_obs (see skv_shape), k.
 * Output : scores float [n_layers][H][n_pre] (raw sums total G or 1 times
 *          (n_window + n_lookahead) per head).
 * Requires n_window + n_lookahead >= 1 and G * (n_window + n_lookahead)
 * <= 2^20; n_pre = 0 is accepted and does nothing (scores may then be NULL). */
skv_status speckv_scores(const skv_shape* shape, const void* q_obs, const void* k, float* scores,
                         void* workspace, size_t workspace_bytes, void* stream);

/* speckv_scores without a workspace, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, results and errors as speckv_scores
 * (bit-identical scores), with a fixed scratch array of 64 MiB inside the
 * library standing in for the workspace: one copy per GPU, held from the
 * first call on that GPU until the process ends.  The call allocates and
 * frees nothing.  It returns SKV_ERR_WORKSPACE when the problem needs more
 * scratch than that (e.g. up to 30 of the 64 layers of the 64K
 * Qwen2.5-32B-shaped workload fit per call, and up to 7 layers of the 128K
 * Llama-3.1-8B-shaped one), and
 * SKV_ERR_PARAM when `stream` belongs to a device other than the current one.
 * Every call on one GPU uses the same scratch: calls that overlap on one GPU
 * (other streams, other threads) race and must be ordered by the caller.
 * Nothing in the scratch needs clearing between calls. */
skv_status speckv_scores_noalloc(const skv_shape* shape, const void* q_obs, const void* k, float* scores,
                                 void* stream);

/* SpecKV selection ("Key designs", SpecKV; "Loss / training strategy",
 * local pooling).  Per head: pooled = pool1d(scores) over the n_pre prefix
 * scores (stride 1, odd pool_kernel in 1 .. 4097, windows truncated at both
 * ends; max or in-range mean; SKV_POOL_NONE copies); then the
 * min(C_max, n_pre) best prefix keys, ordered by pooled score descending and
 * lower index first on ties (-0 equals +0), plus every window key
 * n_pre .. n_in - 1; written ascending.
 * Inputs : scores float [n_layers][H][n_pre] (any finite values, non-negative
 *          from speckv_scores; NULL when n_pre = 0, where the kept list is
 *          the window alone).
 * Outputs: kept int32 [n_layers][H][n_keep]; pooled float
 *          [n_layers][H][n_pre] or NULL.
 * The SpecPC token selection is this call on a shape with n_layers = 1,
 * n_kv_heads = 1 (n_q_heads = 1), n_in = tokens, n_window = 0. */
skv_status speckv_select(const skv_shape* shape, const float* scores, int32_t C_max, int32_t pool,
                         int32_t pool_kernel, int32_t* kept, float* pooled, void* workspace,
                         size_t workspace_bytes, void* stream);

/* SpecKV compaction ("Key designs", SpecKV: keep the selected KV pairs).
 * Per head h < H: out[t] = in[kept[t]] for t < n_keep, for K and V,
 * bit-exact, reading KV head h (or h / G with per_query_head).
 * Out of place: k_out, v_out are [n_layers][H][n_keep][head_dim] and must
 *   not overlap k or v.
 * In place: k_out == k and v_out == v; rows 0 .. n_keep - 1 of every head
 *   slab are overwritten, the stride is unchanged and rows >= n_keep are
 *   left unspecified.  Requires kept ascending (as speckv_select writes it),
 *   and H = n_kv_heads (SKV_ERR_PARAM otherwise).
 * kept int32 [n_layers][H][n_keep], values in [0, n_in); n_keep in 1 .. n_in. */
skv_status speckv_compact(const skv_shape* shape, const void* k, const void* v, const int32_t* kept,
                          int64_t n_keep, void* k_out, void* v_out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Token gather for the SpecKV-PC cascade ("Key designs", SpecKV-PC: SpecPC
 * first cuts the prompt to its kept tokens, then SpecKV works on the
 * target's cache over that shorter prompt).  For every layer and KV head:
 *   k_out[t] = k[tokens[t]], v_out[t] = v[tokens[t]] for t < n_tokens,
 * bit-exact, with one token list shared by every head (as specpc_token_scores
 * and speckv_select produce it).  It stands in for the target's cache of the
 * compressed prompt when a cache over the full prompt is at hand.
 * Uses n_layers, n_kv_heads, head_dim, n_in, kv_head_stride and dtype of
 * the shape (the rest is validated as usual and otherwise ignored).
 * Inputs : k, v [n_layers][n_kv_heads][kv_head_stride] (rows of n_in);
 *          tokens int32 [n_tokens] on the device, values in [0, n_in) (a
 *          token outside that range yields a zero row).
 * Outputs: k_out, v_out [n_layers][n_kv_heads][n_tokens][head_dim],
 *          contiguous; out of place only (SKV_ERR_ALIAS on any overlap).
 * Requires 1 <= n_tokens <= n_in (SKV_ERR_PARAM otherwise). */
skv_status specpc_gather_tokens(const skv_shape* shape, const void* k, const void* v, const int32_t* tokens,
                                int64_t n_tokens, void* k_out, void* v_out, void* stream);

/* SpecKV over keys taken through a row list ("Key designs", SpecKV-PC:
 * SpecKV on the target's cache over the prompt SpecPC kept, without first
 * gathering that cache).  The shape describes the logical problem: n_in is
 * the number of listed rows (the compressed prompt's tokens) and
 * kv_head_stride the stride of the physical head slabs, each holding
 * n_src_rows rows (n_src_rows * head_dim <= kv_head_stride).  Logical key j
 * of every head is physical row rows[j]; rows int32 [n_in] on the device,
 * values in [0, n_src_rows) (a value outside reads a clamped row: the
 * results are then unspecified but memory-safe).
 * speckv_scores_rows equals speckv_scores on the gathered cache
 * (specpc_gather_tokens with the same list), bit for bit, with the same
 * workspace.  speckv_compact_rows writes, out of place only,
 *   out[t] = k[rows[kept[t]]] (and v) for t < n_keep,
 * the kept list holding logical indices as speckv_select writes them (a
 * logical index outside [0, n_in), or a row outside [0, n_src_rows), gives
 * a zero row); outputs as speckv_compact's, SKV_ERR_ALIAS on any overlap. */
skv_status speckv_scores_rows(const skv_shape* shape, const void* q_obs, const void* k, const int32_t* rows,
                              int64_t n_src_rows, float* scores, void* workspace, size_t workspace_bytes,
                              void* stream);
skv_status speckv_compact_rows(const skv_shape* shape, const void* k, const void* v, const int32_t* rows,
                               int64_t n_src_rows, const int32_t* kept, int64_t n_keep, void* k_out,
                               void* v_out, void* stream);

/* SpecPC token scores ("Key designs", SpecPC).
 * The draft's query axis has n_keys = n_in + n_lookahead - 1 positions (the
 * input tokens, then the generated draft tokens but the last; n_keys = n_in
 * when n_lookahead <= 1), and so does its key axis.  For layers
 * l_skip <= l < n_layers and every query head hq, window row i (position
 * p_i = n_keys - W + i, W = n_window) attends causally:
 *   P[l][hq][i][j] = softmax over j <= p_i of scale * <q_i, k_j>, 0 for j > p_i
 *   Abar[i][j]     = mean over (l, hq) of P, for the input tokens j < n_in
 *   token_scores[j] = max over i of w_i * Abar[i][j]
 * query_weights: float [W] on the device, or NULL for w_i = 0.1 + 0.9 i/(W-1)
 * (1 at the end of the window, 0.1 at its far edge; 1 when W = 1).
 * Inputs : q_win [n_layers][n_q_heads][W][head_dim] (all layers, skipped
 *          ones included), k [n_layers][n_kv_heads][kv_head_stride] with
 *          n_keys rows per head (kv_head_stride >= n_keys * head_dim,
 *          SKV_ERR_SHAPE otherwise).  Output: token_scores float [n_in].
 * Requires 0 <= l_skip < n_layers, 1 <= W <= n_in, G * W <= 2^20, and
 * aggregation = per_query_head = 0 (SKV_ERR_PARAM otherwise). */
skv_status specpc_token_scores(const skv_shape* shape, int32_t l_skip, const void* q_win, const void* k,
                               const float* query_weights, float* token_scores, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Decode attention over a (compacted) KV cache ("Background": attention and
 * KV cache cost grow with the context; "Key designs", SpecKV: generation
 * runs over the kept pairs).  For every layer l and query head hq, with
 * cache head h = hq / G (G = n_q_heads / n_kv_heads), or h = hq with
 * per_query_head (one cache per query head, as speckv_compact writes it):
 *   out[l][hq] = sum_{j < n_rows} softmax_j(scale * <q[l][hq], k[l][h][j]>) v[l][h][j]
 * (no mask: every cached row precedes the new token; append the new
 * token's own K/V row to attend it).
 * The shape describes the cache buffers: k, v are [n_layers][H][kv_head_stride]
 * with rows of head_dim elements, H = n_kv_heads (or n_q_heads with
 * per_query_head), n_in rows allocated per head.  After out-of-place
 * compaction pass n_in = n_rows = n_keep; after in-place compaction the
 * prefill shape and n_rows = n_keep.  n_window, n_lookahead and aggregation
 * are ignored.  bf16 or fp32 (the shape's dtype); G <= 16 (SKV_ERR_SHAPE).
 * Inputs : q [n_layers][n_q_heads][head_dim] in the cache dtype; k, v as above.
 * Output : out float [n_layers][n_q_heads][head_dim].
 * Requires 1 <= n_rows <= n_in (SKV_ERR_PARAM).  Long caches are split over
 * several blocks per head, whose partial results go to the workspace;
 * speckv_decode_workspace_bytes reports its size (0 bytes when every head
 * fits one block, e.g. up to 512 rows; NULL is then allowed). */
skv_status speckv_decode_workspace_bytes(const skv_shape* shape, int64_t n_rows, size_t* out_bytes);
skv_status speckv_decode_attention(const skv_shape* shape, int64_t n_rows, const void* q, const void* k,
                                   const void* v, float* out, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Optional per-kernel timing with HIP events, for measurement only.
 * While enabled, every kernel the library launches is bracketed by a pair
 * of events on its stream.  speckv_profile_read synchronizes on the
 * recorded events and reports, per kernel name, the launch count and the
 * summed event time.  Process-wide state, not thread-safe; off by default.
 * If a sample could not be recorded (host memory exhausted), the read
 * returns SKV_ERR_INTERNAL after filling in the totals it has. */
skv_status speckv_profile_enable(int32_t on);
int32_t speckv_profile_count(void);
skv_status speckv_profile_read(int32_t index, const char** name, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* SPECKV_H */
