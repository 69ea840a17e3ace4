/*
 * chunkkv.h -- C-ABI of the MI355X (gfx950) ChunkKV prefill-time KV-cache
 * compression library (libchunkkv.so).
 *
 * The method: page "ChunkKV: Semantic-Preserving KV Cache Compression for
 * Efficient Long-Context LLM Inference" (NeurIPS'25 blog post), section 4.1,
 * Algorithm 1 (inputs Q, K, V, observe window w, chunk size c, compressed
 * length L_max; output K', V') and section 4.2, Algorithm 2 (layer-wise index
 * reuse with N_reuse).  The attention probabilities are equation (1) of
 * section 2 of the page "Kara: Efficient reasoning-LLM serving via
 * sliding-window KV cache compression": softmax(Q K^T / sqrt(d)).
 *
 * What is computed, per layer l, sequence b and KV head h (T = T_b):
 *   1. x[g,r,t] = q[g,r] . k[t] / sqrt(d) for the G = H_q/H_kv query heads of
 *      the group (query head hq belongs to KV head hq / G) and the w window
 *      queries r (positions T-w .. T-1), over ALL T keys, no causal mask;
 *      p = softmax over t of each (g, r) row.
 *   2. C = ceil(T / c) chunks; chunk j covers tokens [j*c, min(j*c+c, T)).
 *   3. S[j] = sum over g, r and the chunk's tokens of p  (fp32).
 *   4. the k = floor(L_max / c) chunks with the largest S are selected
 *      (all C if k >= C, none if k == 0); equal scores: lower chunk id first.
 *   5. the last w tokens are always kept.
 *   6. indices = ascending, duplicate-free list of kept tokens, n of them
 *      (n <= L_cap = min(T, k*c + w)); K'[i] = K[indices[i]], V' likewise.
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned HIP device memory.  The library never
 *     allocates, frees or keeps device memory (the one exception is the fixed
 *     scratch array inside the library that chunkkv_decode_attention_static
 *     uses instead of a workspace).  Host pointers (problem
 *     struct and the arrays it points to, pointer tables) are read during the
 *     call only.  All buffers must stay valid until the work queued on
 *     `stream` (a hipStream_t; NULL = default stream) has finished.  Streams
 *     and events are passed as void pointers so that this header needs no
 *     HIP header: plain C callers and foreign-function bindings use it as is.
 *   - Arguments are validated on the host before anything is launched.  A
 *     non-OK status means nothing was launched and nothing was written;
 *     chunkkv_last_error() then returns a message (thread-local).
 *   - Launches are asynchronous on `stream`; there is no host<->device
 *     synchronisation and no device-side assert.  CHUNKKV_ERR_HIP reports a
 *     failed launch.
 *   - Inputs (Q, K, V) are never written.  Output rows i >= n are left
 *     untouched.
 *   - Element offsets and strides are in elements of the problem's dtype.
 *     Every K/V row and window-query row must start 16-byte aligned and
 *     head_dim * elem_bytes must be a multiple of 16.
 *   - Concurrent calls on different streams must use different workspaces
 *     and outputs.
 */
#ifndef CHUNKKV_H
#define CHUNKKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CHUNKKV_OK = 0,
  CHUNKKV_ERR_INVALID_ARG = 1, /* a value outside the method's domain */
  CHUNKKV_ERR_UNSUPPORTED = 2, /* valid for the method, not supported by this library */
  CHUNKKV_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than planned */
  CHUNKKV_ERR_HIP = 4          /* a HIP runtime call failed */
} chunkkv_status;

typedef enum { CHUNKKV_F32 = 0, CHUNKKV_BF16 = 1 } chunkkv_dtype;

/*
 * The problem of one layer (Algorithm 1's inputs), for a batch of
 * independent sequences packed along the token axis.
 *
 * seq_start  HOST [n_seqs + 1], non-decreasing: sequence b owns key/value
 *            token rows [seq_start[b], seq_start[b+1]); T_b = difference,
 *            1 <= window <= T_b < 2^31.
 * l_max      HOST [n_seqs]: L_max of each sequence, >= 0.  A budget ratio x
 *            is passed as floor(x * T_b).
 * K/V layout element (token row t, KV head h, dim i) at
 *            t*kv_stride_tok + h*kv_stride_head + i.
 * Window queries: element (sequence b, window row r, query head hq, dim i)
 *            at b*q_stride_seq + r*q_stride_row + hq*q_stride_head + i; row r
 *            is the query at position T_b - w + r (Algorithm 1 step 1 reads
 *            only these w rows).
 */
typedef struct {
  int32_t dtype;             /* chunkkv_dtype; Q, K, V, K', V' share it */
  int32_t n_seqs;            /* B >= 1 */
  const int64_t *seq_start;  /* HOST [B + 1] */
  const int64_t *l_max;      /* HOST [B] */
  int32_t n_q_heads;         /* H_q >= 1, multiple of n_kv_heads */
  int32_t n_kv_heads;        /* H_kv >= 1 */
  int32_t head_dim;          /* d: 8..256, d * elem_bytes multiple of 16 */
  int32_t window;            /* w >= 1 */
  int32_t chunk;             /* c >= 1 */
  int32_t reserved;          /* must be 0 (keeps the 64-bit fields aligned; room for a flag) */
  int64_t kv_stride_tok, kv_stride_head;
  int64_t q_stride_seq, q_stride_row, q_stride_head;
} chunkkv_problem;

/*
 * Sizes of one layer's outputs.  "Per scoring layer" buffers (scores,
 * indices, lengths) hold one block per layer that runs selection; K'/V' are
 * per layer.
 *   scores : fp32, element (b, h, j) at score_off[b] + h*C_b + j
 *   indices: int32, element (b, h, i) at index_off[b] + h*L_cap_b + i
 *   lengths: int32, element (b, h) at b*H_kv + h  (= n of that head)
 *   K', V' : rows of head_dim elements; row (b, h, i) is row
 *            index_off[b] + h*L_cap_b + i, i.e. head-major and position
 *            ordered per sequence.
 */
typedef struct {
  int64_t scores_elems;      /* sum_b H_kv * C_b */
  int64_t index_elems;       /* sum_b H_kv * L_cap_b (also the K'/V' row count) */
  int64_t length_elems;      /* B * H_kv */
  size_t workspace_bytes;    /* workspace for chunkkv_score on one layer */
} chunkkv_sizes;

/* Number of phase events chunkkv_compress_layers can record. */
#define CHUNKKV_N_PHASE_EVENTS 4

/*
 * Host-only planning: validates the problem and fills the sizes and, when
 * the arrays are non-NULL, the per-sequence offsets (HOST arrays of n_seqs
 * entries) and L_cap_b = min(T_b, floor(L_max_b / c) * c + w).  The sizes
 * follow ChunkKV page, section 4.1, Algorithm 1: step 2 fixes the chunk count
 * C_b = ceil(T_b / c) (the last chunk may be short, so scores_elems counts
 * C_b per head), step 4 the number of kept chunks k_b = floor(L_max_b / c),
 * and step 5 the w recent tokens that are always kept, so a head keeps at
 * most L_cap_b rows (index_elems counts L_cap_b per head).  Touches no device
 * and needs no GPU.
 *   p          HOST problem (read during the call only)
 *   out        HOST sizes out (required)
 *   score_off, index_off, l_cap  HOST int64 [n_seqs] out, each may be NULL
 * Errors: CHUNKKV_ERR_INVALID_ARG / CHUNKKV_ERR_UNSUPPORTED (out NULL, or
 * the problem outside the method's domain or this library's support),
 * nothing written.
 */
int chunkkv_plan(const chunkkv_problem *p, chunkkv_sizes *out, int64_t *score_off,
                 int64_t *index_off, int64_t *l_cap);

/*
 * Workspace needed by chunkkv_compress_layers to score `n_score_layers`
 * layers per launch (1 <= n_score_layers, counted up to 32; more layers per
 * launch means fewer launches).  Its size follows from the same quantities as
 * chunkkv_plan (ChunkKV page, section 4.1, Algorithm 1 step 2: C_b chunks per
 * head; step 3: the chunk scores are sums of softmax rows normalised over
 * all T_b keys, whose per-row statistics and, where the kernels keep them,
 * per-row chunk partials live here between launches).  Host only.  Returns 0
 * on invalid input (a NULL or invalid problem, n_score_layers < 1).
 */
size_t chunkkv_workspace_bytes(const chunkkv_problem *p, int32_t n_score_layers);

/*
 * Algorithm 1 steps 1-3 (ChunkKV page, section 4.1) with Kara eq. (1):
 * observe-window attention of every (sequence, KV head), summed into the
 * C_b chunk scores.  bf16 caches with head_dim 128 and c <= 3 whose G*w rows
 * fit one 128-row block are scored in two passes over the keys (row
 * statistics, then the final scores) instead of through per-row chunk
 * partials; the workspace is sized for whichever path the problem takes.
 *   q_win     DEVICE window queries (layout in chunkkv_problem)
 *   k         DEVICE keys (layout in chunkkv_problem)
 *   scores    DEVICE fp32 out, scores_elems entries (layout: chunkkv_sizes)
 *   workspace DEVICE scratch of >= chunkkv_sizes.workspace_bytes bytes
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE (ws NULL or too small), HIP.
 */
int chunkkv_score(const chunkkv_problem *p, const void *q_win, const void *k, float *scores,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Algorithm 1 steps 4-6 (ChunkKV page, section 4.1; the TopK -> index form
 * is Kara eqs. (2)-(3)): per (sequence, KV head) select the floor(L_max/c)
 * top-scoring chunks (ties: lower chunk id), add the last w tokens, and write
 * the kept token positions (0-based within the sequence) in ascending order.
 *   scores   DEVICE fp32, as written by chunkkv_score (>= 0).  Any other
 *            values are accepted: a score with the sign bit set counts as 0
 *            and the rest are ordered by their bit patterns (+inf above every
 *            finite score), so exactly min(k, C) chunks are always selected
 *            and every index lies in [0, T_b).
 *   indices  DEVICE int32 out, index_elems entries (entries i >= n untouched)
 *   lengths  DEVICE int32 out, length_elems entries
 * No workspace: a head's scores are held in registers (C_b <= 32768) or
 * re-read from `scores`.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
int chunkkv_select(const chunkkv_problem *p, const float *scores, int32_t *indices,
                   int32_t *lengths, void *stream);

/*
 * Algorithm 1 step 6, index_select (ChunkKV page, section 4.1): byte copy of
 * the kept K and V rows into the compacted caches.
 *   k, v          DEVICE inputs (layout in chunkkv_problem)
 *   indices, lengths  DEVICE, as written by chunkkv_select (any layer's)
 *   k_out, v_out  DEVICE out, index_elems rows of head_dim elements each
 *                 (16-byte aligned); rows i >= n untouched
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.  Indices and lengths as written by
 * chunkkv_select are always valid; other values are clamped (lengths into
 * [0, L_cap_b], index values into [0, T_b)), so no input makes the copy read
 * or write outside the sequence's rows and the head's output rows.
 */
int chunkkv_gather(const chunkkv_problem *p, const void *k, const void *v,
                   const int32_t *indices, const int32_t *lengths, void *k_out, void *v_out,
                   void *stream);

/*
 * Algorithm 2 (ChunkKV page, section 4.2, layer-wise index reuse) over
 * n_layers layers sharing one problem shape: layer l scores and selects iff
 * l mod n_reuse == 0 (an anchor layer); every other layer gathers its OWN
 * K/V with the indices of anchor floor(l / n_reuse) * n_reuse.
 *   q_win, k, v     HOST tables [n_layers] of DEVICE pointers (q_win[l] may be
 *                   NULL where l mod n_reuse != 0)
 *   k_out, v_out    HOST tables [n_layers] of DEVICE outputs
 *   scores, indices, lengths  DEVICE, n_anchor = ceil(n_layers / n_reuse)
 *                   consecutive per-scoring-layer blocks (block a belongs to
 *                   layer a * n_reuse)
 *   workspace       DEVICE scratch of >= chunkkv_workspace_bytes(p, 1) bytes;
 *                   a larger one lets more anchor layers share a launch
 *   phase_events    NULL, or HOST [CHUNKKV_N_PHASE_EVENTS] hipEvent_t handles
 *                   marking, on `stream`, the start of the scoring phase,
 *                   its end, the start of the gather phase and its end (for
 *                   timing; any entry may be NULL).  A phase that is a
 *                   single kernel launch (the bf16 d=128 score kernel over
 *                   every scoring layer, unless the problem is scored in two
 *                   passes; the gather over at most 32 layers; at most 8
 *                   sequences) takes its two events at that
 *                   kernel's own start and end (hipExtLaunchKernel);
 *                   otherwise they are recorded between the phases'
 *                   kernels.  When the
 *                   workspace cannot hold every scoring layer at once, the
 *                   phases interleave and entry 1 is recorded together with
 *                   entry 2.
 * The call allocates nothing and issues no memset or copy, only kernel
 * launches (and the phase events): without phase events it can be captured
 * into a HIP graph, whose replays give the same outputs.
 * Errors: INVALID_ARG (incl. n_layers < 1, n_reuse < 1, a NULL table entry
 * that is needed), UNSUPPORTED, WORKSPACE, HIP.
 */
int chunkkv_compress_layers(const chunkkv_problem *p, int32_t n_layers, int32_t n_reuse,
                            const void *const *q_win, const void *const *k,
                            const void *const *v, void *const *k_out, void *const *v_out,
                            float *scores, int32_t *indices, int32_t *lengths, void *workspace,
                            size_t workspace_bytes, void *stream, void *const *phase_events);

/*
 * The hybrid layer policy (ChunkKV page, section 5.7: chunk-level selection in
 * some layers, token-level selection, i.e. c = 1, in others) as a per-layer
 * chunk size.  layer_chunk is a HOST [n_layers] table of chunk sizes; p->chunk
 * is ignored and every other field of p applies to all layers.  Layers are
 * taken in runs of consecutive layers with the same chunk size, and Algorithm
 * 2 (section 4.2) restarts at each run: in a run starting at layer r0, layer
 * l scores iff (l - r0) mod n_reuse == 0 and otherwise gathers with the
 * indices of anchor r0 + floor((l - r0) / n_reuse) * n_reuse, so indices are
 * never reused across a change of chunk size.
 *
 * Host-only planning of chunkkv_compress_layers_hybrid's buffers.  Anchors
 * are numbered in layer order; anchor a's scores, indices and lengths start at
 * element score_block_off[a], index_block_off[a] and length_block_off[a] of
 * the scores, indices and lengths buffers, each block laid out as
 * chunkkv_sizes describes for the problem with that anchor's chunk size;
 * entry n_anchor of each array holds the buffer's total size in elements.
 * kv_out_rows[l] is the row count of layer l's K'/V' (the index_elems of its
 * chunk size).  workspace_bytes is the largest chunkkv_workspace_bytes(p_c,
 * n_c) over the runs, n_c the run's anchor count: with it every run scores all
 * its anchors (up to 32) in one launch per phase.  Any workspace of at least
 * the largest chunkkv_workspace_bytes(p_c, 1) works, with fewer anchors per
 * launch.
 *   n_anchor          HOST out, may be NULL
 *   *_block_off       HOST int64 [n_layers + 1] out (n_anchor <= n_layers),
 *                     each may be NULL
 *   kv_out_rows       HOST int64 [n_layers] out, may be NULL
 *   workspace_bytes   HOST out, may be NULL
 * Errors: INVALID_ARG (layer_chunk NULL, n_layers < 1, n_reuse < 1, or a
 * layer's problem invalid, as in chunkkv_plan), UNSUPPORTED.
 */
int chunkkv_plan_hybrid(const chunkkv_problem *p, const int32_t *layer_chunk, int32_t n_layers,
                        int32_t n_reuse, int32_t *n_anchor, int64_t *score_block_off,
                        int64_t *index_block_off, int64_t *length_block_off, int64_t *kv_out_rows,
                        size_t *workspace_bytes);

/*
 * chunkkv_compress_layers with a per-layer chunk size (the layer runs and
 * block layout of chunkkv_plan_hybrid): the scoring layers of every run are
 * scored and selected, then every layer is gathered.  Arguments as in
 * chunkkv_compress_layers, with
 *   scores, indices, lengths  DEVICE, the anchors' blocks at the offsets
 *                   chunkkv_plan_hybrid gives (totals in its entry n_anchor)
 *   k_out[l], v_out[l]  DEVICE, kv_out_rows[l] rows each
 *   workspace       DEVICE scratch of >= the largest chunkkv_workspace_bytes
 *                   (p_c, 1) over the chunk sizes used (chunkkv_plan_hybrid's
 *                   workspace_bytes lets each run score all its anchors at once)
 *   phase_events    NULL, or HOST [CHUNKKV_N_PHASE_EVENTS] hipEvent_t
 *                   handles recorded on `stream` before the first scoring
 *                   launch, after the last selection (entries 1 and 2) and
 *                   after the last gather.
 * The call allocates nothing and issues only kernel launches (and the phase
 * events).  Its outputs equal those of one chunkkv_compress_layers call per
 * run with that run's chunk size.
 * Errors: as chunkkv_plan_hybrid, and as chunkkv_compress_layers.
 */
int chunkkv_compress_layers_hybrid(const chunkkv_problem *p, const int32_t *layer_chunk,
                                   int32_t n_layers, int32_t n_reuse, const void *const *q_win,
                                   const void *const *k, const void *const *v,
                                   void *const *k_out, void *const *v_out, float *scores,
                                   int32_t *indices, int32_t *lengths, void *workspace,
                                   size_t workspace_bytes, void *stream,
                                   void *const *phase_events);

/*
 * Workspace needed by chunkkv_decode_attention for problem p: per-block
 * partials of every (sequence, KV head, block of kept rows, query head).
 * Host only.  Returns 0 on invalid input.
 */
size_t chunkkv_decode_workspace_bytes(const chunkkv_problem *p);

/*
 * Decode attention over the compacted cache: the step that consumes it (the
 * ChunkKV page's latency / throughput section decodes over the compressed
 * cache).  For every sequence b and query head hq one new query attends over
 * the kept rows of KV head hq / G with weights softmax(q . k / sqrt(d))
 * (Kara eq. (1)); the output is the weighted sum of the kept value rows.
 * The new token's own key and value are not included (an engine appends
 * them); a head with no kept rows gives zeros.
 *   q_dec         DEVICE [n_seqs][n_q_heads][head_dim], the problem's dtype,
 *                 16-byte aligned
 *   k_out, v_out  DEVICE compacted caches as written by chunkkv_gather
 *                 (rows index_off[b] + h * L_cap_b + i), 16-byte aligned
 *   lengths       DEVICE int32 [n_seqs * n_kv_heads], as written by
 *                 chunkkv_select (other values are clamped into [0, L_cap_b])
 *   out           DEVICE fp32 [n_seqs][n_q_heads][head_dim]
 *   workspace     DEVICE scratch of >= chunkkv_decode_workspace_bytes(p)
 *                 bytes, 16-byte aligned
 * All buffers belong to the caller; the call allocates nothing and only
 * launches kernels on `stream`, so it can be captured into a HIP graph.
 * Errors: INVALID_ARG, UNSUPPORTED (incl. misaligned buffers), WORKSPACE, HIP.
 */
int chunkkv_decode_attention(const chunkkv_problem *p, const void *q_dec, const void *k_out,
                             const void *v_out, const int32_t *lengths, float *out,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Size of the scratch array chunkkv_decode_attention_static uses (per GPU). */
#define CHUNKKV_STATIC_SCRATCH_BYTES (16u << 20)

/*
 * chunkkv_decode_attention without a caller workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments (minus the
 * workspace), same kernels and the same results as chunkkv_decode_attention.
 * The per-block partials go to a file-scope device array of
 * CHUNKKV_STATIC_SCRATCH_BYTES (16 MiB) inside the library, one per GPU the
 * library runs on, held until the process ends.  The call allocates and frees
 * nothing (no hipMalloc, no allocating library routine); its first call on a
 * device looks up that device's copy of the array (hipGetSymbolAddress) and
 * keeps the address.  Every call on a GPU shares that GPU's array and it
 * keeps the last call's contents (no call relies on them): calls that
 * overlap in time on one GPU (other streams, other host threads) race on it
 * and must be ordered by the caller.
 * Errors: as chunkkv_decode_attention; CHUNKKV_ERR_WORKSPACE (before anything
 * is launched) when chunkkv_decode_workspace_bytes(p) exceeds
 * CHUNKKV_STATIC_SCRATCH_BYTES; CHUNKKV_ERR_HIP when the array's address
 * cannot be looked up.
 */
int chunkkv_decode_attention_static(const chunkkv_problem *p, const void *q_dec, const void *k_out,
                                    const void *v_out, const int32_t *lengths, float *out,
                                    void *stream);

/*
 * Paged output: the same copy as chunkkv_gather (ChunkKV page, section 4.1,
 * Algorithm 1 step 6), written into a pool of fixed-size pages of
 * consecutive KV rows, the block layout of PagedAttention (Kara page,
 * section 2), instead of one contiguous run per head.  Kept row i of
 * (sequence b, KV head h) goes to row i % page_rows of page
 * block_table[(b * n_kv_heads + h) * max_pages + i / page_rows].
 *   k, v          DEVICE inputs (layout in chunkkv_problem)
 *   indices, lengths  DEVICE, as written by chunkkv_select (clamped as in
 *                 chunkkv_gather)
 *   block_table   DEVICE int32 [n_seqs * n_kv_heads][max_pages]: the pool
 *                 pages of each (sequence, head) in order; max_pages must
 *                 cover ceil(L_cap_b / page_rows) for every sequence
 *   k_pages, v_pages  DEVICE out [n_pages][page_rows][head_dim], 16-byte
 *                 aligned; only the rows of kept rows are written.  A page id
 *                 outside [0, n_pages) leaves its rows unwritten; pages
 *                 listed twice get the rows of whichever copy lands last.
 * All buffers belong to the caller; the call allocates nothing and only
 * launches kernels on `stream`, so it can be captured into a HIP graph.
 * Errors: INVALID_ARG (incl. page_rows, max_pages or n_pages < 1, a table
 * too short for L_cap), UNSUPPORTED, HIP.
 */
int chunkkv_gather_paged(const chunkkv_problem *p, const void *k, const void *v,
                         const int32_t *indices, const int32_t *lengths,
                         const int32_t *block_table, int32_t max_pages, int32_t page_rows,
                         int64_t n_pages, void *k_pages, void *v_pages, void *stream);

/* Message of this thread's last non-OK status ("" if none). */
const char *chunkkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CHUNKKV_H */
