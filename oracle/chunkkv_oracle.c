/*
 * chunkkv_oracle.c -- plain, slow CPU oracle for ChunkKV prefill-time KV-cache
 * compression.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library under kv_cache_compression_win_amd/) shares no code with it and
 * never calls it.
 *
 * Source of truth: the page "ChunkKV: Semantic-Preserving KV Cache Compression
 * for Efficient Long-Context LLM Inference" (NeurIPS'25 blog post), section 4.1
 * (Algorithm 1, ChunkKV) and section 4.2 (Algorithm 2, layer-wise index
 * reuse); the attention probability definition is equation (1) of section 2 of
 * the page "Kara: Efficient reasoning-LLM serving via sliding-window KV cache
 * compression", and the TopK -> index form is equations (2)-(3) there.
 *
 * Everything is computed in double precision.  bf16 and fp32 inputs are
 * widened exactly.  Nothing is blocked, fused or reordered: scores come from a
 * naive rows x keys x head_dim loop, top-k from a full sort, gather from one
 * memcpy per row.
 *
 * Readings taken where the pages leave a step open (each one is also listed
 * in the design notes of the repository):
 *   - attention rows are softmax(q . k / sqrt(d)) over ALL T keys of the
 *     sequence, no causal mask (Algorithm 1 step 1 states A is w x T_k;
 *     scale and softmax from Kara eq. (1));
 *   - with grouped-query attention, query head hq belongs to KV head
 *     hq / G (G = n_q_heads / n_kv_heads); the rows of all G query heads of
 *     the group are summed into that KV head's chunk scores, each row
 *     normalised on its own;
 *   - the short last chunk is summed, not averaged; every one of the
 *     C = ceil(T/c) chunks is a top-k candidate, window chunks included;
 *   - equal scores are ordered by lower chunk id first;
 *   - the output is the ascending, duplicate-free union of the selected
 *     chunks' tokens and the last w tokens.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ENOMEM 2

/* Exact widening of one stored element to double. */
static double widen(const void *base, int dtype, int64_t idx) {
  if (dtype == ORC_F32) return (double)((const float *)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

int64_t orc_num_chunks(int64_t T, int64_t c) {
  /* Algorithm 1 step 2: C = ceil(T_k / c); the last chunk may be short. */
  return (T + c - 1) / c;
}

int64_t orc_num_keep_chunks(int64_t l_max, int64_t c) {
  /* Algorithm 1 step 4: k = floor(L_max / c). */
  return l_max / c;
}

/*
 * Algorithm 1 steps 1-3 for one sequence and one KV head h.
 *
 * q     : queries of the sequence, element (t, hq, i) at
 *         q[t*q_tok_stride + hq*q_head_stride + i], rows 0..t_q-1; only the
 *         observe window, rows t_q-w .. t_q-1, is read (step 1).
 * k     : keys of the sequence, element (t, h, i) at
 *         k[t*k_tok_stride + h*k_head_stride + i], t < T.
 * scores: out, C doubles, C = ceil(T/c).
 *
 * For every window row of every query head of the group:
 *   x_t = (sum_i q_i k_{t,i}) / sqrt(d)         (Kara eq. (1))
 *   p_t = exp(x_t - max x) / sum_u exp(x_u - max x)
 * and scores[j] += sum of p_t over tokens t of chunk j (step 3).
 */
int orc_chunk_scores(int dtype, int64_t T, int64_t t_q, int n_q_heads,
                     int n_kv_heads, int h, int d, int w, int c, const void *q,
                     int64_t q_tok_stride, int64_t q_head_stride,
                     const void *k, int64_t k_tok_stride,
                     int64_t k_head_stride, double *scores) {
  if (T < 1 || d < 1 || w < 1 || c < 1 || n_kv_heads < 1 ||
      n_q_heads % n_kv_heads != 0 || h < 0 || h >= n_kv_heads || w > T ||
      w > t_q || (dtype != ORC_F32 && dtype != ORC_BF16))
    return ORC_EINVAL;
  const int G = n_q_heads / n_kv_heads;
  const int64_t C = orc_num_chunks(T, c);
  double *x = (double *)malloc((size_t)T * sizeof(double));
  if (!x) return ORC_ENOMEM;
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
  for (int64_t j = 0; j < C; ++j) scores[j] = 0.0;

  for (int g = 0; g < G; ++g) {
    const int hq = h * G + g;
    for (int r = 0; r < w; ++r) {
      const int64_t qt = t_q - w + r; /* observe-window row */
      for (int64_t t = 0; t < T; ++t) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i)
          acc += widen(q, dtype, qt * q_tok_stride + (int64_t)hq * q_head_stride + i) *
                 widen(k, dtype, t * k_tok_stride + (int64_t)h * k_head_stride + i);
        x[t] = acc * inv_sqrt_d;
      }
      double m = x[0];
      for (int64_t t = 1; t < T; ++t)
        if (x[t] > m) m = x[t];
      double s = 0.0;
      for (int64_t t = 0; t < T; ++t) s += exp(x[t] - m);
      for (int64_t t = 0; t < T; ++t) scores[t / c] += exp(x[t] - m) / s;
    }
  }
  free(x);
  return ORC_OK;
}

typedef struct {
  double score;
  int64_t id;
} orc_ranked;

static int cmp_rank(const void *a, const void *b) {
  const orc_ranked *x = (const orc_ranked *)a, *y = (const orc_ranked *)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->id > y->id) - (x->id < y->id);
}

static int cmp_i32(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/*
 * Algorithm 1 step 4 (and Kara eq. (2)): TopK of the C chunk scores with
 * k = floor(L_max / c).  All C ids are sorted by (score descending, id
 * ascending) and the first min(k, C) are kept.  sel receives them in
 * ascending id order; the count is returned (negative on error).
 */
int64_t orc_topk(int64_t C, int64_t k, const double *scores, int32_t *sel) {
  if (C < 1 || k < 0) return -ORC_EINVAL;
  const int64_t n = k < C ? k : C;
  orc_ranked *r = (orc_ranked *)malloc((size_t)C * sizeof(orc_ranked));
  if (!r) return -ORC_ENOMEM;
  for (int64_t j = 0; j < C; ++j) {
    r[j].score = scores[j];
    r[j].id = j;
  }
  qsort(r, (size_t)C, sizeof(orc_ranked), cmp_rank);
  for (int64_t i = 0; i < n; ++i) sel[i] = (int32_t)r[i].id;
  free(r);
  qsort(sel, (size_t)n, sizeof(int32_t), cmp_i32);
  return n;
}

/*
 * Algorithm 1 steps 5-6: every token of a selected chunk is kept, and the
 * last w tokens are always kept.  idx receives the kept token positions in
 * ascending order without duplicates; their number n is returned.
 */
int64_t orc_indices(int64_t T, int w, int c, int64_t nsel, const int32_t *sel,
                    int32_t *idx) {
  if (T < 1 || w < 1 || w > T || c < 1 || nsel < 0) return -ORC_EINVAL;
  unsigned char *keep = (unsigned char *)calloc((size_t)T, 1);
  if (!keep) return -ORC_ENOMEM;
  for (int64_t s = 0; s < nsel; ++s) {
    const int64_t j = sel[s];
    for (int64_t t = j * c; t < j * c + c && t < T; ++t) keep[t] = 1;
  }
  for (int64_t t = T - w; t < T; ++t) keep[t] = 1;
  int64_t n = 0;
  for (int64_t t = 0; t < T; ++t)
    if (keep[t]) idx[n++] = (int32_t)t;
  free(keep);
  return n;
}

/*
 * Algorithm 1 step 6, index_select: row i of dst is a byte copy of token
 * idx[i] of head `head` in src (element (t, head, :) at
 * src[t*tok_stride + head*head_stride], strides in elements).
 */
void orc_gather(int64_t n, const int32_t *idx, int elem_bytes, int d,
                const void *src, int64_t tok_stride, int64_t head_stride,
                int head, void *dst) {
  const size_t row = (size_t)d * (size_t)elem_bytes;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t off = ((int64_t)idx[i] * tok_stride + (int64_t)head * head_stride) * elem_bytes;
    memcpy((char *)dst + (size_t)i * row, (const char *)src + off, row);
  }
}

/*
 * Algorithm 2 (layer-wise index reuse) for one sequence and all KV heads.
 *
 * A layer l with l mod n_reuse == 0 runs Algorithm 1 and stores its index
 * sets; any other layer reuses the sets of layer floor(l / n_reuse) * n_reuse
 * and only gathers -- from its OWN keys and values.
 *
 * Per layer l: q[l] (may be NULL for a reusing layer), k[l], v[l] laid out as
 * in orc_chunk_scores; k_out[l], v_out[l] receive [n_kv_heads][l_cap][d]
 * rows (rows >= lengths are not written).
 * scores  : NULL or [n_layers][n_kv_heads][C] doubles (only anchor layers are
 *           written).
 * indices : [n_layers][n_kv_heads][l_cap] int32, lengths: [n_layers][n_kv_heads].
 * l_cap must be >= min(T, k*c + w).
 */
int orc_compress_layers(int dtype, int64_t T, int64_t t_q, int n_q_heads,
                        int n_kv_heads, int d, int w, int c, int64_t l_max,
                        int n_layers, int n_reuse, const void *const *q,
                        int64_t q_tok_stride, int64_t q_head_stride,
                        const void *const *k, const void *const *v,
                        int64_t kv_tok_stride, int64_t kv_head_stride,
                        void *const *k_out, void *const *v_out, int64_t l_cap,
                        double *scores, int32_t *indices, int64_t *lengths) {
  if (n_layers < 1 || n_reuse < 1 || l_max < 0) return ORC_EINVAL;
  const int64_t C = orc_num_chunks(T, c);
  const int64_t kk = orc_num_keep_chunks(l_max, c);
  const int64_t need = (kk * c + w < T) ? kk * c + w : T;
  if (l_cap < need) return ORC_EINVAL;
  const int eb = dtype == ORC_F32 ? 4 : 2;
  double *sc = (double *)malloc((size_t)C * sizeof(double));
  int32_t *sel = (int32_t *)malloc((size_t)C * sizeof(int32_t));
  if (!sc || !sel) {
    free(sc);
    free(sel);
    return ORC_ENOMEM;
  }
  int rc = ORC_OK;
  for (int l = 0; l < n_layers && rc == ORC_OK; ++l) {
    const int anchor = (l / n_reuse) * n_reuse;
    for (int h = 0; h < n_kv_heads; ++h) {
      int32_t *idx = indices + ((int64_t)l * n_kv_heads + h) * l_cap;
      int64_t n;
      if (l % n_reuse == 0) {
        rc = orc_chunk_scores(dtype, T, t_q, n_q_heads, n_kv_heads, h, d, w, c,
                              q[l], q_tok_stride, q_head_stride, k[l],
                              kv_tok_stride, kv_head_stride, sc);
        if (rc != ORC_OK) break;
        if (scores)
          memcpy(scores + ((int64_t)l * n_kv_heads + h) * C, sc, (size_t)C * sizeof(double));
        const int64_t nsel = orc_topk(C, kk, sc, sel);
        n = orc_indices(T, w, c, nsel, sel, idx);
      } else {
        /* I_l <- I_reuse[floor(l / N_reuse) * N_reuse] */
        const int32_t *src = indices + ((int64_t)anchor * n_kv_heads + h) * l_cap;
        n = lengths[(int64_t)anchor * n_kv_heads + h];
        memcpy(idx, src, (size_t)n * sizeof(int32_t));
      }
      lengths[(int64_t)l * n_kv_heads + h] = n;
      orc_gather(n, idx, eb, d, k[l], kv_tok_stride, kv_head_stride, h,
                 (char *)k_out[l] + (size_t)h * (size_t)l_cap * d * eb);
      orc_gather(n, idx, eb, d, v[l], kv_tok_stride, kv_head_stride, h,
                 (char *)v_out[l] + (size_t)h * (size_t)l_cap * d * eb);
    }
  }
  free(sc);
  free(sel);
  return rc;
}

/*
 * Decode attention over one KV head's compacted cache: the step that consumes
 * the compressed cache (the ChunkKV page's latency / throughput section times
 * decoding over it).  Each of the G query heads of the KV head attends with
 * one new query over the n kept rows: weights softmax(q . k_i / sqrt(d))
 * (Kara eq. (1)), output sum_i weight_i * v_i.  Reading: the new token's own
 * key and value are not part of the cache here (an engine appends them); an
 * empty cache (n == 0) gives zeros.
 * q [G][d], k and v [n][d] (one head's kept rows in order), out [G][d].
 */
int orc_decode_attention(int dtype, int64_t n, int G, int d, const void *q,
                         const void *k, const void *v, double *out) {
  if (n < 0 || G < 1 || d < 1 || (dtype != ORC_F32 && dtype != ORC_BF16))
    return ORC_EINVAL;
  for (int64_t e = 0; e < (int64_t)G * d; ++e) out[e] = 0.0;
  if (n == 0) return ORC_OK;
  double *x = (double *)malloc((size_t)n * sizeof(double));
  if (!x) return ORC_ENOMEM;
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
  for (int g = 0; g < G; ++g) {
    for (int64_t i = 0; i < n; ++i) {
      double acc = 0.0;
      for (int j = 0; j < d; ++j)
        acc += widen(q, dtype, (int64_t)g * d + j) * widen(k, dtype, i * d + j);
      x[i] = acc * inv_sqrt_d;
    }
    double m = x[0];
    for (int64_t i = 1; i < n; ++i)
      if (x[i] > m) m = x[i];
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += exp(x[i] - m);
    for (int64_t i = 0; i < n; ++i) {
      const double p = exp(x[i] - m) / s;
      for (int j = 0; j < d; ++j) out[(int64_t)g * d + j] += p * widen(v, dtype, i * d + j);
    }
  }
  free(x);
  return ORC_OK;
}
