/*
 * A plain C caller of libchunkkv.so: the C-ABI of include/chunkkv.h used with
 * nothing but the HIP runtime's allocation and copy calls, no Python, no torch.
 * Test infrastructure: it also links the CPU oracle (oracle/chunkkv_oracle.c)
 * to check what the library computed.
 *
 *   c_consumer plan   host only: the planner's sizes against the formulas of
 *                     the ChunkKV page (section 4.1, Algorithm 1 steps 2, 4
 *                     and 5) and the validation errors; needs no GPU.
 *   c_consumer run    on the GPU: a two-layer fp32 problem with grouped-query
 *                     attention and index reuse 2 (section 4.2, Algorithm 2),
 *                     compressed by chunkkv_compress_layers and compared with
 *                     the oracle: chunk scores within 1e-5 relative, indices,
 *                     lengths and the gathered rows exactly.
 *
 * Exit status 0 when every check passes; each failure is printed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "chunkkv.h"

/* the oracle's entry point (oracle/chunkkv_oracle.c) */
int orc_compress_layers(int dtype, int64_t T, int64_t t_q, int n_q_heads, int n_kv_heads, int d, int w, int c,
                        int64_t l_max, int n_layers, int n_reuse, const void *const *q, int64_t q_tok_stride,
                        int64_t q_head_stride, const void *const *k, const void *const *v, int64_t kv_tok_stride,
                        int64_t kv_head_stride, void *const *k_out, void *const *v_out, int64_t l_cap,
                        double *scores, int32_t *indices, int64_t *lengths);

static int failures = 0;

#define CHECK(cond, ...)                          \
  do {                                            \
    if (!(cond)) {                                \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);               \
      fprintf(stderr, "\n");                      \
      ++failures;                                 \
    }                                             \
  } while (0)

#define HIP_OK(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "FAIL %s:%d: %s -> %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
      exit(1);                                                                    \
    }                                                                             \
  } while (0)

static chunkkv_problem problem(int dtype, int n_seqs, const int64_t *seq_start, const int64_t *l_max, int hq,
                               int hkv, int d, int w, int c) {
  chunkkv_problem p;
  memset(&p, 0, sizeof p);
  p.dtype = dtype;
  p.n_seqs = n_seqs;
  p.seq_start = seq_start;
  p.l_max = l_max;
  p.n_q_heads = hq;
  p.n_kv_heads = hkv;
  p.head_dim = d;
  p.window = w;
  p.chunk = c;
  p.kv_stride_tok = (int64_t)hkv * d; /* K/V [sum T][H_kv][d] */
  p.kv_stride_head = d;
  p.q_stride_seq = (int64_t)w * hq * d; /* window queries [B][w][H_q][d] */
  p.q_stride_row = (int64_t)hq * d;
  p.q_stride_head = d;
  return p;
}

static int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }

/* ---------------------------------------------------------------- plan -- */
static void plan_checks(void) {
  /* four packed sequences of a 70B-shaped batch: T_b, L_max,b = 20% of T_b */
  const int64_t T[4] = {131072, 65536, 32768, 16384};
  int64_t start[5] = {0, 0, 0, 0, 0}, lm[4];
  for (int b = 0; b < 4; ++b) {
    start[b + 1] = start[b] + T[b];
    lm[b] = T[b] / 5;
  }
  const int hq = 64, hkv = 8, d = 128, w = 64, c = 10;
  chunkkv_problem p = problem(CHUNKKV_BF16, 4, start, lm, hq, hkv, d, w, c);
  chunkkv_sizes sz;
  int64_t so[4], io[4], lc[4];
  CHECK(chunkkv_plan(&p, &sz, so, io, lc) == CHUNKKV_OK, "plan: %s", chunkkv_last_error());
  int64_t s_sum = 0, i_sum = 0;
  for (int b = 0; b < 4; ++b) {
    const int64_t C = (T[b] + c - 1) / c, kk = lm[b] / c;
    CHECK(lc[b] == imin(T[b], kk * c + w), "L_cap of sequence %d: %lld", b, (long long)lc[b]);
    CHECK(so[b] == s_sum && io[b] == i_sum, "offsets of sequence %d", b);
    s_sum += hkv * C;
    i_sum += hkv * lc[b];
  }
  CHECK(sz.scores_elems == s_sum, "scores_elems %lld vs %lld", (long long)sz.scores_elems, (long long)s_sum);
  CHECK(sz.index_elems == i_sum, "index_elems %lld vs %lld", (long long)sz.index_elems, (long long)i_sum);
  CHECK(sz.length_elems == 4 * hkv, "length_elems %lld", (long long)sz.length_elems);
  CHECK(sz.workspace_bytes > 0 && chunkkv_workspace_bytes(&p, 1) == sz.workspace_bytes,
        "workspace for one scoring layer");
  CHECK(chunkkv_workspace_bytes(&p, 8) >= sz.workspace_bytes, "workspace grows with the layers per launch");

  /* budget of at least C chunks keeps every token; budget 0 keeps the window */
  const int64_t s1[2] = {0, 1000};
  int64_t big[1] = {5000}, zero[1] = {0}, one_cap[1];
  chunkkv_problem q1 = problem(CHUNKKV_F32, 1, s1, big, 4, 2, 64, 8, 10);
  CHECK(chunkkv_plan(&q1, &sz, NULL, NULL, one_cap) == CHUNKKV_OK && one_cap[0] == 1000, "k >= C: L_cap = T");
  q1.l_max = zero;
  CHECK(chunkkv_plan(&q1, &sz, NULL, NULL, one_cap) == CHUNKKV_OK && one_cap[0] == 8, "k = 0: L_cap = w");

  /* validation: every failure is reported before anything runs, with a message */
  chunkkv_problem bad = problem(CHUNKKV_F32, 1, s1, big, 4, 2, 64, 1001, 10);
  CHECK(chunkkv_plan(&bad, &sz, NULL, NULL, NULL) == CHUNKKV_ERR_INVALID_ARG, "window longer than T");
  CHECK(strlen(chunkkv_last_error()) > 0, "an error message");
  bad = problem(CHUNKKV_F32, 1, s1, big, 3, 2, 64, 8, 10);
  CHECK(chunkkv_plan(&bad, &sz, NULL, NULL, NULL) == CHUNKKV_ERR_INVALID_ARG, "H_q not a multiple of H_kv");
  bad = problem(CHUNKKV_BF16, 1, s1, big, 4, 2, 100, 8, 10);
  CHECK(chunkkv_plan(&bad, &sz, NULL, NULL, NULL) == CHUNKKV_ERR_UNSUPPORTED, "rows not a multiple of 16 bytes");
  bad = problem(CHUNKKV_F32, 1, s1, big, 4, 2, 64, 8, 0);
  CHECK(chunkkv_plan(&bad, &sz, NULL, NULL, NULL) == CHUNKKV_ERR_INVALID_ARG, "chunk 0");
  CHECK(chunkkv_plan(NULL, &sz, NULL, NULL, NULL) == CHUNKKV_ERR_INVALID_ARG, "NULL problem");
  CHECK(chunkkv_plan(&q1, NULL, NULL, NULL, NULL) == CHUNKKV_ERR_INVALID_ARG, "NULL sizes");
  /* a call with no workspace is refused on the host (nothing is launched) */
  const void *qs[1] = {NULL}, *ks[1] = {NULL}, *vs[1] = {NULL};
  void *kos[1] = {NULL}, *vos[1] = {NULL};
  CHECK(chunkkv_compress_layers(&q1, 1, 1, qs, ks, vs, kos, vos, NULL, NULL, NULL, NULL, 0, NULL, NULL) !=
            CHUNKKV_OK,
        "compress with NULL buffers");
}

/* ----------------------------------------------------------------- run -- */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static float next_normalish(void) {
  /* xorshift64*; sum of four uniforms, centred: a cheap bell-shaped value */
  float s = 0.0f;
  for (int i = 0; i < 4; ++i) {
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    s += (float)((rng_state * 0x2545F4914F6CDD1Dull) >> 40) / (float)(1 << 24);
  }
  return (s - 2.0f) * 1.7f;
}

static void run_checks(void) {
  enum { T = 1000, HQ = 4, HKV = 2, D = 64, W = 8, CH = 10, LAYERS = 2, REUSE = 2 };
  const int64_t start[2] = {0, T}, lm[1] = {100};
  chunkkv_problem p = problem(CHUNKKV_F32, 1, start, lm, HQ, HKV, D, W, CH);
  chunkkv_sizes sz;
  int64_t l_cap = 0;
  if (chunkkv_plan(&p, &sz, NULL, NULL, &l_cap) != CHUNKKV_OK) {
    fprintf(stderr, "FAIL plan: %s\n", chunkkv_last_error());
    exit(1);
  }
  const int64_t C = (T + CH - 1) / CH;
  const size_t kv_n = (size_t)T * HKV * D, q_n = (size_t)W * HQ * D, out_n = (size_t)sz.index_elems * D;

  /* host inputs; a planted chunk (id 37) whose keys lean towards the window queries */
  float *hq[LAYERS], *hk[LAYERS], *hv[LAYERS];
  for (int l = 0; l < LAYERS; ++l) {
    hq[l] = (float *)malloc(q_n * sizeof(float));
    hk[l] = (float *)malloc(kv_n * sizeof(float));
    hv[l] = (float *)malloc(kv_n * sizeof(float));
    for (size_t i = 0; i < q_n; ++i) hq[l][i] = next_normalish();
    for (size_t i = 0; i < kv_n; ++i) hk[l][i] = next_normalish();
    for (size_t i = 0; i < kv_n; ++i) hv[l][i] = next_normalish();
    for (int t = 370; t < 380; ++t)
      for (int h = 0; h < HKV; ++h)
        for (int i = 0; i < D; ++i) hk[l][((size_t)t * HKV + h) * D + i] += 0.5f * hq[l][(size_t)(h * (HQ / HKV)) * D + i];
  }

  /* device buffers: inputs, outputs, workspace */
  void *dq[LAYERS], *dk[LAYERS], *dv[LAYERS], *dko[LAYERS], *dvo[LAYERS];
  for (int l = 0; l < LAYERS; ++l) {
    HIP_OK(hipMalloc(&dq[l], q_n * sizeof(float)));
    HIP_OK(hipMalloc(&dk[l], kv_n * sizeof(float)));
    HIP_OK(hipMalloc(&dv[l], kv_n * sizeof(float)));
    HIP_OK(hipMalloc(&dko[l], out_n * sizeof(float)));
    HIP_OK(hipMalloc(&dvo[l], out_n * sizeof(float)));
    HIP_OK(hipMemcpy(dq[l], hq[l], q_n * sizeof(float), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dk[l], hk[l], kv_n * sizeof(float), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dv[l], hv[l], kv_n * sizeof(float), hipMemcpyHostToDevice));
  }
  const int n_anchor = (LAYERS + REUSE - 1) / REUSE;
  const size_t ws = chunkkv_workspace_bytes(&p, n_anchor);
  float *d_scores;
  int32_t *d_idx, *d_len;
  void *d_ws;
  HIP_OK(hipMalloc((void **)&d_scores, (size_t)n_anchor * sz.scores_elems * sizeof(float)));
  HIP_OK(hipMalloc((void **)&d_idx, (size_t)n_anchor * sz.index_elems * sizeof(int32_t)));
  HIP_OK(hipMalloc((void **)&d_len, (size_t)n_anchor * sz.length_elems * sizeof(int32_t)));
  HIP_OK(hipMalloc(&d_ws, ws));

  const void *qs[LAYERS] = {dq[0], NULL}; /* the reusing layer needs no queries */
  const void *ks[LAYERS] = {dk[0], dk[1]}, *vs[LAYERS] = {dv[0], dv[1]};
  void *kos[LAYERS] = {dko[0], dko[1]}, *vos[LAYERS] = {dvo[0], dvo[1]};
  const int st = chunkkv_compress_layers(&p, LAYERS, REUSE, qs, ks, vs, kos, vos, d_scores, d_idx, d_len, d_ws, ws,
                                         NULL, NULL);
  if (st != CHUNKKV_OK) {
    fprintf(stderr, "FAIL compress_layers: status %d: %s\n", st, chunkkv_last_error());
    exit(1);
  }
  HIP_OK(hipDeviceSynchronize());

  float *g_scores = (float *)malloc((size_t)sz.scores_elems * sizeof(float));
  int32_t *g_idx = (int32_t *)malloc((size_t)sz.index_elems * sizeof(int32_t));
  int32_t g_len[HKV];
  HIP_OK(hipMemcpy(g_scores, d_scores, (size_t)sz.scores_elems * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(g_idx, d_idx, (size_t)sz.index_elems * sizeof(int32_t), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(g_len, d_len, sizeof g_len, hipMemcpyDeviceToHost));

  /* the oracle over the same host inputs */
  double *o_scores = (double *)calloc((size_t)LAYERS * HKV * C, sizeof(double));
  int32_t *o_idx = (int32_t *)calloc((size_t)LAYERS * HKV * l_cap, sizeof(int32_t));
  int64_t o_len[LAYERS * HKV];
  float *o_k[LAYERS], *o_v[LAYERS];
  for (int l = 0; l < LAYERS; ++l) {
    o_k[l] = (float *)calloc(out_n, sizeof(float));
    o_v[l] = (float *)calloc(out_n, sizeof(float));
  }
  const void *oq[LAYERS] = {hq[0], NULL}, *ok_[LAYERS] = {hk[0], hk[1]}, *ov[LAYERS] = {hv[0], hv[1]};
  void *oko[LAYERS] = {o_k[0], o_k[1]}, *ovo[LAYERS] = {o_v[0], o_v[1]};
  /* window row r is position T - W + r; the oracle reads row t_q - W + r of q, so t_q = W */
  CHECK(orc_compress_layers(0, T, W, HQ, HKV, D, W, CH, lm[0], LAYERS, REUSE, oq, (int64_t)HQ * D, D, ok_, ov,
                            (int64_t)HKV * D, D, oko, ovo, l_cap, o_scores, o_idx, o_len) == 0,
        "oracle failed");

  for (int h = 0; h < HKV; ++h) {
    int bad = 0;
    for (int64_t j = 0; j < C; ++j) {
      const double ref = o_scores[(int64_t)h * C + j], got = g_scores[(int64_t)h * C + j];
      if (fabs(got - ref) > 1e-5 * fabs(ref) + 1e-30) ++bad;
    }
    CHECK(bad == 0, "head %d: %d chunk scores outside 1e-5 relative", h, bad);
    CHECK(g_len[h] == o_len[h], "head %d: length %d vs %lld", h, g_len[h], (long long)o_len[h]);
    CHECK(memcmp(g_idx + (int64_t)h * l_cap, o_idx + (int64_t)h * l_cap, (size_t)o_len[h] * sizeof(int32_t)) == 0,
          "head %d: indices differ", h);
    /* the planted chunk's tokens are kept */
    int planted = 0;
    for (int64_t i = 0; i < o_len[h]; ++i) planted += g_idx[(int64_t)h * l_cap + i] == 375;
    CHECK(planted == 1, "head %d: planted chunk not kept", h);
  }
  float *g_rows = (float *)malloc(out_n * sizeof(float));
  for (int l = 0; l < LAYERS; ++l) {
    for (int which = 0; which < 2; ++which) {
      HIP_OK(hipMemcpy(g_rows, which ? dvo[l] : dko[l], out_n * sizeof(float), hipMemcpyDeviceToHost));
      const float *ref = which ? o_v[l] : o_k[l];
      for (int h = 0; h < HKV; ++h) {
        const size_t off = (size_t)h * l_cap * D, n = (size_t)o_len[h] * D;
        CHECK(memcmp(g_rows + off, ref + off, n * sizeof(float)) == 0, "layer %d head %d: gathered %s rows differ",
              l, h, which ? "V" : "K");
      }
    }
  }

  for (int l = 0; l < LAYERS; ++l) {
    HIP_OK(hipFree(dq[l]));
    HIP_OK(hipFree(dk[l]));
    HIP_OK(hipFree(dv[l]));
    HIP_OK(hipFree(dko[l]));
    HIP_OK(hipFree(dvo[l]));
    free(hq[l]);
    free(hk[l]);
    free(hv[l]);
    free(o_k[l]);
    free(o_v[l]);
  }
  HIP_OK(hipFree(d_scores));
  HIP_OK(hipFree(d_idx));
  HIP_OK(hipFree(d_len));
  HIP_OK(hipFree(d_ws));
  free(g_scores);
  free(g_idx);
  free(g_rows);
  free(o_scores);
  free(o_idx);
}

int main(int argc, char **argv) {
  if (argc != 2 || (strcmp(argv[1], "plan") != 0 && strcmp(argv[1], "run") != 0)) {
    fprintf(stderr, "usage: %s plan|run\n", argv[0]);
    return 2;
  }
  if (strcmp(argv[1], "plan") == 0)
    plan_checks();
  else
    run_checks();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("c_consumer %s: all checks passed\n", argv[1]);
  return 0;
}
