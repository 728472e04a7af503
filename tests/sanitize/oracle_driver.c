/*
 * Runs every function of the oracle (oracle/ngram_oracle.c) once per edge
 * case on exactly-sized heap buffers, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer: an access outside a buffer or an undefined
 * operation aborts with the sanitizer's report.  The values are not checked
 * here (the oracle's pins do that); a few invariants that hold for any input
 * are, so that a silently wrong path still fails.  Test code only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t orc_compress(const int32_t* raw, int64_t n, const int32_t* lut, int32_t vocab,
                     int32_t vocab_c, int32_t pad_id, int32_t* comp);
void orc_hash(const int32_t* comp, int32_t B, int32_t T, const int32_t* hist, int32_t hist_len,
              int32_t pad_id, int32_t n_orders, const int32_t* orders, int32_t heads,
              const int64_t* rows, const uint64_t* mult, int32_t* row_idx);
double orc_fp8_e4m3_value(uint32_t byte);
void orc_gather(const int32_t* row_idx, int64_t n_tok, int32_t n_tables, const void* const* tables,
                int32_t dtype, int32_t row_dim, const float* scales, double* e);
void orc_project(const double* e, int64_t n_tok, int32_t mem, const void* w, int32_t dtype,
                 int32_t d, double* out);
void orc_gate(const void* hidden, int32_t dtype, int64_t tok_stride, int64_t branch_stride,
              const double* k, int64_t n_tok, int32_t nb, int32_t d, const void* gamma_q,
              const void* gamma_k, double eps, double* gate);
void orc_gated_value(const double* gate, const double* v, int64_t n_tok, int32_t nb, int32_t d,
                     double* u);
void orc_conv_block(const double* u, int32_t B, int32_t T, int32_t nb, int32_t d, const void* w,
                    int32_t w_dtype, int32_t kernel, int32_t dil, const void* gamma_u, double eps,
                    const double* state, double* delta);
void orc_normalise_rows(const double* u, int64_t rows, int32_t d, const void* gamma, int32_t dtype,
                        double eps, double* out);
void orc_conv_block_backward(const double* u, int32_t B, int32_t T, int32_t nb, int32_t d,
                             const void* w, int32_t w_dtype, int32_t kernel, int32_t dil,
                             const void* gamma_u, double eps, const double* state,
                             const double* d_delta, double* d_u, double* d_w, double* d_gamma_u);
void orc_gated_value_backward(const double* gate, const double* v, const double* d_u,
                              int64_t n_tok, int32_t nb, int32_t d, double* d_gate, double* d_v);
void orc_gate_backward(const void* hidden, int32_t dtype, int64_t tok_stride,
                       int64_t branch_stride, const double* k, int64_t n_tok, int32_t nb,
                       int32_t d, const void* gamma_q, const void* gamma_k, double eps,
                       const double* d_gate, double* d_k, double* d_hidden, double* d_gamma_q,
                       double* d_gamma_k);
void orc_project_backward(const double* e, int64_t n_tok, int32_t mem, const void* w,
                          int32_t dtype, int32_t d, const double* d_out, double* d_e,
                          double* d_w);
void orc_scatter_add(const int32_t* row_idx, int64_t n_tok, int32_t n_tables, const double* d_e,
                     int32_t row_dim, double* const* d_tables);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return rng_state;
}
static double next_unit(void) { return (double)(next_u64() >> 11) * 0x1p-53 * 2.0 - 1.0; }

static void* xmalloc(size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}
static double* dvec(int64_t n, double scale) {
  double* p = (double*)xmalloc(sizeof(double) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) p[i] = scale * next_unit();
  return p;
}
static float* fvec(int64_t n, double scale) {
  float* p = (float*)xmalloc(sizeof(float) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) p[i] = (float)(scale * next_unit());
  return p;
}
static uint16_t* bvec(int64_t n, double scale) { /* bf16 bits, truncated fp32 */
  uint16_t* p = (uint16_t*)xmalloc(sizeof(uint16_t) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) {
    float f = (float)(scale * next_unit());
    uint32_t b;
    memcpy(&b, &f, 4);
    p[i] = (uint16_t)(b >> 16);
  }
  return p;
}

static int failures = 0;
#define CHECK(cond, what)                             \
  do {                                                \
    if (!(cond)) {                                    \
      fprintf(stderr, "invariant failed: %s\n", what); \
      ++failures;                                     \
    }                                                 \
  } while (0)

/* one forward + backward chain at the given shape */
static void chain(int32_t B, int32_t T, int32_t nb, int32_t nbh, int32_t d, int32_t row_dim,
                  int32_t n_orders, const int32_t* orders, int32_t heads, int32_t dtype,
                  int with_hist, int with_state, int with_gamma) {
  const int32_t vocab = 97, vocab_c = 75, pad = 0;
  const int32_t n_tables = n_orders * heads, max_order = orders[n_orders - 1];
  const int32_t mem = n_tables * row_dim, dil = max_order, kernel = 4;
  const int64_t n = (int64_t)B * T;
  /* ids: a few out of range on purpose */
  int32_t* raw = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) raw[i] = (int32_t)(next_u64() % (vocab + 4)) - 2;
  int32_t* lut = (int32_t*)xmalloc(sizeof(int32_t) * vocab);
  for (int32_t i = 0; i < vocab; ++i) lut[i] = i == 0 ? 0 : 1 + (i % (vocab_c - 1));
  int32_t* comp = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)n);
  const int64_t bad = orc_compress(raw, n, lut, vocab, vocab_c, pad, comp);
  CHECK(bad >= 0 && bad <= n, "compress count");
  for (int64_t i = 0; i < n; ++i) CHECK(comp[i] >= 0 && comp[i] < vocab_c, "compressed range");
  const int32_t hist_len = max_order - 1;
  int32_t* hist = NULL;
  if (with_hist && hist_len > 0) {
    hist = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)(B * hist_len));
    for (int32_t i = 0; i < B * hist_len; ++i) hist[i] = (int32_t)(next_u64() % vocab_c);
  }
  int64_t rows[16];
  uint64_t mult[16 * 4];
  for (int32_t j = 0; j < n_tables; ++j) rows[j] = 101 + 2 * j; /* any sizes: ranges only */
  for (int32_t i = 0; i < 16 * 4; ++i) mult[i] = next_u64() | 1u;
  int32_t* ridx = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)(n * n_tables));
  orc_hash(comp, B, T, hist, hist ? hist_len : 0, pad, n_orders, orders, heads, rows, mult, ridx);
  for (int64_t i = 0; i < n * n_tables; ++i)
    CHECK(ridx[i] >= 0 && ridx[i] < rows[i % n_tables], "row id range");
  /* tables in the storage dtype */
  void* tabs[16];
  float scales[16];
  for (int32_t j = 0; j < n_tables; ++j) {
    const int64_t cnt = rows[j] * row_dim;
    if (dtype == 0) {
      tabs[j] = fvec(cnt, 0.02);
    } else if (dtype == 1) {
      tabs[j] = bvec(cnt, 0.02);
    } else {
      uint8_t* q = (uint8_t*)xmalloc((size_t)cnt);
      for (int64_t i = 0; i < cnt; ++i) {  /* any E4M3 code but the NaNs */
        q[i] = (uint8_t)next_u64();
        if ((q[i] & 0x7F) == 0x7F) q[i] ^= 1;
      }
      tabs[j] = q;
    }
    scales[j] = 0.25f;
  }
  double* e = (double*)xmalloc(sizeof(double) * (size_t)(n * mem));
  orc_gather(ridx, n, n_tables, (const void* const*)tabs, dtype, row_dim,
             dtype == 2 ? scales : NULL, e);
  const int32_t adt = dtype == 2 ? 1 : dtype; /* activations */
  void* wk = adt == 0 ? (void*)fvec((int64_t)nb * mem * d, 0.1) : (void*)bvec((int64_t)nb * mem * d, 0.1);
  void* wv = adt == 0 ? (void*)fvec((int64_t)mem * d, 0.1) : (void*)bvec((int64_t)mem * d, 0.1);
  double* k = (double*)xmalloc(sizeof(double) * (size_t)(n * nb * d));
  double* kb = (double*)xmalloc(sizeof(double) * (size_t)(n * d));
  for (int32_t b = 0; b < nb; ++b) {
    const size_t off = (size_t)b * mem * d * (adt == 0 ? 4 : 2);
    orc_project(e, n, mem, (const char*)wk + off, adt, d, kb);
    for (int64_t t = 0; t < n; ++t) memcpy(k + (t * nb + b) * d, kb + t * d, sizeof(double) * d);
  }
  double* v = (double*)xmalloc(sizeof(double) * (size_t)(n * d));
  orc_project(e, n, mem, wv, adt, d, v);
  void* hidden = adt == 0 ? (void*)fvec(n * nbh * d, 1.0) : (void*)bvec(n * nbh * d, 1.0);
  void* gq = NULL;
  void* gk = NULL;
  void* gu = NULL;
  if (with_gamma) {
    gq = adt == 0 ? (void*)fvec(d, 1.0) : (void*)bvec(d, 1.0);
    gk = adt == 0 ? (void*)fvec(d, 1.0) : (void*)bvec(d, 1.0);
    gu = adt == 0 ? (void*)fvec(d, 1.0) : (void*)bvec(d, 1.0);
  }
  double* gate = (double*)xmalloc(sizeof(double) * (size_t)(n * nb));
  orc_gate(hidden, adt, (int64_t)nbh * d, nbh == 1 ? 0 : d, k, n, nb, d, gq, gk, 1e-6, gate);
  for (int64_t i = 0; i < n * nb; ++i) CHECK(gate[i] > 0.0 && gate[i] < 1.0, "gate range");
  double* u = (double*)xmalloc(sizeof(double) * (size_t)(n * nb * d));
  orc_gated_value(gate, v, n, nb, d, u);
  const int32_t span = (kernel - 1) * dil;
  double* state = with_state ? dvec((int64_t)B * span * nb * d, 1.0) : NULL;
  void* cw = adt == 0 ? (void*)fvec(kernel * d, 0.5) : (void*)bvec(kernel * d, 0.5);
  double* delta = (double*)xmalloc(sizeof(double) * (size_t)(n * nb * d));
  orc_conv_block(u, B, T, nb, d, cw, adt, kernel, dil, gu, 1e-6, state, delta);
  double* nrm = (double*)xmalloc(sizeof(double) * (size_t)(n * nb * d));
  orc_normalise_rows(u, n * nb, d, gu, adt, 1e-6, nrm);
  for (int64_t i = 0; i < n * nb * d; ++i) CHECK(isfinite(delta[i]) && isfinite(nrm[i]), "finite");
  /* backward */
  double* dd = dvec(n * nb * d, 1.0);
  double* du = (double*)xmalloc(sizeof(double) * (size_t)(n * nb * d));
  double* dw = (double*)calloc((size_t)(kernel * d), sizeof(double));
  double* dgu = (double*)calloc((size_t)d, sizeof(double));
  orc_conv_block_backward(u, B, T, nb, d, cw, adt, kernel, dil, gu, 1e-6, state, dd, du, dw, dgu);
  double* dgate = (double*)xmalloc(sizeof(double) * (size_t)(n * nb));
  double* dv = (double*)xmalloc(sizeof(double) * (size_t)(n * d));
  orc_gated_value_backward(gate, v, du, n, nb, d, dgate, dv);
  double* dk = (double*)xmalloc(sizeof(double) * (size_t)(n * nb * d));
  double* dh = (double*)calloc((size_t)(n * nbh * d), sizeof(double));
  double* dgq = (double*)calloc((size_t)d, sizeof(double));
  double* dgk = (double*)calloc((size_t)d, sizeof(double));
  orc_gate_backward(hidden, adt, (int64_t)nbh * d, nbh == 1 ? 0 : d, k, n, nb, d, gq, gk, 1e-6,
                    dgate, dk, dh, dgq, dgk);
  double* de = (double*)calloc((size_t)(n * mem), sizeof(double));
  double* dwv = (double*)calloc((size_t)(mem * d), sizeof(double));
  orc_project_backward(e, n, mem, wv, adt, d, dv, de, dwv);
  double* dtab[16];
  for (int32_t j = 0; j < n_tables; ++j) dtab[j] = (double*)calloc((size_t)(rows[j] * row_dim), sizeof(double));
  orc_scatter_add(ridx, n, n_tables, de, row_dim, dtab);
  for (int32_t j = 0; j < n_tables; ++j) {
    free(dtab[j]);
    free(tabs[j]);
  }
  free(raw); free(lut); free(comp); free(hist); free(ridx); free(e); free(wk); free(wv); free(k);
  free(kb); free(v); free(hidden); free(gq); free(gk); free(gu); free(gate); free(u); free(state);
  free(cw); free(delta); free(nrm); free(dd); free(du); free(dw); free(dgu); free(dgate); free(dv);
  free(dk); free(dh); free(dgq); free(dgk); free(de); free(dwv);
}

int main(void) {
  for (uint32_t b = 0; b < 256; ++b) {
    const double x = orc_fp8_e4m3_value(b);
    CHECK(((b & 0x7F) == 0x7F) ? isnan(x) : (isfinite(x) && fabs(x) <= 448.0), "fp8 decode");
  }
  const int32_t o23[2] = {2, 3}, o234[3] = {2, 3, 4}, o1[1] = {1}, o12[2] = {1, 2};
  /*     B  T  nb nbh  d  row  orders    heads dtype hist state gamma */
  chain(1, 1, 1, 1, 8, 4, 2, o23, 2, 0, 1, 1, 1);     /* one token, history, state */
  chain(3, 17, 1, 1, 8, 4, 2, o23, 2, 0, 0, 0, 0);    /* ragged, nothing optional */
  chain(2, 13, 2, 2, 16, 8, 2, o23, 1, 1, 1, 1, 1);   /* bf16, per-branch queries */
  chain(2, 9, 3, 1, 16, 16, 2, o23, 2, 2, 0, 1, 1);   /* fp8 tables, shared query */
  chain(2, 20, 1, 1, 8, 4, 3, o234, 1, 0, 1, 1, 0);   /* dilation 4 */
  chain(1, 7, 1, 1, 8, 4, 1, o1, 3, 1, 0, 1, 1);      /* order 1: dilation 1 */
  chain(2, 5, 2, 2, 8, 4, 2, o12, 2, 0, 1, 0, 1);     /* orders {1, 2} */
  if (failures) {
    fprintf(stderr, "%d invariant failures\n", failures);
    return 1;
  }
  printf("oracle driver: all paths ran clean\n");
  return 0;
}
