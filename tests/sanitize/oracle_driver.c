/*
 * The oracle under the address and undefined-behaviour sanitizers: every entry
 * point on small ragged shapes, each buffer allocated at exactly the size the
 * call needs, so that any read or write past it is reported.  The entry points
 * are also checked against each other where they must agree (split partials
 * merged = whole rows, the unbounded window = plain attention, the (-1, 0)
 * window = causal, bf16 row sampling = the fp64 path on the same values).
 * Exit status: the number of failed checks.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attention_f64(const double* Q, const double* K, const double* V, double* O, double* LSE, int B, int H,
                         int n_q, int n_k, int d, int causal, double scale);
int oracle_attention_rows_bf16(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const int64_t* rows,
                               int64_t n_rows, double* O_rows, double* LSE_rows, int B, int H, int n_q, int n_k,
                               int d, int causal, double scale);
int oracle_partial_f64(const double* Q, const double* K, const double* V, double* acc, double* m, double* l, int B,
                       int H, int n_q, int n_k, int d, int causal, double scale, int key_begin, int key_end);
int oracle_merge_f64(const double* acc, const double* m, const double* l, double* O, double* LSE, int n_parts,
                     int64_t n_rows, int d);
int oracle_probs_f64(const double* Q, const double* K, double* P, int B, int H, int n_q, int n_k, int d, int causal,
                     double scale);
int oracle_attention_window_f64(const double* Q, const double* K, const double* V, double* O, double* LSE, int B,
                                int H, int n_q, int n_k, int d, int wl, int wr, double scale);
int oracle_attention_window_rows_bf16(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const int64_t* rows,
                                      int64_t n_rows, double* O_rows, double* LSE_rows, int B, int H, int n_q,
                                      int n_k, int d, int wl, int wr, double scale);
int64_t oracle_window_pairs(int n_q, int n_k, int wl, int wr);
int oracle_attention_blockmask_f64(const double* Q, const double* K, const double* V, double* O, double* LSE,
                                   int B, int H, int n_q, int n_k, int d, const uint8_t* M, int Mb, int Mh, int bq,
                                   int bk, int wl, int wr, double scale);
int oracle_attention_blockmask_rows_bf16(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                         const int64_t* rows, int64_t n_rows, double* O_rows, double* LSE_rows,
                                         int B, int H, int n_q, int n_k, int d, const uint8_t* M, int Mb, int Mh,
                                         int bq, int bk, int wl, int wr, double scale);
int64_t oracle_blockmask_pairs(int n_q, int n_k, const uint8_t* M, int Mb, int Mh, int b, int h, int bq, int bk,
                               int wl, int wr);
int oracle_backward_f64(const double* Q, const double* K, const double* V, const double* dO, double* dQ, double* dK,
                        double* dV, int B, int H, int n_q, int n_k, int d, int causal, double scale);
void oracle_bf16_to_f64(const uint16_t* src, double* dst, int64_t n);
uint8_t oracle_e4m3_encode(float y);
double oracle_e4m3_decode(uint8_t c);
int oracle_quantize_fp8(const uint16_t* X, uint8_t* codes, float* descale, int B, int H, int n, int d);
int oracle_attention_fp8_rows(const uint8_t* Qc, const uint8_t* Kc, const uint8_t* Vc, const float* descale_q,
                              const float* descale_k, const float* descale_v, const int64_t* rows, int64_t n_rows,
                              double* O_rows, double* LSE_rows, int B, int H, int n_q, int n_k, int d, int causal,
                              double scale);

static int failures = 0;
#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                                \
    }                                                                            \
  } while (0)

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double uniform(void) {  /* xorshift64*, in (-2, 2) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return ((double)((rng * 0x2545f4914f6cdd1dull) >> 11) / 9007199254740992.0) * 4.0 - 2.0;
}
/* bf16 bit pattern of a double, truncated (any pattern is a valid input) */
static uint16_t to_bf16(double x) {
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
static void* alloc(size_t bytes) { return malloc(bytes ? bytes : 1); }
static double maxdiff(const double* a, const double* b, int64_t n) {
  double m = 0.0;
  for (int64_t i = 0; i < n; ++i) m = fmax(m, fabs(a[i] - b[i]));
  return m;
}

static void run_shape(int B, int H, int nq, int nk, int d) {
  const int64_t nQ = (int64_t)B * H * nq * d, nK = (int64_t)B * H * nk * d, R = (int64_t)B * H * nq;
  const double scale = 1.0 / sqrt((double)d);
  uint16_t *Qb = alloc(nQ * 2), *Kb = alloc(nK * 2), *Vb = alloc(nK * 2);
  double *Q = alloc(nQ * 8), *K = alloc(nK * 8), *V = alloc(nK * 8), *dO = alloc(nQ * 8);
  for (int64_t i = 0; i < nQ; ++i) Qb[i] = to_bf16(uniform());
  for (int64_t i = 0; i < nK; ++i) Kb[i] = to_bf16(uniform()), Vb[i] = to_bf16(uniform());
  for (int64_t i = 0; i < nQ; ++i) dO[i] = uniform();
  oracle_bf16_to_f64(Qb, Q, nQ);
  oracle_bf16_to_f64(Kb, K, nK);
  oracle_bf16_to_f64(Vb, V, nK);
  double *O = alloc(nQ * 8), *L = alloc(R * 8), *O2 = alloc(nQ * 8), *L2 = alloc(R * 8);
  for (int causal = 0; causal < 2; ++causal) {
    CHECK(oracle_attention_f64(Q, K, V, O, L, B, H, nq, nk, d, causal, scale) == 0);
    /* windows that reduce to plain and causal attention */
    CHECK(oracle_attention_window_f64(Q, K, V, O2, L2, B, H, nq, nk, d, -1, causal ? 0 : -1, scale) == 0);
    CHECK(maxdiff(O, O2, nQ) < 1e-12 && maxdiff(L, L2, R) < 1e-12);
    /* every row through the bf16 sampling entry point, in reverse order */
    int64_t* rows = alloc(R * 8);
    for (int64_t r = 0; r < R; ++r) rows[r] = R - 1 - r;
    double *Or = alloc(nQ * 8), *Lr = alloc(R * 8);
    CHECK(oracle_attention_rows_bf16(Qb, Kb, Vb, rows, R, Or, Lr, B, H, nq, nk, d, causal, scale) == 0);
    double err = 0.0;
    for (int64_t r = 0; r < R; ++r) {
      err = fmax(err, fabs(Lr[r] - L[rows[r]]));
      for (int c = 0; c < d; ++c) err = fmax(err, fabs(Or[r * d + c] - O[rows[r] * d + c]));
    }
    CHECK(err < 1e-12);
    /* three key chunks (the last one may be empty), merged */
    const int S = 3, len = (nk + S - 1) / S;
    double *acc = alloc((size_t)S * nQ * 8), *m = alloc((size_t)S * R * 8), *l = alloc((size_t)S * R * 8);
    for (int c = 0; c < S; ++c) {
      const int j0 = c * len < nk ? c * len : nk, j1 = (c + 1) * len < nk ? (c + 1) * len : nk;
      CHECK(oracle_partial_f64(Q, K, V, acc + c * nQ, m + c * R, l + c * R, B, H, nq, nk, d, causal, scale, j0,
                               j1) == 0);
    }
    CHECK(oracle_merge_f64(acc, m, l, O2, L2, S, R, d) == 0);
    CHECK(maxdiff(O, O2, nQ) < 1e-12 && maxdiff(L, L2, R) < 1e-12);
    /* probabilities: rows sum to one */
    double* P = alloc((size_t)R * nk * 8);
    CHECK(oracle_probs_f64(Q, K, P, B, H, nq, nk, d, causal, scale) == 0);
    for (int64_t r = 0; r < R; ++r) {
      double s = 0.0;
      for (int j = 0; j < nk; ++j) s += P[r * nk + j];
      CHECK(fabs(s - 1.0) < 1e-12);
    }
    /* backward */
    double *dQ = alloc(nQ * 8), *dK = alloc(nK * 8), *dV = alloc(nK * 8);
    CHECK(oracle_backward_f64(Q, K, V, dO, dQ, dK, dV, B, H, nq, nk, d, causal, scale) == 0);
    for (int64_t i = 0; i < nQ; ++i) CHECK(isfinite(dQ[i]));
    for (int64_t i = 0; i < nK; ++i) CHECK(isfinite(dK[i]) && isfinite(dV[i]));
    /* FP8: quantise Q, K, V and attend every row */
    uint8_t *Qc = alloc(nQ), *Kc = alloc(nK), *Vc = alloc(nK);
    float *sq = alloc((size_t)B * H * 4), *sk = alloc((size_t)B * H * 4), *sv = alloc((size_t)B * H * 4);
    CHECK(oracle_quantize_fp8(Qb, Qc, sq, B, H, nq, d) == 0);
    CHECK(oracle_quantize_fp8(Kb, Kc, sk, B, H, nk, d) == 0);
    CHECK(oracle_quantize_fp8(Vb, Vc, sv, B, H, nk, d) == 0);
    CHECK(oracle_attention_fp8_rows(Qc, Kc, Vc, sq, sk, sv, rows, R, Or, Lr, B, H, nq, nk, d, causal, scale) == 0);
    for (int64_t r = 0; r < R; ++r) CHECK(isfinite(Lr[r]));
    free(Qc), free(Kc), free(Vc), free(sq), free(sk), free(sv);
    free(dQ), free(dK), free(dV), free(P), free(acc), free(m), free(l), free(rows), free(Or), free(Lr);
  }
  /* windows with empty rows and both edges, sampled and whole */
  const int win[][2] = {{0, 0}, {2, 1}, {0, -1}, {-1, 3}, {5, 0}, {1 << 30, 1 << 30}};
  for (size_t w = 0; w < sizeof win / sizeof win[0]; ++w) {
    const int wl = win[w][0], wr = win[w][1];
    CHECK(oracle_attention_window_f64(Q, K, V, O, L, B, H, nq, nk, d, wl, wr, scale) == 0);
    int64_t* rows = alloc(R * 8);
    for (int64_t r = 0; r < R; ++r) rows[r] = r;
    double *Or = alloc(nQ * 8), *Lr = alloc(R * 8);
    CHECK(oracle_attention_window_rows_bf16(Qb, Kb, Vb, rows, R, Or, Lr, B, H, nq, nk, d, wl, wr, scale) == 0);
    CHECK(maxdiff(O, Or, nQ) < 1e-12);
    for (int64_t r = 0; r < R; ++r) CHECK((isinf(L[r]) && isinf(Lr[r])) || fabs(L[r] - Lr[r]) < 1e-12);
    CHECK(oracle_window_pairs(nq, nk, wl, wr) >= 0);
    free(rows), free(Or), free(Lr);
  }
  /* block masks of every broadcast shape and block size, exactly sized, whole and sampled */
  const int blk[][2] = {{1, 1}, {2, 3}, {4, 2}, {64, 64}};
  for (size_t t = 0; t < sizeof blk / sizeof blk[0]; ++t) {
    const int bq = blk[t][0], bk = blk[t][1];
    const int n_qb = (nq + bq - 1) / bq, n_kb = (nk + bk - 1) / bk;
    for (int Mb = 1; Mb <= B; Mb += (B > 1 ? B - 1 : 1))
      for (int Mh = 1; Mh <= H; Mh += (H > 1 ? H - 1 : 1)) {
        uint8_t* M = alloc((size_t)Mb * Mh * n_qb * n_kb);
        for (int64_t e = 0; e < (int64_t)Mb * Mh * n_qb * n_kb; ++e) M[e] = (uint8_t)((e * 7 + t) % 3 != 0);
        CHECK(oracle_attention_blockmask_f64(Q, K, V, O, L, B, H, nq, nk, d, M, Mb, Mh, bq, bk, 3, 2, scale) == 0);
        int64_t* rows = alloc(R * 8);
        for (int64_t r = 0; r < R; ++r) rows[r] = r;
        double *Or = alloc(nQ * 8), *Lr = alloc(R * 8);
        CHECK(oracle_attention_blockmask_rows_bf16(Qb, Kb, Vb, rows, R, Or, Lr, B, H, nq, nk, d, M, Mb, Mh, bq, bk,
                                                   3, 2, scale) == 0);
        CHECK(maxdiff(O, Or, nQ) < 1e-12);
        for (int64_t r = 0; r < R; ++r) CHECK((isinf(L[r]) && isinf(Lr[r])) || fabs(L[r] - Lr[r]) < 1e-12);
        CHECK(oracle_blockmask_pairs(nq, nk, M, Mb, Mh, B - 1, H - 1, bq, bk, 3, 2) >= 0);
        CHECK(oracle_attention_blockmask_f64(Q, K, V, O, L, B, H, nq, nk, d, M, 2 * B + 1, Mh, bq, bk, -1, -1,
                                             scale) != 0);
        free(M), free(rows), free(Or), free(Lr);
      }
  }
  free(Qb), free(Kb), free(Vb), free(Q), free(K), free(V), free(dO), free(O), free(L), free(O2), free(L2);
}

int main(void) {
  run_shape(1, 1, 1, 1, 1);
  run_shape(1, 2, 5, 7, 4);
  run_shape(2, 1, 17, 3, 8);
  run_shape(1, 3, 9, 33, 16);
  /* e4m3: every code decodes to a value that encodes back to the same code (NaN codes excepted) */
  for (int c = 0; c < 256; ++c) {
    if ((c & 0x7f) == 0x7f) continue;
    const double v = oracle_e4m3_decode((uint8_t)c);
    if (v == 0.0) continue;  /* +0 and -0 */
    CHECK(oracle_e4m3_encode((float)v) == (uint8_t)c);
  }
  /* shape errors are reported, not read past */
  CHECK(oracle_attention_f64(NULL, NULL, NULL, NULL, NULL, 0, 1, 1, 1, 1, 0, 1.0) != 0);
  CHECK(oracle_merge_f64(NULL, NULL, NULL, NULL, NULL, 0, 1, 1) != 0);
  if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
  else printf("oracle checks passed\n");
  return failures;
}
