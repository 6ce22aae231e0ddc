/*
 * Exact-attention oracle: plain, slow, obviously correct fp64 CPU code.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this file; only the test suite, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * What it computes (FlashAttention-2 walkthrough page, "kernel main loop"
 * section: the online-softmax pseudocode and the remark that v1 and v2 follow
 * the same online-softmax mathematics; the result is exact attention):
 *
 *   s_ij      = scale * sum_k q_ik * k_jk                 (fp64)
 *   allowed   = { j : j < N_k and (not causal or j <= i) } (top-left causal)
 *   m_i       = max_{j allowed} s_ij
 *   l_i       = sum_{j allowed} exp(s_ij - m_i)
 *   O_i       = (sum_{j allowed} exp(s_ij - m_i) * v_j) / l_i
 *   LSE_i     = m_i + ln l_i
 *
 * This is the textbook two-pass softmax (max, then exponentials), not the
 * online recurrence the GPU path uses; the two reach the same result up to
 * rounding.  Tensors are contiguous [B][H][N][d]; LSE is [B][H][N_q].
 *
 * A key-range variant returns the unnormalised partial (acc, m, l) over
 * [key_begin, key_end) and a merge routine combines such partials; these
 * follow the "FA2 cross-paper synthesis" page, section 5 item 5 (split the
 * key/value sequence for single-query decode) with the same rescaling algebra
 * as the online recurrence (walkthrough page, main-loop pseudocode).  An
 * empty key range yields m = -inf, l = 0, acc = 0 and contributes nothing.
 *
 * The sliding-window functions at the end generalise the causal mask to a
 * band of keys around each query row (see the comment there).
 *
 * Parity pins: every function here is pinned by CPU tests (brute force at 50
 * digits, closed forms, invariants, torch's fp64 CPU attention, a float64
 * transcription of the pages' recurrence); none is "parity unpinned".
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 bit pattern -> double, exactly (a bf16 is the top half of a float). */
static double bf16_bits_to_double(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

void oracle_bf16_to_f64(const uint16_t* src, double* dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) dst[i] = bf16_bits_to_double(src[i]);
}

/* Number of keys row i may attend to: the allowed set is always a prefix. */
static int64_t allowed_prefix(int64_t i, int64_t n_k, int causal) {
  if (!causal) return n_k;
  return (i + 1 < n_k) ? i + 1 : n_k;
}

/*
 * One query row against keys [j0, j1) (already clipped to the allowed set).
 * Writes the unnormalised partial: acc[d] = sum exp(s_j - m) v_j, *m, *l.
 * s is caller scratch of at least j1 - j0 doubles.
 */
static void partial_row(const double* q, const double* K, const double* V, int64_t j0, int64_t j1,
                        int d, double scale, double* s, double* acc, double* m_out, double* l_out) {
  for (int c = 0; c < d; ++c) acc[c] = 0.0;
  if (j1 <= j0) {
    *m_out = -INFINITY;
    *l_out = 0.0;
    return;
  }
  /* pass 1: scores and their maximum */
  double m = -INFINITY;
  for (int64_t j = j0; j < j1; ++j) {
    const double* kj = K + j * d;
    double dot = 0.0;
    for (int c = 0; c < d; ++c) dot += q[c] * kj[c];
    s[j - j0] = scale * dot;
    if (s[j - j0] > m) m = s[j - j0];
  }
  /* pass 2: exponentials, their sum, and the weighted sum of values */
  double l = 0.0;
  for (int64_t j = j0; j < j1; ++j) {
    double p = exp(s[j - j0] - m);
    l += p;
    const double* vj = V + j * d;
    for (int c = 0; c < d; ++c) acc[c] += p * vj[c];
  }
  *m_out = m;
  *l_out = l;
}

/* Full attention for one row: normalise the partial over the allowed prefix. */
static void attend_row(const double* q, const double* K, const double* V, int64_t n_allowed, int d,
                       double scale, double* s, double* o, double* lse) {
  double m, l;
  partial_row(q, K, V, 0, n_allowed, d, scale, s, o, &m, &l);
  for (int c = 0; c < d; ++c) o[c] /= l;
  *lse = m + log(l);
}

static int check_shape(int B, int H, int n_q, int n_k, int d) {
  return (B >= 1 && H >= 1 && n_q >= 0 && n_k >= 1 && d >= 1) ? 0 : -1;
}

/*
 * O, LSE for all rows.  Q, K, V are fp64 values (the exact values of the
 * bf16 inputs, or any reals for pins).  Returns 0, or -1 on a bad shape.
 */
int oracle_attention_f64(const double* Q, const double* K, const double* V, double* O, double* LSE,
                         int B, int H, int n_q, int n_k, int d, int causal, double scale) {
  if (check_shape(B, H, n_q, n_k, d)) return -1;
  const int64_t rows_per_block = 64;
  const int64_t n_blocks = (n_q + rows_per_block - 1) / rows_per_block;
  const int64_t n_tasks = (int64_t)B * H * n_blocks;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)n_k);
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < n_tasks; ++t) {
      const int64_t bh = t / n_blocks, blk = t % n_blocks;
      const double* Kh = K + bh * (int64_t)n_k * d;
      const double* Vh = V + bh * (int64_t)n_k * d;
      const int64_t i_end = (blk + 1) * rows_per_block < n_q ? (blk + 1) * rows_per_block : n_q;
      for (int64_t i = blk * rows_per_block; i < i_end; ++i) {
        const int64_t row = bh * n_q + i;
        attend_row(Q + row * d, Kh, Vh, allowed_prefix(i, n_k, causal), d, scale, s, O + row * d, LSE + row);
      }
    }
    free(s);
  }
  return 0;
}

/*
 * Same result for a chosen set of rows of bf16 inputs.  Q, K, V hold bf16 bit
 * patterns of the whole [B][H][N][d] tensors; rows[r] = (b*H + h)*N_q + i.
 * Only the heads the listed rows touch are converted.  O_rows is [n_rows][d],
 * LSE_rows is [n_rows].  Returns 0, or -1 on a bad shape / row index.
 */
int oracle_attention_rows_bf16(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const int64_t* rows,
                               int64_t n_rows, double* O_rows, double* LSE_rows, int B, int H, int n_q, int n_k,
                               int d, int causal, double scale) {
  if (check_shape(B, H, n_q, n_k, d)) return -1;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= (int64_t)B * H * n_q) return -1;
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)n_k);
    double* q = (double*)malloc(sizeof(double) * (size_t)d);
    double* Kh = (double*)malloc(sizeof(double) * (size_t)n_k * d);
    double* Vh = (double*)malloc(sizeof(double) * (size_t)n_k * d);
    int64_t cached_bh = -1;
    if (!s || !q || !Kh || !Vh) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (failed) continue;
      const int64_t bh = rows[r] / n_q, i = rows[r] % n_q;
      if (bh != cached_bh) {
        oracle_bf16_to_f64(K + bh * (int64_t)n_k * d, Kh, (int64_t)n_k * d);
        oracle_bf16_to_f64(V + bh * (int64_t)n_k * d, Vh, (int64_t)n_k * d);
        cached_bh = bh;
      }
      oracle_bf16_to_f64(Q + rows[r] * d, q, d);
      attend_row(q, Kh, Vh, allowed_prefix(i, n_k, causal), d, scale, s, O_rows + r * d, LSE_rows + r);
    }
    free(s); free(q); free(Kh); free(Vh);
  }
  return failed ? -1 : 0;
}

/*
 * Unnormalised partial over keys [key_begin, key_end) intersected with the
 * allowed set, for every row: acc [B][H][N_q][d], m and l [B][H][N_q].
 */
int oracle_partial_f64(const double* Q, const double* K, const double* V, double* acc, double* m, double* l,
                       int B, int H, int n_q, int n_k, int d, int causal, double scale, int key_begin,
                       int key_end) {
  if (check_shape(B, H, n_q, n_k, d) || key_begin < 0 || key_end < key_begin) return -1;
  const int64_t n_rows = (int64_t)B * H * n_q;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)n_k);
#pragma omp for schedule(static)
    for (int64_t row = 0; row < n_rows; ++row) {
      const int64_t bh = row / n_q, i = row % n_q;
      const int64_t n_allowed = allowed_prefix(i, n_k, causal);
      const int64_t j0 = key_begin;
      const int64_t j1 = key_end < n_allowed ? key_end : n_allowed;
      partial_row(Q + row * d, K + bh * (int64_t)n_k * d, V + bh * (int64_t)n_k * d, j0, j1, d, scale, s,
                  acc + row * d, m + row, l + row);
    }
    free(s);
  }
  return 0;
}

/*
 * Merge n_parts partials per row (part-major: acc [n_parts][n_rows][d], m and
 * l [n_parts][n_rows]) into O [n_rows][d] and LSE [n_rows]:
 *   M = max_c m_c;  w_c = exp(m_c - M) (0 for an empty part);
 *   l = sum_c w_c l_c;  O = (sum_c w_c acc_c) / l;  LSE = M + ln l.
 */
int oracle_merge_f64(const double* acc, const double* m, const double* l, double* O, double* LSE, int n_parts,
                     int64_t n_rows, int d) {
  if (n_parts < 1 || n_rows < 0 || d < 1) return -1;
  for (int64_t row = 0; row < n_rows; ++row) {
    double M = -INFINITY;
    for (int c = 0; c < n_parts; ++c)
      if (m[c * n_rows + row] > M) M = m[c * n_rows + row];
    double lsum = 0.0;
    for (int k = 0; k < d; ++k) O[row * d + k] = 0.0;
    for (int c = 0; c < n_parts; ++c) {
      const double mc = m[c * n_rows + row];
      if (mc == -INFINITY) continue; /* empty part: weight 0 */
      const double w = exp(mc - M);
      lsum += w * l[c * n_rows + row];
      for (int k = 0; k < d; ++k) O[row * d + k] += w * acc[(c * n_rows + row) * d + k];
    }
    for (int k = 0; k < d; ++k) O[row * d + k] /= lsum;
    LSE[row] = M + log(lsum);
  }
  return 0;
}

/*
 * The probability matrix P [B][H][N_q][N_k] (zero where not allowed), for
 * small shapes in tests: P_ij = exp(s_ij - m_i) / l_i.
 */
int oracle_probs_f64(const double* Q, const double* K, double* P, int B, int H, int n_q, int n_k, int d,
                     int causal, double scale) {
  if (check_shape(B, H, n_q, n_k, d)) return -1;
  double* s = (double*)malloc(sizeof(double) * (size_t)n_k);
  if (!s) return -1;
  for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
    for (int64_t i = 0; i < n_q; ++i) {
      const double* q = Q + (bh * n_q + i) * d;
      double* prow = P + (bh * n_q + i) * n_k;
      const int64_t n_allowed = allowed_prefix(i, n_k, causal);
      double m = -INFINITY;
      for (int64_t j = 0; j < n_allowed; ++j) {
        const double* kj = K + (bh * n_k + j) * d;
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += q[c] * kj[c];
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
      }
      double l = 0.0;
      for (int64_t j = 0; j < n_allowed; ++j) l += exp(s[j] - m);
      for (int64_t j = 0; j < n_k; ++j) prow[j] = (j < n_allowed) ? exp(s[j] - m) / l : 0.0;
    }
  }
  free(s);
  return 0;
}

/*
 * Sliding-window attention (the synthesis page, section 5 item 4: extend the
 * causal block skip to a sliding window).  Key j is visible to query i iff
 *   j < N_k,  (wl < 0 or j >= i - wl)  and  (wr < 0 or j <= i + wr),
 * with top-left alignment as for the causal mask: wl = wr = -1 is plain
 * attention, wl = -1 and wr = 0 is the causal mask.  The visible keys of a row
 * form one contiguous range [j0, j1).  A row that sees no key gets O = 0 and
 * LSE = -inf (the empty sum).
 */
static void window_range(int64_t i, int64_t n_k, int wl, int wr, int64_t* j0, int64_t* j1) {
  int64_t lo = 0, hi = n_k; /* [lo, hi) */
  if (wl >= 0 && i - wl > lo) lo = i - wl;
  if (wr >= 0 && i + wr + 1 < hi) hi = i + wr + 1;
  if (hi < lo) hi = lo;
  *j0 = lo;
  *j1 = hi;
}

static void attend_range_row(const double* q, const double* K, const double* V, int64_t j0, int64_t j1, int d,
                             double scale, double* s, double* o, double* lse) {
  double m, l;
  partial_row(q, K, V, j0, j1, d, scale, s, o, &m, &l);
  if (j1 <= j0) {
    *lse = -INFINITY; /* o is already zero */
    return;
  }
  for (int c = 0; c < d; ++c) o[c] /= l;
  *lse = m + log(l);
}

int oracle_attention_window_f64(const double* Q, const double* K, const double* V, double* O, double* LSE, int B,
                                int H, int n_q, int n_k, int d, int wl, int wr, double scale) {
  if (check_shape(B, H, n_q, n_k, d)) return -1;
  const int64_t n_rows = (int64_t)B * H * n_q;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)n_k);
#pragma omp for schedule(dynamic, 16)
    for (int64_t row = 0; row < n_rows; ++row) {
      const int64_t bh = row / n_q, i = row % n_q;
      int64_t j0, j1;
      window_range(i, n_k, wl, wr, &j0, &j1);
      attend_range_row(Q + row * d, K + bh * (int64_t)n_k * d, V + bh * (int64_t)n_k * d, j0, j1, d, scale, s,
                       O + row * d, LSE + row);
    }
    free(s);
  }
  return 0;
}

/* The windowed result for chosen rows of bf16 inputs (as oracle_attention_rows_bf16). */
int oracle_attention_window_rows_bf16(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const int64_t* rows,
                                      int64_t n_rows, double* O_rows, double* LSE_rows, int B, int H, int n_q,
                                      int n_k, int d, int wl, int wr, double scale) {
  if (check_shape(B, H, n_q, n_k, d)) return -1;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= (int64_t)B * H * n_q) return -1;
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)n_k);
    double* q = (double*)malloc(sizeof(double) * (size_t)d);
    double* Kh = (double*)malloc(sizeof(double) * (size_t)n_k * d);
    double* Vh = (double*)malloc(sizeof(double) * (size_t)n_k * d);
    int64_t cached_bh = -1;
    if (!s || !q || !Kh || !Vh) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (failed) continue;
      const int64_t bh = rows[r] / n_q, i = rows[r] % n_q;
      if (bh != cached_bh) {
        oracle_bf16_to_f64(K + bh * (int64_t)n_k * d, Kh, (int64_t)n_k * d);
        oracle_bf16_to_f64(V + bh * (int64_t)n_k * d, Vh, (int64_t)n_k * d);
        cached_bh = bh;
      }
      oracle_bf16_to_f64(Q + rows[r] * d, q, d);
      int64_t j0, j1;
      window_range(i, n_k, wl, wr, &j0, &j1);
      attend_range_row(q, Kh, Vh, j0, j1, d, scale, s, O_rows + r * d, LSE_rows + r);
    }
    free(s); free(q); free(Kh); free(Vh);
  }
  return failed ? -1 : 0;
}

/* Number of visible (query, key) pairs of one head under the window (for FLOP counts). */
int64_t oracle_window_pairs(int n_q, int n_k, int wl, int wr) {
  int64_t total = 0;
  for (int64_t i = 0; i < n_q; ++i) {
    int64_t j0, j1;
    window_range(i, n_k, wl, wr, &j0, &j1);
    total += j1 - j0;
  }
  return total;
}

/*
 * Backward pass (the synthesis page, section 3 item 1 and section 5 item 2:
 * the gradients of exact attention from the stored LSE; FA2's five products).
 * For a scalar loss with upstream gradient dO of the output O, per (b, h):
 *   P_ij  = exp(s_ij - LSE_i) over allowed j, 0 elsewhere   (s_ij = scale q_i . k_j)
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   D_i   = sum_c dO_ic O_ic            (= sum_j P_ij dP_ij)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 * O and LSE are recomputed here in fp64 (plain two-pass softmax) rather than
 * taken from the caller, so the gradients are those of exact attention.
 * Causal masking is top-left as in the forward.  Returns 0, or -1.
 */
int oracle_backward_f64(const double* Q, const double* K, const double* V, const double* dO, double* dQ,
                        double* dK, double* dV, int B, int H, int n_q, int n_k, int d, int causal, double scale) {
  if (check_shape(B, H, n_q, n_k, d)) return -1;
  double* P = (double*)malloc(sizeof(double) * (size_t)n_q * n_k);
  double* dS = (double*)malloc(sizeof(double) * (size_t)n_q * n_k);
  if (!P || !dS) {
    free(P); free(dS);
    return -1;
  }
  /* heads one after another; the loops over rows inside a head run in parallel */
  for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
    const double* q = Q + bh * (int64_t)n_q * d;
    const double* k = K + bh * (int64_t)n_k * d;
    const double* v = V + bh * (int64_t)n_k * d;
    const double* go = dO + bh * (int64_t)n_q * d;
    double* gq = dQ + bh * (int64_t)n_q * d;
    double* gk = dK + bh * (int64_t)n_k * d;
    double* gv = dV + bh * (int64_t)n_k * d;
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t i = 0; i < n_q; ++i) {
      const int64_t n_allowed = allowed_prefix(i, n_k, causal);
      double* prow = P + i * n_k;
      double m = -INFINITY;
      for (int64_t j = 0; j < n_allowed; ++j) {
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += q[i * d + c] * k[j * d + c];
        prow[j] = scale * dot;
        if (prow[j] > m) m = prow[j];
      }
      double l = 0.0;
      for (int64_t j = 0; j < n_allowed; ++j) l += exp(prow[j] - m);
      const double lse = m + log(l);
      for (int64_t j = 0; j < n_k; ++j) prow[j] = (j < n_allowed) ? exp(prow[j] - lse) : 0.0;
      /* D_i = dO_i . O_i with O_i = sum_j P_ij v_j */
      double Di = 0.0;
      for (int c = 0; c < d; ++c) {
        double oc = 0.0;
        for (int64_t j = 0; j < n_allowed; ++j) oc += prow[j] * v[j * d + c];
        Di += go[i * d + c] * oc;
      }
      /* dS_ij = P_ij (dO_i . v_j - D_i) */
      for (int64_t j = 0; j < n_k; ++j) {
        if (j >= n_allowed) { dS[i * n_k + j] = 0.0; continue; }
        double dp = 0.0;
        for (int c = 0; c < d; ++c) dp += go[i * d + c] * v[j * d + c];
        dS[i * n_k + j] = prow[j] * (dp - Di);
      }
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_q; ++i)
      for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < n_k; ++j) acc += dS[i * n_k + j] * k[j * d + c];
        gq[i * d + c] = scale * acc;
      }
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n_k; ++j)
      for (int c = 0; c < d; ++c) {
        double acck = 0.0, accv = 0.0;
        for (int64_t i = 0; i < n_q; ++i) {
          acck += dS[i * n_k + j] * q[i * d + c];
          accv += P[i * n_k + j] * go[i * d + c];
        }
        gk[j * d + c] = scale * acck;
        gv[j * d + c] = accv;
      }
  }
  free(P); free(dS);
  return 0;
}

/*
 * FP8 (e4m3) inputs.  The improvements page (section 三 on FlashAttention-3,
 * and section 四, point ③) says FP8 doubles matrix throughput and that the
 * precision it loses must be controlled by scaling; it gives no recipe, so
 * this is the plainest one.  The format is OCP e4m3fn: sign, 4 exponent bits
 * (bias 7), 3 mantissa bits, subnormals, largest finite 448, no infinities
 * (codes 0x7f and 0xff are NaN and are never produced here).
 *
 * Scaling is per (batch, head) tensor slice: amax = max |x| over the slice,
 * inv = fp32(448 / amax) and descale = fp32(amax / 448) (both 1 when
 * amax = 0).  The code of x is e4m3 round-to-nearest-even of the fp32
 * product fp32(x) * inv; its value is decode(code) * descale.
 *
 * Attention on FP8 inputs is exact attention (the definition at the top of
 * this file) applied to the dequantised values q = decode(Qc) * descale_q,
 * k = decode(Kc) * descale_k, v = decode(Vc) * descale_v, in fp64.
 */
static uint8_t e4m3_rne(float y) {
  /* round-to-nearest-even onto the e4m3fn grid, |y| <= 448 assumed */
  const uint8_t sign = (y < 0.f || (y == 0.f && signbit(y))) ? 0x80 : 0;
  double a = fabs((double)y);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);              /* a = f * 2^e, f in [0.5, 1) */
  int E = e - 1;             /* a in [2^E, 2^(E+1)) */
  if (E < -6) E = -6;        /* subnormal range shares the spacing of E = -6 */
  const double ulp = ldexp(1.0, E - 3);
  double q = a / ulp;        /* exact: a and ulp are binary */
  double fl = floor(q);
  double r = q - fl;
  if (r > 0.5 || (r == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
  double v = fl * ulp;       /* rounded magnitude */
  if (v > 448.0) v = 448.0;  /* not reached for |y| <= 448 */
  /* encode v */
  if (v < ldexp(1.0, -6)) return sign | (uint8_t)(int)(v / ldexp(1.0, -9)); /* subnormal: m * 2^-9 */
  int ev;
  double fv = frexp(v, &ev); /* v = fv * 2^ev, fv in [0.5, 1) */
  const int expo = ev - 1 + 7;
  const int mant = (int)((fv * 2.0 - 1.0) * 8.0 + 0.5);
  return sign | (uint8_t)(expo << 3) | (uint8_t)mant;
}

uint8_t oracle_e4m3_encode(float y) { return e4m3_rne(y); }

double oracle_e4m3_decode(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  const double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Per-head quantisation of bf16 X [B][H][N][d] into codes [B][H][N][d] and
 * descale [B][H].  Returns 0. */
int oracle_quantize_fp8(const uint16_t* X, uint8_t* codes, float* descale, int B, int H, int n, int d) {
  for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
    const uint16_t* x = X + bh * (int64_t)n * d;
    float amax = 0.f;
    for (int64_t i = 0; i < (int64_t)n * d; ++i) {
      const float a = fabsf((float)bf16_bits_to_double(x[i]));
      if (a > amax) amax = a;
    }
    const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
    descale[bh] = amax > 0.f ? amax / 448.0f : 1.0f;
    for (int64_t i = 0; i < (int64_t)n * d; ++i) {
      const float y = (float)bf16_bits_to_double(x[i]) * inv;
      codes[bh * (int64_t)n * d + i] = e4m3_rne(y);
    }
  }
  return 0;
}

/*
 * Attention on FP8 inputs for a chosen set of rows.  Qc, Kc, Vc hold e4m3
 * codes of the whole [B][H][N][d] tensors (V in the same row layout as K);
 * descale_* are [B][H]; rows[r] = (b*H + h)*N_q + i; the visible keys of row i
 * are j < N_k and, if causal, j <= i.  O_rows [n_rows][d], LSE_rows [n_rows].
 * Returns 0, or -1 on a bad shape / row index.
 */
int oracle_attention_fp8_rows(const uint8_t* Qc, const uint8_t* Kc, const uint8_t* Vc, const float* descale_q,
                              const float* descale_k, const float* descale_v, const int64_t* rows, int64_t n_rows,
                              double* O_rows, double* LSE_rows, int B, int H, int n_q, int n_k, int d, int causal,
                              double scale) {
  if (check_shape(B, H, n_q, n_k, d)) return -1;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= (int64_t)B * H * n_q) return -1;
  double table[256];
  for (int c = 0; c < 256; ++c) table[c] = oracle_e4m3_decode((uint8_t)c);
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)n_k);
    double* q = (double*)malloc(sizeof(double) * (size_t)d);
    double* Kh = (double*)malloc(sizeof(double) * (size_t)n_k * d);
    double* Vh = (double*)malloc(sizeof(double) * (size_t)n_k * d);
    int64_t cached_bh = -1;
    if (!s || !q || !Kh || !Vh) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (failed) continue;
      const int64_t bh = rows[r] / n_q, i = rows[r] % n_q;
      if (bh != cached_bh) {
        const uint8_t* kc = Kc + bh * (int64_t)n_k * d;
        const uint8_t* vc = Vc + bh * (int64_t)n_k * d;
        for (int64_t e = 0; e < (int64_t)n_k * d; ++e) {
          Kh[e] = table[kc[e]] * (double)descale_k[bh];
          Vh[e] = table[vc[e]] * (double)descale_v[bh];
        }
        cached_bh = bh;
      }
      for (int c = 0; c < d; ++c) q[c] = table[Qc[rows[r] * d + c]] * (double)descale_q[bh];
      attend_row(q, Kh, Vh, allowed_prefix(i, n_k, causal), d, scale, s, O_rows + r * d, LSE_rows + r);
    }
    free(s); free(q); free(Kh); free(Vh);
  }
  return failed ? -1 : 0;
}

/* Threads the parallel regions above use (reported beside CPU timings). */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
#else
int oracle_num_threads(void) { return 1; }
#endif

/*
 * Block-sparse attention (the synthesis page, section 5 item 4: the causal
 * block skip extended to sliding windows and dilated patterns, as one
 * sparse-block-skip mechanism).  A byte mask M selects (query block, key
 * block) pairs: query rows are grouped in blocks of bq, keys in blocks of bk,
 * and M has shape [Mb][Mh][ceil(N_q/bq)][ceil(N_k/bk)] with Mb in {1, B} and
 * Mh in {1, H} (a size-1 dimension is shared by every batch or head).  Key j
 * is visible to query i of (b, h) iff
 *   j < N_k,
 *   M[b mod Mb][h mod Mh][i / bq][j / bk] != 0, and
 *   the band (wl, wr) admits it: (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr).
 * The softmax runs over the visible keys only (two passes: maximum, then the
 * exponentials); a row that sees no key gets O = 0 and LSE = -inf.
 */
static int blockmask_visible(const uint8_t* mrow, int64_t i, int64_t j, int bk, int wl, int wr) {
  if (wl >= 0 && j < i - wl) return 0;
  if (wr >= 0 && j > i + wr) return 0;
  return mrow[j / bk] != 0;
}

static void attend_masked_row(const double* q, const double* K, const double* V, int64_t n_k, int d,
                              double scale, const uint8_t* mrow, int bk, int64_t i, int wl, int wr, double* s,
                              double* o, double* lse) {
  for (int c = 0; c < d; ++c) o[c] = 0.0;
  double m = -INFINITY;
  for (int64_t j = 0; j < n_k; ++j) {
    if (!blockmask_visible(mrow, i, j, bk, wl, wr)) continue;
    const double* kj = K + j * d;
    double dot = 0.0;
    for (int c = 0; c < d; ++c) dot += q[c] * kj[c];
    s[j] = scale * dot;
    if (s[j] > m) m = s[j];
  }
  if (m == -INFINITY) {
    *lse = -INFINITY; /* no visible key: O stays zero */
    return;
  }
  double l = 0.0;
  for (int64_t j = 0; j < n_k; ++j) {
    if (!blockmask_visible(mrow, i, j, bk, wl, wr)) continue;
    const double p = exp(s[j] - m);
    l += p;
    const double* vj = V + j * d;
    for (int c = 0; c < d; ++c) o[c] += p * vj[c];
  }
  for (int c = 0; c < d; ++c) o[c] /= l;
  *lse = m + log(l);
}

static int check_blockmask(int B, int H, int Mb, int Mh, int bq, int bk) {
  if (bq < 1 || bk < 1) return -1;
  if (!(Mb == 1 || Mb == B) || !(Mh == 1 || Mh == H)) return -1;
  return 0;
}

/* The mask row of query i of (b, h): M[b mod Mb][h mod Mh][i / bq][.] */
static const uint8_t* blockmask_row(const uint8_t* M, int64_t b, int64_t h, int64_t i, int Mb, int Mh, int bq,
                                    int64_t n_qb, int64_t n_kb) {
  return M + (((b % Mb) * Mh + (h % Mh)) * n_qb + i / bq) * n_kb;
}

int oracle_attention_blockmask_f64(const double* Q, const double* K, const double* V, double* O, double* LSE,
                                   int B, int H, int n_q, int n_k, int d, const uint8_t* M, int Mb, int Mh, int bq,
                                   int bk, int wl, int wr, double scale) {
  if (check_shape(B, H, n_q, n_k, d) || check_blockmask(B, H, Mb, Mh, bq, bk)) return -1;
  const int64_t n_rows = (int64_t)B * H * n_q;
  const int64_t n_qb = (n_q + bq - 1) / bq, n_kb = (n_k + bk - 1) / bk;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)n_k);
#pragma omp for schedule(dynamic, 16)
    for (int64_t row = 0; row < n_rows; ++row) {
      const int64_t bh = row / n_q, i = row % n_q;
      const uint8_t* mrow = blockmask_row(M, bh / H, bh % H, i, Mb, Mh, bq, n_qb, n_kb);
      attend_masked_row(Q + row * d, K + bh * (int64_t)n_k * d, V + bh * (int64_t)n_k * d, n_k, d, scale, mrow,
                        bk, i, wl, wr, s, O + row * d, LSE + row);
    }
    free(s);
  }
  return 0;
}

/* The block-sparse result for chosen rows of bf16 inputs (as oracle_attention_rows_bf16). */
int oracle_attention_blockmask_rows_bf16(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                         const int64_t* rows, int64_t n_rows, double* O_rows, double* LSE_rows,
                                         int B, int H, int n_q, int n_k, int d, const uint8_t* M, int Mb, int Mh,
                                         int bq, int bk, int wl, int wr, double scale) {
  if (check_shape(B, H, n_q, n_k, d) || check_blockmask(B, H, Mb, Mh, bq, bk)) return -1;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= (int64_t)B * H * n_q) return -1;
  const int64_t n_qb = (n_q + bq - 1) / bq, n_kb = (n_k + bk - 1) / bk;
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)n_k);
    double* q = (double*)malloc(sizeof(double) * (size_t)d);
    double* Kh = (double*)malloc(sizeof(double) * (size_t)n_k * d);
    double* Vh = (double*)malloc(sizeof(double) * (size_t)n_k * d);
    int64_t cached_bh = -1;
    if (!s || !q || !Kh || !Vh) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (failed) continue;
      const int64_t bh = rows[r] / n_q, i = rows[r] % n_q;
      if (bh != cached_bh) {
        oracle_bf16_to_f64(K + bh * (int64_t)n_k * d, Kh, (int64_t)n_k * d);
        oracle_bf16_to_f64(V + bh * (int64_t)n_k * d, Vh, (int64_t)n_k * d);
        cached_bh = bh;
      }
      oracle_bf16_to_f64(Q + rows[r] * d, q, d);
      const uint8_t* mrow = blockmask_row(M, bh / H, bh % H, i, Mb, Mh, bq, n_qb, n_kb);
      attend_masked_row(q, Kh, Vh, n_k, d, scale, mrow, bk, i, wl, wr, s, O_rows + r * d, LSE_rows + r);
    }
    free(s); free(q); free(Kh); free(Vh);
  }
  return failed ? -1 : 0;
}

/* Visible (query, key) pairs of one (b, h) under the block mask and band. */
int64_t oracle_blockmask_pairs(int n_q, int n_k, const uint8_t* M, int Mb, int Mh, int b, int h, int bq, int bk,
                               int wl, int wr) {
  const int64_t n_qb = (n_q + bq - 1) / bq, n_kb = (n_k + bk - 1) / bk;
  int64_t n = 0;
  for (int64_t i = 0; i < n_q; ++i) {
    const uint8_t* mrow = blockmask_row(M, b, h, i, Mb, Mh, bq, n_qb, n_kb);
    for (int64_t j = 0; j < n_k; ++j) n += blockmask_visible(mrow, i, j, bk, wl, wr);
  }
  return n;
}
