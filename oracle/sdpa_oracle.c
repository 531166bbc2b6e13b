/*
 * sdpa_oracle.c — plain fp64 CPU definition of scaled dot-product attention and its
 * hand-derived backward.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.  It is deliberately slow and
 * literal: one query row at a time, every score written out, no tiling, no online
 * softmax, no fusion.  It shares no code with the GPU library.
 *
 * What it follows (page titles and sections of the source pages):
 *  - "Scaled dot-product attention (forward and backward)" (tinyllm L5.1), §2 Principles
 *    (symbol table: S = alpha Q K^T, P = softmax(S) over keys, O = P V,
 *    D_i = sum_j P_ij dP_ij), §2.1 (default alpha = 1/sqrt(d)), §2.2 Masking (blocked
 *    scores are -inf before the softmax, the row max is subtracted, a fully blocked row
 *    gives zeros), §2.3 The backward pass (dV = P^T dO, dP = dO V^T,
 *    dS = P o (dP - D), dQ = alpha dS K, dK = alpha dS^T Q), §2.4 (leading dims are
 *    independent problems).
 *  - Lucid "ScaledDotProductAttentionBackward", Notes (the mask is additive, -inf at
 *    excluded positions; is_causal adds an upper-triangular -inf so query i sees keys
 *    j <= i) and forward (q.shape[-1] == k.shape[-1], k.shape[-2] == v.shape[-2]).
 *  - "Understanding PyTorch Scaled Dot-Product Attention" §3 (causal = tril, diagonal
 *    included) and §4 (GQA: KV head g serves query heads g*G .. g*G+G-1, the
 *    repeat_interleave order).  The gradient of a shared KV head is the sum over the
 *    query heads it serves: the chain rule through that repetition.
 *  - cuDNN "Attention", Support Matrix glossary note on padded layouts and the forward
 *    Configurable Options (padding mask: per-batch seq_len_q / seq_len_kv; positions at
 *    or past the length are masked out; a length of 0 skips the batch) and the forward
 *    Python API return values (stats = max + ln sum exp(s - max), natural log, fp32).
 *  - torch "flex_attention", parameters (scale defaults to 1/sqrt(E), E = query/key
 *    width; lse has shape (B, Hq, L)).
 *  - cuDNN "Attention", forward Configurable Options, diagonal masking: with the
 *    BOTTOM_RIGHT alignment the diagonal ends at the bottom-right corner of the actual
 *    (per-batch) sequence lengths, and right bound 0 masks every column past it, so query
 *    i sees key j iff j <= i + (len_kv - len_q).
 *  - cuDNN "Attention", forward Configurable Options, diagonal masking: a sliding window
 *    of length W is the causal right bound 0 plus the left bound W, which masks every
 *    column at or before row_idx - W (row_idx on the diagonal's alignment), so query i
 *    sees key j iff i + off - W < j <= i + off.
 *
 * Readings where the pages are silent: a query row at or past len_q is empty (O = 0,
 * LSE = -inf, no gradient); an empty or fully blocked row has LSE = -inf (ln 0);
 * disallowed pairs read neither K nor V; mask entries that are NaN or +inf are rejected.
 */
#include "sdpa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX4(a, b, c, d, B1, B2, B3) ((((int64_t)(a) * (B1) + (b)) * (B2) + (c)) * (B3) + (d))

static int check_problem(const oracle_problem* p, const int32_t* len_q, const int32_t* len_kv) {
  if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->Lq < 0 || p->Lk < 0 || p->Dk < 1 || p->Dv < 1)
    return -1;
  if (p->Hq % p->Hkv != 0) return -1;
  if (isinf(p->scale)) return -1;
  if (p->is_causal < 0 || p->is_causal > 2) return -1;
  if (p->window < 0 || (p->window > 0 && !p->is_causal)) return -1;
  for (int b = 0; b < p->B; ++b) {
    if (len_q && (len_q[b] < 0 || len_q[b] > p->Lq)) return -1;
    if (len_kv && (len_kv[b] < 0 || len_kv[b] > p->Lk)) return -1;
  }
  return 0;
}

/* alpha: the explicit scale, or 1/sqrt(d) of the query/key width when none is given. */
static double resolve_scale(const oracle_problem* p) {
  return isnan(p->scale) ? 1.0 / sqrt((double)p->Dk) : p->scale;
}

/*
 * One query row (b, h, i): fills P[0..Lk) with the attention weights and returns the
 * row's LSE through *lse.  Returns 0, or -2 for an undefined mask entry.
 *   allowed(j) = (j < len_kv[b]) and (not causal or j <= i + off) and (no window or
 *   j > i + off - W), and the row itself must satisfy i < len_q[b]; off = 0 for the
 *   top-left diagonal and len_kv[b] - len_q[b] for the bottom-right one;
 *   s_j = alpha * (q_i . k_g,j) + M[b,h,i,j]   if allowed, else -inf;
 *   m = max_j s_j; a row with m = -inf (or an empty row) has P = 0 and LSE = -inf;
 *   otherwise P_j = exp(s_j - m) / sum_t exp(s_t - m) and LSE = m + ln sum_t exp(s_t - m).
 */
static int row_weights(const oracle_problem* p, double alpha, const double* q, const double* k,
                       const double* mask, const int32_t* len_q, const int32_t* len_kv, int b,
                       int h, int i, double* s, double* P, double* lse) {
  const int G = p->Hq / p->Hkv;
  const int g = h / G;
  const int kv_len = len_kv ? len_kv[b] : p->Lk;
  const int q_len = len_q ? len_q[b] : p->Lq;
  const int row_valid = i < q_len;
  const int off = (p->is_causal == 2) ? kv_len - q_len : 0;
  const double* qi = q + IDX4(b, h, i, 0, p->Hq, p->Lq, p->Dk);

  double m = -INFINITY;
  for (int j = 0; j < p->Lk; ++j) {
    int allowed = row_valid && j < kv_len && (!p->is_causal || j <= i + off) &&
                  (!p->window || j > i + off - p->window);
    if (!allowed) {
      s[j] = -INFINITY;
      continue;
    }
    const double* kj = k + IDX4(b, g, j, 0, p->Hkv, p->Lk, p->Dk);
    double dot = 0.0;
    for (int t = 0; t < p->Dk; ++t) dot += qi[t] * kj[t];
    double sj = alpha * dot;
    if (mask) {
      double mv = mask[b * p->mask_stride[0] + h * p->mask_stride[1] + (int64_t)i * p->mask_stride[2] +
                       (int64_t)j * p->mask_stride[3]];
      if (isnan(mv) || (isinf(mv) && mv > 0)) return -2;
      sj += mv;
    }
    s[j] = sj;
    if (sj > m) m = sj;
  }

  if (m == -INFINITY) {
    for (int j = 0; j < p->Lk; ++j) P[j] = 0.0;
    *lse = -INFINITY;
    return 0;
  }
  double l = 0.0;
  for (int j = 0; j < p->Lk; ++j) {
    P[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
    l += P[j];
  }
  for (int j = 0; j < p->Lk; ++j) P[j] /= l;
  *lse = m + log(l);
  return 0;
}

/* O_i = sum_j P_ij v_j over the keys with nonzero weight (blocked keys are never read). */
static void row_output(const oracle_problem* p, const double* v, const double* P, int b, int g,
                       double* oi) {
  for (int t = 0; t < p->Dv; ++t) oi[t] = 0.0;
  for (int j = 0; j < p->Lk; ++j) {
    if (P[j] == 0.0) continue;
    const double* vj = v + IDX4(b, g, j, 0, p->Hkv, p->Lk, p->Dv);
    for (int t = 0; t < p->Dv; ++t) oi[t] += P[j] * vj[t];
  }
}

int oracle_sdpa_forward(const oracle_problem* p, const double* q, const double* k,
                        const double* v, const double* mask, const int32_t* len_q,
                        const int32_t* len_kv, double* o, double* lse) {
  if (check_problem(p, len_q, len_kv)) return -1;
  const double alpha = resolve_scale(p);
  const int G = p->Hq / p->Hkv;
  const int64_t nrows = (int64_t)p->B * p->Hq * p->Lq;
  int status = 0;
#pragma omp parallel reduction(min : status)
  {
    double* s = (double*)malloc(sizeof(double) * (p->Lk + 1));
    double* P = (double*)malloc(sizeof(double) * (p->Lk + 1));
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
      int i = (int)(r % p->Lq);
      int h = (int)((r / p->Lq) % p->Hq);
      int b = (int)(r / ((int64_t)p->Lq * p->Hq));
      double row_lse;
      int st = row_weights(p, alpha, q, k, mask, len_q, len_kv, b, h, i, s, P, &row_lse);
      if (st) status = st;
      lse[r] = row_lse;
      row_output(p, v, P, b, h / G, o + r * p->Dv);
    }
    free(s);
    free(P);
  }
  return status;
}

int oracle_sdpa_forward_rows(const oracle_problem* p, const double* q, const double* k,
                             const double* v, const double* mask, const int32_t* len_q,
                             const int32_t* len_kv, int64_t nrows, const int32_t* rows,
                             double* o_rows, double* lse_rows) {
  if (check_problem(p, len_q, len_kv)) return -1;
  for (int64_t r = 0; r < nrows; ++r) {
    const int32_t* bhi = rows + 3 * r;
    if (bhi[0] < 0 || bhi[0] >= p->B || bhi[1] < 0 || bhi[1] >= p->Hq || bhi[2] < 0 ||
        bhi[2] >= p->Lq)
      return -1;
  }
  const double alpha = resolve_scale(p);
  const int G = p->Hq / p->Hkv;
  int status = 0;
#pragma omp parallel reduction(min : status)
  {
    double* s = (double*)malloc(sizeof(double) * (p->Lk + 1));
    double* P = (double*)malloc(sizeof(double) * (p->Lk + 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      const int32_t* bhi = rows + 3 * r;
      double row_lse;
      int st = row_weights(p, alpha, q, k, mask, len_q, len_kv, bhi[0], bhi[1], bhi[2], s, P,
                           &row_lse);
      if (st) status = st;
      lse_rows[r] = row_lse;
      row_output(p, v, P, bhi[0], bhi[1] / G, o_rows + r * p->Dv);
    }
    free(s);
    free(P);
  }
  return status;
}

/*
 * Backward, one (batch b, KV head g) at a time so that each task owns dK_g and dV_g.
 * For every query head h served by g and every row i, P_i is recomputed from the
 * definition, then
 *   dP_ij = dO_i . v_j,   D_i = sum_j P_ij dP_ij,   dS_ij = P_ij (dP_ij - D_i),
 *   dQ_i  = alpha sum_j dS_ij k_j,
 *   dK_j += alpha dS_ij q_i,   dV_j += P_ij dO_i.
 * Keys with zero weight contribute nothing (dS_ij = 0 there) and are not read.
 */
int oracle_sdpa_backward(const oracle_problem* p, const double* q, const double* k,
                         const double* v, const double* mask, const int32_t* len_q,
                         const int32_t* len_kv, const double* dO, double* dq, double* dk,
                         double* dv, double* dsum) {
  if (check_problem(p, len_q, len_kv)) return -1;
  const double alpha = resolve_scale(p);
  const int G = p->Hq / p->Hkv;
  const int ngroups = p->B * p->Hkv;
  int status = 0;
#pragma omp parallel reduction(min : status)
  {
    double* s = (double*)malloc(sizeof(double) * (p->Lk + 1));
    double* P = (double*)malloc(sizeof(double) * (p->Lk + 1));
    double* dP = (double*)malloc(sizeof(double) * (p->Lk + 1));
#pragma omp for schedule(dynamic, 1)
    for (int bg = 0; bg < ngroups; ++bg) {
      const int b = bg / p->Hkv, g = bg % p->Hkv;
      double* dkg = dk + IDX4(b, g, 0, 0, p->Hkv, p->Lk, p->Dk);
      double* dvg = dv + IDX4(b, g, 0, 0, p->Hkv, p->Lk, p->Dv);
      memset(dkg, 0, sizeof(double) * (size_t)p->Lk * p->Dk);
      memset(dvg, 0, sizeof(double) * (size_t)p->Lk * p->Dv);
      for (int h = g * G; h < (g + 1) * G; ++h) {
        for (int i = 0; i < p->Lq; ++i) {
          const int64_t r = ((int64_t)b * p->Hq + h) * p->Lq + i;
          const double* qi = q + r * p->Dk;
          const double* dOi = dO + r * p->Dv;
          double* dqi = dq + r * p->Dk;
          double row_lse;
          int st = row_weights(p, alpha, q, k, mask, len_q, len_kv, b, h, i, s, P, &row_lse);
          if (st) status = st;

          double D = 0.0;
          for (int j = 0; j < p->Lk; ++j) {
            dP[j] = 0.0;
            if (P[j] == 0.0) continue;
            const double* vj = v + IDX4(b, g, j, 0, p->Hkv, p->Lk, p->Dv);
            double dot = 0.0;
            for (int t = 0; t < p->Dv; ++t) dot += dOi[t] * vj[t];
            dP[j] = dot;
            D += P[j] * dot;
          }
          if (dsum) dsum[r] = D;

          for (int t = 0; t < p->Dk; ++t) dqi[t] = 0.0;
          for (int j = 0; j < p->Lk; ++j) {
            if (P[j] == 0.0) continue;
            const double dS = P[j] * (dP[j] - D);
            const double* kj = k + IDX4(b, g, j, 0, p->Hkv, p->Lk, p->Dk);
            double* dkj = dkg + (int64_t)j * p->Dk;
            double* dvj = dvg + (int64_t)j * p->Dv;
            for (int t = 0; t < p->Dk; ++t) {
              dqi[t] += alpha * dS * kj[t];
              dkj[t] += alpha * dS * qi[t];
            }
            for (int t = 0; t < p->Dv; ++t) dvj[t] += P[j] * dOi[t];
          }
        }
      }
    }
    free(s);
    free(P);
    free(dP);
  }
  return status;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
