/*
 * sdpa_oracle.h — plain fp64 CPU definition of scaled dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the yardstick the GPU path is measured
 * against: only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  It shares no header, helper or constant with the GPU library.
 *
 * All arrays are host memory, fp64, contiguous row-major:
 *   q  (B, Hq,  Lq, Dk)     k  (B, Hkv, Lk, Dk)     v  (B, Hkv, Lk, Dv)
 *   o  (B, Hq,  Lq, Dv)     lse (B, Hq, Lq)         dO (B, Hq, Lq, Dv)
 *   dq like q, dk like k, dv like v, dsum (B, Hq, Lq)
 * mask: additive, any broadcast of (B, Hq, Lq, Lk) described by element strides
 *   mask_stride[0..3] for (b, h, i, j); a stride of 0 broadcasts that dimension.
 * len_q / len_kv: optional per-batch valid lengths (NULL = full length).
 *
 * Return value: 0 on success, -1 on an invalid problem (bad sizes, Hq % Hkv != 0,
 * a length outside [0, L]), -2 if an allowed mask entry is NaN or +inf (undefined
 * for an additive -inf mask).
 */
#ifndef SDPA_ORACLE_H
#define SDPA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t B, Hq, Hkv, Lq, Lk, Dk, Dv;
  int64_t mask_stride[4];
  double scale;      /* NaN selects the default 1/sqrt(Dk) */
  int32_t is_causal; /* 0: none; 1 top-left: key j visible to query i iff j <= i;
                        2 bottom-right: iff j <= i + (len_kv - len_q) of the batch */
  int32_t window;    /* 0: none; W > 0 (with is_causal): also j > i + off - W, i.e. a row
                        sees the last W keys up to its diagonal (off as above) */
} oracle_problem;

int oracle_sdpa_forward(const oracle_problem* p, const double* q, const double* k,
                        const double* v, const double* mask, const int32_t* len_q,
                        const int32_t* len_kv, double* o, double* lse);

/* Forward restricted to an explicit list of rows: rows[3r..3r+2] = (b, h, i).
 * o_rows is (nrows, Dv), lse_rows is (nrows). */
int oracle_sdpa_forward_rows(const oracle_problem* p, const double* q, const double* k,
                             const double* v, const double* mask, const int32_t* len_q,
                             const int32_t* len_kv, int64_t nrows, const int32_t* rows,
                             double* o_rows, double* lse_rows);

/* Backward from the definition; recomputes P itself.  dsum (may be NULL) receives
 * D_i = sum_j P_ij dP_ij for every row. */
int oracle_sdpa_backward(const oracle_problem* p, const double* q, const double* k,
                         const double* v, const double* mask, const int32_t* len_q,
                         const int32_t* len_kv, const double* dO, double* dq, double* dk,
                         double* dv, double* dsum);

/* Number of OpenMP threads the oracle runs on (1 if built without OpenMP). */
int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
