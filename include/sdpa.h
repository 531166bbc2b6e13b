/*
 * sdpa.h — C ABI of the MI355X (gfx950) scaled dot-product attention library.
 *
 * Operation (forward), per batch b, query head h, query row i:
 *   S_ij = scale * q_i . k_j + M_bhij   for every key j the row may attend to,
 *   P_i  = softmax over keys of S_i (row max subtracted),  O_i = sum_j P_ij v_j,
 *   LSE_i = max_j S_ij + ln sum_j exp(S_ij - max_j S_ij)          (natural log, fp32).
 * Sources: "Scaled dot-product attention (forward and backward)" (tinyllm L5.1),
 * section 2 Principles and 2.2 Masking; cuDNN "Attention", SDPA FP16/BF16 Forward
 * (Python API return values: stats = max + ln sum exp, shape (B, Hq, Sq, 1); Tensors
 * table); torch "flex_attention" parameters (default scale 1/sqrt(E), lse (B, Hq, L)).
 *
 * Backward: dV = P^T dO, dP = dO V^T, dS = P o (dP - D) with D_i = rowsum(dO o O)_i,
 *   dQ = scale dS K, dK = scale dS^T Q.  Source: tinyllm L5.1 section 2.3 The backward
 *   pass; cuDNN "Attention", SDPA FP16/BF16 Backward (takes the forward's O and stats).
 *
 * Which keys a row may attend to (all conditions at once):
 *  - additive mask: an entry of -inf blocks the pair, a finite entry is added as a bias
 *    (Lucid ScaledDotProductAttentionBackward, Notes; cuDNN "Attention", Bias mask);
 *  - is_causal = 1 (SDPA_CAUSAL_TOP_LEFT): key j is visible to query i iff j <= i;
 *    is_causal = 2 (SDPA_CAUSAL_BOTTOM_RIGHT): iff j <= i + (len_kv - len_q), with the
 *    batch's actual lengths, so the diagonal ends in the bottom-right corner (cuDNN
 *    "Attention", forward Configurable Options, diagonal masking: BOTTOM_RIGHT alignment
 *    with right bound 0 -- a prefill chunk against its KV cache; rows that end up with no
 *    key are empty);
 *    ("Understanding PyTorch Scaled Dot-Product Attention" section 3, tril);
 *  - sliding_window = W > 0 (with is_causal 1 or 2): key j is also visible only if
 *    j > i + offset - W, offset being the diagonal's (0, or len_kv - len_q): each row sees
 *    the last W keys up to its diagonal (cuDNN "Attention", forward Configurable Options,
 *    diagonal masking: sliding window = right bound 0 with left bound W, which masks the
 *    columns at or before row_idx - W);
 *  - per-batch lengths: keys j >= seq_lens_kv[b] are blocked and query rows
 *    i >= seq_lens_q[b] are empty (cuDNN "Attention", Support Matrix glossary note on
 *    padded layouts; Configurable Options, Padding mask).  Rows and keys past a length
 *    are never read.
 * A row with no visible key (empty or fully masked) yields O = 0, LSE = -inf and zero
 * gradients, never NaN (tinyllm L5.1 section 2.2).
 *
 * GQA: Hq must be a multiple of Hkv; query head h reads KV head h / (Hq / Hkv), the
 * repeat_interleave order ("Understanding PyTorch Scaled Dot-Product Attention"
 * section 4).  dK/dV of a shared head sum over the query heads it serves.
 *
 * Layout: every tensor is logically (B, H, L, D) with the element strides given below for
 * (b, h, l); the innermost (d) stride is 1.  dO shares O's strides, dQ/dK/dV share
 * Q/K/V's strides.  The mask is logically (B, Hq, Lq, Lk) with strides for (b, h, i) and a
 * unit stride along keys; a stride of 0 broadcasts a dimension ((B|1, Hq|1, Lq, Lk)).
 * LSE is contiguous (B, Hq, Lq) fp32.  One element type for q, k, v, o, dO, dq, dk, dv and
 * the mask.
 *
 * Ownership and threading: every data pointer is a device pointer owned by the caller.
 * The library allocates no device memory, keeps no handles, never synchronises the
 * device, and launches only on the given stream (a hipStream_t; NULL = default stream).
 * It is re-entrant; its only global state is a thread-local error message.
 *
 * Errors: every condition checkable on the host is validated before anything is
 * launched; on failure the call returns a status, launches nothing and records a
 * message readable with sdpa_last_error().  Device-resident preconditions are not
 * checked: 0 <= seq_lens <= L, finite q/k/v/dO (rows past a length may hold anything),
 * mask entries finite or -inf.
 */
#ifndef SDPA_H
#define SDPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SDPA_OK = 0,
  SDPA_ERR_INVALID_ARGUMENT = 1,   /* malformed problem or pointer */
  SDPA_ERR_UNSUPPORTED = 2,        /* well-formed but outside what the kernels cover */
  SDPA_ERR_WORKSPACE_TOO_SMALL = 3,
  SDPA_ERR_HIP = 4                 /* a launch failed; see sdpa_last_error() */
} sdpa_status;

typedef enum { SDPA_DTYPE_F32 = 0, SDPA_DTYPE_BF16 = 1 } sdpa_dtype;
/* values of sdpa_problem.is_causal */
typedef enum { SDPA_CAUSAL_NONE = 0, SDPA_CAUSAL_TOP_LEFT = 1, SDPA_CAUSAL_BOTTOM_RIGHT = 2 } sdpa_causal;

typedef struct {
  int32_t dtype;                    /* sdpa_dtype */
  int32_t B, Hq, Hkv, Lq, Lk, Dqk, Dv;
  int64_t q_stride[3];              /* (b, h, l) element strides of q (and dq) */
  int64_t k_stride[3];              /* of k (and dk) */
  int64_t v_stride[3];              /* of v (and dv) */
  int64_t o_stride[3];              /* of o (and dO) */
  int64_t mask_stride[3];           /* (b, h, i) of the mask; keys have unit stride */
  float scale;                      /* NaN selects 1/sqrt(Dqk); else finite and > 0 */
  int32_t is_causal;                /* 0 none, 1 top-left, 2 bottom-right (see above) */
  int32_t sliding_window;           /* 0 none; W > 0 needs is_causal 1 or 2 (see above) */
} sdpa_problem;

/*
 * Supported by the kernels (SDPA_ERR_UNSUPPORTED otherwise):
 *   bf16: Dqk == Dv in {64, 128};  fp32: Dqk == Dv in {32, 64, 128}.
 *   bf16: q/k/v/o (and dO, dq, dk, dv) base pointers 16-byte aligned and their (b, h, l)
 *   strides multiples of 8 elements along every dimension of size > 1; row strides (l, and
 *   the mask's i) below 2^24 elements.  fp32: 4-byte aligned, any strides.
 *   The mask may have any (b, h, i) strides (16-byte copies are used when its rows allow).
 */

/* Device workspace (bytes) the forward needs: 0 for prefill; split-KV partial results
 * when Lq == 1 (decode).  The caller allocates it; it may be reused after the call's
 * work on the stream has finished. */
size_t sdpa_forward_workspace_bytes(const sdpa_problem* p);

/* Device workspace (bytes) the backward takes: per query row, D = rowsum(dO o O) and
 * LSE * log2(e), both fp32; then, for bf16 at Dqk = Dv = 128 when it stays within 8 GiB, a
 * buffer of bf16 dS blocks.  With that buffer, sdpa_backward (and sdpa_backward_main)
 * write dS = P o (dP - D) from the dK/dV pass, rounded to bf16 as the dK and dQ products
 * take it, and form dQ = scale dS K from it instead of recomputing S, P and dP in a second
 * pass (tinyllm L5.1 section 2.3 gives dQ = scale dS K; cuDNN "Attention", SDPA FP16/BF16
 * Backward, lists a backward workspace).  Buffer size: 2 KB per 32 x 32 block of every
 * (batch, query head), i.e. B * Hq * 2ceil(Lq/64) * 4ceil(Lk/128) * 2048 bytes.  The
 * result stays deterministic. */
size_t sdpa_backward_workspace_bytes(const sdpa_problem* p);

/* The least workspace (bytes) the backward accepts: the per-row values alone.  A workspace
 * smaller than sdpa_backward_workspace_bytes runs dQ as its own pass, which recomputes
 * S, P and dP (the same gradients within rounding: the fp32 accumulation order of dQ
 * differs). */
size_t sdpa_backward_workspace_bytes_min(const sdpa_problem* p);

/*
 * Forward.  q (B,Hq,Lq,Dqk), k (B,Hkv,Lk,Dqk), v (B,Hkv,Lk,Dv), o (B,Hq,Lq,Dv) in the io
 * dtype; lse (B,Hq,Lq) fp32 (may be NULL when not wanted); mask_or_null additive;
 * seq_lens_q_or_null / seq_lens_kv_or_null (B) int32 device arrays.  O and LSE are fully
 * written, including zeros / -inf for empty rows.  The result is bitwise repeatable.
 */
sdpa_status sdpa_forward(const sdpa_problem* p, const void* q, const void* k, const void* v,
                         const void* mask_or_null, const int32_t* seq_lens_q_or_null,
                         const int32_t* seq_lens_kv_or_null, void* o, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * The forward without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Arguments and results are those of sdpa_forward; where sdpa_forward needs a
 * workspace (the single-query decode's split partial results), this call uses a scratch
 * array built into the library instead: 16 MiB of device memory per GPU, held from the
 * first call on that GPU until the process ends.  It allocates nothing, neither on the host
 * nor on the device.
 *   Limit: a problem whose sdpa_forward_workspace_bytes exceeds 16 MiB (decode partials of
 *   more than about 32k (batch, query head, split) rows at D = 128) is rejected with
 *   SDPA_ERR_UNSUPPORTED before anything is launched.
 *   Every call on one GPU shares that GPU's scratch, which keeps the last call's contents:
 *   calls that overlap on one GPU (on different streams) race and must be ordered by the
 *   caller.  Calls on the same stream are ordered by the stream.
 */
sdpa_status sdpa_forward_noalloc(const sdpa_problem* p, const void* q, const void* k, const void* v,
                                 const void* mask_or_null, const int32_t* seq_lens_q_or_null,
                                 const int32_t* seq_lens_kv_or_null, void* o, float* lse,
                                 void* stream);

/*
 * Backward.  Takes the forward's o and lse (same problem, mask, causal flag and lengths)
 * and dO (B,Hq,Lq,Dv); writes dq, dk, dv (shapes and strides of q, k, v).  Every element
 * of dq, dk, dv is written (zeros where no gradient flows).  Deterministic: no atomics.
 */
sdpa_status sdpa_backward(const sdpa_problem* p, const void* q, const void* k, const void* v,
                          const void* o, const void* dO, const float* lse,
                          const void* mask_or_null, const int32_t* seq_lens_q_or_null,
                          const int32_t* seq_lens_kv_or_null, void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * The stages sdpa_backward runs, for callers that schedule them themselves.  Same
 * arguments, validation and workspace as sdpa_backward.
 *   prep: D_i = rowsum(dO o O)_i and LSE_i * log2(e) (fp32, into the workspace; D = 0 and
 *         +inf for empty rows);
 *   dkdv: dK and dV (reads D from the workspace; stores dS when the workspace holds the
 *         dS buffer);
 *   dq:   dQ       (reads D from the workspace; with the dS buffer, reads the dS that dkdv
 *         stored).
 *   main: dkdv and dq in one call (after prep), which is what sdpa_backward runs after its
 *         prep: at d = 64 without a mask the two passes share one launch, dQ work filling
 *         the CUs that the dK/dV work leaves idle; at d = 128 with the dS buffer, dkdv
 *         storing dS, then dQ from it; otherwise dkdv then dq.
 * With the dS buffer in the workspace (sdpa_backward_workspace_bytes at d = 128), dq must
 * follow dkdv on the same workspace.  With the least workspace
 * (sdpa_backward_workspace_bytes_min), dkdv and dq are independent of each other once prep
 * has finished and may run concurrently on two streams.  Source: the backward of tinyllm L5.1 section 2.3, with D
 * computed from the output as that section's identity D_i = dO_i . o_i allows.
 */
sdpa_status sdpa_backward_prep(const sdpa_problem* p, const void* q, const void* k,
                               const void* v, const void* o, const void* dO, const float* lse,
                               const void* mask_or_null, const int32_t* seq_lens_q_or_null,
                               const int32_t* seq_lens_kv_or_null, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, void* stream);
sdpa_status sdpa_backward_dkdv(const sdpa_problem* p, const void* q, const void* k,
                               const void* v, const void* o, const void* dO, const float* lse,
                               const void* mask_or_null, const int32_t* seq_lens_q_or_null,
                               const int32_t* seq_lens_kv_or_null, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, void* stream);
sdpa_status sdpa_backward_dq(const sdpa_problem* p, const void* q, const void* k,
                             const void* v, const void* o, const void* dO, const float* lse,
                             const void* mask_or_null, const int32_t* seq_lens_q_or_null,
                             const int32_t* seq_lens_kv_or_null, void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, void* stream);
sdpa_status sdpa_backward_main(const sdpa_problem* p, const void* q, const void* k,
                               const void* v, const void* o, const void* dO, const float* lse,
                               const void* mask_or_null, const int32_t* seq_lens_q_or_null,
                               const int32_t* seq_lens_kv_or_null, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Ragged (packed) sequences.  The operation and every argument shared with sdpa_forward /
 * sdpa_backward are theirs; what changes is where a batch's rows live.  Variable-length
 * sequences are stored one after another without padding, the THD layout (cuDNN
 * "Attention", Support Matrix glossary note 3, Ragged Layout): with offsets_q,
 *   q[b, h, i, :] is row offsets_q[b] + i of the packed tensor, at element offset
 *   (offsets_q[b] + i) * q_stride[2] + h * q_stride[1],
 * likewise o, dO and dq with their own row stride (o_stride[2]); with offsets_kv the same
 * for k, v, dk, dv.  The batch strides of a ragged side are ignored.  Either side may be
 * ragged alone (the other keeps its (b, h, l) strides).
 *   offsets_q, offsets_kv: (B + 1) int32 device arrays of starting ROWS (tokens), not
 *   elements: the page's offsets divided by the row stride, which this layout takes per
 *   tensor (the page's offset multiplier).  NULL = that side is padded; at least one is
 *   non-NULL.
 *   Lengths: seq_lens_q / seq_lens_kv when given (batches may then leave gaps between them,
 *   the page's partially packed layout), else offsets[b + 1] - offsets[b], the cumulative
 *   sequence lengths of a fully packed batch.  Lq, Lk are the maximum lengths: longer
 *   batches are cut to Lq, Lk rows.
 *   Output rows of a ragged side are written only for each batch's valid rows (a gap row
 *   is the caller's and is left as it is); lse stays padded (B, Hq, Lq), -inf past a
 *   batch's length; the mask, when given, is the padded (B, Hq, Lq, Lk) one; the workspace
 *   is the one sdpa_forward_workspace_bytes / sdpa_backward_workspace_bytes give for p.
 * Device-resident preconditions (not checked): offsets non-decreasing within the packed
 * tensors, and every batch's rows inside them.  Bitwise equal to the padded entry points
 * on the same data.
 */
sdpa_status sdpa_forward_ragged(const sdpa_problem* p, const void* q, const void* k,
                                const void* v, const void* mask_or_null,
                                const int32_t* seq_lens_q_or_null,
                                const int32_t* seq_lens_kv_or_null, const int32_t* offsets_q,
                                const int32_t* offsets_kv, void* o, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream);
sdpa_status sdpa_backward_ragged(const sdpa_problem* p, const void* q, const void* k,
                                 const void* v, const void* o, const void* dO, const float* lse,
                                 const void* mask_or_null, const int32_t* seq_lens_q_or_null,
                                 const int32_t* seq_lens_kv_or_null, const int32_t* offsets_q,
                                 const int32_t* offsets_kv, void* dq, void* dk, void* dv,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Single-query decode against a paged KV cache.  The operation is that of sdpa_forward with
 * Lq = 1, no mask, not causal (equivalently the bottom-right diagonal, which leaves every
 * cached key visible), with per-batch KV lengths; only the cache's storage differs.  The
 * keys and values of sequence b live in fixed-size pages of two containers, located through
 * a page table (cuDNN "Attention", forward Configurable Options, Paged attention, offset
 * calculation):
 *   K_cache[b, h, s, d] = k_pages[page_table[b, s / page_size], h, s mod page_size, d]
 *   V_cache[b, h, s, d] = v_pages[page_table[b, s / page_size], h, s mod page_size, d]
 * for s < seq_lens_kv[b].  sliding_window = W > 0 restricts the query to the keys
 * s >= seq_lens_kv[b] - W (the sliding window of sdpa_problem on the bottom-right diagonal,
 * which for one query row ends at the last key).
 *   q (B, Hq, D), o (B, Hq, D) bf16 with (b, h) strides; lse (B, Hq) fp32 or NULL;
 *   k_pages, v_pages (num_pages, Hkv, page_size, D) bf16 with (page, h, s) strides;
 *   page_table (B, max_pages) int32 device array, row-major; seq_lens_kv (B) int32 device
 *   array, 0 <= len <= max_pages * page_size.
 * Device-resident preconditions are not checked: a page-table entry outside
 * [0, num_pages) is clamped into it (the result is then meaningless, but no memory outside
 * the containers is read).  A length of 0 gives O = 0, LSE = -inf.  Bitwise repeatable,
 * and bitwise equal to sdpa_forward on the same cache stored contiguously.
 */
typedef struct {
  int32_t B, Hq, Hkv, D;     /* bf16 only; D in {64, 128}; Hq % Hkv == 0, Hq / Hkv <= 16 */
  int32_t page_size;         /* keys per page: a positive multiple of 32 */
  int32_t num_pages;         /* pages in each container */
  int32_t max_pages;         /* page-table entries per sequence */
  int64_t q_stride[2];       /* (b, h) element strides of q */
  int64_t o_stride[2];       /* (b, h) element strides of o */
  int64_t k_stride[3];       /* (page, h, s) element strides of k_pages */
  int64_t v_stride[3];       /* (page, h, s) element strides of v_pages */
  float scale;               /* NaN selects 1/sqrt(D); else finite and > 0 */
  int32_t sliding_window;    /* 0 none; W > 0: only the last W keys of each sequence */
} sdpa_paged_decode;

/* Device workspace (bytes) of sdpa_decode_paged: the split-KV partial results. */
size_t sdpa_decode_paged_workspace_bytes(const sdpa_paged_decode* p);

sdpa_status sdpa_decode_paged(const sdpa_paged_decode* p, const void* q, const void* k_pages,
                              const void* v_pages, const int32_t* page_table,
                              const int32_t* seq_lens_kv, void* o, float* lse_or_null,
                              void* workspace, size_t workspace_bytes, void* stream);

const char* sdpa_status_string(sdpa_status s);

/* Text of the last failure on the calling thread ("" if none). */
const char* sdpa_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int sdpa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SDPA_H */
