// attn_f32.hip — fp32 forward and backward (accuracy path for fp32 inputs), gfx950.
//
// Same operation as the bf16 kernels, computed entirely in fp32 on the vector ALUs with
// one thread per query row (forward, dQ) or per key row (dK, dV).  Sources:
// "Scaled dot-product attention (forward and backward)", section 2 Principles (S, P, O),
// 2.2 Masking (-inf before the softmax, max subtracted, empty rows are zero) and 2.3 The
// backward pass (dV = P^T dO, dP = dO V^T, dS = P o (dP - D), dQ = a dS K, dK = a dS^T Q,
// D_i = dO_i . O_i).  The backward recomputes P_ij = exp(S_ij - LSE_i) from the forward's
// LSE, as the FlashAttention-2 row of that page's "Going further" table describes.
//
// A workgroup is one wave of 64 rows of one (batch, head) (keys of one (batch, KV head) for
// dK, dV).  The rows its 64 threads loop over (keys, or query rows) are the same for every
// thread, so they are staged through LDS in chunks and read back as broadcasts; each
// thread's arithmetic is the plain per-row definition (two passes for the forward: the row
// max, then the weights and the weighted sum).
#include "kern_common.h"
#include "launch.h"

namespace sdpa {
namespace {

constexpr int kTpb = 64;

// rows staged per chunk: 8 KB of fp32 per staged matrix
template <int D>
constexpr int chunk_rows() { return 2048 / D; }

struct RowCtx {
  int b, h, g, i;
  int q_end, kv_end;
  int start, stop;  // keys [start, stop) are visible (before the mask)
  int coff;         // causal diagonal offset: key j visible iff j <= i + coff
};

// First key row i sees under a sliding window of W keys (0 without one).
__device__ __forceinline__ int window_start(const Problem& p, int i, int coff) {
  return (p.causal && p.window > 0) ? max(0, i + coff - p.window + 1) : 0;
}

__device__ __forceinline__ RowCtx row_ctx(const Problem& p, int b, int h, int i) {
  RowCtx r;
  r.b = b;
  r.h = h;
  r.i = i;
  r.g = h / p.G;
  r.q_end = seq_len_q(p, b);
  r.kv_end = seq_len_kv(p, b);
  r.coff = causal_offset(p.causal, r.q_end, r.kv_end);
  r.stop = (i < r.q_end) ? (p.causal ? max(0, min(r.kv_end, i + 1 + r.coff)) : r.kv_end) : 0;
  r.start = window_start(p, i, r.coff);
  return r;
}

// Keys [block_start, block_stop) cover every key some row of the workgroup's block
// [i0, i0 + 64) can see (uniform).
__device__ __forceinline__ int block_start(const Problem& p, const RowCtx& r, int i0) {
  return window_start(p, i0, r.coff);
}
__device__ __forceinline__ int block_stop(const Problem& p, const RowCtx& r, int i0) {
  const int last = min(i0 + kTpb, r.q_end) - 1;
  if (last < i0) return 0;
  return p.causal ? max(0, min(r.kv_end, last + 1 + r.coff)) : r.kv_end;
}

// a . b over D elements as four interleaved partial sums (shorter dependency chains than
// one running sum; the four are added pairwise at the end)
template <int D>
__device__ __forceinline__ float dot4(const float* a, const float* b) {
  float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
  for (int t = 0; t < D; t += 4) {
    d0 = fmaf(a[t], b[t], d0);
    d1 = fmaf(a[t + 1], b[t + 1], d1);
    d2 = fmaf(a[t + 2], b[t + 2], d2);
    d3 = fmaf(a[t + 3], b[t + 3], d3);
  }
  return (d0 + d1) + (d2 + d3);
}

// Copy rows [j0, j0 + n) of a row-major fp32 matrix (row stride ld) into LDS rows of D.
template <int D>
__device__ __forceinline__ void stage_rows(float* dst, const float* src, int64_t ld, int j0, int n) {
  for (int e = threadIdx.x; e < n * D; e += kTpb) dst[e] = src[(int64_t)(j0 + e / D) * ld + e % D];
}

__device__ __forceinline__ float mask_at(const Problem& p, const RowCtx& r, int j) {
  const float* m = reinterpret_cast<const float*>(p.mask) + r.b * p.m_sb + r.h * p.m_sh +
                   (int64_t)r.i * p.m_si;
  return m[j];
}

// Score of (row, staged key row kj) in natural-log units (-inf where the mask blocks it).
template <int D>
__device__ __forceinline__ float score(const Problem& p, const RowCtx& r, const float* qv,
                                       const float* kj, int j) {
  float s = dot4<D>(qv, kj) * p.scale;
  if (p.mask) s += mask_at(p, r, j);
  return s;
}

// Workgroup -> (batch, head, first row) in a grid of n_rb row blocks per (batch, head).
__device__ __forceinline__ void block_rows(int n_rb, int H, int& b, int& h, int& i0) {
  const int bh = blockIdx.x / n_rb;
  i0 = (blockIdx.x - bh * n_rb) * kTpb;
  b = bh / H;
  h = bh - b * H;
}

template <int D>
__global__ __launch_bounds__(kTpb) void fwd_f32_kernel(FwdArgs a, int n_rb) {
  constexpr int CH = chunk_rows<D>();
  __shared__ float Ks[CH * D], Vs[CH * D];
  const Problem& p = a.p;
  int b, h, i0;
  block_rows(n_rb, p.Hq, b, h, i0);
  const int i = i0 + threadIdx.x;
  const RowCtx r = row_ctx(p, b, h, i);
  const int start_blk = block_start(p, r, i0), stop_blk = block_stop(p, r, i0);
  const bool live = i < r.q_end;
  const float* qrow = reinterpret_cast<const float*>(a.q) + q_base(p, b) + h * p.q_sh +
                      (int64_t)i * p.q_sl;
  const float* kbase = reinterpret_cast<const float*>(a.k) + k_base(p, b) + r.g * p.k_sh;
  const float* vbase = reinterpret_cast<const float*>(a.v) + v_base(p, b) + r.g * p.v_sh;
  float qv[D], acc[D];
#pragma unroll
  for (int t = 0; t < D; ++t) {
    qv[t] = live ? qrow[t] : 0.f;
    acc[t] = 0.f;
  }
  // pass 1: row max
  float m = kNegInf;
  for (int c0 = start_blk; c0 < stop_blk; c0 += CH) {
    const int n = min(CH, stop_blk - c0);
    __syncthreads();
    stage_rows<D>(Ks, kbase, p.k_sl, c0, n);
    __syncthreads();
    for (int jj = 0; jj < n; ++jj)
      if (c0 + jj >= r.start && c0 + jj < r.stop) m = fmaxf(m, score<D>(p, r, qv, Ks + jj * D, c0 + jj));
  }
  // pass 2: weights and weighted sum of values (a masked pair has weight exp(-inf) = 0)
  float l = 0.f;
  for (int c0 = start_blk; c0 < stop_blk; c0 += CH) {
    const int n = min(CH, stop_blk - c0);
    __syncthreads();
    stage_rows<D>(Ks, kbase, p.k_sl, c0, n);
    stage_rows<D>(Vs, vbase, p.v_sl, c0, n);
    __syncthreads();
    if (m == kNegInf) continue;
    for (int jj = 0; jj < n; ++jj) {
      if (c0 + jj < r.start || c0 + jj >= r.stop) continue;
      const float e = expf(score<D>(p, r, qv, Ks + jj * D, c0 + jj) - m);
      l += e;
      const float* vj = Vs + jj * D;
#pragma unroll
      for (int t = 0; t < D; ++t) acc[t] = fmaf(e, vj[t], acc[t]);
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (i < q_rows_out(p, r.q_end)) {
    float* orow = reinterpret_cast<float*>(a.o) + o_base(p, b) + h * p.o_sh + (int64_t)i * p.o_sl;
#pragma unroll
    for (int t = 0; t < D; ++t) orow[t] = acc[t] * inv;
  }
  if (a.lse && i < p.Lq) a.lse[((int64_t)b * p.Hq + h) * p.Lq + i] = l > 0.f ? m + logf(l) : kNegInf;
}

// D_i = dO_i . O_i: one thread per query row (0 for empty rows).
template <int D>
__global__ __launch_bounds__(kTpb) void bwd_prep_f32_kernel(BwdArgs a, int n_rb) {
  const Problem& p = a.p;
  int b, h, i0;
  block_rows(n_rb, p.Hq, b, h, i0);
  const int i = i0 + threadIdx.x;
  if (i >= p.Lq) return;
  const int q_end = seq_len_q(p, b);
  float Di = 0.f;
  if (i < q_end) {
    const int64_t ooff = o_base(p, b) + h * p.o_sh + (int64_t)i * p.o_sl;
    const float* orow = reinterpret_cast<const float*>(a.o) + ooff;
    const float* drow = reinterpret_cast<const float*>(a.dO) + ooff;
#pragma unroll
    for (int t = 0; t < D; ++t) Di = fmaf(drow[t], orow[t], Di);
  }
  a.dsum[((int64_t)b * p.Hq + h) * p.Lq + i] = Di;
}

// dQ_i: one thread per query row.
template <int D>
__global__ __launch_bounds__(kTpb) void bwd_dq_f32_kernel(BwdArgs a, int n_rb) {
  constexpr int CH = chunk_rows<D>();
  __shared__ float Ks[CH * D], Vs[CH * D];
  const Problem& p = a.p;
  int b, h, i0;
  block_rows(n_rb, p.Hq, b, h, i0);
  const int i = i0 + threadIdx.x;
  const RowCtx r = row_ctx(p, b, h, i);
  const int start_blk = block_start(p, r, i0), stop_blk = block_stop(p, r, i0);
  const int64_t qoff = q_base(p, b) + h * p.q_sh + (int64_t)i * p.q_sl;
  const int64_t ooff = o_base(p, b) + h * p.o_sh + (int64_t)i * p.o_sl;
  const float* kbase = reinterpret_cast<const float*>(a.k) + k_base(p, b) + r.g * p.k_sh;
  const float* vbase = reinterpret_cast<const float*>(a.v) + v_base(p, b) + r.g * p.v_sh;
  float qv[D], dov[D], dq[D];
  const bool ok = i < r.q_end;
#pragma unroll
  for (int t = 0; t < D; ++t) {
    qv[t] = ok ? reinterpret_cast<const float*>(a.q)[qoff + t] : 0.f;
    dov[t] = ok ? reinterpret_cast<const float*>(a.dO)[ooff + t] : 0.f;
    dq[t] = 0.f;
  }
  const int64_t row = ((int64_t)b * p.Hq + h) * p.Lq + i;
  const float Di = ok ? a.dsum[row] : 0.f;
  const float lse = ok ? a.lse[row] : kNegInf;
  for (int c0 = start_blk; c0 < stop_blk; c0 += CH) {
    const int n = min(CH, stop_blk - c0);
    __syncthreads();
    stage_rows<D>(Ks, kbase, p.k_sl, c0, n);
    stage_rows<D>(Vs, vbase, p.v_sl, c0, n);
    __syncthreads();
    if (lse == kNegInf) continue;
    for (int jj = 0; jj < n; ++jj) {
      if (c0 + jj < r.start || c0 + jj >= r.stop) continue;
      const float* kj = Ks + jj * D;
      const float P = expf(score<D>(p, r, qv, kj, c0 + jj) - lse);  // 0 for a masked pair
      const float* vj = Vs + jj * D;
      const float dS = P * (dot4<D>(dov, vj) - Di);
#pragma unroll
      for (int t = 0; t < D; ++t) dq[t] = fmaf(dS, kj[t], dq[t]);
    }
  }
  if (i < q_rows_out(p, r.q_end)) {
    float* dqrow = reinterpret_cast<float*>(a.dq) + qoff;
#pragma unroll
    for (int t = 0; t < D; ++t) dqrow[t] = dq[t] * p.scale;
  }
}

// dK_j and dV_j: one thread per key row of a KV head, summing over the query heads it
// serves and over their rows.
template <int D>
__global__ __launch_bounds__(kTpb) void bwd_dkdv_f32_kernel(BwdArgs a, int n_kb) {
  constexpr int CH = chunk_rows<D>();
  __shared__ float Qs[CH * D], Gs[CH * D], Ls[CH], Ds[CH];
  const Problem& p = a.p;
  int b, g, j0;
  block_rows(n_kb, p.Hkv, b, g, j0);
  const int j = j0 + threadIdx.x;
  const int kv_end = seq_len_kv(p, b);
  const int q_end = seq_len_q(p, b);
  const int coff = causal_offset(p.causal, q_end, kv_end);
  const int64_t koff = k_base(p, b) + g * p.k_sh + (int64_t)j * p.k_sl;
  const int64_t voff = v_base(p, b) + g * p.v_sh + (int64_t)j * p.v_sl;
  const bool ok = j < kv_end;
  float kv[D], vv[D], dk[D], dv[D];
#pragma unroll
  for (int t = 0; t < D; ++t) {
    kv[t] = ok ? reinterpret_cast<const float*>(a.k)[koff + t] : 0.f;
    vv[t] = ok ? reinterpret_cast<const float*>(a.v)[voff + t] : 0.f;
    dk[t] = 0.f;
    dv[t] = 0.f;
  }
  // first query row that sees key j (row i sees it iff i >= j - offset); the block's first
  // key bounds the staged rows
  const int i_begin = p.causal ? max(0, j - coff) : 0;
  const int i_blk = p.causal ? max(0, j0 - coff) : 0;
  // under a sliding window of W keys row i sees key j only if i <= j - coff + W - 1
  const bool win = p.causal && p.window > 0;
  const int i_stop = win ? min(q_end, max(j - coff + p.window, 0)) : q_end;
  const int i_stop_blk = win ? min(q_end, max(min(j0 + kTpb, kv_end) - 1 - coff + p.window, 0)) : q_end;
  if (j0 < kv_end) {
    for (int hh = 0; hh < p.G; ++hh) {
      const int h = g * p.G + hh;
      const float* qb = reinterpret_cast<const float*>(a.q) + q_base(p, b) + h * p.q_sh;
      const float* gb = reinterpret_cast<const float*>(a.dO) + o_base(p, b) + h * p.o_sh;
      const int64_t rb = ((int64_t)b * p.Hq + h) * p.Lq;
      const float* mrow = p.mask ? reinterpret_cast<const float*>(p.mask) + b * p.m_sb + h * p.m_sh
                                 : nullptr;
      for (int c0 = i_blk; c0 < i_stop_blk; c0 += CH) {
        const int n = min(CH, i_stop_blk - c0);
        __syncthreads();
        stage_rows<D>(Qs, qb, p.q_sl, c0, n);
        stage_rows<D>(Gs, gb, p.o_sl, c0, n);
        for (int e = threadIdx.x; e < n; e += kTpb) {
          Ls[e] = a.lse[rb + c0 + e];
          Ds[e] = a.dsum[rb + c0 + e];
        }
        __syncthreads();
        if (!ok) continue;
        for (int ii = 0; ii < n; ++ii) {
          const int i = c0 + ii;
          if (i < i_begin || i >= i_stop) continue;
          const float lse = Ls[ii];
          const float* qi = Qs + ii * D;
          const float* doi = Gs + ii * D;
          float s = dot4<D>(qi, kv) * p.scale;
          if (mrow) s += mrow[(int64_t)i * p.m_si + j];
          // a row with no visible key (LSE = -inf) or a masked pair gets P = 0
          const float P = (lse == kNegInf || s == kNegInf) ? 0.f : expf(s - lse);
          const float dS = P * (dot4<D>(doi, vv) - Ds[ii]);
#pragma unroll
          for (int t = 0; t < D; ++t) {
            dv[t] = fmaf(P, doi[t], dv[t]);
            dk[t] = fmaf(dS, qi[t], dk[t]);
          }
        }
      }
    }
  }
  if (j < kv_rows_out(p, kv_end)) {
    float* dkrow = reinterpret_cast<float*>(a.dk) + koff;
    float* dvrow = reinterpret_cast<float*>(a.dv) + voff;
#pragma unroll
    for (int t = 0; t < D; ++t) {
      dkrow[t] = dk[t] * p.scale;
      dvrow[t] = dv[t];
    }
  }
}

template <int D>
hipError_t fwd_d(const FwdArgs& a, hipStream_t s) {
  const int n_rb = (a.p.Lq + kTpb - 1) / kTpb;
  const int64_t grid = (int64_t)n_rb * a.p.B * a.p.Hq;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3((unsigned)grid), dim3(kTpb), 0, s, a, n_rb);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(const BwdArgs& a, int stages, hipStream_t s) {
  const int n_rb = (a.p.Lq + kTpb - 1) / kTpb, n_kb = (a.p.Lk + kTpb - 1) / kTpb;
  const int64_t qgrid = (int64_t)n_rb * a.p.B * a.p.Hq, kgrid = (int64_t)n_kb * a.p.B * a.p.Hkv;
  if ((stages & kBwdPrep) && qgrid > 0) {
    hipLaunchKernelGGL((bwd_prep_f32_kernel<D>), dim3((unsigned)qgrid), dim3(kTpb), 0, s, a, n_rb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((stages & kBwdDkdv) && kgrid > 0) {
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D>), dim3((unsigned)kgrid), dim3(kTpb), 0, s, a, n_kb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((stages & kBwdDq) && qgrid > 0) {
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D>), dim3((unsigned)qgrid), dim3(kTpb), 0, s, a, n_rb);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  switch (a.p.D) {
    case 32: return fwd_d<32>(a, s);
    case 64: return fwd_d<64>(a, s);
    case 128: return fwd_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_f32(const BwdArgs& a, int stages, hipStream_t s) {
  switch (a.p.D) {
    case 32: return bwd_d<32>(a, stages, s);
    case 64: return bwd_d<64>(a, stages, s);
    case 128: return bwd_d<128>(a, stages, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdpa
