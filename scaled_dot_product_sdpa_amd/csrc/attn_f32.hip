// attn_f32.hip — fp32 forward and backward (accuracy path for fp32 inputs), gfx950.
//
// Same operation as the bf16 kernels, computed entirely in fp32 on the vector ALUs with
// one thread per query row (forward, dQ) or per key row (dK, dV).  Sources:
// "Scaled dot-product attention (forward and backward)", section 2 Principles (S, P, O),
// 2.2 Masking (-inf before the softmax, max subtracted, empty rows are zero) and 2.3 The
// backward pass (dV = P^T dO, dP = dO V^T, dS = P o (dP - D), dQ = a dS K, dK = a dS^T Q,
// D_i = dO_i . O_i).  The backward recomputes P_ij = exp(S_ij - LSE_i) from the forward's
// LSE, as the FlashAttention-2 row of that page's "Going further" table describes.
#include "kern_common.h"
#include "launch.h"

namespace sdpa {
namespace {

constexpr int kTpb = 64;

struct RowCtx {
  int b, h, g, i;
  int q_end, kv_end, stop;  // stop: keys [0, stop) are candidates
  int coff;                 // causal diagonal offset: key j visible iff j <= i + coff
};

__device__ __forceinline__ bool key_visible(const Problem& p, const RowCtx& r, int j) {
  return j < r.kv_end && r.i < r.q_end && (!p.causal || j <= r.i + r.coff);
}

__device__ __forceinline__ RowCtx row_ctx(const Problem& p, int64_t row) {
  RowCtx r;
  r.i = (int)(row % p.Lq);
  r.h = (int)((row / p.Lq) % p.Hq);
  r.b = (int)(row / ((int64_t)p.Lq * p.Hq));
  r.g = r.h / p.G;
  r.q_end = seq_len_q(p, r.b);
  r.kv_end = seq_len_kv(p, r.b);
  r.coff = causal_offset(p.causal, r.q_end, r.kv_end);
  r.stop = (r.i < r.q_end) ? (p.causal ? max(0, min(r.kv_end, r.i + 1 + r.coff)) : r.kv_end) : 0;
  return r;
}

// Score of (row, key j) in natural-log units, -inf if the pair is blocked.
template <int D>
__device__ __forceinline__ float score(const Problem& p, const RowCtx& r, const float* qv,
                                       const float* kbase, int j) {
  if (!key_visible(p, r, j)) return kNegInf;
  const float* kj = kbase + (int64_t)j * p.k_sl;
  float dot = 0.f;
#pragma unroll
  for (int t = 0; t < D; ++t) dot = fmaf(qv[t], kj[t], dot);
  float s = dot * p.scale;
  if (p.mask) {
    const float* m = reinterpret_cast<const float*>(p.mask) + r.b * p.m_sb + r.h * p.m_sh +
                     (int64_t)r.i * p.m_si;
    s += m[j];
  }
  return s;
}

template <int D>
__global__ __launch_bounds__(kTpb) void fwd_f32_kernel(FwdArgs a) {
  const Problem& p = a.p;
  const int64_t row = (int64_t)blockIdx.x * kTpb + threadIdx.x;
  if (row >= (int64_t)p.B * p.Hq * p.Lq) return;
  const RowCtx r = row_ctx(p, row);
  const float* qrow = reinterpret_cast<const float*>(a.q) + q_base(p, r.b) + r.h * p.q_sh +
                      (int64_t)r.i * p.q_sl;
  const float* kbase = reinterpret_cast<const float*>(a.k) + k_base(p, r.b) + r.g * p.k_sh;
  const float* vbase = reinterpret_cast<const float*>(a.v) + v_base(p, r.b) + r.g * p.v_sh;
  float qv[D], acc[D];
#pragma unroll
  for (int t = 0; t < D; ++t) {
    qv[t] = (r.i < r.q_end) ? qrow[t] : 0.f;
    acc[t] = 0.f;
  }
  // pass 1: row max
  float m = kNegInf;
  for (int j = 0; j < r.stop; ++j) m = fmaxf(m, score<D>(p, r, qv, kbase, j));
  // pass 2: weights and weighted sum of values
  float l = 0.f;
  if (m != kNegInf) {
    for (int j = 0; j < r.stop; ++j) {
      const float s = score<D>(p, r, qv, kbase, j);
      if (s == kNegInf) continue;
      const float e = expf(s - m);
      l += e;
      const float* vj = vbase + (int64_t)j * p.v_sl;
#pragma unroll
      for (int t = 0; t < D; ++t) acc[t] = fmaf(e, vj[t], acc[t]);
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (r.i < q_rows_out(p, r.q_end)) {
    float* orow = reinterpret_cast<float*>(a.o) + o_base(p, r.b) + r.h * p.o_sh + (int64_t)r.i * p.o_sl;
#pragma unroll
    for (int t = 0; t < D; ++t) orow[t] = acc[t] * inv;
  }
  if (a.lse) a.lse[row] = l > 0.f ? m + logf(l) : kNegInf;
}

// D_i = dO_i . O_i: one thread per query row (0 for empty rows).
template <int D>
__global__ __launch_bounds__(kTpb) void bwd_prep_f32_kernel(BwdArgs a) {
  const Problem& p = a.p;
  const int64_t row = (int64_t)blockIdx.x * kTpb + threadIdx.x;
  if (row >= (int64_t)p.B * p.Hq * p.Lq) return;
  const RowCtx r = row_ctx(p, row);
  float Di = 0.f;
  if (r.i < r.q_end) {
    const int64_t ooff = o_base(p, r.b) + r.h * p.o_sh + (int64_t)r.i * p.o_sl;
    const float* orow = reinterpret_cast<const float*>(a.o) + ooff;
    const float* drow = reinterpret_cast<const float*>(a.dO) + ooff;
#pragma unroll
    for (int t = 0; t < D; ++t) Di = fmaf(drow[t], orow[t], Di);
  }
  a.dsum[row] = Di;
}

// dQ_i: one thread per query row.
template <int D>
__global__ __launch_bounds__(kTpb) void bwd_dq_f32_kernel(BwdArgs a) {
  const Problem& p = a.p;
  const int64_t row = (int64_t)blockIdx.x * kTpb + threadIdx.x;
  if (row >= (int64_t)p.B * p.Hq * p.Lq) return;
  const RowCtx r = row_ctx(p, row);
  const int64_t qoff = q_base(p, r.b) + r.h * p.q_sh + (int64_t)r.i * p.q_sl;
  const int64_t ooff = o_base(p, r.b) + r.h * p.o_sh + (int64_t)r.i * p.o_sl;
  const float* kbase = reinterpret_cast<const float*>(a.k) + k_base(p, r.b) + r.g * p.k_sh;
  const float* vbase = reinterpret_cast<const float*>(a.v) + v_base(p, r.b) + r.g * p.v_sh;
  float qv[D], dov[D], dq[D];
  const bool ok = r.i < r.q_end;
#pragma unroll
  for (int t = 0; t < D; ++t) {
    qv[t] = ok ? reinterpret_cast<const float*>(a.q)[qoff + t] : 0.f;
    dov[t] = ok ? reinterpret_cast<const float*>(a.dO)[ooff + t] : 0.f;
    dq[t] = 0.f;
  }
  const float Di = a.dsum[row];
  const float lse = a.lse[row];
  if (ok && lse != kNegInf) {
    for (int j = 0; j < r.stop; ++j) {
      const float s = score<D>(p, r, qv, kbase, j);
      if (s == kNegInf) continue;
      const float P = expf(s - lse);
      const float* vj = vbase + (int64_t)j * p.v_sl;
      float dP = 0.f;
#pragma unroll
      for (int t = 0; t < D; ++t) dP = fmaf(dov[t], vj[t], dP);
      const float dS = P * (dP - Di);
      const float* kj = kbase + (int64_t)j * p.k_sl;
#pragma unroll
      for (int t = 0; t < D; ++t) dq[t] = fmaf(dS, kj[t], dq[t]);
    }
  }
  if (r.i < q_rows_out(p, r.q_end)) {
    float* dqrow = reinterpret_cast<float*>(a.dq) + qoff;
#pragma unroll
    for (int t = 0; t < D; ++t) dqrow[t] = dq[t] * p.scale;
  }
}

// dK_j and dV_j: one thread per key row of a KV head, summing over the query heads it
// serves and over their rows.
template <int D>
__global__ __launch_bounds__(kTpb) void bwd_dkdv_f32_kernel(BwdArgs a) {
  const Problem& p = a.p;
  const int64_t krow = (int64_t)blockIdx.x * kTpb + threadIdx.x;
  if (krow >= (int64_t)p.B * p.Hkv * p.Lk) return;
  const int j = (int)(krow % p.Lk);
  const int g = (int)((krow / p.Lk) % p.Hkv);
  const int b = (int)(krow / ((int64_t)p.Lk * p.Hkv));
  const int kv_end = seq_len_kv(p, b);
  const int q_end = seq_len_q(p, b);
  const int64_t koff = k_base(p, b) + g * p.k_sh + (int64_t)j * p.k_sl;
  const int64_t voff = v_base(p, b) + g * p.v_sh + (int64_t)j * p.v_sl;
  float kv[D], vv[D], dk[D], dv[D];
#pragma unroll
  for (int t = 0; t < D; ++t) {
    const bool ok = j < kv_end;
    kv[t] = ok ? reinterpret_cast<const float*>(a.k)[koff + t] : 0.f;
    vv[t] = ok ? reinterpret_cast<const float*>(a.v)[voff + t] : 0.f;
    dk[t] = 0.f;
    dv[t] = 0.f;
  }
  if (j < kv_end) {
    // first query row that sees key j (row i sees it iff i >= j - offset)
    const int i_begin = p.causal ? max(0, j - causal_offset(p.causal, q_end, kv_end)) : 0;
    for (int hh = 0; hh < p.G; ++hh) {
      const int h = g * p.G + hh;
      for (int i = i_begin; i < q_end; ++i) {
        const int64_t row = ((int64_t)b * p.Hq + h) * p.Lq + i;
        const float lse = a.lse[row];
        if (lse == kNegInf) continue;
        const float* qi = reinterpret_cast<const float*>(a.q) + q_base(p, b) + h * p.q_sh + (int64_t)i * p.q_sl;
        const float* doi = reinterpret_cast<const float*>(a.dO) + o_base(p, b) + h * p.o_sh + (int64_t)i * p.o_sl;
        float dot = 0.f;
#pragma unroll
        for (int t = 0; t < D; ++t) dot = fmaf(qi[t], kv[t], dot);
        float s = dot * p.scale;
        if (p.mask) {
          const float* m = reinterpret_cast<const float*>(p.mask) + b * p.m_sb + h * p.m_sh + (int64_t)i * p.m_si;
          s += m[j];
        }
        if (s == kNegInf) continue;
        const float P = expf(s - lse);
        float dP = 0.f;
#pragma unroll
        for (int t = 0; t < D; ++t) dP = fmaf(doi[t], vv[t], dP);
        const float dS = P * (dP - a.dsum[row]);
#pragma unroll
        for (int t = 0; t < D; ++t) {
          dv[t] = fmaf(P, doi[t], dv[t]);
          dk[t] = fmaf(dS, qi[t], dk[t]);
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
  const int64_t rows = (int64_t)a.p.B * a.p.Hq * a.p.Lq;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3((unsigned)((rows + kTpb - 1) / kTpb)), dim3(kTpb), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(const BwdArgs& a, int stages, hipStream_t s) {
  const int64_t qrows = (int64_t)a.p.B * a.p.Hq * a.p.Lq;
  const int64_t krows = (int64_t)a.p.B * a.p.Hkv * a.p.Lk;
  const dim3 qgrid((unsigned)((qrows + kTpb - 1) / kTpb)), kgrid((unsigned)((krows + kTpb - 1) / kTpb));
  if ((stages & kBwdPrep) && qrows > 0) {
    hipLaunchKernelGGL((bwd_prep_f32_kernel<D>), qgrid, dim3(kTpb), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((stages & kBwdDkdv) && krows > 0) {
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D>), kgrid, dim3(kTpb), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((stages & kBwdDq) && qrows > 0) {
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D>), qgrid, dim3(kTpb), 0, s, a);
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
