// fwd_bf16.hip — prefill forward, bf16 in / fp32 accumulate, gfx950.
//
// Computes O = softmax(scale * Q K^T + mask) V and LSE per row ("Scaled dot-product
// attention (forward and backward)", section 2 Principles and 2.2 Masking; LSE as in
// cuDNN "Attention", SDPA FP16/BF16 Forward, Python API return values) with the
// one-pass online softmax (running max and sum; the page's "Going further" table names
// Milakov and Gimelshein's online normaliser).
//
// Work decomposition: one workgroup = 4 waves = BM query rows of one (batch, head); each
// wave owns NQB blocks of 32 query rows and keeps their Q operand, O accumulator and
// running max / sum in registers.  K/V tiles of BN = 64 keys stream through LDS
// (coalesced 16-byte loads, prefetched into registers one tile ahead).
//
//   S^T = K Q^T   (keys x queries): A = K rows from LDS (row-permuted, see kern_common.h),
//                 B = Q held in registers; lane l ends up with 16 consecutive keys of
//                 query l%32, so the row max needs one in-register reduction plus one
//                 permlane32 swap, and the row sum is kept per half-wave until the end.
//   O^T += V^T P^T (d x queries): A = V^T read with ds_read_b64_tr_b16, B = bf16(P) taken
//                 straight from the S accumulator registers.  O^T keeps one query per
//                 lane, so the rescale by exp(m_old - m_new) is a per-lane multiply.
//
// Scores are kept in log2 units (scale * log2 e folded into one multiply) and
// exponentiated with v_exp_f32.  Tiles entirely above the causal diagonal or past the
// key length are never visited; only tiles touching the diagonal or a length boundary
// evaluate per-element predicates.  Rows with no visible key produce O = 0, LSE = -inf.
// The output is normalised by the sum of the bf16-rounded weights actually fed to the
// PV product, so each output row is an exact convex combination of value rows.
#include "kern_common.h"
#include "launch.h"

namespace sdpa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;  // keys per K/V tile (two 32-key MFMA blocks)

template <int D>
struct FwdTile {
  static constexpr int KP = D + 8;  // LDS row pitch of the K tile (elements)
  static constexpr int VP = D + 8;  // LDS row pitch of the V tile (elements)
  static constexpr int CPR = D / 8; // 16-byte chunks per row
  static constexpr int NCH = kBN * CPR / kThreads;  // chunks per thread per tensor
};

template <int D, int NQB, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(FwdArgs a) {
  using T = FwdTile<D>;
  constexpr int BM = kWaves * 32 * NQB;
  __shared__ __attribute__((aligned(16))) bf16 Ks[kBN * T::KP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[kBN * T::VP];

  const Problem& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;  // which half of the wave

  // ---- work item: heavy causal tiles first; the heads of one KV group are adjacent.
  const int n_qt = (p.Lq + BM - 1) / BM;
  const int bh_count = p.B * p.Hq;
  const int rank = blockIdx.x / bh_count;
  const int bh = blockIdx.x % bh_count;
  const int qt = CAUSAL ? (n_qt - 1 - rank) : rank;
  const int b = bh / p.Hq;
  const int h = bh % p.Hq;
  const int g = h / p.G;

  const int q_end = p.len_q ? min(p.len_q[b], p.Lq) : p.Lq;
  const int kv_end = p.len_kv ? min(p.len_kv[b], p.Lk) : p.Lk;
  const int i0 = qt * BM;

  const bf16* qb = reinterpret_cast<const bf16*>(a.q) + b * p.q_sb + h * p.q_sh;
  const bf16* kb_ = reinterpret_cast<const bf16*>(a.k) + b * p.k_sb + g * p.k_sh;
  const bf16* vb_ = reinterpret_cast<const bf16*>(a.v) + b * p.v_sb + g * p.v_sh;
  bf16* ob = reinterpret_cast<bf16*>(a.o) + b * p.o_sb + h * p.o_sh;
  const bf16* mb_ = MASK ? reinterpret_cast<const bf16*>(p.mask) + b * p.m_sb + h * p.m_sh : nullptr;
  float* lseb = a.lse ? a.lse + ((int64_t)b * p.Hq + h) * p.Lq : nullptr;

  // Keys this tile of queries can see.
  int kv_stop = kv_end;
  if (CAUSAL) kv_stop = min(kv_stop, min(i0 + BM, q_end));
  if (i0 >= q_end) kv_stop = 0;
  const int n_tiles = kv_stop > 0 ? (kv_stop + kBN - 1) / kBN : 0;

  // ---- Q operand (B of S^T = K Q^T): lane holds query row, 8 consecutive d per k-step.
  bf16x8 qreg[NQB][D / 16];
  int qrow[NQB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    qrow[nb] = i0 + wave * 32 * NQB + nb * 32 + l32;
    const bool ok = qrow[nb] < q_end;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 x = ok ? ld16(qb + (int64_t)qrow[nb] * p.q_sl + kk * 16 + 8 * hi) : zero16();
      qreg[nb][kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 oacc[NQB][D / 32];
  // running max (log2 units), sum of the bf16-rounded weights (normalises O) and sum of
  // the fp32 weights (gives LSE)
  float mrow[NQB], lrow[NQB], frow[NQB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    mrow[nb] = kNegInf;
    lrow[nb] = 0.f;
    frow[nb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[nb][mb] = f32x16{};
  }

  // ---- K/V tile staging: thread handles NCH 16-byte chunks of each tensor.
  u32x4 kst[T::NCH], vst[T::NCH];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int u = 0; u < T::NCH; ++u) {
      const int idx = tid + u * kThreads;
      const int r = idx / T::CPR, c = idx % T::CPR;
      const int row = j0 + r;
      const bool ok = row < kv_stop;
      kst[u] = ok ? ld16(kb_ + (int64_t)row * p.k_sl + c * 8) : zero16();
      vst[u] = ok ? ld16(vb_ + (int64_t)row * p.v_sl + c * 8) : zero16();
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < T::NCH; ++u) {
      const int idx = tid + u * kThreads;
      const int r = idx / T::CPR, c = idx % T::CPR;
      *reinterpret_cast<u32x4*>(&Ks[r * T::KP + c * 8]) = kst[u];
      *reinterpret_cast<u32x4*>(&Vs[r * T::VP + c * 8]) = vst[u];
    }
  };

  if (n_tiles > 0) load_tile(0);

  for (int t = 0; t < n_tiles; ++t) {
    const int j0 = t * kBN;
    store_tile();
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(j0 + kBN);

    // ---- S^T = K Q^T for the two 32-key blocks of the tile.
    f32x16 sacc[NQB][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) sacc[nb][kb] = f32x16{};
      const bf16* krow = &Ks[(kb * 32 + perm_row(l32)) * T::KP + 8 * hi];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        bf16x8 kop = *reinterpret_cast<const bf16x8*>(krow + kk * 16);
#pragma unroll
        for (int nb = 0; nb < NQB; ++nb) sacc[nb][kb] = mfma32(kop, qreg[nb][kk], sacc[nb][kb]);
      }
    }

    // ---- online softmax; lane holds keys j0 + kb*32 + 16*hi + v of query qrow[nb].
    const bool partial = (j0 + kBN > kv_end) || (CAUSAL && j0 + kBN - 1 > i0) ||
                         (i0 + BM > q_end);
    bf16x8 pop[NQB][2][2];
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
      const int qi = qrow[nb];
      float s[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key0 = j0 + kb * 32 + 16 * hi;
        float mv[16];
        if (MASK) {
          if (p.mask_vec && qi < q_end && key0 + 16 <= p.Lk) {
            const bf16* mp = mb_ + (int64_t)qi * p.m_si + key0;
            u32x4 m0 = ld16(mp), m1 = ld16(mp + 8);
            bf16x8 b0 = __builtin_bit_cast(bf16x8, m0), b1 = __builtin_bit_cast(bf16x8, m1);
#pragma unroll
            for (int v = 0; v < 8; ++v) { mv[v] = bf2f(b0[v]); mv[v + 8] = bf2f(b1[v]); }
          } else {
#pragma unroll
            for (int v = 0; v < 16; ++v)
              mv[v] = (qi < q_end && key0 + v < kv_end) ? bf2f(mb_[(int64_t)qi * p.m_si + key0 + v]) : 0.f;
          }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = sacc[nb][kb][v] * p.scale_log2;
          if (MASK) x += mv[v] * kLog2e;
          if (partial) {
            const int key = key0 + v;
            const bool ok = key < kv_end && qi < q_end && (!CAUSAL || key <= qi);
            x = ok ? x : kNegInf;
          }
          s[kb][v] = x;
        }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
      mx = xhalf_max(mx);
      const float m_new = fmaxf(mrow[nb], mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float corr = fast_exp2(mrow[nb] - m_use);
      mrow[nb] = m_new;
      float psum = 0.f, fsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 pb;
#pragma unroll
          for (int t8 = 0; t8 < 8; ++t8) {
            const float pf = fast_exp2(s[kb][half * 8 + t8] - m_use);
            const bf16 e = (bf16)pf;
            pb[t8] = e;
            psum += bf2f(e);
            fsum += pf;
          }
          pop[nb][kb][half] = pb;
        }
      }
      lrow[nb] = lrow[nb] * corr + psum;
      frow[nb] = frow[nb] * corr + fsum;
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) oacc[nb][mb] *= corr;
    }

    // ---- O^T += V^T P^T.  V^T operand via transposing LDS reads: lane (within its
    // 16-lane block) supplies row  key_base + (lane%16)/4, columns d_base + 4*(lane%4).
    {
      const int blk = lane >> 4;
      const int arow = (lane & 15) >> 2;
      const int acol = 4 * (lane & 3) + 16 * (blk & 1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const bf16* vrow = &Vs[(kb * 32 + 16 * hi + 8 * half + arow) * T::VP + acol];
#pragma unroll
          for (int mb = 0; mb < D / 32; ++mb) {
            i16x4 lo = lds_read_tr4(vrow + mb * 32);
            i16x4 hi4 = lds_read_tr4(vrow + 4 * T::VP + mb * 32);
            bf16x8 vop = join_tr(lo, hi4);
#pragma unroll
            for (int nb = 0; nb < NQB; ++nb) oacc[nb][mb] = mfma32(vop, pop[nb][kb][half], oacc[nb][mb]);
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l (0 for empty rows), LSE = ln2 * (m + log2 l).
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    const int qi = qrow[nb];
    const float lt = xhalf_sum(lrow[nb]);
    const float ft = xhalf_sum(frow[nb]);
    const bool live = qi < q_end && lt > 0.f;
    const float inv = live ? 1.f / lt : 0.f;
    if (qi < p.Lq) {
      bf16* orow = ob + (int64_t)qi * p.o_sl;
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (bf16)(oacc[nb][mb][v4 * 4 + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + mb * 32 + v4 * 8 + hi * 4) = w;
        }
      }
      if (lseb && hi == 0) lseb[qi] = live ? (mrow[nb] * kLn2 + logf(ft)) : kNegInf;
    }
  }
}

template <int D, int NQB, bool CAUSAL, bool MASK>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
  constexpr int BM = kWaves * 32 * NQB;
  const int n_qt = (a.p.Lq + BM - 1) / BM;
  const int grid = n_qt * a.p.B * a.p.Hq;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NQB, CAUSAL, MASK>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  const bool causal = a.p.causal != 0;
  const bool mask = a.p.mask != nullptr;
  if (causal) return mask ? launch_t<D, 1, true, true>(a, s) : launch_t<D, 1, true, false>(a, s);
  return mask ? launch_t<D, 1, false, true>(a, s) : launch_t<D, 1, false, false>(a, s);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  if (a.p.Lq == 0) return hipSuccess;
  switch (a.p.D) {
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdpa
