// fwd_bf16.hip — prefill forward, bf16 in / fp32 accumulate, gfx950.
//
// Computes O = softmax(scale * Q K^T + mask) V and LSE per row ("Scaled dot-product
// attention (forward and backward)", section 2 Principles and 2.2 Masking; LSE as in
// cuDNN "Attention", SDPA FP16/BF16 Forward, Python API return values) with the
// one-pass online softmax (running max and sum; the page's "Going further" table names
// Milakov and Gimelshein's online normaliser).
//
// Work decomposition: a workgroup of NW waves owns BM = NW * 32 * NQB query rows of one
// (batch, head); each wave owns NQB blocks of 32 query rows and keeps their Q operand, O
// accumulator and running statistics in registers.  K/V tiles of 64 keys stream
// HBM -> LDS with global_load_lds (16 bytes per lane, no staging registers) into two
// LDS buffers: tile t+1 is in flight while tile t is computed, one barrier per tile.
// Tiles are stored unpadded with XOR-swizzled 16-byte chunks (kern_common.h) so the MFMA
// operand reads are free of bank conflicts.  With NQB = 2 every K/V operand read from
// LDS feeds two MFMAs, which halves LDS traffic per flop.
//
//   S^T = K Q^T   (keys x queries): A = K rows from LDS (row-permuted, see kern_common.h),
//                 B = Q held in registers; lane l ends up with 16 consecutive keys of
//                 query l%32, so the row max needs v_max3 reductions in registers plus one
//                 permlane32 swap, and the row sums stay per half-wave until the end.
//   O^T += V^T P^T (d x queries): A = V^T read with ds_read_b64_tr_b16, B = bf16(P) taken
//                 straight from the S accumulator registers.  O^T keeps one query per
//                 lane, so a rescale is a per-lane multiply.
//
// Softmax arithmetic per score: one FMA folds scale * log2(e) and the reference max into
// the exp2 argument; v_exp_f32; v_cvt_pk_bf16_f32; the bf16 weights are summed with
// v_dot2 (this sum normalises O, so each output row is an exact convex combination of
// value rows) and the fp32 weights with one add (this sum gives LSE).  The reference max
// is only moved when a row's max grows by more than 2^8 (weights stay <= 256, exact in
// fp32 sums and in bf16 range), so the O rescale runs on a few tiles only.
//
// Tiles entirely above the causal diagonal or past the key length are never visited, and
// a wave skips the 32-key blocks that none of its rows can see.  Only tiles touching the
// diagonal or a length boundary evaluate per-element predicates.  Rows with no visible
// key produce O = 0, LSE = -inf.
#include "kern_common.h"
#include "launch.h"

namespace sdpa {
namespace {

constexpr int kBN = 64;             // keys per K/V tile (two 32-key MFMA blocks)
constexpr float kRescaleLog2 = 8.f; // move the reference max only past this growth

template <int D, int NW>
struct FwdTile {
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int TILE = kBN * D;       // elements per K (or V) tile
};

template <int D, int NW, int NQB, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(64 * NW, 1) void fwd_bf16_kernel(FwdArgs a) {
  using T = FwdTile<D, NW>;
  constexpr int BM = NW * 32 * NQB;
  __shared__ __attribute__((aligned(16))) bf16 K0[T::TILE];
  __shared__ __attribute__((aligned(16))) bf16 K1[T::TILE];
  __shared__ __attribute__((aligned(16))) bf16 V0[T::TILE];
  __shared__ __attribute__((aligned(16))) bf16 V1[T::TILE];

  const Problem& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;  // which half of the wave

  // ---- work item; the heads of one KV group are adjacent in launch order.
  const int bh_count = p.B * p.Hq;
  const int rank = blockIdx.x / bh_count;
  const int bh = blockIdx.x % bh_count;
  const int b = bh / p.Hq;
  const int h = bh % p.Hq;
  const int g = h / p.G;

  const int q_end = p.len_q ? min(p.len_q[b], p.Lq) : p.Lq;
  const int kv_end = p.len_kv ? min(p.len_kv[b], p.Lk) : p.Lk;
  // Rows of this workgroup.  Non-causal: query tile `rank` of BM rows.  Causal, large
  // grids: tile n_qt - 1 - rank (heavy tiles launch first and the scheduler evens the
  // load).  Causal, grids of about one round (pair_rows): the half-tiles (BM/2 rows)
  // `rank` and `n_half - 1 - rank`, one per half of the waves, so every workgroup carries
  // the same causal work (a middle half-tile pairs with nothing).
  int wq_lo, row_lo, row_hi;  // this wave's first row; the workgroup's row span
  if (CAUSAL && !p.pair_rows) {
    const int qt = (p.Lq + BM - 1) / BM - 1 - rank;
    wq_lo = qt * BM + wave * 32 * NQB;
    row_lo = qt * BM;
    row_hi = row_lo + BM;
  } else if (CAUSAL) {
    constexpr int HB = BM / 2;
    const int n_half = (p.Lq + HB - 1) / HB;
    const int heavy = n_half - 1 - rank;
    const int mine = wave < NW / 2 ? rank : heavy;
    wq_lo = (wave >= NW / 2 && heavy == rank) ? p.Lq : mine * HB + (wave % (NW / 2)) * 32 * NQB;
    row_lo = rank * HB;
    row_hi = (heavy + 1) * HB;
  } else {
    wq_lo = rank * BM + wave * 32 * NQB;
    row_lo = rank * BM;
    row_hi = row_lo + BM;
  }
  const int wq_hi = min(wq_lo + 32 * NQB, q_end) - 1;     // this wave's last live row

  const bf16* qb = reinterpret_cast<const bf16*>(a.q) + b * p.q_sb + h * p.q_sh;
  const bf16* kb_ = reinterpret_cast<const bf16*>(a.k) + b * p.k_sb + g * p.k_sh;
  const bf16* vb_ = reinterpret_cast<const bf16*>(a.v) + b * p.v_sb + g * p.v_sh;
  bf16* ob = reinterpret_cast<bf16*>(a.o) + b * p.o_sb + h * p.o_sh;
  const bf16* mb_ = MASK ? reinterpret_cast<const bf16*>(p.mask) + b * p.m_sb + h * p.m_sh : nullptr;
  float* lseb = a.lse ? a.lse + ((int64_t)b * p.Hq + h) * p.Lq : nullptr;

  // Keys this tile of queries can see.
  int kv_stop = kv_end;
  if (CAUSAL) kv_stop = min(kv_stop, min(row_hi, q_end));
  if (row_lo >= q_end) kv_stop = 0;
  const int n_tiles = kv_stop > 0 ? (kv_stop + kBN - 1) / kBN : 0;

  // ---- Q operand (B of S^T = K Q^T): lane holds query row, 8 consecutive d per k-step.
  bf16x8 qreg[NQB][D / 16];
  int qrow[NQB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    qrow[nb] = wq_lo + nb * 32 + l32;
    const bool ok = qrow[nb] < q_end;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 x = ok ? ld16(qb + (int64_t)qrow[nb] * p.q_sl + kk * 16 + 8 * hi) : zero16();
      qreg[nb][kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // reference max (log2 units), sum of bf16 weights (normalises O), sum of fp32 weights
  // (gives LSE); both sums are relative to the reference max.
  f32x16 oacc[NQB][D / 32];
  float mref[NQB], lrow[NQB], frow[NQB];
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    mref[nb] = kNegInf;
    lrow[nb] = 0.f;
    frow[nb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[nb][mb] = f32x16{};
  }

  // ---- K/V tiles: HBM -> LDS, double-buffered.
  auto load_tile = [&](int j0, bf16* Kd, bf16* Vd) {
    tile_to_lds_swz<kBN, D, NW>(kb_, p.k_sl, j0, kv_stop, Kd, wave, lane);
    tile_to_lds_swz<kBN, D, NW>(vb_, p.v_sl, j0, kv_stop, Vd, wave, lane);
  };
  if (n_tiles > 0) load_tile(0, K0, V0);
  const float c2 = p.scale_log2;
  const bf16x2 ones2 = {(bf16)1.f, (bf16)1.f};
  // K operand read: row kb*32 + perm_row(l32), logical chunk 2*kk + hi
  const int krow_l = perm_row(l32);
  // V^T operand (transposing read): row key_base + arow, logical chunk vchunk, half vhalf
  const int blk = lane >> 4;
  const int arow = (lane & 15) >> 2;
  const int vchunk = ((lane & 3) >> 1) + 2 * (blk & 1);
  const int vhalf = 4 * (lane & 1);

  // One tile step; the loop below is unrolled by two so that the buffer being read and
  // the one being filled are distinct LDS objects at compile time (the compiler then
  // does not make the reads of tile t wait for the copies of tile t+1).
  auto step = [&](int t, const bf16* Kt, const bf16* Vt, bf16* Kn, bf16* Vn)
                  __attribute__((always_inline)) {
    const int j0 = t * kBN;
    wait_vmem();       // this wave's copies of tile t have landed
    __syncthreads();   // ... and everyone's; the other buffer is no longer being read
    if (t + 1 < n_tiles) load_tile(j0 + kBN, Kn, Vn);

    // The tile's two 32-key blocks one after the other: S^T, softmax, then PV.
    const bool partial_t = (j0 + kBN > kv_end) || (CAUSAL && j0 + kBN - 1 > wq_lo) ||
                           (wq_lo + 32 * NQB > q_end);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key_lo = j0 + kb * 32;
      // a block none of this wave's rows can see is skipped (wave-uniform)
      if (!(wq_lo < q_end && key_lo < kv_stop && (!CAUSAL || key_lo <= wq_hi))) continue;

      // ---- S^T = K Q^T for keys key_lo .. key_lo + 31
      f32x16 sacc[NQB];
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) sacc[nb] = f32x16{};
      {
        // all K operands of the block first, so the LDS reads are in flight together
        const int kr = kb * 32 + krow_l;
        bf16x8 kop[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) kop[kk] = tile_row8<D>(Kt, kr, 2 * kk + hi);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
          for (int nb = 0; nb < NQB; ++nb) sacc[nb] = mfma32(kop[kk], qreg[nb][kk], sacc[nb]);
      }

      // ---- online softmax; lane holds keys key0 + v (v < 16) of query qrow[nb].
      const int key0 = key_lo + 16 * hi;
      bf16x8 pop[NQB][2];
#pragma unroll
      for (int nb = 0; nb < NQB; ++nb) {
        const int qi = qrow[nb];
        // x: raw dot products (no mask) or log2-unit scores (mask)
        float x[16];
        if (MASK) {
          float mv[16];
          if (p.mask_vec && qi < q_end && key0 + 16 <= p.Lk) {
            const bf16* mp = mb_ + (int64_t)qi * p.m_si + key0;
            bf16x8 b0 = __builtin_bit_cast(bf16x8, ld16(mp)), b1 = __builtin_bit_cast(bf16x8, ld16(mp + 8));
#pragma unroll
            for (int v = 0; v < 8; ++v) { mv[v] = bf2f(b0[v]); mv[v + 8] = bf2f(b1[v]); }
          } else {
#pragma unroll
            for (int v = 0; v < 16; ++v)
              mv[v] = (qi < q_end && key0 + v < kv_end) ? bf2f(mb_[(int64_t)qi * p.m_si + key0 + v]) : 0.f;
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) x[v] = fmaf(sacc[nb][v], c2, mv[v] * kLog2e);
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v) x[v] = sacc[nb][v];
        }
        if (partial_t) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = key0 + v;
            const bool ok = key < kv_end && qi < q_end && (!CAUSAL || key <= qi);
            x[v] = ok ? x[v] : kNegInf;
          }
        }
        float mx = kNegInf;
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, x[v]);
        mx = xhalf_max(mx);
        const float mt = MASK ? mx : mx * c2;  // block max in log2 units (c2 > 0)
        // lazy rescale: move the reference only when some row grew past the threshold
        const bool need = mt > mref[nb] + kRescaleLog2;
        if (__builtin_amdgcn_ballot_w64(need)) {
          const float mnew = need ? mt : mref[nb];
          const float corr = need ? fast_exp2(mref[nb] - mnew) : 1.f;
          mref[nb] = mnew;
          lrow[nb] *= corr;
          frow[nb] *= corr;
#pragma unroll
          for (int mb = 0; mb < D / 32; ++mb) oacc[nb][mb] *= corr;
        }
        const float m_use = (mref[nb] == kNegInf) ? 0.f : mref[nb];
        float psum = lrow[nb], fsum = frow[nb];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 pb;
#pragma unroll
          for (int t2 = 0; t2 < 4; ++t2) {
            const int v = half * 8 + 2 * t2;
            f32x2 e;
            if (MASK) {
              e[0] = fast_exp2(x[v] - m_use);
              e[1] = fast_exp2(x[v + 1] - m_use);
            } else {
              e[0] = fast_exp2(fmaf(x[v], c2, -m_use));
              e[1] = fast_exp2(fmaf(x[v + 1], c2, -m_use));
            }
            const bf16x2 e2 = __builtin_convertvector(e, bf16x2);
            psum = __builtin_amdgcn_fdot2_f32_bf16(e2, ones2, psum, false);
            fsum += e[0];
            fsum += e[1];
            pb[2 * t2] = e2[0];
            pb[2 * t2 + 1] = e2[1];
          }
          pop[nb][half] = pb;
        }
        lrow[nb] = psum;
        frow[nb] = fsum;
      }

      // ---- O^T += V^T P^T.  V^T operand via transposing LDS reads: lane (within its
      // 16-lane block) supplies row  key_base + (lane%16)/4, columns d_base + 4*(lane%4).
      bf16x8 vop[2][D / 32];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int vr = kb * 32 + 16 * hi + 8 * half + arow;  // rows vr .. vr + 7
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) vop[half][mb] = tile_tr8<D>(Vt, vr, vchunk + 4 * mb, vhalf);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
          for (int nb = 0; nb < NQB; ++nb) oacc[nb][mb] = mfma32(vop[half][mb], pop[nb][half], oacc[nb][mb]);
    }
  };
  for (int t = 0; t < n_tiles; t += 2) {
    step(t, K0, V0, K1, V1);
    if (t + 1 < n_tiles) step(t + 1, K1, V1, K0, V0);
  }

  // ---- epilogue: O = O^T / l (0 for empty rows), LSE = ln2 * (mref + log2 f).
#pragma unroll
  for (int nb = 0; nb < NQB; ++nb) {
    const int qi = qrow[nb];
    const float lt = xhalf_sum(lrow[nb]);
    const float ft = xhalf_sum(frow[nb]);
    const bool rowlive = qi < q_end && lt > 0.f;
    const float inv = rowlive ? 1.f / lt : 0.f;
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
      if (lseb && hi == 0) lseb[qi] = rowlive ? (mref[nb] * kLn2 + logf(ft)) : kNegInf;
    }
  }
}

template <int D, int NW, int NQB, bool CAUSAL, bool MASK>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
  constexpr int BM = NW * 32 * NQB;
  const int n_qt = (a.p.Lq + BM - 1) / BM;
  FwdArgs args = a;
  // pair half-tiles when whole tiles would give about one round of workgroups
  args.p.pair_rows = CAUSAL && (int64_t)n_qt * a.p.B * a.p.Hq <= 512;
  const int n_wg = args.p.pair_rows ? ((a.p.Lq + BM / 2 - 1) / (BM / 2) + 1) / 2 : n_qt;
  const int grid = n_wg * a.p.B * a.p.Hq;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, NQB, CAUSAL, MASK>), dim3(grid), dim3(64 * NW), 0, s, args);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool MASK>
hipError_t launch_shape(const FwdArgs& a, hipStream_t s) {
  // 8 waves of 32 query rows per workgroup: two waves per SIMD hide each other's LDS and
  // MFMA latencies, which measured faster than 64 rows per wave at one wave per SIMD.
  return launch_t<D, 8, 1, CAUSAL, MASK>(a, s);
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  const bool causal = a.p.causal != 0;
  const bool mask = a.p.mask != nullptr;
  if (causal) return mask ? launch_shape<D, true, true>(a, s) : launch_shape<D, true, false>(a, s);
  return mask ? launch_shape<D, false, true>(a, s) : launch_shape<D, false, false>(a, s);
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
