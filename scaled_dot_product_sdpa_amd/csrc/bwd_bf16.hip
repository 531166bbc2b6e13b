// bwd_bf16.hip — backward, bf16 in / fp32 accumulate, gfx950.
//
// Gradients of O = softmax(scale Q K^T + mask) V ("Scaled dot-product attention (forward
// and backward)", section 2.3 The backward pass):
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  D_i = rowsum(dO o O)_i,
//   dQ = scale dS K,  dK = scale dS^T Q.
// P is never stored: it is recomputed tile by tile as P_ij = exp(S_ij - LSE_i) from the
// forward's LSE (that page's "Going further" table: the FlashAttention-2 backward
// recomputes P from saved row statistics and uses D = rowsum(dO o O)).
//
// Three kernels, no atomics (the result is deterministic):
//  1. prep:  D_i = sum_t dO_it O_it in fp32 (zero for empty rows).
//  2. dkdv:  key-stationary.  A workgroup owns 128 keys of one (batch, KV head); each wave
//            keeps 32 keys' K and V operands and their dK^T, dV^T accumulators in
//            registers, and walks the query heads of the group and their query tiles
//            (Q, dO staged through LDS).  Per 32x32 block:
//              S = Q K^T, P = exp2(S*scale*log2e - LSE*log2e),  dP = dO V^T,
//              dS = P o (dP - D),  dV^T += dO^T P,  dK^T += Q^T dS
//            with dO^T and Q^T read from LDS by ds_read_b64_tr_b16.
//  3. dq:    query-stationary (the forward's decomposition).  Per 64-key tile:
//              S^T = K Q^T,  P^T,  dP^T = V dO^T,  dS^T = P^T o (dP^T - D),
//              dQ^T += K^T dS^T   (K^T via transposing LDS reads).
// Rows and keys past the lengths, and pairs above the causal diagonal, carry P = 0; whole
// tiles that are blocked are skipped.
#include "kern_common.h"
#include "launch.h"

namespace sdpa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// ---------------------------------------------------------------------------------------
// 1. D = rowsum(dO o O)
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(BwdArgs a) {
  const Problem& p = a.p;
  constexpr int CPR = D / 8;                  // threads per row (one 16-byte chunk each)
  constexpr int RPB = kThreads / CPR;         // rows per block
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / CPR;
  const int c = threadIdx.x % CPR;
  const int64_t nrows = (int64_t)p.B * p.Hq * p.Lq;
  float acc = 0.f;
  int i = 0, b = 0, h = 0;
  if (row < nrows) {
    i = (int)(row % p.Lq);
    h = (int)((row / p.Lq) % p.Hq);
    b = (int)(row / ((int64_t)p.Lq * p.Hq));
    const int q_end = p.len_q ? min(p.len_q[b], p.Lq) : p.Lq;
    if (i < q_end) {
      const int64_t off = b * p.o_sb + h * p.o_sh + (int64_t)i * p.o_sl + c * 8;
      bf16x8 o8 = __builtin_bit_cast(bf16x8, ld16(reinterpret_cast<const bf16*>(a.o) + off));
      bf16x8 d8 = __builtin_bit_cast(bf16x8, ld16(reinterpret_cast<const bf16*>(a.dO) + off));
#pragma unroll
      for (int t = 0; t < 8; ++t) acc = fmaf(bf2f(o8[t]), bf2f(d8[t]), acc);
    }
  }
#pragma unroll
  for (int w = CPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, CPR);
  if (row < nrows && c == 0) a.dsum[row] = acc;
}

// ---------------------------------------------------------------------------------------
// 2. dK, dV (key-stationary)
// ---------------------------------------------------------------------------------------
constexpr int kKT = 128;  // keys per workgroup (32 per wave)
constexpr int kQT = 32;   // query rows per inner tile

template <int D>
struct DkdvTile {
  static constexpr int QP = D + 8;        // LDS pitch of the Q / dO tiles
  static constexpr int MP = kKT + 8;      // LDS pitch of the mask tile
  static constexpr int CPR = D / 8;
  static constexpr int NCH = kQT * CPR / kThreads;  // 16-byte chunks per thread (Q or dO)
  static constexpr int MCH = kQT * (kKT / 8) / kThreads;  // mask chunks per thread
};

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using T = DkdvTile<D>;
  __shared__ __attribute__((aligned(16))) bf16 Qs[kQT * T::QP];
  __shared__ __attribute__((aligned(16))) bf16 dOs[kQT * T::QP];
  __shared__ __attribute__((aligned(16))) bf16 Ms[MASK ? kQT * T::MP : 8];
  __shared__ float lse_s[kQT];
  __shared__ float dsum_s[kQT];

  const Problem& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int n_kt = (p.Lk + kKT - 1) / kKT;
  const int bg_count = p.B * p.Hkv;
  const int rank = blockIdx.x / bg_count;
  const int bg = blockIdx.x % bg_count;
  // Causal: low key tiles see the most queries, so launch them first.
  const int kt = rank;
  (void)n_kt;
  const int b = bg / p.Hkv;
  const int g = bg % p.Hkv;
  const int q_end = p.len_q ? min(p.len_q[b], p.Lq) : p.Lq;
  const int kv_end = p.len_kv ? min(p.len_kv[b], p.Lk) : p.Lk;
  const int j0 = kt * kKT;
  const int jw = j0 + wave * 32;  // this wave's first key
  const int myk = jw + l32;       // this lane's key (N index of S, dP)

  const bf16* kbase = reinterpret_cast<const bf16*>(a.k) + b * p.k_sb + g * p.k_sh;
  const bf16* vbase = reinterpret_cast<const bf16*>(a.v) + b * p.v_sb + g * p.v_sh;

  // K and V operands of this lane's key (B operands of S = Q K^T and dP = dO V^T).
  bf16x8 kreg[D / 16], vreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const bool ok = myk < kv_end;
    kreg[kk] = __builtin_bit_cast(bf16x8, ok ? ld16(kbase + (int64_t)myk * p.k_sl + kk * 16 + 8 * hi) : zero16());
    vreg[kk] = __builtin_bit_cast(bf16x8, ok ? ld16(vbase + (int64_t)myk * p.v_sl + kk * 16 + 8 * hi) : zero16());
  }

  f32x16 dk_acc[D / 32], dv_acc[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) { dk_acc[mb] = f32x16{}; dv_acc[mb] = f32x16{}; }

  // Query tiles that can see any key of this workgroup.
  const int kstop = min(kv_end, j0 + kKT);  // keys [j0, kstop) exist
  int qt_begin = 0;
  if (CAUSAL) qt_begin = j0 / kQT;
  const int qt_end = (j0 < kstop) ? (q_end + kQT - 1) / kQT : 0;
  const int n_q_tiles = qt_end > qt_begin ? qt_end - qt_begin : 0;
  const int total = n_q_tiles * p.G;

  u32x4 qst[T::NCH], dost[T::NCH], mst[MASK ? T::MCH : 1];
  float lse_st = 0.f, dsum_st = 0.f;
  auto load_tile = [&](int it) {
    const int hh = it / n_q_tiles;
    const int i0 = (qt_begin + it % n_q_tiles) * kQT;
    const int h = g * p.G + hh;
    const bf16* qb = reinterpret_cast<const bf16*>(a.q) + b * p.q_sb + h * p.q_sh;
    const bf16* dob = reinterpret_cast<const bf16*>(a.dO) + b * p.o_sb + h * p.o_sh;
#pragma unroll
    for (int u = 0; u < T::NCH; ++u) {
      const int idx = tid + u * kThreads;
      const int r = idx / T::CPR, c = idx % T::CPR;
      const int row = i0 + r;
      const bool ok = row < q_end;
      qst[u] = ok ? ld16(qb + (int64_t)row * p.q_sl + c * 8) : zero16();
      dost[u] = ok ? ld16(dob + (int64_t)row * p.o_sl + c * 8) : zero16();
    }
    if (MASK) {
      const bf16* mb = reinterpret_cast<const bf16*>(p.mask) + b * p.m_sb + h * p.m_sh;
#pragma unroll
      for (int u = 0; u < T::MCH; ++u) {
        const int idx = tid + u * kThreads;
        const int r = idx / (kKT / 8), c = idx % (kKT / 8);
        const int row = i0 + r, col = j0 + c * 8;
        const bool ok = p.mask_vec && row < q_end && col + 8 <= p.Lk;
        if (ok) {
          mst[u] = ld16(mb + (int64_t)row * p.m_si + col);
        } else {
          // ragged key tail: gather element by element inside the key length
          bf16x8 t8;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            t8[e] = (row < q_end && col + e < kv_end) ? mb[(int64_t)row * p.m_si + col + e] : (bf16)0.f;
          mst[u] = __builtin_bit_cast(u32x4, t8);
        }
      }
    }
    if (tid < kQT) {
      const int row = i0 + tid;
      const int64_t r = ((int64_t)b * p.Hq + h) * p.Lq + row;
      float l = (row < q_end) ? a.lse[r] : kNegInf;
      // exp2(s - (+inf)) = 0 makes empty rows contribute nothing
      lse_st = (l == kNegInf) ? __builtin_inff() : l * kLog2e;
      dsum_st = (row < q_end) ? a.dsum[r] : 0.f;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < T::NCH; ++u) {
      const int idx = tid + u * kThreads;
      const int r = idx / T::CPR, c = idx % T::CPR;
      *reinterpret_cast<u32x4*>(&Qs[r * T::QP + c * 8]) = qst[u];
      *reinterpret_cast<u32x4*>(&dOs[r * T::QP + c * 8]) = dost[u];
    }
    if (MASK) {
#pragma unroll
      for (int u = 0; u < T::MCH; ++u) {
        const int idx = tid + u * kThreads;
        const int r = idx / (kKT / 8), c = idx % (kKT / 8);
        *reinterpret_cast<u32x4*>(&Ms[r * T::MP + c * 8]) = mst[u];
      }
    }
    if (tid < kQT) { lse_s[tid] = lse_st; dsum_s[tid] = dsum_st; }
  };

  if (total > 0) load_tile(0);
  const int blk = lane >> 4;
  const int arow = (lane & 15) >> 2;
  const int acol = 4 * (lane & 3) + 16 * (blk & 1);

  for (int it = 0; it < total; ++it) {
    const int i0 = (qt_begin + it % n_q_tiles) * kQT;
    store_tile();
    __syncthreads();
    if (it + 1 < total) load_tile(it + 1);

    // this wave's keys [jw, jw+32) against queries [i0, i0+32)
    const bool any = (jw < kv_end) && (!CAUSAL || i0 + kQT - 1 >= jw);
    if (any) {
      // S = Q K^T and dP = dO V^T: A = Q / dO rows (row-permuted), B = K / V in registers.
      f32x16 s_acc = f32x16{}, dp_acc = f32x16{};
      const int qr = perm_row(l32);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        bf16x8 qa = *reinterpret_cast<const bf16x8*>(&Qs[qr * T::QP + kk * 16 + 8 * hi]);
        bf16x8 da = *reinterpret_cast<const bf16x8*>(&dOs[qr * T::QP + kk * 16 + 8 * hi]);
        s_acc = mfma32(qa, kreg[kk], s_acc);
        dp_acc = mfma32(da, vreg[kk], dp_acc);
      }
      // lane holds key myk and queries i0 + 16*hi + v
      const bool partial = (myk >= kv_end) || (jw + 32 > kv_end) || (i0 + kQT > q_end) ||
                           (CAUSAL && i0 < jw + 31);
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) {
          const int v = half * 8 + t8;
          const int ql = 16 * hi + v;
          float x = s_acc[v] * p.scale_log2;
          if (MASK) x += bf2f(Ms[ql * T::MP + wave * 32 + l32]) * kLog2e;
          if (partial) {
            const int qi = i0 + ql;
            const bool ok = myk < kv_end && qi < q_end && (!CAUSAL || myk <= qi);
            x = ok ? x : kNegInf;
          }
          const float pv = fast_exp2(x - lse_s[ql]);
          const float ds = pv * (dp_acc[v] - dsum_s[ql]);
          pb[half][t8] = (bf16)pv;
          dsb[half][t8] = (bf16)ds;
        }
      }
      // dV^T += dO^T P,  dK^T += Q^T dS   (A operands: transposing LDS reads)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int rbase = (16 * hi + 8 * half + arow) * T::QP + acol;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) {
          bf16x8 doT = join_tr(lds_read_tr4(&dOs[rbase + mb * 32]), lds_read_tr4(&dOs[rbase + 4 * T::QP + mb * 32]));
          bf16x8 qT = join_tr(lds_read_tr4(&Qs[rbase + mb * 32]), lds_read_tr4(&Qs[rbase + 4 * T::QP + mb * 32]));
          dv_acc[mb] = mfma32(doT, pb[half], dv_acc[mb]);
          dk_acc[mb] = mfma32(qT, dsb[half], dk_acc[mb]);
        }
      }
    }
    __syncthreads();
  }

  // Epilogue: lane holds key myk, d = mb*32 + (v/4)*8 + 4*hi + v%4.
  if (myk < p.Lk) {
    bf16* dkrow = reinterpret_cast<bf16*>(a.dk) + b * p.k_sb + g * p.k_sh + (int64_t)myk * p.k_sl;
    bf16* dvrow = reinterpret_cast<bf16*>(a.dv) + b * p.v_sb + g * p.v_sh + (int64_t)myk * p.v_sl;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        bf16x4 wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[e] = (bf16)(dk_acc[mb][v4 * 4 + e] * p.scale);
          wv[e] = (bf16)(dv_acc[mb][v4 * 4 + e]);
        }
        *reinterpret_cast<bf16x4*>(dkrow + mb * 32 + v4 * 8 + hi * 4) = wk;
        *reinterpret_cast<bf16x4*>(dvrow + mb * 32 + v4 * 8 + hi * 4) = wv;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// 3. dQ (query-stationary)
// ---------------------------------------------------------------------------------------
constexpr int kBN = 64;

template <int D>
struct DqTile {
  static constexpr int KP = D + 8;
  static constexpr int VP = D + 8;
  static constexpr int CPR = D / 8;
  static constexpr int NCH = kBN * CPR / kThreads;
};

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(BwdArgs a) {
  using T = DqTile<D>;
  constexpr int BM = kWaves * 32;
  __shared__ __attribute__((aligned(16))) bf16 Ks[kBN * T::KP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[kBN * T::VP];

  const Problem& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

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
  const bf16* dob = reinterpret_cast<const bf16*>(a.dO) + b * p.o_sb + h * p.o_sh;
  const bf16* kb_ = reinterpret_cast<const bf16*>(a.k) + b * p.k_sb + g * p.k_sh;
  const bf16* vb_ = reinterpret_cast<const bf16*>(a.v) + b * p.v_sb + g * p.v_sh;
  const bf16* mb_ = MASK ? reinterpret_cast<const bf16*>(p.mask) + b * p.m_sb + h * p.m_sh : nullptr;

  int kv_stop = kv_end;
  if (CAUSAL) kv_stop = min(kv_stop, min(i0 + BM, q_end));
  if (i0 >= q_end) kv_stop = 0;
  const int n_tiles = kv_stop > 0 ? (kv_stop + kBN - 1) / kBN : 0;

  const int qi = i0 + wave * 32 + l32;  // this lane's query (N index)
  const bool qok = qi < q_end;
  bf16x8 qreg[D / 16], doreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qreg[kk] = __builtin_bit_cast(bf16x8, qok ? ld16(qb + (int64_t)qi * p.q_sl + kk * 16 + 8 * hi) : zero16());
    doreg[kk] = __builtin_bit_cast(bf16x8, qok ? ld16(dob + (int64_t)qi * p.o_sl + kk * 16 + 8 * hi) : zero16());
  }
  const int64_t rowid = ((int64_t)b * p.Hq + h) * p.Lq + qi;
  float lse_l2 = __builtin_inff(), dsum = 0.f;
  if (qok) {
    const float l = a.lse[rowid];
    lse_l2 = (l == kNegInf) ? __builtin_inff() : l * kLog2e;
    dsum = a.dsum[rowid];
  }

  f32x16 dq_acc[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) dq_acc[mb] = f32x16{};

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
  const int blk = lane >> 4;
  const int arow = (lane & 15) >> 2;
  const int acol = 4 * (lane & 3) + 16 * (blk & 1);

  for (int t = 0; t < n_tiles; ++t) {
    const int j0 = t * kBN;
    store_tile();
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(j0 + kBN);

    const bool partial = (j0 + kBN > kv_end) || (CAUSAL && j0 + kBN - 1 > i0) || (i0 + BM > q_end);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T = K Q^T and dP^T = V dO^T for keys j0 + kb*32 + perm
      f32x16 s_acc = f32x16{}, dp_acc = f32x16{};
      const int kr = (kb * 32 + perm_row(l32));
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[kr * T::KP + kk * 16 + 8 * hi]);
        bf16x8 va = *reinterpret_cast<const bf16x8*>(&Vs[kr * T::VP + kk * 16 + 8 * hi]);
        s_acc = mfma32(ka, qreg[kk], s_acc);
        dp_acc = mfma32(va, doreg[kk], dp_acc);
      }
      // lane holds query qi and keys key0 + v
      const int key0 = j0 + kb * 32 + 16 * hi;
      float mv[16];
      if (MASK) {
        if (p.mask_vec && qok && key0 + 16 <= p.Lk) {
          const bf16* mp = mb_ + (int64_t)qi * p.m_si + key0;
          bf16x8 b0 = __builtin_bit_cast(bf16x8, ld16(mp)), b1 = __builtin_bit_cast(bf16x8, ld16(mp + 8));
#pragma unroll
          for (int v = 0; v < 8; ++v) { mv[v] = bf2f(b0[v]); mv[v + 8] = bf2f(b1[v]); }
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            mv[v] = (qok && key0 + v < kv_end) ? bf2f(mb_[(int64_t)qi * p.m_si + key0 + v]) : 0.f;
        }
      }
      bf16x8 dsb[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) {
          const int v = half * 8 + t8;
          float x = s_acc[v] * p.scale_log2;
          if (MASK) x += mv[v] * kLog2e;
          if (partial) {
            const int key = key0 + v;
            const bool ok = key < kv_end && qok && (!CAUSAL || key <= qi);
            x = ok ? x : kNegInf;
          }
          const float pv = fast_exp2(x - lse_l2);
          dsb[half][t8] = (bf16)(pv * (dp_acc[v] - dsum));
        }
      }
      // dQ^T += K^T dS^T  (K^T via transposing LDS reads)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16* krow = &Ks[(kb * 32 + 16 * hi + 8 * half + arow) * T::KP + acol];
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) {
          bf16x8 kT = join_tr(lds_read_tr4(krow + mb * 32), lds_read_tr4(krow + 4 * T::KP + mb * 32));
          dq_acc[mb] = mfma32(kT, dsb[half], dq_acc[mb]);
        }
      }
    }
    __syncthreads();
  }

  if (qi < p.Lq) {
    bf16* dqrow = reinterpret_cast<bf16*>(a.dq) + b * p.q_sb + h * p.q_sh + (int64_t)qi * p.q_sl;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(qok ? dq_acc[mb][v4 * 4 + e] * p.scale : 0.f);
        *reinterpret_cast<bf16x4*>(dqrow + mb * 32 + v4 * 8 + hi * 4) = w;
      }
    }
  }
}

template <int D, bool CAUSAL, bool MASK>
hipError_t launch_main(const BwdArgs& a, int stages, hipStream_t s) {
  const int n_kt = (a.p.Lk + kKT - 1) / kKT;
  if ((stages & kBwdDkdv) && n_kt > 0) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, MASK>), dim3(n_kt * a.p.B * a.p.Hkv), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_qt = (a.p.Lq + 127) / 128;
  if ((stages & kBwdDq) && n_qt > 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, MASK>), dim3(n_qt * a.p.B * a.p.Hq), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdArgs& a, int stages, hipStream_t s) {
  const int64_t rows = (int64_t)a.p.B * a.p.Hq * a.p.Lq;
  if ((stages & kBwdPrep) && rows > 0) {
    constexpr int RPB = kThreads / (D / 8);
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(stages & (kBwdDkdv | kBwdDq))) return hipSuccess;
  const bool causal = a.p.causal != 0, mask = a.p.mask != nullptr;
  if (causal) return mask ? launch_main<D, true, true>(a, stages, s) : launch_main<D, true, false>(a, stages, s);
  return mask ? launch_main<D, false, true>(a, stages, s) : launch_main<D, false, false>(a, stages, s);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, int stages, hipStream_t s) {
  switch (a.p.D) {
    case 64: return launch_d<64>(a, stages, s);
    case 128: return launch_d<128>(a, stages, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdpa
