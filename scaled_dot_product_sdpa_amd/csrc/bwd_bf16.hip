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
//  1. prep:  per row, D_i = sum_t dO_it O_it and lse2_i = LSE_i * log2(e) (+inf for a row
//            with no visible key or past the length, so that exp2(s - lse2) = 0 there),
//            both fp32 into the workspace.
//  2. dkdv:  key-stationary.  A workgroup owns 32 * NW keys of one (batch, KV head); each
//            wave keeps its 32 keys' K and V operands and their dK^T, dV^T accumulators in
//            registers, and walks the query heads of the group and their 32-row query
//            tiles.  Q, dO (and lse2, D) tiles stream HBM -> LDS with global_load_lds into
//            two buffers (tile t+1 in flight while tile t is computed).  Per 32x32 block:
//              S = Q K^T,  P = exp2(S * scale * log2e - lse2),  dP = dO V^T,
//              dS = P o (dP - D),  dV^T += dO^T P,  dK^T += Q^T dS
//            with dO^T and Q^T read from LDS by ds_read_b64_tr_b16.
//  3. dq:    query-stationary (the forward's decomposition, 8 waves of 32 rows).  Per
//            32-key block of a double-buffered 64-key K/V tile:
//              S^T = K Q^T,  P^T,  dP^T = V dO^T,  dS^T = P^T o (dP^T - D),
//              dQ^T += K^T dS^T   (K^T via transposing LDS reads).
// Rows and keys past the lengths and pairs above the causal diagonal carry P = 0; blocks
// that are blocked as a whole are skipped.  LDS tiles are unpadded with XOR-swizzled
// 16-byte chunks (kern_common.h).
#include "kern_common.h"
#include "launch.h"

namespace sdpa {
namespace {

// ---------------------------------------------------------------------------------------
// 1. D = rowsum(dO o O) and lse2
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  const Problem& p = a.p;
  constexpr int CPR = D / 8;         // threads per row (one 16-byte chunk each)
  constexpr int RPB = 256 / CPR;     // rows per block
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / CPR;
  const int c = threadIdx.x % CPR;
  const int64_t nrows = (int64_t)p.B * p.Hq * p.Lq;
  float acc = 0.f;
  bool valid = false;
  if (row < nrows) {
    const int i = (int)(row % p.Lq);
    const int h = (int)((row / p.Lq) % p.Hq);
    const int b = (int)(row / ((int64_t)p.Lq * p.Hq));
    const int q_end = p.len_q ? min(p.len_q[b], p.Lq) : p.Lq;
    if (i < q_end) {
      valid = true;
      const int64_t off = b * p.o_sb + h * p.o_sh + (int64_t)i * p.o_sl + c * 8;
      bf16x8 o8 = __builtin_bit_cast(bf16x8, ld16(reinterpret_cast<const bf16*>(a.o) + off));
      bf16x8 d8 = __builtin_bit_cast(bf16x8, ld16(reinterpret_cast<const bf16*>(a.dO) + off));
#pragma unroll
      for (int t = 0; t < 8; ++t) acc = fmaf(bf2f(o8[t]), bf2f(d8[t]), acc);
    }
  }
#pragma unroll
  for (int w = CPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, CPR);
  if (row < nrows && c == 0) {
    a.dsum[row] = acc;
    const float l = valid ? a.lse[row] : kNegInf;
    a.lse2[row] = (l == kNegInf) ? __builtin_inff() : l * kLog2e;
  }
}

// ---------------------------------------------------------------------------------------
// 2. dK, dV (key-stationary)
// ---------------------------------------------------------------------------------------
constexpr int kQT = 32;  // query rows per inner tile

template <int D, int NW, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(64 * NW) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int KT = 32 * NW;   // keys per workgroup
  constexpr int CPR = D / 8;
  constexpr int TILE = kQT * D;
  __shared__ __attribute__((aligned(16))) bf16 Q0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 Q1[TILE];
  __shared__ __attribute__((aligned(16))) bf16 G0[TILE];  // dO
  __shared__ __attribute__((aligned(16))) bf16 G1[TILE];
  __shared__ __attribute__((aligned(16))) float S0[2 * kQT];  // lse2 rows, then D rows
  __shared__ __attribute__((aligned(16))) float S1[2 * kQT];
  // mask tiles (kQT rows x KT keys, unswizzled), used when mask rows allow 16-byte copies
  __shared__ __attribute__((aligned(16))) bf16 M0[MASK ? kQT * KT : 8];
  __shared__ __attribute__((aligned(16))) bf16 M1[MASK ? kQT * KT : 8];

  const Problem& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Low key tiles see the most (causal) queries: they are launched first.
  const int bg_count = p.B * p.Hkv;
  const int kt = blockIdx.x / bg_count;
  const int bg = blockIdx.x % bg_count;
  const int b = bg / p.Hkv;
  const int g = bg % p.Hkv;
  const int q_end = p.len_q ? min(p.len_q[b], p.Lq) : p.Lq;
  const int kv_end = p.len_kv ? min(p.len_kv[b], p.Lk) : p.Lk;
  const int j0 = kt * KT;
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
  const int kstop = min(kv_end, j0 + KT);
  const int qt_begin = CAUSAL ? j0 / kQT : 0;
  const int qt_end = (j0 < kstop) ? (q_end + kQT - 1) / kQT : 0;
  const int n_q_tiles = qt_end > qt_begin ? qt_end - qt_begin : 0;
  const int total = n_q_tiles * p.G;

  auto tile_rows = [&](int it, int& h, int& i0) {
    h = g * p.G + it / n_q_tiles;
    i0 = (qt_begin + it % n_q_tiles) * kQT;
  };
  auto load_tile = [&](int it, bf16* Qd, bf16* Gd, float* Sd, bf16* Md) {
    int h, i0;
    tile_rows(it, h, i0);
    const bf16* qb = reinterpret_cast<const bf16*>(a.q) + b * p.q_sb + h * p.q_sh;
    const bf16* dob = reinterpret_cast<const bf16*>(a.dO) + b * p.o_sb + h * p.o_sh;
    tile_to_lds_swz<kQT, D, NW>(qb, p.q_sl, i0, q_end, Qd, wave, lane);
    tile_to_lds_swz<kQT, D, NW>(dob, p.o_sl, i0, q_end, Gd, wave, lane);
    if (MASK && p.mask_vec) {
      // rows past Lq and 8-key chunks past Lk (Lk % 8 == 0 here) repeat valid memory;
      // the pairs they stand for are masked by the predicates
      constexpr int CPRM = KT / 8, NBLK = kQT * CPRM / 64;
      const bf16* mb = reinterpret_cast<const bf16*>(p.mask) + b * p.m_sb + h * p.m_sh;
#pragma unroll
      for (int i = 0; i < NBLK / NW; ++i) {
        const int blk = wave * (NBLK / NW) + i;
        const int ci = blk * 64 + lane;
        const int row = min(i0 + ci / CPRM, p.Lq - 1);
        const int col = min(j0 + (ci % CPRM) * 8, p.Lk - 8);
        global_to_lds16(mb + (int64_t)row * p.m_si + col, Md + blk * 512);
      }
    }
    if (wave == NW - 1) {
      // lse2 (lanes 0..31) and D (lanes 32..63) of the tile's rows; rows past Lq repeat
      // the last row and are masked by the predicates
      const int64_t rb = ((int64_t)b * p.Hq + h) * p.Lq;
      const int row = min(i0 + l32, p.Lq - 1);
      const float* src = (hi ? a.dsum : a.lse2) + rb + row;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)Sd, 4, 0, 0);
    }
  };

  const float c2 = p.scale_log2;
  const int qr = perm_row(l32);              // Q / dO row read by this lane (S, dP)

  const int blk = lane >> 4;
  const int arow = (lane & 15) >> 2;
  const int tchunk = ((lane & 3) >> 1) + 2 * (blk & 1);
  const int thalf = 4 * (lane & 1);

  auto step = [&](int it, const bf16* Qt, const bf16* Gt, const float* St, const bf16* Mt,
                  bf16* Qn, bf16* Gn, float* Sn, bf16* Mn) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
    if (it + 1 < total) load_tile(it + 1, Qn, Gn, Sn, Mn);
    int h, i0;
    tile_rows(it, h, i0);
    // this wave's keys [jw, jw + 32) against queries [i0, i0 + 32)
    if (!(jw < kv_end && (!CAUSAL || i0 + kQT - 1 >= jw))) return;

    // S = Q K^T and dP = dO V^T: A = Q / dO rows (row-permuted), B = K / V in registers.
    f32x16 s_acc = f32x16{}, dp_acc = f32x16{};
    {
      bf16x8 op[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        op[kk] = tile_row8<D>(Qt, qr, 2 * kk + hi);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) s_acc = mfma32(op[kk], kreg[kk], s_acc);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        op[kk] = tile_row8<D>(Gt, qr, 2 * kk + hi);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) dp_acc = mfma32(op[kk], vreg[kk], dp_acc);
    }

    // lane holds key myk and queries i0 + 16*hi + v
    const bool partial = (jw + 32 > kv_end) || (i0 + kQT > q_end) || (CAUSAL && i0 < jw + 31);
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const f32x4* lrow = reinterpret_cast<const f32x4*>(St + 16 * hi + 8 * half);
      const f32x4* drow = reinterpret_cast<const f32x4*>(St + kQT + 16 * hi + 8 * half);
      const f32x4 l_a = lrow[0], l_b = lrow[1], d_a = drow[0], d_b = drow[1];
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {
        const int v = half * 8 + t8;
        const int qi = i0 + 16 * hi + v;
        const float l2 = t8 < 4 ? l_a[t8] : l_b[t8 - 4];
        const float dd = t8 < 4 ? d_a[t8] : d_b[t8 - 4];
        float bias = -l2;
        if (MASK) {
          if (p.mask_vec) {
            bias += bf2f(Mt[(16 * hi + v) * KT + wave * 32 + l32]) * kLog2e;
          } else {
            const bf16* mrow = reinterpret_cast<const bf16*>(p.mask) + b * p.m_sb + h * p.m_sh;
            const bool in = qi < q_end && myk < kv_end;
            bias += in ? bf2f(mrow[(int64_t)qi * p.m_si + myk]) * kLog2e : 0.f;
          }
        }
        float x = fmaf(s_acc[v], c2, bias);
        if (partial) {
          const bool ok = myk < kv_end && qi < q_end && (!CAUSAL || myk <= qi);
          x = ok ? x : kNegInf;
        }
        const float pv = fast_exp2(x);
        pb[half][t8] = (bf16)pv;
        dsb[half][t8] = (bf16)(pv * (dp_acc[v] - dd));
      }
    }
    // dV^T += dO^T P,  dK^T += Q^T dS   (A operands: transposing LDS reads)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int tr = 16 * hi + 8 * half + arow;  // rows tr .. tr + 7 (two quads)
      bf16x8 gT[D / 32], qT[D / 32];
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) {
        gT[mb] = tile_tr8<D>(Gt, tr, tchunk + 4 * mb, thalf);
        qT[mb] = tile_tr8<D>(Qt, tr, tchunk + 4 * mb, thalf);
      }
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) {
        dv_acc[mb] = mfma32(gT[mb], pb[half], dv_acc[mb]);
        dk_acc[mb] = mfma32(qT[mb], dsb[half], dk_acc[mb]);
      }
    }
  };

  if (total > 0) load_tile(0, Q0, G0, S0, M0);
  for (int it = 0; it < total; it += 2) {
    step(it, Q0, G0, S0, M0, Q1, G1, S1, M1);
    if (it + 1 < total) step(it + 1, Q1, G1, S1, M1, Q0, G0, S0, M0);
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

template <int D, int NW, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(64 * NW) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BM = NW * 32;
  constexpr int CPR = D / 8;
  constexpr int TILE = kBN * D;
  __shared__ __attribute__((aligned(16))) bf16 K0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 K1[TILE];
  __shared__ __attribute__((aligned(16))) bf16 V0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 V1[TILE];

  const Problem& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int bh_count = p.B * p.Hq;
  const int rank = blockIdx.x / bh_count;
  const int bh = blockIdx.x % bh_count;
  const int b = bh / p.Hq;
  const int h = bh % p.Hq;
  const int g = h / p.G;
  const int q_end = p.len_q ? min(p.len_q[b], p.Lq) : p.Lq;
  const int kv_end = p.len_kv ? min(p.len_kv[b], p.Lk) : p.Lk;
  // Rows: as in the forward (heavy tiles first, or paired half-tiles for small grids).
  int wq_lo, row_lo, row_hi;
  if (CAUSAL && !p.pair_rows) {
    const int qt = (p.Lq + BM - 1) / BM - 1 - rank;
    wq_lo = qt * BM + wave * 32;
    row_lo = qt * BM;
    row_hi = row_lo + BM;
  } else if (CAUSAL) {
    constexpr int HB = BM / 2;
    const int n_half = (p.Lq + HB - 1) / HB;
    const int heavy = n_half - 1 - rank;
    const int mine = wave < NW / 2 ? rank : heavy;
    wq_lo = (wave >= NW / 2 && heavy == rank) ? p.Lq : mine * HB + (wave % (NW / 2)) * 32;
    row_lo = rank * HB;
    row_hi = (heavy + 1) * HB;
  } else {
    wq_lo = rank * BM + wave * 32;
    row_lo = rank * BM;
    row_hi = row_lo + BM;
  }
  const int wq_hi = min(wq_lo + 32, q_end) - 1;

  const bf16* qb = reinterpret_cast<const bf16*>(a.q) + b * p.q_sb + h * p.q_sh;
  const bf16* dob = reinterpret_cast<const bf16*>(a.dO) + b * p.o_sb + h * p.o_sh;
  const bf16* kb_ = reinterpret_cast<const bf16*>(a.k) + b * p.k_sb + g * p.k_sh;
  const bf16* vb_ = reinterpret_cast<const bf16*>(a.v) + b * p.v_sb + g * p.v_sh;
  const bf16* mb_ = MASK ? reinterpret_cast<const bf16*>(p.mask) + b * p.m_sb + h * p.m_sh : nullptr;

  int kv_stop = kv_end;
  if (CAUSAL) kv_stop = min(kv_stop, min(row_hi, q_end));
  if (row_lo >= q_end) kv_stop = 0;
  const int n_tiles = kv_stop > 0 ? (kv_stop + kBN - 1) / kBN : 0;

  const int qi = wq_lo + l32;  // this lane's query (N index)
  const bool qok = qi < q_end;
  bf16x8 qreg[D / 16], doreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qreg[kk] = __builtin_bit_cast(bf16x8, qok ? ld16(qb + (int64_t)qi * p.q_sl + kk * 16 + 8 * hi) : zero16());
    doreg[kk] = __builtin_bit_cast(bf16x8, qok ? ld16(dob + (int64_t)qi * p.o_sl + kk * 16 + 8 * hi) : zero16());
  }
  const int64_t rowid = ((int64_t)b * p.Hq + h) * p.Lq + qi;
  const float lse2 = qok ? a.lse2[rowid] : __builtin_inff();
  const float dsum = qok ? a.dsum[rowid] : 0.f;

  f32x16 dq_acc[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) dq_acc[mb] = f32x16{};

  auto load_tile = [&](int j0, bf16* Kd, bf16* Vd) {
    tile_to_lds_swz<kBN, D, NW>(kb_, p.k_sl, j0, kv_stop, Kd, wave, lane);
    tile_to_lds_swz<kBN, D, NW>(vb_, p.v_sl, j0, kv_stop, Vd, wave, lane);
  };
  const float c2 = p.scale_log2;
  const int krow_l = perm_row(l32);
  const int blk = lane >> 4;
  const int arow = (lane & 15) >> 2;
  const int tchunk = ((lane & 3) >> 1) + 2 * (blk & 1);
  const int thalf = 4 * (lane & 1);

  auto step = [&](int t, const bf16* Kt, const bf16* Vt, bf16* Kn, bf16* Vn)
                  __attribute__((always_inline)) {
    const int j0 = t * kBN;
    wait_vmem();
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(j0 + kBN, Kn, Vn);
    const bool partial_t = (j0 + kBN > kv_end) || (CAUSAL && j0 + kBN - 1 > wq_lo) ||
                           (wq_lo + 32 > q_end);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key_lo = j0 + kb * 32;
      if (!(wq_lo < q_end && key_lo < kv_stop && (!CAUSAL || key_lo <= wq_hi))) continue;
      // S^T = K Q^T and dP^T = V dO^T for keys key_lo + perm
      f32x16 s_acc = f32x16{}, dp_acc = f32x16{};
      {
        const int kr = kb * 32 + krow_l;

        bf16x8 op[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
          op[kk] = tile_row8<D>(Kt, kr, 2 * kk + hi);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) s_acc = mfma32(op[kk], qreg[kk], s_acc);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
          op[kk] = tile_row8<D>(Vt, kr, 2 * kk + hi);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) dp_acc = mfma32(op[kk], doreg[kk], dp_acc);
      }
      // lane holds query qi and keys key0 + v
      const int key0 = key_lo + 16 * hi;
      float mv[16];
      if (MASK) {
        if (p.mask_vec && qok && key0 + 16 <= p.Lk) {
          const bf16* mp = mb_ + (int64_t)qi * p.m_si + key0;
          bf16x8 b0 = __builtin_bit_cast(bf16x8, ld16(mp)), b1 = __builtin_bit_cast(bf16x8, ld16(mp + 8));
#pragma unroll
          for (int v = 0; v < 8; ++v) { mv[v] = bf2f(b0[v]) * kLog2e; mv[v + 8] = bf2f(b1[v]) * kLog2e; }
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            mv[v] = (qok && key0 + v < kv_end) ? bf2f(mb_[(int64_t)qi * p.m_si + key0 + v]) * kLog2e : 0.f;
        }
      }
      bf16x8 dsb[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) {
          const int v = half * 8 + t8;
          float x = fmaf(s_acc[v], c2, MASK ? mv[v] - lse2 : -lse2);
          if (partial_t) {
            const int key = key0 + v;
            const bool ok = key < kv_end && qok && (!CAUSAL || key <= qi);
            x = ok ? x : kNegInf;
          }
          const float pv = fast_exp2(x);
          dsb[half][t8] = (bf16)(pv * (dp_acc[v] - dsum));
        }
      }
      // dQ^T += K^T dS^T  (K^T via transposing LDS reads)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int tr = kb * 32 + 16 * hi + 8 * half + arow;  // rows tr .. tr + 7
        bf16x8 kT[D / 32];
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) kT[mb] = tile_tr8<D>(Kt, tr, tchunk + 4 * mb, thalf);
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) dq_acc[mb] = mfma32(kT[mb], dsb[half], dq_acc[mb]);
      }
    }
  };

  if (n_tiles > 0) load_tile(0, K0, V0);
  for (int t = 0; t < n_tiles; t += 2) {
    step(t, K0, V0, K1, V1);
    if (t + 1 < n_tiles) step(t + 1, K1, V1, K0, V0);
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

// Waves per workgroup of the two main kernels.
template <int D> struct BwdShape;
template <> struct BwdShape<64> { static constexpr int KV_NW = 4; static constexpr int Q_NW = 8; };
template <> struct BwdShape<128> { static constexpr int KV_NW = 4; static constexpr int Q_NW = 8; };

template <int D, bool CAUSAL, bool MASK>
hipError_t launch_main(const BwdArgs& a, int stages, hipStream_t s) {
  constexpr int KNW = BwdShape<D>::KV_NW, QNW = BwdShape<D>::Q_NW;
  const int n_kt = (a.p.Lk + 32 * KNW - 1) / (32 * KNW);
  if ((stages & kBwdDkdv) && n_kt > 0) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, KNW, CAUSAL, MASK>), dim3(n_kt * a.p.B * a.p.Hkv),
                       dim3(64 * KNW), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  constexpr int BM = 32 * QNW;
  const int n_qt = (a.p.Lq + BM - 1) / BM;
  BwdArgs args = a;
  args.p.pair_rows = CAUSAL && (int64_t)n_qt * a.p.B * a.p.Hq <= 512;
  const int n_wg = args.p.pair_rows ? ((a.p.Lq + BM / 2 - 1) / (BM / 2) + 1) / 2 : n_qt;
  if ((stages & kBwdDq) && n_wg > 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, QNW, CAUSAL, MASK>), dim3(n_wg * a.p.B * a.p.Hq),
                       dim3(64 * QNW), 0, s, args);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdArgs& a, int stages, hipStream_t s) {
  const int64_t rows = (int64_t)a.p.B * a.p.Hq * a.p.Lq;
  if ((stages & kBwdPrep) && rows > 0) {
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, a);
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
