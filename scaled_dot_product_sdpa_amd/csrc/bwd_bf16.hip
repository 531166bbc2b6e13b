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
// Three kernels (a fourth with the dS buffer), no atomics (the result is deterministic):
//  1. prep:  per row, D_i = sum_t dO_it O_it and lse2_i = LSE_i * log2(e) (+inf for a row
//            with no visible key or past the length, so that exp2(s - lse2) = 0 there),
//            both fp32 into the workspace.
//  2. dkdv:  key-stationary.  A workgroup owns 32 * NW keys of one (batch, KV head); each
//            wave keeps its 32 keys' K and V operands and their dK^T, dV^T accumulators in
//            registers, and walks the query heads of the group and their 64-row query
//            tiles.  Q, dO (and lse2, D) tiles stream HBM -> LDS with buffer loads through
//            three buffers (one barrier per tile).  Per 32x32 block:
//              S = Q K^T,  P = exp2(S * scale * log2e - lse2),  dP = dO V^T,
//              dS = P o (dP - D),  dV^T += dO^T P,  dK^T += Q^T dS
//            with dO^T and Q^T read from LDS by ds_read_b64_tr_b16.  Inside a wave the
//            blocks are software-pipelined: the dV, dK MFMAs of block b-1 run with the P, dS
//            arithmetic of block b, and the S, dP MFMAs of block b+1 with the rest of it.
//            At D = 128 (with a mask, when its rows allow 16-byte copies) each 32-key slice
//            is split over a pair of waves (S, P, dV in one; dP, dS, dK in the other, P
//            handed over through LDS), which fits two waves per SIMD where one wave holding
//            both needs ~320 registers.
//  3. dq:    query-stationary (the forward's decomposition, 4 waves of 32 rows).  Per
//            32-key block of a 64-key K/V tile (three LDS buffers, buffer-load copies):
//              S^T = K Q^T,  P^T,  dP^T = V dO^T,  dS^T = P^T o (dP^T - D),
//              dQ^T += K^T dS^T   (K^T via transposing LDS reads).
//            At D = 64 the blocks are software-pipelined inside each wave like the other
//            kernels (dQ one block late); at D = 128 that form needs more than the 256
//            registers two waves per SIMD allow, so each block runs start to finish.
//  4. dq from stored dS (D = 128, with the dS buffer in the workspace): the paired dK/dV
//            kernel also writes each bf16 dS block it forms, and dQ^T += K^T dS^T is then
//            one product per block that streams the stored blocks instead of recomputing
//            S, P and dP (see section 3c).  Still no atomics: each dQ element is written by
//            one lane.
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
    int i, h, b;
    if (nrows < ((int64_t)1 << 31)) {  // 32-bit index arithmetic (64-bit division is slow)
      const uint32_t r32 = (uint32_t)row, bh = r32 / (uint32_t)p.Lq;
      i = (int)(r32 - bh * (uint32_t)p.Lq);
      b = (int)(bh / (uint32_t)p.Hq);
      h = (int)(bh - (uint32_t)b * (uint32_t)p.Hq);
    } else {
      i = (int)(row % p.Lq);
      h = (int)((row / p.Lq) % p.Hq);
      b = (int)(row / ((int64_t)p.Lq * p.Hq));
    }
    const int q_end = seq_len_q(p, b);
    if (i < q_end) {
      valid = true;
      const int64_t off = o_base(p, b) + h * p.o_sh + (int64_t)i * p.o_sl + c * 8;
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
    // with a mask the kernels subtract LSE in natural units (see dkdv_body)
    a.lse2[row] = (l == kNegInf) ? __builtin_inff() : (a.p.mask ? l : l * kLog2e);
  }
}

// ---------------------------------------------------------------------------------------
// 2. dK, dV (key-stationary)
// ---------------------------------------------------------------------------------------
constexpr int kQT = 64;  // query rows per LDS tile (two 32-row blocks)

// LDS bytes of the dK/dV body: three Q, dO tiles, lse2/D rows and (with a mask) mask tiles.
template <int D, int NW, bool MASK>
constexpr int dkdv_lds_bytes() {
  return 3 * (2 * kQT * D * 2 + 2 * kQT * 4 + (MASK ? kQT * 32 * NW : 8) * 2);
}

// Workgroup `bid` of `nblk` (the dK/dV grid), LDS at smem.
template <int D, int NW, int CM, bool MASK>
__device__ __forceinline__ void dkdv_body(const BwdArgs& a, int bid, int nblk, char* smem) {
  constexpr bool CAUSAL = CM != 0;  // CM: 0 no diagonal, 1 causal, 2 causal + sliding window
  constexpr int KT = 32 * NW;    // keys per workgroup
  constexpr int TILE = kQT * D;
  constexpr int NS = D / 16;     // MFMAs of one S (or dP) block
  constexpr int NT = D / 32;     // MFMAs of one half of a dV (or dK) block
  constexpr int R1 = 4 * NT;     // slots of region 1 (dV, dK MFMAs)
  constexpr int R2 = 2 * NS;     // slots of region 2 (S, dP MFMAs)
  constexpr int E1 = 16 / R1;    // scores per lane per region-1 slot
  constexpr int MT = MASK ? kQT * KT : 8;
  // LDS operand reads issued ahead of their MFMA (transposed dV/dK operands, S/dP A
  // operands): an MFMA takes 32 cycles, a 16-byte LDS read several times that, and with
  // one wave per SIMD nothing else covers the wait; d = 128 has no registers to spare.
  constexpr int TPRE = D == 64 ? 3 : 2;
  constexpr int APRE = D == 64 ? 4 : 2;
  bf16* const Q0 = reinterpret_cast<bf16*>(smem);
  bf16* const Q1 = Q0 + TILE;
  bf16* const Q2 = Q1 + TILE;
  bf16* const G0 = Q2 + TILE;  // dO
  bf16* const G1 = G0 + TILE;
  bf16* const G2 = G1 + TILE;
  float* const R0 = reinterpret_cast<float*>(G2 + TILE);  // lse2 rows, then D rows
  float* const R1s = R0 + 2 * kQT;
  float* const R2s = R1s + 2 * kQT;
  // mask tiles (kQT rows x KT keys, unswizzled), used when mask rows allow 16-byte copies
  bf16* const M0 = reinterpret_cast<bf16*>(R2s + 2 * kQT);
  bf16* const M1 = M0 + MT;
  bf16* const M2 = M1 + MT;
  static_assert(6 * TILE * 2 + 6 * kQT * 4 + 3 * MT * 2 == dkdv_lds_bytes<D, NW, MASK>(), "LDS layout");

  const Problem& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Work item: (batch, KV head) group, then key tile kt; low key tiles see the most
  // (causal) queries and are launched first.
  int bg, kt;
  xcd_item(bid, p.B * p.Hkv, nblk / (p.B * p.Hkv), 1, !CAUSAL, bg, kt);
  const int b = batch_by_work(p, bg / p.Hkv);
  const int g = bg % p.Hkv;
  const int q_end = seq_len_q(p, b);
  const int kv_end = seq_len_kv(p, b);
  const int j0 = kt * KT;
  const int jw = j0 + wave * 32;  // this wave's first key
  const int myk = jw + l32;       // this lane's key (N index of S, dP)

  const bf16* kbase = reinterpret_cast<const bf16*>(a.k) + k_base(p, b) + g * p.k_sh;
  const bf16* vbase = reinterpret_cast<const bf16*>(a.v) + v_base(p, b) + g * p.v_sh;

  // Query tiles that can see any key of this workgroup; the G heads of the group in turn.
  const int kstop = min(kv_end, j0 + KT);
  // first query tile with a row that sees key j0 (row i sees it iff i >= j0 - coff)
  const int coff = CAUSAL ? causal_offset(p.causal, q_end, kv_end) : 0;
  const int qt_begin = CAUSAL ? max(j0 - coff, 0) / kQT : 0;
  // sliding window of W keys: row i sees key j only if i <= j - coff + W - 1, so rows past
  // kstop - coff + W - 2 see none of this workgroup's keys
  const int W = CM == 2 ? p.window : 0;
  const int q_last = W > 0 ? min(q_end, max(kstop - coff + W - 1, 0)) : q_end;
  const int qt_end = (j0 < kstop) ? (q_last + kQT - 1) / kQT : 0;
  const int n_q_tiles = qt_end > qt_begin ? qt_end - qt_begin : 0;
  const int total = n_q_tiles * p.G;
  // The query tiles of each head are walked last to first: every key tile of the group
  // starts at the same (last) query tile and walks the same sequence, so the workgroups of
  // a group that run at once on one XCD read each Q / dO tile from its L2 (walking from
  // each key tile's own diagonal instead, they would stream the rows out of step and
  // thrash the L2).
  auto tile_rows = [&](int it, int& h, int& i0) {
    h = g * p.G + it / n_q_tiles;
    i0 = (qt_end - 1 - it % n_q_tiles) * kQT;
  };

  // ---- tiles HBM -> LDS: Q and dO rows (swizzled), lse2 and D rows, mask rows.
  TileCopy<kQT, D, NW> qcopy, gcopy;
  qcopy.init(p.q_sl, wave, lane);
  gcopy.init(p.o_sl, wave, lane);
  constexpr int MCPR = KT / 8, MPW = kQT * MCPR / 64 / NW;  // mask: 16-byte chunks per row, per wave
  uint32_t mvoff[MASK ? MPW : 1];
  if (MASK) {
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
      const int ci = (wave * MPW + i) * 64 + lane;
      mvoff[i] = (uint32_t)((ci / MCPR) * p.m_si * 2 + (ci % MCPR) * 16);
    }
  }
  auto load_tile = [&](int it, bf16* Qd, bf16* Gd, float* Rd, bf16* Md) {
    int h, i0;
    tile_rows(it, h, i0);
    const bf16* qb = reinterpret_cast<const bf16*>(a.q) + q_base(p, b) + h * p.q_sh;
    const bf16* dob = reinterpret_cast<const bf16*>(a.dO) + o_base(p, b) + h * p.o_sh;
    qcopy.copy(rows_rsrc<D, kQT>(qb, p.q_sl, i0, q_end), Qd, wave);
    gcopy.copy(rows_rsrc<D, kQT>(dob, p.o_sl, i0, q_end), Gd, wave);
    const int uw = __builtin_amdgcn_readfirstlane(wave);
    if (uw < 2) {
      // lse2 (wave 0) and D (wave 1) of the tile's rows; rows past Lq arrive as zeros and
      // are masked by the predicates
      const int64_t rb = ((int64_t)b * p.Hq + h) * p.Lq + i0;
      const float* src = (uw ? a.dsum : a.lse2) + rb;
      buffer_to_lds<4>(raw_rsrc(src, (int64_t)max(min(p.Lq - i0, kQT), 0) * 4), Rd, uw * kQT * 4, lane * 4);
    }
    if (MASK && p.mask_vec) {
      // keys past Lk read the next row (or zeros past the end); those pairs are masked
      const bf16* mb = reinterpret_cast<const bf16*>(p.mask) + b * p.m_sb + h * p.m_sh +
                       (int64_t)i0 * p.m_si + j0;
      const int nr = min(p.Lq - i0, kQT);
      const i32x4 rs = raw_rsrc(mb, nr > 0 ? (int64_t)(nr - 1) * p.m_si * 2 + (p.Lk - j0) * 2 : 0);
      const int mw = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
      for (int i = 0; i < MPW; ++i) buffer_to_lds<16>(rs, Md, (mw * MPW + i) * 1024, mvoff[i]);
    }
  };

  // Tile 0 and the K, V operands of this lane's key (B operands of S = Q K^T and
  // dP = dO V^T) land first; tile 1 streams in behind the first block.
  if (total > 0) load_tile(0, Q0, G0, R0, M0);
  bf16x8 kreg[NS], vreg[NS];
#pragma unroll
  for (int kk = 0; kk < NS; ++kk) {
    const bool ok = myk < kv_end;
    kreg[kk] = __builtin_bit_cast(bf16x8, ok ? ld16(kbase + (int64_t)myk * p.k_sl + kk * 16 + 8 * hi) : zero16());
    vreg[kk] = __builtin_bit_cast(bf16x8, ok ? ld16(vbase + (int64_t)myk * p.v_sl + kk * 16 + 8 * hi) : zero16());
  }
  wait_vmem();
  if (total > 1) load_tile(1, Q1, G1, R1s, M1);

  f32x16 dk_acc[NT], dv_acc[NT];
#pragma unroll
  for (int mb = 0; mb < NT; ++mb) { dk_acc[mb] = f32x16{}; dv_acc[mb] = f32x16{}; }

  const float c2 = p.scale_log2;
  const float sc = p.scale;
  const int qr = perm_row(l32);  // Q / dO row read by this lane (A operands of S, dP)
  const int blk = lane >> 4;
  const int arow = (lane & 15) >> 2;
  const int tchunk = ((lane & 3) >> 1) + 2 * (blk & 1);
  const int thalf = 4 * (lane & 1);

  // dV, dK of a block run one block late: B operands bf16 P and dS (zero before the first
  // block), A operands transposed dO and Q read from the block's tile just in time.
  bf16x8 pd_a[4], pd_b[4];  // P half 0, P half 1, dS half 0, dS half 1
#pragma unroll
  for (int i = 0; i < 4; ++i) { pd_a[i] = bf16x8{}; pd_b[i] = bf16x8{}; }
  // MFMA j of a block's dV, dK: dV half 0, dK half 0, dV half 1, dK half 1, NT d-blocks each
  OpOffsets<D> ofs;  // operand reads (A operands of row qr, transposed dO and Q)
  ofs.init(qr, hi, arow, tchunk, thalf);
  auto tr_op = [&](int j, const bf16* Qt, const bf16* Gt, int kb) {
    const int half = j / (2 * NT), which = (j / NT) % 2, mb = j % NT;
    return ofs.tr8(which ? Qt : Gt, kb * 32 + 8 * half, mb);  // rows kb*32 + 16hi + 8half + arow ..
  };
  auto dvdk_mfma = [&](int j, bf16x8 op, const bf16x8 (&pd)[4]) {
    const int half = j / (2 * NT), which = (j / NT) % 2, mb = j % NT;
    if (which == 0) dv_acc[mb] = mfma32(op, pd[half], dv_acc[mb]);
    else dk_acc[mb] = mfma32(op, pd[2 + half], dk_acc[mb]);
  };

  // ---- one pipeline phase for block bi (rows kb*32.. of the tile in Qc/Gc/Rc/Mc; the
  // next block's rows kbn*32.. of Qn/Gn).  Region 1: dV, dK MFMAs of block bi-1 with the
  // P and dS arithmetic of block bi.  Region 2: S, dP MFMAs of block bi+1 with the rest of
  // that arithmetic, the A-operand reads of block bi+1 and the transposed reads of block bi.
  // All blocks of the tiles are computed (pairs a wave cannot see get P = 0), so every
  // phase has the same shape; S, dP of the block after a wave's last are never used.
  auto phase = [&](int bi, const bf16* Qp, const bf16* Gp, int kbp, const bf16* Qc, const bf16* Gc,
                   const float* Rc, const bf16* Mc, int kb, const bf16* Qn, const bf16* Gn, int kbn,
                   f32x16& s, f32x16& dp, f32x16& s_nx, f32x16& dp_nx, const bf16x8 (&pd_prev)[4],
                   bf16x8 (&pd)[4]) __attribute__((always_inline)) {
    const int it = bi >> 1;
    int h, i0;
    tile_rows(it, h, i0);
    const int r0 = i0 + kb * 32;  // first query row of the block
    // lane holds key myk and queries r0 + 16*hi + v
    // lse2 and D of the lane's 16 rows, four at a time, read a few slots ahead of use
    const f32x4* lr = reinterpret_cast<const f32x4*>(Rc + kb * 32 + 16 * hi);
    const f32x4* dr = reinterpret_cast<const f32x4*>(Rc + kQT + kb * 32 + 16 * hi);
    f32x4 l4[4], d4[4];
    l4[0] = lr[0];
    d4[0] = dr[0];
    float mbias[16];
    if (MASK) {
      if (p.mask_vec) {
#pragma unroll
        for (int v = 0; v < 16; ++v) mbias[v] = bf2f(Mc[(kb * 32 + 16 * hi + v) * KT + wave * 32 + l32]);
      } else {
        const bf16* mrow = reinterpret_cast<const bf16*>(p.mask) + b * p.m_sb + h * p.m_sh;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int qi = r0 + 16 * hi + v;
          const bool in = qi < q_end && myk < kv_end;
          mbias[v] = in ? bf2f(mrow[(int64_t)qi * p.m_si + myk]) : 0.f;
        }
      }
    }
    const bool partial = (jw + 32 > kv_end) || (r0 + 32 > q_end) || (CAUSAL && r0 + coff < jw + 31) ||
                         (W > 0 && jw <= r0 + 31 + coff - W);
    if (partial) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int qi = r0 + 16 * hi + v;
        const bool ok = (myk < kv_end) & (qi < q_end) & (!CAUSAL | (myk <= qi + coff)) &
                        ((W == 0) | (myk > qi + coff - W));
        s[v] = ok ? s[v] : kNegInf;
      }
    }
    // P and dS in three stages one slot apart: A (exp2 argument, dP - D), B (exp2),
    // C (dS and the bf16 operands)
    float xv[16], dd[16];
    // The exp2 argument.  With a mask, scale * s + m - LSE is formed in natural units (the
    // prep kernel then stores LSE itself) and only the difference goes to log2 units: m
    // near the bottom of the fp32 range times log2(e) would overflow.
    auto st_a = [&](int e) {
      const float l2 = l4[e / 4][e % 4];
      xv[e] = MASK ? (fmaf(s[e], sc, mbias[e]) - l2) * kLog2e : fmaf(s[e], c2, -l2);
      dd[e] = dp[e] - d4[e / 4][e % 4];
    };
    auto st_b = [&](int e) { xv[e] = fast_exp2(xv[e]); };
    auto st_c = [&](int e) {
      dd[e] = xv[e] * dd[e];
      if (e & 1) {
        const int half = e / 8, t = e % 8;
        f32x2 pp = {xv[e - 1], xv[e]}, ss = {dd[e - 1], dd[e]};
        const bf16x2 p2 = __builtin_convertvector(pp, bf16x2), s2 = __builtin_convertvector(ss, bf16x2);
        pd[half][t - 1] = p2[0];
        pd[half][t] = p2[1];
        pd[2 + half][t - 1] = s2[0];
        pd[2 + half][t] = s2[1];
      }
    };
    // region 1
    bf16x8 aop[R2], top[R1];
#pragma unroll
    for (int j = 0; j < TPRE; ++j) top[j] = tr_op(j, Qp, Gp, kbp);
#pragma unroll
    for (int j = 0; j < R1; ++j) {
      if (j + TPRE < R1) top[j + TPRE] = tr_op(j + TPRE, Qp, Gp, kbp);
      if (j >= R1 - APRE) {  // the first A operands of block bi+1
        const int i = j - (R1 - APRE);
        aop[i] = ofs.row8((i & 1) ? Gn : Qn, kbn * 32, i >> 1);
      }
      if ((j * E1) % 4 == 0 && j * E1 / 4 + 1 < 4) {
        l4[j * E1 / 4 + 1] = lr[j * E1 / 4 + 1];
        d4[j * E1 / 4 + 1] = dr[j * E1 / 4 + 1];
      }
      dvdk_mfma(j, top[j], pd_prev);
#pragma unroll
      for (int e = j * E1; e < (j + 1) * E1; ++e) st_a(e);
#pragma unroll
      for (int e = (j - 1) * E1; e < j * E1; ++e)
        if (e >= 0) st_b(e);
#pragma unroll
      for (int e = (j - 2) * E1; e < (j - 1) * E1; ++e)
        if (e >= 0) st_c(e);
      __builtin_amdgcn_sched_barrier(0);
    }
    // region 2
    s_nx = f32x16{};
    dp_nx = f32x16{};
#pragma unroll
    for (int i = 0; i < R2; ++i) {
      if (i + APRE < R2) {
        const int n = i + APRE;
        aop[n] = ofs.row8((n & 1) ? Gn : Qn, kbn * 32, n >> 1);
      }
      if (i & 1) dp_nx = mfma32(aop[i], vreg[i >> 1], dp_nx);
      else s_nx = mfma32(aop[i], kreg[i >> 1], s_nx);
      if (i == 0) {
#pragma unroll
        for (int e = (R1 - 1) * E1; e < R1 * E1; ++e) st_b(e);
#pragma unroll
        for (int e = (R1 - 2) * E1; e < (R1 - 1) * E1; ++e) st_c(e);
      }
      if (i == 1) {
#pragma unroll
        for (int e = (R1 - 1) * E1; e < R1 * E1; ++e) st_c(e);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // this block's P and dS stay computed inside this phase (see pin)
#pragma unroll
    for (int i = 0; i < 4; ++i) pin(pd[i]);
  };

  // One tile step (two blocks); unrolled by three over the LDS buffers (see the forward).
  f32x16 s_a = f32x16{}, dp_a = f32x16{}, s_b = f32x16{}, dp_b = f32x16{};
  // Tile t-1 (the previous block's transposed operands) is only overwritten after the
  // barrier in the middle of step t.
  auto step = [&](int t, const bf16* Qp, const bf16* Gp, const bf16* Qc, const bf16* Gc,
                  const float* Rc, const bf16* Mc, const bf16* Qn, const bf16* Gn, bf16* Ql,
                  bf16* Gl, float* Rl, bf16* Ml) __attribute__((always_inline)) {
    ofs.repin();
    phase(2 * t, Qp, Gp, 1, Qc, Gc, Rc, Mc, 0, Qc, Gc, 1, s_a, dp_a, s_b, dp_b, pd_b, pd_a);
    if (t + 1 < total) wait_vmem();
    __syncthreads();
    if (t + 2 < total) load_tile(t + 2, Ql, Gl, Rl, Ml);
    phase(2 * t + 1, Qc, Gc, 0, Qc, Gc, Rc, Mc, 1, Qn, Gn, 0, s_b, dp_b, s_a, dp_a, pd_a, pd_b);
  };

  if (total > 0) {
    // the first phase runs the dV, dK MFMAs of "block -1" (rows 32..63 of buffer 2) with
    // zero weights: those rows are zeroed so the products are exactly zero
    lds_zero<32 * D * 2, 64 * NW>(Q2 + 32 * D, tid);
    lds_zero<32 * D * 2, 64 * NW>(G2 + 32 * D, tid);
    __syncthreads();  // every wave's share of tile 0 has landed; the zeros are visible
#pragma unroll
    for (int i = 0; i < R2; ++i) {
      const bf16x8 op = ofs.row8((i & 1) ? G0 : Q0, 0, i >> 1);
      if (i & 1) dp_a = mfma32(op, vreg[i >> 1], dp_a);
      else s_a = mfma32(op, kreg[i >> 1], s_a);
    }
  }
  for (int t = 0; t < total; t += 3) {
    step(t, Q2, G2, Q0, G0, R0, M0, Q1, G1, Q2, G2, R2s, M2);
    if (t + 1 < total) step(t + 1, Q0, G0, Q1, G1, R1s, M1, Q2, G2, Q0, G0, R0, M0);
    if (t + 2 < total) step(t + 2, Q1, G1, Q2, G2, R2s, M2, Q0, G0, Q1, G1, R1s, M1);
  }
  // the last block's dV, dK (second block of tile total-1, buffer (total-1) % 3)
  if (total > 0) {
    const int lb = (total - 1) % 3;
    const bf16* Ql = lb == 0 ? Q0 : (lb == 1 ? Q1 : Q2);
    const bf16* Gl = lb == 0 ? G0 : (lb == 1 ? G1 : G2);
#pragma unroll
    for (int j = 0; j < R1; ++j) dvdk_mfma(j, tr_op(j, Ql, Gl, 1), pd_b);
  }

  // Epilogue: lane holds key myk, d = mb*32 + (v/4)*8 + 4*hi + v%4.
  if (myk < kv_rows_out(p, kv_end)) {
    bf16* dkrow = reinterpret_cast<bf16*>(a.dk) + k_base(p, b) + g * p.k_sh + (int64_t)myk * p.k_sl;
    bf16* dvrow = reinterpret_cast<bf16*>(a.dv) + v_base(p, b) + g * p.v_sh + (int64_t)myk * p.v_sl;
#pragma unroll
    for (int mb = 0; mb < NT; ++mb) {
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

template <int D, int NW, int CM, bool MASK>
__global__ __launch_bounds__(64 * NW, 1) void bwd_dkdv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[dkdv_lds_bytes<D, NW, MASK>()];
  dkdv_body<D, NW, CM, MASK>(a, blockIdx.x, gridDim.x, smem);
}

// ---------------------------------------------------------------------------------------
// 2b. dK, dV with each 32-key slice worked by a pair of waves
// ---------------------------------------------------------------------------------------
// Same decomposition and grid as the dK/dV body (a workgroup owns 32 * NP keys of one
// (batch, KV head) and walks the group's query tiles through three LDS buffers), but each
// 32-key slice is split over two waves by the products it feeds:
//   wave w < NP ("P wave"):   S = Q K^T,  P = exp2(S * scale * log2e - lse2),  dV^T += dO^T P
//                             (with a mask, P = exp2((S * scale + m - LSE) * log2e))
//   wave w + NP ("dS wave"):  dP = dO V^T,  dS = P o (dP - D),                  dK^T += Q^T dS
// The P wave hands P (fp32, in its own accumulator layout: lane = key, 16 query rows) to
// its partner through LDS, one barrier per 32-row block.  Each wave then holds one operand
// (K or V) and one accumulator (dV^T or dK^T) instead of both, which fits two waves per SIMD
// (the single-wave form needs ~320 registers); the two waves of a SIMD are one P wave and
// one dS wave, so the exponentials of one run under the other's MFMAs.  dS is formed from
// the same fp32 P and dP as in the single-wave body, so both give the same results.
//
// Phase k (between barriers k-1 and k) runs the S, P (or dP) of block k and the dV (or dK)
// of block k-1; the dS wave forms dS of block k-1 from the P its partner stored in phase
// k-1.  Block k is rows (k % 2) * 32 of tile k / 2.  Tile t+2 is copied into the buffer of
// tile t-1 after barrier 2t (the last phase reading tile t-1 is 2t) and must have landed by
// barrier 2t+3.
// With a mask (rows that allow 16-byte copies), each block's 32 mask rows of the workgroup's
// keys are copied by the eight waves (one 1 KB copy each) into three 8 KB buffers: block
// k+3's after barrier k, into the buffer block k used, landed by barrier k+2 (the copy of a
// block goes before the tile copied with it, so waiting for it leaves the tile in flight).
template <int D, int NP, bool MASK>
constexpr int dkdv_pair_lds_bytes() {
  return 3 * (2 * kQT * D * 2 + 2 * kQT * 4) + 2 * NP * 64 * 16 * 4 + (MASK ? 3 * 32 * 32 * NP * 2 : 0);
}

// A compile-time flag passed as an argument, so that the generic phase and step lambdas
// below are instantiated separately for the first and last phases.
template <bool V> struct Role { static constexpr bool value = V; };

// The waves of one role (PW: P waves, else dS waves).  STORE: the dS waves also write each
// block's bf16 dS to the dS buffer (BwdArgs::ds) for the dQ-from-dS kernel, and the P waves
// alone copy the tiles and masks.  The vector-memory counter completes loads, copies and
// stores in issue order, so a wave's copy cannot count as landed before that wave's earlier
// stores are acknowledged, which for stores that go out to HBM takes longer than the copy
// pipeline allows (measured: the copy waits then stall the kernel by a sixth).  The dS
// waves therefore issue no copies and never wait on the counter; the barriers order them.
template <bool PW, int D, int NP, int CM, bool MASK, bool STORE>
__device__ __forceinline__ void dkdv_pair_wave(const BwdArgs& a, int bid, int nblk, char* smem) {
  constexpr bool CAUSAL = CM != 0;
  constexpr int NW = 2 * NP;
  constexpr int KT = 32 * NP;    // keys per workgroup
  constexpr int TILE = kQT * D;
  constexpr int NS = D / 16;     // MFMAs of one S (or dP) block
  constexpr int NT = D / 32;     // d-blocks of dV (or dK)
  constexpr int NM = NS + 2 * NT;  // MFMAs of one phase
  constexpr int PRE = 3;         // LDS operand reads issued ahead of their MFMA
  bf16* const Q0 = reinterpret_cast<bf16*>(smem);
  bf16* const Q1 = Q0 + TILE;
  bf16* const Q2 = Q1 + TILE;
  bf16* const G0 = Q2 + TILE;  // dO
  bf16* const G1 = G0 + TILE;
  bf16* const G2 = G1 + TILE;
  float* const R0 = reinterpret_cast<float*>(G2 + TILE);  // lse2 rows, then D rows
  float* const R1s = R0 + 2 * kQT;
  float* const R2s = R1s + 2 * kQT;
  char* const Pex = reinterpret_cast<char*>(R2s + 2 * kQT);  // [2][NP][64 lanes x 16 fp32]
  constexpr int MBLK = 32 * KT;  // mask rows of one block
  bf16* const Mk = reinterpret_cast<bf16*>(Pex + 2 * NP * 4096);  // [3][32 rows x KT keys]
  static_assert(6 * TILE * 2 + 6 * kQT * 4 + 2 * NP * 4096 + (MASK ? 3 * MBLK * 2 : 0) ==
                    dkdv_pair_lds_bytes<D, NP, MASK>(), "LDS layout");

  const Problem& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int pair = wave % NP;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int bg, kt;
  xcd_item(bid, p.B * p.Hkv, nblk / (p.B * p.Hkv), 1, !CAUSAL, bg, kt);
  const int b = batch_by_work(p, bg / p.Hkv);
  const int g = bg % p.Hkv;
  const int q_end = seq_len_q(p, b);
  const int kv_end = seq_len_kv(p, b);
  const int j0 = kt * KT;
  const int jw = j0 + pair * 32;  // the pair's first key
  const int myk = jw + l32;       // this lane's key

  const int kstop = min(kv_end, j0 + KT);
  const int coff = CAUSAL ? causal_offset(p.causal, q_end, kv_end) : 0;
  const int qt_begin = CAUSAL ? max(j0 - coff, 0) / kQT : 0;
  const int W = CM == 2 ? p.window : 0;
  const int q_last = W > 0 ? min(q_end, max(kstop - coff + W - 1, 0)) : q_end;
  const int qt_end = (j0 < kstop) ? (q_last + kQT - 1) / kQT : 0;
  const int n_q_tiles = qt_end > qt_begin ? qt_end - qt_begin : 0;
  const int total = n_q_tiles * p.G;
  // query tiles last to first, the group's heads in turn (see the dK/dV body)
  auto tile_rows = [&](int it, int& h, int& i0) __attribute__((always_inline)) {
    h = g * p.G + it / n_q_tiles;
    i0 = (qt_end - 1 - it % n_q_tiles) * kQT;
  };

  // Tiles HBM -> LDS by the CW copying waves (all NW, or the P waves of a storing kernel).
  // The row copies (lse2 by wave 0, D by wave 1) go first, so that every wave has at most
  // TPW copies of a tile issued after the previous tile's.
  constexpr bool CP = !STORE || PW;  // this wave copies
  constexpr int CW = STORE ? NP : NW;
  static_assert(NP >= 2, "waves 0 and 1 (P waves) copy the row values");
  TileCopy<kQT, D, CW> qcopy, gcopy;
  qcopy.init(p.q_sl, CP ? wave : 0, lane);
  gcopy.init(p.o_sl, CP ? wave : 0, lane);
  auto load_tile = [&](int it, bf16* Qd, bf16* Gd, float* Rd) __attribute__((always_inline)) {
    int h, i0;
    tile_rows(it, h, i0);
    const int uw = __builtin_amdgcn_readfirstlane(wave);
    if (uw < 2) {
      const int64_t rb = ((int64_t)b * p.Hq + h) * p.Lq + i0;
      const float* src = (uw ? a.dsum : a.lse2) + rb;
      buffer_to_lds<4>(raw_rsrc(src, (int64_t)max(min(p.Lq - i0, kQT), 0) * 4), Rd, uw * kQT * 4, lane * 4);
    }
    const bf16* qb = reinterpret_cast<const bf16*>(a.q) + q_base(p, b) + h * p.q_sh;
    const bf16* dob = reinterpret_cast<const bf16*>(a.dO) + o_base(p, b) + h * p.o_sh;
    if constexpr (CP) {
      qcopy.copy(rows_rsrc<D, kQT>(qb, p.q_sl, i0, q_end), Qd, wave);
      gcopy.copy(rows_rsrc<D, kQT>(dob, p.o_sl, i0, q_end), Gd, wave);
    }
  };
  constexpr int TPW = 2 * TileCopy<kQT, D, CW>::PER_WAVE;  // tile copies per copying wave
  // Mask rows of block k (32 rows x KT keys, 16-byte chunks, row-major) into Mk[k % 3]:
  // chunks (wave * MPW + i) * 64 + lane; keys past Lk read the next row (or zeros past the
  // end), and those pairs are masked by the predicates.
  const int nb = 2 * total;
  constexpr int MPW = 32 * KT / 8 / (64 * CW);  // mask copies per copying wave and block
  static_assert(!MASK || MPW * 64 * CW == 32 * KT / 8, "whole mask chunks per lane and block");
  uint32_t mvoff[MPW];
#pragma unroll
  for (int i = 0; i < MPW; ++i) {
    const int ci = ((CP ? wave : 0) * MPW + i) * 64 + lane;
    mvoff[i] = MASK ? (uint32_t)((ci / (KT / 8)) * p.m_si * 2 + (ci % (KT / 8)) * 16) : 0u;
  }
  auto load_mask = [&](int k) __attribute__((always_inline)) {
    if (!MASK || !CP || k >= nb) return;
    int h, i0;
    tile_rows(k >> 1, h, i0);
    const int r0 = i0 + (k & 1) * 32;
    const bf16* mb = reinterpret_cast<const bf16*>(p.mask) + b * p.m_sb + h * p.m_sh + (int64_t)r0 * p.m_si + j0;
    const int nr = min(p.Lq - r0, 32);
    const i32x4 rs = raw_rsrc(mb, nr > 0 ? (int64_t)(nr - 1) * p.m_si * 2 + (p.Lk - j0) * 2 : 0);
#pragma unroll
    for (int i = 0; i < MPW; ++i) buffer_to_lds<16>(rs, Mk + (k % 3) * MBLK, (wave * MPW + i) * 1024, mvoff[i]);
  };
  // Wait until the copies issued after the mask (or tile) that the next barrier publishes
  // are the only ones in flight: one tile's copies (one more for the waves that also copy
  // the row values) and one block's mask.
  auto wait_tile_and_mask = [&]() __attribute__((always_inline)) {
    if (wave < 2) wait_vmem_le<TPW + MPW + 1>();
    else wait_vmem_le<TPW + MPW>();
  };

  const float c2 = p.scale_log2;
  const float sc = p.scale;
  const int qr = perm_row(l32);
  const int blk = lane >> 4;
  const int arow = (lane & 15) >> 2;
  const int tchunk = ((lane & 3) >> 1) + 2 * (blk & 1);
  const int thalf = 4 * (lane & 1);
  const uint32_t dso = (uint32_t)(l32 * 64 + hi * 32);  // this lane's bytes of a dS^T block

  {
    // K (P wave) or V (dS wave) of this lane's key: B operand of S or dP
    if (total > 0) load_tile(0, Q0, G0, R0);
    load_mask(0);
    load_mask(1);
    bf16x8 kv[NS];
    {
      const bf16* base = reinterpret_cast<const bf16*>(PW ? a.k : a.v) +
                         (PW ? k_base(p, b) + g * p.k_sh : v_base(p, b) + g * p.v_sh);
      const int64_t sl = PW ? p.k_sl : p.v_sl;
      const bool ok = myk < kv_end;
#pragma unroll
      for (int kk = 0; kk < NS; ++kk)
        kv[kk] = __builtin_bit_cast(bf16x8, ok ? ld16(base + (int64_t)myk * sl + kk * 16 + 8 * hi) : zero16());
    }
    wait_vmem();
    load_mask(2);
    if (total > 1) load_tile(1, Q1, G1, R1s);

    f32x16 acc[NT];
#pragma unroll
    for (int mb = 0; mb < NT; ++mb) acc[mb] = f32x16{};
    // The dO tiles follow the three Q tiles; the operand offsets of the dO reads (transposed
    // in the P wave, rows in the dS wave) carry the Q tiles' bytes and the reads go through
    // dO pointers moved back by as much, so every read's buffer lies within its 16-bit
    // offset field.
    constexpr int GB = 3 * TILE;
    OpOffsets<D> ofs;
    ofs.init(qr, hi, arow, tchunk, thalf, PW ? 0 : GB * 2, PW ? GB * 2 : 0);

    // One phase.  FIRST: no block k-1; LAST: no block k.  Cur/kb: tile and rows of block k;
    // Prv/kbp: those of block k-1.  P wave: cur_bf receives bf16 P of block k, prv_bf holds
    // that of block k-1.  dS wave: cur_dp receives dP of block k, prv_dp holds dP of block
    // k-1.
    auto phase = [&](auto first_t, auto last_t, int k, const bf16* Qc, const bf16* Gc, const float* Rc, int kb,
                     const bf16* Qp, const bf16* Gp, const float* Rp, int kbp, bf16x8 (&cur_bf)[2],
                     const bf16x8 (&prv_bf)[2], f32x16& cur_dp, f32x16& prv_dp) __attribute__((always_inline)) {
      constexpr bool FIRST = decltype(first_t)::value, LAST = decltype(last_t)::value;
      constexpr int n_lo = LAST ? NS : 0, n_hi = FIRST ? NS : NM;
      // operand n: A of the S/dP MFMAs (rows of Q or dO), then the transposed A of the
      // dV/dK MFMAs (dO^T or Q^T of block k-1)
      auto opr = [&](int n) __attribute__((always_inline)) {
        if (n < NS) return ofs.row8(PW ? Qc : Gc - GB, kb * 32, n);
        const int j = n - NS;
        return ofs.tr8(PW ? Gp - GB : Qp, kbp * 32 + 8 * (j / NT), j % NT);
      };
      bf16x8 op[NM];
#pragma unroll
      for (int n = n_lo; n < n_lo + PRE && n < n_hi; ++n) op[n] = opr(n);
      f32x16 s = f32x16{};  // S (P wave) or dP (dS wave) of block k
      char* const pex_w = Pex + ((k & 1) * NP + pair) * 4096 + lane * 16;      // block k
      const char* const pex_r = Pex + (((k + 1) & 1) * NP + pair) * 4096 + lane * 16;  // block k-1
      float xv[16];
      bf16x8 ds[2];
      f32x4 d4[4];
      if constexpr (!PW && !FIRST) {
        // P of block k-1 (stored by the partner before the last barrier) and D of its rows
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const f32x4 pc = *reinterpret_cast<const f32x4*>(pex_r + c * 1024);
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[4 * c + e] = pc[e];
          d4[c] = reinterpret_cast<const f32x4*>(Rp + kQT + kbp * 32 + 16 * hi)[c];
        }
      }
      // dS of block k-1 for the scores of slot n (E per slot), into the bf16 B operands
      constexpr int E = 16 / NS;
      auto ds_slot = [&](int n) __attribute__((always_inline)) {
#pragma unroll
        for (int e = n * E; e < (n + 1) * E; e += 2) {
          xv[e] *= prv_dp[e] - d4[e / 4][e % 4];
          xv[e + 1] *= prv_dp[e + 1] - d4[e / 4][(e + 1) % 4];
          const f32x2 ss = {xv[e], xv[e + 1]};
          const bf16x2 s2 = __builtin_convertvector(ss, bf16x2);
          ds[e / 8][e % 8] = s2[0];
          ds[e / 8][e % 8 + 1] = s2[1];
        }
      };
      // Block k-1's dS to the dS buffer as its 32 x 32 dS^T block: this lane's key row, its
      // 16 queries (one 32-byte half of the 64-byte row).  The storing waves issue no copies,
      // so these stores hold up no copy wait.
      auto store_ds = [&]() __attribute__((always_inline)) {
        if constexpr (STORE && !PW && !FIRST) {
          int hp, i0p;
          tile_rows((k - 1) >> 1, hp, i0p);
          const int qb = (i0p >> 5) + kbp;
          const int64_t blk_i = (((int64_t)b * p.Hq + hp) * a.ds_nqb + qb) * a.ds_nkb + (jw >> 5);
          const reg_rsrc_t rs = reg_rsrc(reinterpret_cast<const bf16*>(a.ds) + blk_i * 1024, 2048);
          // non-temporal: 2 bytes per visible pair that the dQ pass reads once, after this
          // kernel; they should not push the group's Q and dO rows out of L2
          reg_st16<kNonTemporalPolicy>(rs, dso, 0, __builtin_bit_cast(u32x4, ds[0]));
          reg_st16<kNonTemporalPolicy>(rs, dso + 16, 0, __builtin_bit_cast(u32x4, ds[1]));
        }
      };
      if constexpr (!PW && LAST) {
#pragma unroll
        for (int n = 0; n < NS; ++n) ds_slot(n);
        store_ds();
      }
      // P of block k (P wave): lane holds key myk and query rows r0 + 16*hi + v.  The
      // exponentials run in the dV MFMA slots once S is complete (after the loop in the
      // first phase, which has no dV slots); each finished group of four is stored for the
      // partner.
      int r0 = 0;
      f32x4 l4[4];
      if constexpr (PW && !LAST) {
        int h, i0;
        tile_rows(k >> 1, h, i0);
        (void)h;
        r0 = i0 + kb * 32;
#pragma unroll
        for (int c = 0; c < 4; ++c) l4[c] = reinterpret_cast<const f32x4*>(Rc + kb * 32 + 16 * hi)[c];
      }
      // the mask values of the lane's key and rows (copied before the last barrier)
      float mbias[16];
      if constexpr (PW && !LAST && MASK) {
        const bf16* mc = Mk + (k % 3) * MBLK + 16 * hi * KT + pair * 32 + l32;
#pragma unroll
        for (int v = 0; v < 16; ++v) mbias[v] = bf2f(mc[v * KT]);
      }
      auto p_mask = [&]() __attribute__((always_inline)) {
        const bool partial = (jw + 32 > kv_end) || (r0 + 32 > q_end) || (CAUSAL && r0 + coff < jw + 31) ||
                             (W > 0 && jw <= r0 + 31 + coff - W);
        if (partial) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int qi = r0 + 16 * hi + v;
            const bool ok = (myk < kv_end) & (qi < q_end) & (!CAUSAL | (myk <= qi + coff)) &
                            ((W == 0) | (myk > qi + coff - W));
            s[v] = ok ? s[v] : kNegInf;
          }
        }
      };
      auto p_scores = [&](int e0, int e1) __attribute__((always_inline)) {
#pragma unroll
        for (int e = e0; e < e1; e += 2) {
          // with a mask, scale * s + m - LSE in natural units (the prep kernel then stores
          // LSE itself), and only the difference goes to log2 units
          if constexpr (MASK) {
            xv[e] = fast_exp2((fmaf(s[e], sc, mbias[e]) - l4[e / 4][e % 4]) * kLog2e);
            xv[e + 1] = fast_exp2((fmaf(s[e + 1], sc, mbias[e + 1]) - l4[e / 4][(e + 1) % 4]) * kLog2e);
          } else {
            xv[e] = fast_exp2(fmaf(s[e], c2, -l4[e / 4][e % 4]));
            xv[e + 1] = fast_exp2(fmaf(s[e + 1], c2, -l4[e / 4][(e + 1) % 4]));
          }
          const f32x2 pp = {xv[e], xv[e + 1]};
          const bf16x2 p2 = __builtin_convertvector(pp, bf16x2);
          cur_bf[e / 8][e % 8] = p2[0];
          cur_bf[e / 8][e % 8 + 1] = p2[1];
          if ((e + 2) % 4 == 0) {
            const int c = e / 4;
            *reinterpret_cast<f32x4*>(pex_w + c * 1024) = f32x4{xv[4 * c], xv[4 * c + 1], xv[4 * c + 2], xv[4 * c + 3]};
          }
        }
      };
      constexpr int E2 = 16 / (2 * NT);  // scores per dV slot
#pragma unroll
      for (int n = n_lo; n < n_hi; ++n) {
        if (n + PRE < n_hi) op[n + PRE] = opr(n + PRE);
        if (n < NS) {
          s = mfma32(op[n], kv[n], s);
          if constexpr (!PW && !FIRST) ds_slot(n);
          if (n == NS - 1) store_ds();
        } else {
          const int j = n - NS;
          acc[j % NT] = mfma32(op[n], PW ? prv_bf[j / NT] : ds[j / NT], acc[j % NT]);
          if constexpr (PW && !LAST) {
            if (j == 0) p_mask();
            p_scores(j * E2, (j + 1) * E2);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (!PW && !LAST) cur_dp = s;
      if constexpr (PW && FIRST) {
        p_mask();
        p_scores(0, 16);
      }
      if constexpr (PW && !LAST) {
        pin(cur_bf[0]);
        pin(cur_bf[1]);
      }
    };

    bf16x8 pa[2] = {bf16x8{}, bf16x8{}}, pb[2] = {bf16x8{}, bf16x8{}};
    f32x16 dpa = f32x16{}, dpb = f32x16{};
    using T = Role<true>;
    using F = Role<false>;
    // tile t: phase 2t (block 2t; block 2t-1 of tile t-1), barrier, copy of tile t+2 into
    // tile t-1's buffer, phase 2t+1 (block 2t+1; block 2t), wait for tile t+1, barrier.
    // With a mask, the mask of block k+3 is copied after barrier k, and the barrier before
    // phase k waits for the mask of block k: behind it are then only the copies issued after
    // barrier k-2 (a tile, if one was, and a mask).
    auto step = [&](auto first_t, int t, const bf16* Qp, const bf16* Gp, const float* Rp, const bf16* Qc,
                    const bf16* Gc, const float* Rc, bf16* Ql, bf16* Gl, float* Rl) __attribute__((always_inline)) {
      ofs.repin();
      phase(first_t, F{}, 2 * t, Qc, Gc, Rc, 0, Qp, Gp, Rp, 1, pa, pb, dpa, dpb);
      if constexpr (MASK && CP) {
        if (t + 1 < total) wait_tile_and_mask();  // tile t+1 and the mask of block 2t+2 behind
        else wait_vmem();
      }
      __syncthreads();
      load_mask(2 * t + 3);
      if (t + 2 < total) load_tile(t + 2, Ql, Gl, Rl);
      phase(F{}, F{}, 2 * t + 1, Qc, Gc, Rc, 1, Qc, Gc, Rc, 0, pb, pa, dpb, dpa);
      if constexpr (CP) {
        if (t + 2 < total) {
          if constexpr (MASK) wait_tile_and_mask();  // the mask of block 2t+3 and tile t+2 behind
          else wait_vmem_le<TPW>();
        } else if (MASK && 2 * t + 3 < nb) {
          wait_vmem_le<MPW>();  // the mask of block 2t+3 behind
        } else {
          wait_vmem();
        }
      }
      __syncthreads();
      load_mask(2 * t + 4);
    };
    if (total > 0) {
      __syncthreads();  // every wave's share of tile 0 has landed
      step(T{}, 0, Q2, G2, R2s, Q0, G0, R0, Q2, G2, R2s);
    }
    for (int t = 1; t < total; t += 3) {
      step(F{}, t, Q0, G0, R0, Q1, G1, R1s, Q0, G0, R0);
      if (t + 1 < total) step(F{}, t + 1, Q1, G1, R1s, Q2, G2, R2s, Q1, G1, R1s);
      if (t + 2 < total) step(F{}, t + 2, Q2, G2, R2s, Q0, G0, R0, Q2, G2, R2s);
    }
    if (total > 0) {
      // block 2 total - 1 (rows 32.. of tile total-1)
      const int lb = (total - 1) % 3;
      const bf16* Ql = lb == 0 ? Q0 : (lb == 1 ? Q1 : Q2);
      const bf16* Gl = lb == 0 ? G0 : (lb == 1 ? G1 : G2);
      const float* Rl = lb == 0 ? R0 : (lb == 1 ? R1s : R2s);
      phase(F{}, T{}, 2 * total, Ql, Gl, Rl, 0, Ql, Gl, Rl, 1, pa, pb, dpa, dpb);
    }

    // Epilogue: lane holds key myk, d = mb*32 + (v/4)*8 + 4*hi + v%4.
    if (myk < kv_rows_out(p, kv_end)) {
      bf16* row = PW ? reinterpret_cast<bf16*>(a.dv) + v_base(p, b) + g * p.v_sh + (int64_t)myk * p.v_sl
                     : reinterpret_cast<bf16*>(a.dk) + k_base(p, b) + g * p.k_sh + (int64_t)myk * p.k_sl;
      const float f = PW ? 1.f : p.scale;
#pragma unroll
      for (int mb = 0; mb < NT; ++mb) {
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[mb][v4 * 4 + e] * f);
          *reinterpret_cast<bf16x4*>(row + mb * 32 + v4 * 8 + hi * 4) = w;
        }
      }
    }
  }
}

template <int D, int NP, int CM, bool MASK, bool STORE>
__device__ __forceinline__ void dkdv_pair_body(const BwdArgs& a, int bid, int nblk, char* smem) {
  if (__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) < NP)
    dkdv_pair_wave<true, D, NP, CM, MASK, STORE>(a, bid, nblk, smem);
  else
    dkdv_pair_wave<false, D, NP, CM, MASK, STORE>(a, bid, nblk, smem);
}

template <int D, int NP, int CM, bool MASK, bool STORE>
__global__ __launch_bounds__(128 * NP, 1) void bwd_dkdv_pair_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[dkdv_pair_lds_bytes<D, NP, MASK>()];
  dkdv_pair_body<D, NP, CM, MASK, STORE>(a, blockIdx.x, gridDim.x, smem);
}

// ---------------------------------------------------------------------------------------
// 3. dQ (query-stationary)
// ---------------------------------------------------------------------------------------
constexpr int kBN = 64;

// LDS bytes of the pipelined dQ body: three K and two V tiles.  The phase of block bi
// computes S and dP of block bi+1 and dQ of block bi-1, so K of tile t is read by the phases
// of blocks 2t-1 .. 2t+2 and V of tile t by those of blocks 2t-1 and 2t.  Tile t+2 is
// requested after the barrier that follows the phase of block 2t: it takes the K buffer of
// tile t-1 (last read in that phase) and the V buffer of tile t.
template <int D>
constexpr int dq_lds_bytes() { return 5 * kBN * D * 2; }

template <int D, int NW, int CM, bool MASK>
__device__ __forceinline__ void dq_body(const BwdArgs& a, int bid, int nblk, char* smem) {
  constexpr bool CAUSAL = CM != 0;  // CM: 0 no diagonal, 1 causal, 2 causal + sliding window
  constexpr int BM = NW * 32;
  constexpr int TILE = kBN * D;
  constexpr int NS = D / 16;   // MFMAs of one S^T (or dP^T) block
  constexpr int NT = D / 32;   // MFMAs of one half of a dQ^T block
  constexpr int R1 = 2 * NT;   // slots of region 1 (dQ MFMAs)
  constexpr int R2 = 2 * NS;   // slots of region 2 (S^T, dP^T MFMAs)
  constexpr int E1 = 16 / R1;  // scores per lane per region-1 slot
  bf16* const K0 = reinterpret_cast<bf16*>(smem);
  bf16* const K1 = K0 + TILE;
  bf16* const K2 = K1 + TILE;
  bf16* const V0 = K2 + TILE;
  bf16* const V1 = V0 + TILE;
  static_assert(5 * TILE * 2 == dq_lds_bytes<D>(), "LDS layout");

  const Problem& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index stays a vector value here: as a scalar, the per-wave block tests become
  // branches whose joins copy the accumulators (a vector test runs both sides under exec)
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Work item: (batch, KV head) group, then query tile `rank` of head h of the group.
  int gi, r;
  xcd_item(bid, p.B * p.Hkv, nblk / (p.B * p.Hkv), p.G, !CAUSAL, gi, r);
  const int b = batch_by_work(p, gi / p.Hkv);
  const int g = gi % p.Hkv;
  const int h = g * p.G + r % p.G;
  const int rank = r / p.G;
  const int q_end = seq_len_q(p, b);
  const int kv_end = seq_len_kv(p, b);
  // Rows: query tile `rank` of BM rows, heavy tiles first on causal grids (as the forward).
  const int qt = CAUSAL ? (p.Lq + BM - 1) / BM - 1 - rank : rank;
  const int wq_lo = qt * BM + wave * 32;  // this wave's first row
  const int row_lo = qt * BM, row_hi = row_lo + BM;
  const int wq_hi = min(wq_lo + 32, q_end) - 1;

  const bf16* qb = reinterpret_cast<const bf16*>(a.q) + q_base(p, b) + h * p.q_sh;
  const bf16* dob = reinterpret_cast<const bf16*>(a.dO) + o_base(p, b) + h * p.o_sh;
  const bf16* kb_ = reinterpret_cast<const bf16*>(a.k) + k_base(p, b) + g * p.k_sh;
  const bf16* vb_ = reinterpret_cast<const bf16*>(a.v) + v_base(p, b) + g * p.v_sh;
  const bf16* mb_ = MASK ? reinterpret_cast<const bf16*>(p.mask) + b * p.m_sb + h * p.m_sh : nullptr;

  int kv_stop = kv_end;
  const int coff = CAUSAL ? causal_offset(p.causal, q_end, kv_end) : 0;  // diagonal offset
  if (CAUSAL) kv_stop = min(kv_stop, min(row_hi, q_end) + coff);
  if (row_lo >= q_end) kv_stop = 0;
  const int n_tiles = kv_stop > 0 ? (kv_stop + kBN - 1) / kBN : 0;
  // sliding window: tiles before the first row's window are skipped (as the forward)
  const int W = CM == 2 ? p.window : 0;
  const int t0 = W > 0 ? min(max(row_lo + coff - W + 1, 0) / kBN, n_tiles) : 0;
  int vis_stop = wq_lo < q_end ? kv_stop : 0;
  if (CAUSAL) vis_stop = min(vis_stop, wq_hi + 1 + coff);
  const int nvis = vis_stop > 0 ? (vis_stop + 31) / 32 : 0;  // 32-key blocks this wave works on (a prefix)

  TileCopy<kBN, D, NW> kcopy, vcopy;
  kcopy.init(p.k_sl, wave, lane);
  vcopy.init(p.v_sl, wave, lane);
  auto load_tile = [&](int j0, bf16* Kd, bf16* Vd) {
    kcopy.copy(rows_rsrc<D, kBN>(kb_, p.k_sl, j0, kv_stop), Kd, wave);
    vcopy.copy(rows_rsrc<D, kBN>(vb_, p.v_sl, j0, kv_stop), Vd, wave);
  };
  // tile 0 and this lane's row operands land first; tile 1 streams in behind
  if (n_tiles > t0) load_tile(t0 * kBN, K0, V0);
  const int qi = wq_lo + l32;  // this lane's query (N index)
  const bool qok = qi < q_end;
  bf16x8 qreg[NS], doreg[NS];
#pragma unroll
  for (int kk = 0; kk < NS; ++kk) {
    qreg[kk] = __builtin_bit_cast(bf16x8, qok ? ld16(qb + (int64_t)qi * p.q_sl + kk * 16 + 8 * hi) : zero16());
    doreg[kk] = __builtin_bit_cast(bf16x8, qok ? ld16(dob + (int64_t)qi * p.o_sl + kk * 16 + 8 * hi) : zero16());
  }
  const int64_t rowid = ((int64_t)b * p.Hq + h) * p.Lq + qi;
  const float nl2 = qok ? -a.lse2[rowid] : kNegInf;  // exp2 offset of this lane's row
  const float dsum = qok ? a.dsum[rowid] : 0.f;
  // Mask values of block bi for this lane (keys 32*bi + 16*hi + 0..15), read two blocks
  // ahead into the registers of the block's parity (mk_e, mk_o): each load is issued
  // before the wait ahead of the tile barrier that precedes its use, so it adds no wait of
  // its own (the compiler cannot see the tile copies and would otherwise wait for all of
  // them, the next tile's included, before the first use).
  auto mask_vec_ok = [&](int bi) { return p.mask_vec && qok && 32 * bi + 16 * hi + 16 <= p.Lk; };
  auto load_mask = [&](int bi, u32x4 (&m)[2]) {
    if (MASK && bi < nvis && mask_vec_ok(bi)) {
      const bf16* mp = mb_ + (int64_t)qi * p.m_si + 32 * bi + 16 * hi;
      m[0] = ld16(mp);
      m[1] = ld16(mp + 8);
    } else {
      m[0] = zero16();
      m[1] = zero16();
    }
  };
  u32x4 mk_e[2], mk_o[2];
  load_mask(2 * t0, mk_e);
  load_mask(2 * t0 + 1, mk_o);
  wait_vmem();
  if (n_tiles > t0 + 1) load_tile((t0 + 1) * kBN, K1, V1);

  f32x16 dq_acc[NT];
#pragma unroll
  for (int mb = 0; mb < NT; ++mb) dq_acc[mb] = f32x16{};

  const float c2 = p.scale_log2;
  const float sc = p.scale;
  const int krow_l = perm_row(l32);
  const int blk = lane >> 4;
  const int arow = (lane & 15) >> 2;
  const int tchunk = ((lane & 3) >> 1) + 2 * (blk & 1);
  const int thalf = 4 * (lane & 1);

  // dQ^T of a block runs one block late: B operand bf16 dS^T (zero before the first
  // block), A operand K^T read from the block's tile just in time.
  bf16x8 ds_a[2], ds_b[2];
  ds_a[0] = ds_a[1] = ds_b[0] = ds_b[1] = bf16x8{};
  OpOffsets<D> ofs;  // operand reads (A operands of row krow_l, transposed K)
  ofs.init(krow_l, hi, arow, tchunk, thalf);
  auto kt_op = [&](int j, const bf16* Kt, int kb) {
    const int half = j / NT, mb = j % NT;
    return ofs.tr8(Kt, kb * 32 + 8 * half, mb);  // rows kb*32 + 16hi + 8half + arow ..
  };
  auto dq_mfma = [&](int j, bf16x8 op, const bf16x8 (&ds)[2]) {
    const int half = j / NT, mb = j % NT;
    dq_acc[mb] = mfma32(op, ds[half], dq_acc[mb]);
  };

  // ---- one pipeline phase for block bi (keys kb*32.. of Kc/Vc; the previous block's keys
  // kbp*32.. of Kp; the next block's keys kbn*32.. of Kn/Vn).  Region 1: dQ MFMAs of block
  // bi-1 with the P, dS arithmetic of block bi.  Region 2: S^T, dP^T MFMAs of block bi+1
  // with the rest of it.  The S^T, dP^T of the block after a wave's last are never used.
  auto phase = [&](int bi, const bf16* Kp, int kbp, const bf16* Kn, const bf16* Vn, int kbn,
                   f32x16& s, f32x16& dp, f32x16& s_nx, f32x16& dp_nx, const bf16x8 (&ds_prev)[2],
                   bf16x8 (&ds)[2], u32x4 (&mk)[2]) __attribute__((always_inline)) {
    if (bi >= nvis) {
      // the wave's last block: its dQ, while its K tile is still resident
      if (bi == nvis && bi > 2 * t0) {
#pragma unroll
        for (int j = 0; j < R1; ++j) dq_mfma(j, kt_op(j, Kp, kbp), ds_prev);
      }
      return;
    }
    const int key0 = 32 * bi + 16 * hi;  // lane holds query qi and keys key0 + v
    float mbias[16];
    if (MASK) {
      if (mask_vec_ok(bi)) {
        const bf16x8 b0 = __builtin_bit_cast(bf16x8, mk[0]), b1 = __builtin_bit_cast(bf16x8, mk[1]);
#pragma unroll
        for (int v = 0; v < 8; ++v) { mbias[v] = bf2f(b0[v]); mbias[v + 8] = bf2f(b1[v]); }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          mbias[v] = (qok && key0 + v < kv_end) ? bf2f(mb_[(int64_t)qi * p.m_si + key0 + v]) : 0.f;
      }
      load_mask(bi + 2, mk);
    }
    const bool partial = (32 * bi + 32 > kv_end) || (CAUSAL && 32 * bi + 31 > wq_lo + coff) ||
                         (wq_lo + 32 > q_end) || (W > 0 && 32 * bi <= wq_hi + coff - W);
    if (partial) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = key0 + v;
        const bool ok = (key < kv_end) & qok & (!CAUSAL | (key <= qi + coff)) &
                        ((W == 0) | (key > qi + coff - W));
        s[v] = ok ? s[v] : kNegInf;
      }
    }
    float xv[16], dd[16];
    auto st_a = [&](int e) {
      // with a mask in natural units (nl2 then holds -LSE; see dkdv_body)
      xv[e] = MASK ? (fmaf(s[e], sc, mbias[e]) + nl2) * kLog2e : fmaf(s[e], c2, nl2);
      dd[e] = dp[e] - dsum;
    };
    auto st_b = [&](int e) { xv[e] = fast_exp2(xv[e]); };
    auto st_c = [&](int e) {
      dd[e] = xv[e] * dd[e];
      if (e & 1) {
        f32x2 ss = {dd[e - 1], dd[e]};
        const bf16x2 s2 = __builtin_convertvector(ss, bf16x2);
        ds[e / 8][e % 8 - 1] = s2[0];
        ds[e / 8][e % 8] = s2[1];
      }
    };
    // region 1
    bf16x8 aop[R2], top[R1];
    top[0] = kt_op(0, Kp, kbp);
#pragma unroll
    for (int j = 0; j < R1; ++j) {
      if (j + 1 < R1) top[j + 1] = kt_op(j + 1, Kp, kbp);
      dq_mfma(j, top[j], ds_prev);
#pragma unroll
      for (int e = j * E1; e < (j + 1) * E1; ++e) st_a(e);
#pragma unroll
      for (int e = (j - 1) * E1; e < j * E1; ++e)
        if (e >= 0) st_b(e);
#pragma unroll
      for (int e = (j - 2) * E1; e < (j - 1) * E1; ++e)
        if (e >= 0) st_c(e);
      if (j == R1 - 1) aop[0] = ofs.row8(Kn, kbn * 32, 0);  // first A operand of bi+1
      __builtin_amdgcn_sched_barrier(0);
    }
    // region 2
    s_nx = f32x16{};
    dp_nx = f32x16{};
#pragma unroll
    for (int i = 0; i < R2; ++i) {
      if (i + 1 < R2) {
        const int n = i + 1;
        aop[n] = ofs.row8((n & 1) ? Vn : Kn, kbn * 32, n >> 1);
      }
      if (i & 1) dp_nx = mfma32(aop[i], doreg[i >> 1], dp_nx);
      else s_nx = mfma32(aop[i], qreg[i >> 1], s_nx);
      if (i == 0) {
#pragma unroll
        for (int e = (R1 - 1) * E1; e < R1 * E1; ++e) st_b(e);
#pragma unroll
        for (int e = (R1 - 2) * E1; e < (R1 - 1) * E1; ++e) st_c(e);
      }
      if (i == 1) {
#pragma unroll
        for (int e = (R1 - 1) * E1; e < R1 * E1; ++e) st_c(e);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One tile step (two blocks); unrolled by three over the LDS buffers (see the forward).
  f32x16 s_a = f32x16{}, dp_a = f32x16{}, s_b = f32x16{}, dp_b = f32x16{};
  auto step = [&](int t, const bf16* Kp, const bf16* Kc, const bf16* Vc, const bf16* Kn,
                  const bf16* Vn, bf16* Kl, bf16* Vl) __attribute__((always_inline)) {
    ofs.repin();
    phase(2 * t, Kp, 1, Kc, Vc, 1, s_a, dp_a, s_b, dp_b, ds_b, ds_a, mk_e);
    // tile t+1 has landed for every wave, and no wave still reads tile t-1 (unconditional,
    // so that the compiler sees every earlier load complete on every path)
    wait_vmem();
    __syncthreads();
    if (t + 2 < n_tiles) load_tile((t + 2) * kBN, Kl, Vl);
    phase(2 * t + 1, Kc, 0, Kn, Vn, 0, s_b, dp_b, s_a, dp_a, ds_a, ds_b, mk_o);
  };

  if (n_tiles > t0) {
    // the first phase runs the dQ MFMAs of "block -1" (rows 32..63 of buffer 2) with zero
    // weights: those rows are zeroed so the products are exactly zero
    lds_zero<32 * D * 2, 64 * NW>(K2 + 32 * D, tid);
    __syncthreads();  // every wave's share of the first tile has landed; the zeros are visible
    if (nvis > 2 * t0) {
#pragma unroll
      for (int i = 0; i < R2; ++i) {
        const bf16x8 op = ofs.row8((i & 1) ? V0 : K0, 0, i >> 1);
        if (i & 1) dp_a = mfma32(op, doreg[i >> 1], dp_a);
        else s_a = mfma32(op, qreg[i >> 1], s_a);
      }
    }
  }
  // unrolled by six (three K and two V buffers), so every buffer is a compile-time choice
  bf16* const Kb[3] = {K0, K1, K2};
  bf16* const Vb[2] = {V0, V1};
  for (int tl = 0; tl < n_tiles - t0; tl += 6) {
#pragma unroll
    for (int u = 0; u < 6; ++u)
      if (tl + u < n_tiles - t0)
        step(t0 + tl + u, Kb[(u + 2) % 3], Kb[u % 3], Vb[u % 2], Kb[(u + 1) % 3], Vb[(u + 1) % 2],
             Kb[(u + 2) % 3], Vb[u % 2]);
  }
  // a wave whose last block is the workgroup's last: that block's dQ (second block of
  // tile n_tiles-1, buffer (n_tiles-1-t0) % 3, never overwritten)
  if (nvis > 2 * t0 && nvis == 2 * n_tiles) {
    const int lt = (n_tiles - 1 - t0) % 3;
    const bf16* Kl = lt == 0 ? K0 : (lt == 1 ? K1 : K2);
#pragma unroll
    for (int j = 0; j < R1; ++j) dq_mfma(j, kt_op(j, Kl, 1), ds_b);
  }

  if (qi < q_rows_out(p, q_end)) {
    bf16* dqrow = reinterpret_cast<bf16*>(a.dq) + q_base(p, b) + h * p.q_sh + (int64_t)qi * p.q_sl;
#pragma unroll
    for (int mb = 0; mb < NT; ++mb) {
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

// ---------------------------------------------------------------------------------------
// 3b. dQ, block-sequential form (for head dims where the pipelined form's registers do
//     not fit two waves per SIMD): each 32-key block's S^T, dP^T, dS^T and dQ^T in turn.
// ---------------------------------------------------------------------------------------

template <int D, int NW, int CM, bool MASK>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[dq_lds_bytes<D>()];
  dq_body<D, NW, CM, MASK>(a, blockIdx.x, gridDim.x, smem);
}

// dK/dV and dQ in one launch: workgroups [0, n_dkdv) run the dK/dV body (heavy key tiles
// first), the rest the dQ body, so dQ work fills the CUs that the dK/dV tail leaves idle
// and no launch boundary separates the two.  Both bodies fit two waves per SIMD (d = 64).
// n_dkdv is a multiple of 8 whenever the XCD-aware item order is used, so the dQ items
// keep their XCD.
template <int D, int NW, int CM, bool MASK>
__global__ __launch_bounds__(64 * NW, 2) void bwd_fused_kernel(BwdArgs a, int n_dkdv) {
  constexpr int kL1 = dkdv_lds_bytes<D, NW, MASK>(), kL2 = dq_lds_bytes<D>();
  __shared__ __attribute__((aligned(16))) char smem[kL1 > kL2 ? kL1 : kL2];
  if ((int)blockIdx.x < n_dkdv) dkdv_body<D, NW, CM, MASK>(a, blockIdx.x, n_dkdv, smem);
  else dq_body<D, NW, CM, MASK>(a, blockIdx.x - n_dkdv, gridDim.x - n_dkdv, smem);
}

template <int D, int NW, int CM, bool MASK>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dq_seq_kernel(BwdArgs a) {
  constexpr bool CAUSAL = CM != 0;  // CM: 0 no diagonal, 1 causal, 2 causal + sliding window
  constexpr int BM = NW * 32;
  constexpr int CPR = D / 8;
  constexpr int TILE = kBN * D;
  __shared__ __attribute__((aligned(16))) bf16 K0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 K1[TILE];
  __shared__ __attribute__((aligned(16))) bf16 V0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 V1[TILE];
  // With a mask whose rows allow 16-byte copies: each wave's 32 mask rows of the tile's two
  // 32-key blocks, one 2 KB region per (wave, block) (see load_mask)
  constexpr int MREG = 32 * 32;
  __shared__ __attribute__((aligned(16))) bf16 Ms[MASK ? NW * 2 * MREG : 8];

  const Problem& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index stays a vector value here: as a scalar, the per-wave block tests become
  // branches whose joins copy the accumulators (a vector test runs both sides under exec)
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Work item: (batch, KV head) group, then query tile `rank` of head h of the group.
  int gi, r;
  xcd_item(blockIdx.x, p.B * p.Hkv, (int)(gridDim.x / (p.B * p.Hkv)), p.G, !CAUSAL, gi, r);
  const int b = batch_by_work(p, gi / p.Hkv);
  const int g = gi % p.Hkv;
  const int h = g * p.G + r % p.G;
  const int rank = r / p.G;
  const int q_end = seq_len_q(p, b);
  const int kv_end = seq_len_kv(p, b);
  // Rows: query tile `rank` of BM rows, heavy tiles first on causal grids (as the forward).
  const int qt = CAUSAL ? (p.Lq + BM - 1) / BM - 1 - rank : rank;
  const int wq_lo = qt * BM + wave * 32;  // this wave's first row
  const int row_lo = qt * BM, row_hi = row_lo + BM;
  const int wq_hi = min(wq_lo + 32, q_end) - 1;

  const bf16* qb = reinterpret_cast<const bf16*>(a.q) + q_base(p, b) + h * p.q_sh;
  const bf16* dob = reinterpret_cast<const bf16*>(a.dO) + o_base(p, b) + h * p.o_sh;
  const bf16* kb_ = reinterpret_cast<const bf16*>(a.k) + k_base(p, b) + g * p.k_sh;
  const bf16* vb_ = reinterpret_cast<const bf16*>(a.v) + v_base(p, b) + g * p.v_sh;
  const bf16* mb_ = MASK ? reinterpret_cast<const bf16*>(p.mask) + b * p.m_sb + h * p.m_sh : nullptr;

  int kv_stop = kv_end;
  const int coff = CAUSAL ? causal_offset(p.causal, q_end, kv_end) : 0;  // diagonal offset
  if (CAUSAL) kv_stop = min(kv_stop, min(row_hi, q_end) + coff);
  if (row_lo >= q_end) kv_stop = 0;
  const int n_tiles = kv_stop > 0 ? (kv_stop + kBN - 1) / kBN : 0;
  // sliding window: tiles before the first row's window are skipped
  const int W = CM == 2 ? p.window : 0;
  const int t0 = W > 0 ? min(max(row_lo + coff - W + 1, 0) / kBN, n_tiles) : 0;

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

  TileCopy<kBN, D, NW> kcopy, vcopy;
  kcopy.init(p.k_sl, wave, lane);
  vcopy.init(p.v_sl, wave, lane);
  auto load_tile = [&](int j0, bf16* Kd, bf16* Vd) {
    kcopy.copy(rows_rsrc<D, kBN>(kb_, p.k_sl, j0, kv_stop), Kd, wave);
    vcopy.copy(rows_rsrc<D, kBN>(vb_, p.v_sl, j0, kv_stop), Vd, wave);
  };
  const float c2 = p.scale_log2;
  const float sc = p.scale;
  const int krow_l = perm_row(l32);
  const int blk = lane >> 4;
  const int arow = (lane & 15) >> 2;
  const int tchunk = ((lane & 3) >> 1) + 2 * (blk & 1);
  const int thalf = 4 * (lane & 1);
  OpOffsets<D> ofs;  // operand reads (A operands of row krow_l, transposed K)
  ofs.init(krow_l, hi, arow, tchunk, thalf);

  // ---- mask staging (MASK and 16-byte mask rows).  Only this wave reads its rows, so it
  // fills its own regions without a barrier: the mask of block kb of tile t+1 is copied
  // into region (wave, kb) as soon as the wave has read that block of tile t, and is waited
  // for with explicit counts of the copies issued after it (the compiler cannot see them).
  // Per wave, in issue order: tile t+1's K/V copies (NC), then the mask of tile t+1's
  // block 0 (two copies, during block 0 of tile t), then its block 1 (two copies).
  // A region holds rows r = 0..31 as four 16-byte chunks; logical chunk c of row r sits at
  // chunk 4r + (c ^ ((r >> 2) & 3)), so the 16-lane phases of a read (sixteen rows at one
  // chunk) hit sixteen distinct bank groups.
  const bool mstage = MASK && p.mask_vec;
  constexpr int NC = 2 * TileCopy<kBN, D, NW>::PER_WAVE;
  uint32_t mvo[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int pc = 64 * i + lane, r = pc >> 2, c = (pc & 3) ^ ((r >> 2) & 3);
    mvo[i] = (uint32_t)(((int64_t)r * p.m_si + 8 * c) * 2);
  }
  auto load_mask = [&](int key_lo, int kb) {
    const int nr = min(p.Lq - wq_lo, 32);
    const int64_t bytes = nr > 0 && key_lo < p.Lk ? (int64_t)(nr - 1) * p.m_si * 2 + (p.Lk - key_lo) * 2 : 0;
    const i32x4 rs = raw_rsrc(mb_ + (int64_t)wq_lo * p.m_si + key_lo, bytes);
    const int uw = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int i = 0; i < 2; ++i) buffer_to_lds<16>(rs, Ms, ((uw * 2 + kb) * 2 + i) * 1024, mvo[i]);
  };
  // tile t's K/V copies have landed (with staging, the four mask copies after them may not)
  auto wait_tile = [&]() {
    if (mstage) wait_vmem_le<4>();
    else wait_vmem();
  };
  // the mask copies of the block now in use have landed: after them come the other block's
  // two copies and, unless this is the last tile, the next tile's K/V copies
  auto wait_mask = [&](bool next_tile) {
    if (next_tile) wait_vmem_le<NC + 2>();
    else wait_vmem_le<2>();
  };

  auto step = [&](int t, const bf16* Kt, const bf16* Vt, bf16* Kn, bf16* Vn)
                  __attribute__((always_inline)) {
    const int j0 = t * kBN;
    ofs.repin();
    wait_tile();
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(j0 + kBN, Kn, Vn);
    const bool partial_t = (j0 + kBN > kv_end) || (CAUSAL && j0 + kBN - 1 > wq_lo + coff) ||
                           (wq_lo + 32 > q_end) || (W > 0 && j0 <= wq_hi + coff - W);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key_lo = j0 + kb * 32;
      if (!(wq_lo < q_end && key_lo < kv_stop && (!CAUSAL || key_lo <= wq_hi + coff) &&
            (W == 0 || key_lo + 31 > wq_lo + coff - W))) {
        if (mstage) load_mask(key_lo + kBN, kb);
        continue;
      }
      // S^T = K Q^T and dP^T = V dO^T for keys key_lo + perm
      f32x16 s_acc = f32x16{}, dp_acc = f32x16{};
      {
        bf16x8 op[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) op[kk] = ofs.row8(Kt, kb * 32, kk);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) s_acc = mfma32(op[kk], qreg[kk], s_acc);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) op[kk] = ofs.row8(Vt, kb * 32, kk);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) dp_acc = mfma32(op[kk], doreg[kk], dp_acc);
      }
      // lane holds query qi and keys key0 + v
      const int key0 = key_lo + 16 * hi;
      // with a mask, s_acc becomes the exp2 argument here: scale * s + m - LSE in natural
      // units (lse2 then holds LSE; see dkdv_body), converted to log2 units
      if (MASK) {
        if (mstage) {
          wait_mask(t + 1 < n_tiles);
          const bf16* mr = Ms + (wave * 2 + kb) * MREG + 4 * 8 * l32;
          const int sw = (l32 >> 2) & 3;
          const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(mr + 8 * ((2 * hi) ^ sw));
          const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(mr + 8 * ((2 * hi + 1) ^ sw));
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            s_acc[v] = (fmaf(s_acc[v], sc, bf2f(b0[v])) - lse2) * kLog2e;
            s_acc[v + 8] = (fmaf(s_acc[v + 8], sc, bf2f(b1[v])) - lse2) * kLog2e;
          }
          // the region is refilled only after these reads have returned
          wait_lds();
          load_mask(key_lo + kBN, kb);
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float mv = (qok && key0 + v < kv_end) ? bf2f(mb_[(int64_t)qi * p.m_si + key0 + v]) : 0.f;
            s_acc[v] = (fmaf(s_acc[v], sc, mv) - lse2) * kLog2e;
          }
        }
      }
      bf16x8 dsb[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) {
          const int v = half * 8 + t8;
          float x = MASK ? s_acc[v] : fmaf(s_acc[v], c2, -lse2);
          if (partial_t) {
            const int key = key0 + v;
            const bool ok = (key < kv_end) & qok & (!CAUSAL | (key <= qi + coff)) &
                            ((W == 0) | (key > qi + coff - W));
            x = ok ? x : kNegInf;
          }
          const float pv = fast_exp2(x);
          dsb[half][t8] = (bf16)(pv * (dp_acc[v] - dsum));
        }
      }
      // dQ^T += K^T dS^T  (K^T via transposing LDS reads)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8 kT[D / 32];
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) kT[mb] = ofs.tr8(Kt, kb * 32 + 8 * half, mb);
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) dq_acc[mb] = mfma32(kT[mb], dsb[half], dq_acc[mb]);
      }
    }
  };

  if (n_tiles > t0) {
    load_tile(t0 * kBN, K0, V0);
    if (mstage) {
      load_mask(t0 * kBN, 0);
      load_mask(t0 * kBN + 32, 1);
    }
  }
  for (int t = t0; t < n_tiles; t += 2) {
    step(t, K0, V0, K1, V1);
    if (t + 1 < n_tiles) step(t + 1, K1, V1, K0, V0);
  }
  // the last tile's mask copies (of keys past the tiles) must land before the workgroup
  // ends and its LDS is handed to another
  if (mstage) wait_vmem();

  if (qi < q_rows_out(p, q_end)) {
    bf16* dqrow = reinterpret_cast<bf16*>(a.dq) + q_base(p, b) + h * p.q_sh + (int64_t)qi * p.q_sl;
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

// ---------------------------------------------------------------------------------------
// 3c. dQ from the stored dS blocks (d = 128, when dK/dV and dQ run in one call)
// ---------------------------------------------------------------------------------------
// The paired dK/dV kernel forms every bf16 dS block of the problem anyway (the operand of its
// dK product, rounded as the dQ product takes it); with a dS buffer it also writes them out
// (BwdArgs::ds).  dQ = scale dS K then needs one product per block, without recomputing S,
// P and dP (two of the query-stationary pass's three products, and its exponentials): this
// kernel streams each row block's dS^T blocks from HBM once, through LDS, and reads them
// back transposed (ds_read_b64_tr_b16) as the B operand of dQ^T += K^T dS^T, with K^T read
// as in the other dQ kernels.  Its cost is the dS traffic: 2 bytes per visible pair written
// and read again, instead of 4 D flops and an exponential per pair recomputed.
//
// A wave (32 query rows) visits the key blocks [lo, hi) in which some row sees some key:
// the union of the rows' visible keys is one interval (consecutive rows' windows overlap),
// so every such block holds a visible pair.  The dK/dV kernel has written each of them: a
// visible pair (i, j) lies in a query tile (64 rows) and key workgroup it visits.
// Workgroup: NW waves of 32 rows of one head (the other dQ kernels' items and order); each
// step copies one 32-key K block (shared) and each wave's dS block into one of kDsBufs
// buffers, kDsBufs - 1 blocks ahead.  Eight waves share each K block and three buffers
// (72 KB of LDS, two workgroups and sixteen waves per CU): measured against four waves with
// three, four or five buffers (the fewer buffers, the more workgroups per CU and the
// faster), 215 against 229-239 us on the causal GQA 4k step, equal on the padded 2k one.
// Grids too small to give every CU two such workgroups (a 512-row prefill chunk) take
// four-wave ones (48 KB, three per CU).
constexpr int kDsBufs = 3;
constexpr int kNumCu = 256;

template <int D, int NW, int CM>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dq_ds_kernel(BwdArgs a) {
  constexpr bool CAUSAL = CM != 0;
  constexpr int BM = NW * 32;
  constexpr int KB = 32 * D;  // elements of a 32-key K block
  __shared__ __attribute__((aligned(16))) bf16 Ks[kDsBufs * KB];
  __shared__ __attribute__((aligned(16))) bf16 Ss[kDsBufs * NW * 1024];

  const Problem& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int gi, r;
  xcd_item(blockIdx.x, p.B * p.Hkv, (int)(gridDim.x / (p.B * p.Hkv)), p.G, !CAUSAL, gi, r);
  const int b = batch_by_work(p, gi / p.Hkv);
  const int g = gi % p.Hkv;
  const int h = g * p.G + r % p.G;
  const int rank = r / p.G;
  const int q_end = seq_len_q(p, b);
  const int kv_end = seq_len_kv(p, b);
  const int qt = CAUSAL ? (p.Lq + BM - 1) / BM - 1 - rank : rank;
  const int row_lo = qt * BM;
  const int coff = CAUSAL ? causal_offset(p.causal, q_end, kv_end) : 0;
  const int W = CM == 2 ? p.window : 0;

  // key blocks [lo, hi_) with a visible pair for the 32 rows from r0: the rows' visible keys
  // together are [first, stop)
  auto blocks = [&](int r0, int& lo, int& hi_) __attribute__((always_inline)) {
    lo = hi_ = 0;
    if (r0 >= q_end) return;
    int stop = kv_end;
    if (CAUSAL) stop = min(stop, min(r0 + 32, q_end) + coff);
    const int first = W > 0 ? max(r0 + coff - W + 1, 0) : 0;
    if (stop <= first) return;
    lo = first >> 5;
    hi_ = (stop + 31) >> 5;
  };
  int my_lo, my_hi;
  blocks(row_lo + 32 * wave, my_lo, my_hi);
  int kb0 = 0, kb1 = 0;  // the workgroup's blocks: the union of its waves' ranges
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    int lo, hi_;
    blocks(row_lo + 32 * w, lo, hi_);
    if (hi_ > lo) {
      kb0 = kb1 > kb0 ? min(kb0, lo) : lo;
      kb1 = max(kb1, hi_);
    }
  }
  const int nblk = kb1 > kb0 ? kb1 - kb0 : 0;

  const bf16* kbase = reinterpret_cast<const bf16*>(a.k) + k_base(p, b) + g * p.k_sh;
  // this wave's row of dS blocks (query block row_lo / 32 + wave of head h)
  const bf16* dsrow = reinterpret_cast<const bf16*>(a.ds) +
                      (((int64_t)b * p.Hq + h) * a.ds_nqb + (row_lo >> 5) + wave) * a.ds_nkb * 1024;
  TileCopy<32, D, NW> kcopy;
  kcopy.init(p.k_sl, wave, lane);
  constexpr int CPB = TileCopy<32, D, NW>::PER_WAVE + 2;  // copies per wave and block
  auto issue = [&](int i) __attribute__((always_inline)) {
    const int kb = kb0 + i;
    const int buf = i % kDsBufs;
    kcopy.copy(rows_rsrc<D, 32>(kbase, p.k_sl, kb * 32, kv_end), Ks + buf * KB, wave);
    // a block this wave does not visit is copied from an empty range (zeros, no traffic)
    const bool mine = kb >= my_lo && kb < my_hi;
    const i32x4 rs = raw_rsrc(dsrow + (int64_t)kb * 1024, mine ? 2048 : 0);
    bf16* dst = Ss + (buf * NW + wave) * 1024;
    buffer_to_lds<16, true>(rs, dst, 0, lane * 16);
    buffer_to_lds<16, true>(rs, dst, 1024, 1024 + lane * 16);
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) acc[mb] = f32x16{};
  const int blk = lane >> 4;
  const int arow = (lane & 15) >> 2;
  const int tchunk = ((lane & 3) >> 1) + 2 * (blk & 1);
  const int thalf = 4 * (lane & 1);
  OpOffsets<D> ofs;
  ofs.init(perm_row(l32), hi, arow, tchunk, thalf);
  // B operand of k-step `half` (keys 16 hi + 8 half + t, t = 0..7, of query l32): each
  // 16-lane block reads four key rows of its sixteen queries; lane j supplies the address of
  // key row 16 hi + j / 4 (+ 8 half, + 4 for the second read), queries 16 (blk & 1) + 4 (j % 4)
  // .. + 3 (one 64-byte row per key; a 32-lane phase reads four whole rows, every bank once)
  const uint32_t dso = (uint32_t)((16 * hi + arow) * 64 + 32 * (blk & 1) + 8 * (lane & 3));

#pragma unroll
  for (int i = 0; i < kDsBufs - 1; ++i)
    if (i < nblk) issue(i);
  for (int i = 0; i < nblk; ++i) {
    // block i has landed when only the copies of the blocks issued after it are in flight
    static_assert(kDsBufs == 3, "the wait below covers one block in flight");
    if (i + 1 < nblk) wait_vmem_le<CPB>();
    else wait_vmem();
    __syncthreads();
    // into the buffer of block i - 1, which every wave has finished reading
    if (i + kDsBufs - 1 < nblk) issue(i + kDsBufs - 1);
    const int kb = kb0 + i;
    if (kb >= my_lo && kb < my_hi) {
      const bf16* Kt = Ks + (i % kDsBufs) * KB;
      const char* St = reinterpret_cast<const char*>(Ss + ((i % kDsBufs) * NW + wave) * 1024);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 bop = join_tr(lds_read_tr4(reinterpret_cast<const bf16*>(St + dso + half * 512)),
                                   lds_read_tr4(reinterpret_cast<const bf16*>(St + dso + half * 512 + 256)));
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) acc[mb] = mfma32(ofs.tr8(Kt, 8 * half, mb), bop, acc[mb]);
      }
    }
  }

  const int qi = row_lo + 32 * wave + l32;
  if (qi < q_rows_out(p, q_end)) {
    const bool qok = qi < q_end;
    bf16* dqrow = reinterpret_cast<bf16*>(a.dq) + q_base(p, b) + h * p.q_sh + (int64_t)qi * p.q_sl;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(qok ? acc[mb][v4 * 4 + e] * p.scale : 0.f);
        *reinterpret_cast<bf16x4*>(dqrow + mb * 32 + v4 * 8 + hi * 4) = w;
      }
    }
  }
}

// Waves per workgroup of the two main kernels.  dQ runs two 4-wave workgroups per CU (two
// waves per SIMD; the workgroups' barriers are independent), measured faster than one
// 8-wave workgroup on the MHA 1k and padded 2k workloads and equal on GQA 4k.
template <int D> struct BwdShape;
// PIPE_DQ / PIPE_DQ_MASK: dQ runs the software-pipelined kernel (else the block-sequential
// one) without / with a mask; it needs two waves per SIMD, which its registers allow except
// with a mask at D = 128.  FUSE: dK/dV and dQ in one launch (bwd_fused_kernel), whose
// bodies fit two waves per SIMD only at D = 64.
// PAIR_DKDV: dK/dV runs the paired-wave kernel (two waves per 32-key slice), with a mask
// when its rows allow 16-byte copies (the mask is staged per 32-row block).
template <> struct BwdShape<64> {
  static constexpr int KV_NW = 4, Q_NW = 4;
  static constexpr bool PIPE_DQ = true, PIPE_DQ_MASK = true, FUSE = true, PAIR_DKDV = false;
};
template <> struct BwdShape<128> {
  static constexpr int KV_NW = 4, Q_NW = 4;
  static constexpr bool PIPE_DQ = true, PIPE_DQ_MASK = false, FUSE = false, PAIR_DKDV = true;
};

template <int D, int CM, bool MASK>
hipError_t launch_main(const BwdArgs& a, int stages, hipStream_t s) {
  constexpr int KNW = BwdShape<D>::KV_NW, QNW = BwdShape<D>::Q_NW;
  const int n_kt = (a.p.Lk + 32 * KNW - 1) / (32 * KNW);
  constexpr int BM = 32 * QNW;
  const int n_qt = (a.p.Lq + BM - 1) / BM;
  if constexpr (BwdShape<D>::FUSE && KNW == QNW && !MASK) {
    // both passes in one launch (see bwd_fused_kernel)
    if ((stages & kBwdDkdv) && (stages & kBwdDq)) {
      const int n_dkdv = n_kt * a.p.B * a.p.Hkv, n_dq = n_qt * a.p.B * a.p.Hq;
      if (n_dkdv + n_dq > 0)
        hipLaunchKernelGGL((bwd_fused_kernel<D, KNW, CM, MASK>), dim3(n_dkdv + n_dq), dim3(64 * KNW), 0, s,
                           a, n_dkdv);
      return hipGetLastError();
    }
  }
  // With a dS buffer (d = 128, where dK/dV runs the paired kernel) the dK/dV pass stores
  // dS and dQ is formed from it: the dq stage then reads what the dkdv stage wrote.
  bool ds_path = false;
  if constexpr (BwdShape<D>::PAIR_DKDV) {
    static_assert(32 * KNW == kDsKeysPerGroup, "dS buffer key blocks follow the dK/dV workgroups");
    ds_path = a.ds != nullptr && (!MASK || a.p.mask_vec);
  }
  if ((stages & kBwdDkdv) && n_kt > 0) {
    bool paired = false;
    if constexpr (BwdShape<D>::PAIR_DKDV) {
      if (ds_path) {
        hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, KNW, CM, MASK, true>), dim3(n_kt * a.p.B * a.p.Hkv),
                           dim3(128 * KNW), 0, s, a);
        paired = true;
      } else if (!MASK || a.p.mask_vec) {
        hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, KNW, CM, MASK, false>), dim3(n_kt * a.p.B * a.p.Hkv),
                           dim3(128 * KNW), 0, s, a);
        paired = true;
      }
    }
    if (!paired)
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, KNW, CM, MASK>), dim3(n_kt * a.p.B * a.p.Hkv),
                         dim3(64 * KNW), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((stages & kBwdDq) && n_qt > 0) {
    if constexpr (BwdShape<D>::PAIR_DKDV) {
      if (ds_path) {
        // eight-wave workgroups where they still give every CU two; else four waves
        const int n8 = ((a.p.Lq + 255) / 256) * a.p.B * a.p.Hq;
        if (n8 >= 2 * kNumCu)
          hipLaunchKernelGGL((bwd_dq_ds_kernel<D, 8, CM>), dim3(n8), dim3(512), 0, s, a);
        else
          hipLaunchKernelGGL((bwd_dq_ds_kernel<D, 4, CM>), dim3(n_qt * a.p.B * a.p.Hq), dim3(256), 0, s, a);
        return hipGetLastError();
      }
    }
    if constexpr (MASK ? BwdShape<D>::PIPE_DQ_MASK : BwdShape<D>::PIPE_DQ)
      hipLaunchKernelGGL((bwd_dq_kernel<D, QNW, CM, MASK>), dim3(n_qt * a.p.B * a.p.Hq),
                         dim3(64 * QNW), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dq_seq_kernel<D, QNW, CM, MASK>), dim3(n_qt * a.p.B * a.p.Hq),
                         dim3(64 * QNW), 0, s, a);
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
  const bool mask = a.p.mask != nullptr;
  // the window's checks are compiled only into the windowed kernels
  if (a.p.causal && a.p.window > 0)
    return mask ? launch_main<D, 2, true>(a, stages, s) : launch_main<D, 2, false>(a, stages, s);
  if (a.p.causal) return mask ? launch_main<D, 1, true>(a, stages, s) : launch_main<D, 1, false>(a, stages, s);
  return mask ? launch_main<D, 0, true>(a, stages, s) : launch_main<D, 0, false>(a, stages, s);
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
