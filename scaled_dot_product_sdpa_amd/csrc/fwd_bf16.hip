// fwd_bf16.hip — prefill forward, bf16 in / fp32 accumulate, gfx950.
//
// Computes O = softmax(scale * Q K^T + mask) V and LSE per row ("Scaled dot-product
// attention (forward and backward)", section 2 Principles and 2.2 Masking; LSE as in
// cuDNN "Attention", SDPA FP16/BF16 Forward, Python API return values) with the
// one-pass online softmax (running max and sum; the page's "Going further" table names
// Milakov and Gimelshein's online normaliser).
//
// Work decomposition: a workgroup of NW waves owns BM = NW * 32 query rows of one
// (batch, head); each wave owns 32 query rows and keeps their Q operand, O accumulator
// and running statistics in registers.  K/V tiles of 64 keys stream HBM -> LDS with
// buffer loads straight into LDS (16 bytes per lane, no staging registers): while tile t
// is computed, tile t+1 is landing and tile t+2 is requested after the one barrier of the
// step, into two K and three V buffers.  Tiles are stored unpadded with XOR-swizzled
// 16-byte chunks (kern_common.h) so the MFMA operand reads are free of bank conflicts.
// The (batch, KV head) groups are spread over the XCDs so that a group's K/V stay in one
// L2 while all of its query tiles stream them.
//
//   S^T = K Q^T   (keys x queries): A = K rows from LDS (row-permuted, see kern_common.h),
//                 B = Q held in registers; lane l ends up with 16 consecutive keys of
//                 query l%32, so the row max needs v_max3 reductions in registers plus one
//                 permlane32 swap, and the row sums stay per half-wave until the end.
//   O^T += V^T P^T (d x queries): A = V^T read with ds_read_b64_tr_b16, B = bf16(P) taken
//                 straight from the S accumulator registers.  O^T keeps one query per
//                 lane, so a rescale is a per-lane multiply.
//
// Software pipeline inside each wave: the softmax of a 32-key block costs about as many
// SIMD cycles (16 exponentials and ~70 other vector ops per lane) as its 16 MFMAs, so
// the S MFMAs of block b+1 are issued interleaved with the softmax arithmetic of block b
// and the matrix and vector units of the SIMD work at the same time; the PV MFMAs of
// block b follow.
//
// Softmax arithmetic per score: one FMA folds scale * log2(e) and the reference max into
// the exp2 argument; v_exp_f32; v_cvt_pk_bf16_f32 (the B operand of the PV product); one
// add into the fp32 row sum, which both normalises O and gives LSE.  (The PV product
// weighs V with the bf16-rounded weights, so O's row weights sum to 1 within the bf16
// rounding of the weights, |error| <= 2^-9 of |O|.)  The reference max is only moved when
// a row's max grows by more than 2^8 (weights stay <= 256, exact in fp32 sums and in bf16
// range), so the O rescale runs on a few blocks only.
//
// Tiles entirely above the causal diagonal or past the key length are never visited, and
// a wave works only on the 32-key blocks that some of its rows can see (a prefix of the
// key range).  Only blocks touching the diagonal or a length boundary evaluate
// per-element predicates.  Rows with no visible key produce O = 0, LSE = -inf.
#include "kern_common.h"
#include "launch.h"

namespace sdpa {
namespace {

constexpr int kBN = 64;             // keys per K/V tile (two 32-key MFMA blocks)
constexpr float kRescaleLog2 = 8.f; // move the reference max only past this growth

template <int D, int NW, int WPE, int CM, bool MASK>
__global__ __launch_bounds__(64 * NW, WPE) void fwd_bf16_kernel(FwdArgs a) {
  constexpr bool CAUSAL = CM != 0;  // CM: 0 no diagonal, 1 causal, 2 causal + sliding window
  constexpr int BM = NW * 32;
  constexpr int TILE = kBN * D;
  // Tile t's K is read by the phases of blocks 2t-1 (the next block's scores) and 2t; its V
  // by those of blocks 2t and 2t+1.  Tile t+2 is requested after the barrier in the middle
  // of step t, so K needs two buffers (tile t's is free by then) and V three.
  // One LDS array, V buffers first: operand reads address their buffer with a constant in
  // the instruction's 16-bit offset field (see OpOffsets), which reaches the three V buffers
  // and the first K buffer.
  __shared__ __attribute__((aligned(16))) bf16 lds[5 * TILE];
  bf16* const Vb[3] = {lds, lds + TILE, lds + 2 * TILE};
  bf16* const Kb[2] = {lds + 3 * TILE, lds + 4 * TILE};

  const Problem& p = a.p;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int l32 = lane & 31;
  const int hi = lane >> 5;  // which half of the wave

  // ---- work item: (batch, KV head) group, then query tile `rank` of head h of the group
  // (the G heads of one rank adjacent in launch order).
  int gi, r;
  xcd_item(blockIdx.x, p.B * p.Hkv, (int)(gridDim.x / (p.B * p.Hkv)), p.G, !CAUSAL, gi, r);
  const int b = batch_by_work(p, gi / p.Hkv);
  const int g = gi % p.Hkv;
  const int h = g * p.G + r % p.G;
  const int rank = r / p.G;

  const int q_end = seq_len_q(p, b);
  const int kv_end = seq_len_kv(p, b);
  // Rows of this workgroup: query tile `rank` of BM rows; causal grids run the tiles
  // heavy first (tile n_qt - 1 - rank) and the scheduler evens the load.
  const int qt = CAUSAL ? (p.Lq + BM - 1) / BM - 1 - rank : rank;
  const int wq_lo = qt * BM + wave * 32;  // this wave's first row
  const int row_lo = qt * BM, row_hi = row_lo + BM;  // the workgroup's row span
  const int wq_hi = min(wq_lo + 32, q_end) - 1;  // this wave's last live row

  const bf16* qb = reinterpret_cast<const bf16*>(a.q) + q_base(p, b) + h * p.q_sh;
  const bf16* kb_ = reinterpret_cast<const bf16*>(a.k) + k_base(p, b) + g * p.k_sh;
  const bf16* vb_ = reinterpret_cast<const bf16*>(a.v) + v_base(p, b) + g * p.v_sh;
  bf16* ob = reinterpret_cast<bf16*>(a.o) + o_base(p, b) + h * p.o_sh;
  const bf16* mb_ = MASK ? reinterpret_cast<const bf16*>(p.mask) + b * p.m_sb + h * p.m_sh : nullptr;
  float* lseb = a.lse ? a.lse + ((int64_t)b * p.Hq + h) * p.Lq : nullptr;

  // Keys this tile of queries can see.
  int kv_stop = kv_end;
  const int coff = CAUSAL ? causal_offset(p.causal, q_end, kv_end) : 0;  // diagonal offset
  if (CAUSAL) kv_stop = min(kv_stop, min(row_hi, q_end) + coff);
  if (row_lo >= q_end) kv_stop = 0;
  const int n_tiles = kv_stop > 0 ? (kv_stop + kBN - 1) / kBN : 0;
  // Sliding window of W keys: the workgroup's first row sees no key before
  // row_lo + coff - W + 1, so the tiles before that one are skipped.
  const int W = CM == 2 ? p.window : 0;
  const int t0 = W > 0 ? min(max(row_lo + coff - W + 1, 0) / kBN, n_tiles) : 0;
  // 32-key blocks this wave works on: a prefix of the keys (from block 2 * t0).
  int vis_stop = wq_lo < q_end ? kv_stop : 0;
  if (CAUSAL) vis_stop = min(vis_stop, wq_hi + 1 + coff);
  const int nvis = vis_stop > 0 ? (vis_stop + 31) / 32 : 0;
  // The fewest blocks any wave of the workgroup works on (wave 0's on a causal diagonal; 0
  // if a wave's rows all lie past the length): tiles before t_full are whole for every wave.
  int vis_min = row_lo + 32 * (NW - 1) < q_end ? kv_stop : 0;
  if (CAUSAL) vis_min = min(vis_min, min(row_lo + 32, q_end) + coff);
  const int t_full = min(vis_min > 0 ? (vis_min + 31) / 32 / 2 : 0, n_tiles);

  // ---- K/V tiles: HBM -> LDS (rows past kv_stop arrive as zeros).
  TileCopy<kBN, D, NW> kcopy, vcopy;
  kcopy.init(p.k_sl, wave, lane);
  vcopy.init(p.v_sl, wave, lane);
  auto load_tile = [&](int j0, bf16* Kd, bf16* Vd) {
    kcopy.copy(rows_rsrc<D, kBN>(kb_, p.k_sl, j0, kv_stop), Kd, wave);
    vcopy.copy(rows_rsrc<D, kBN>(vb_, p.v_sl, j0, kv_stop), Vd, wave);
  };
  // ---- tile 0 and the Q operand (B of S^T = K Q^T: lane holds query row, 8 consecutive d
  // per k-step) land first; tile 1 streams in behind the first block.
  if (n_tiles > t0) load_tile(t0 * kBN, Kb[0], Vb[0]);
  const int qrow = wq_lo + l32;

  // Mask values of block `bi` for this lane (keys 32*bi + 16*hi + 0..15 of row qrow),
  // read two blocks ahead (see body).  Rows whose mask cannot be read with 16-byte loads
  // take the element path in pre_scores.
  // A block's mask values come as two 16-byte loads per lane when its 32 keys lie within the
  // mask rows (a test on the block alone, so that the whole wave takes one path); rows past
  // the last one read the last row instead, their scores being hidden by the predicates.
  auto mask_vec_ok = [&](int bi) { return p.mask_vec && 32 * bi + 32 <= p.Lk; };
  auto load_mask = [&](int bi, u32x4 (&m)[2]) {
    if (MASK && bi < nvis && mask_vec_ok(bi)) {
      const bf16* mp = mb_ + (int64_t)min(qrow, p.Lq - 1) * p.m_si + 32 * bi + 16 * hi;
      m[0] = ld16(mp);
      m[1] = ld16(mp + 8);
    } else {
      m[0] = zero16();
      m[1] = zero16();
    }
  };

  // Even blocks keep their mask values in mk_e, odd blocks in mk_o; the first two land
  // with the Q rows.
  u32x4 mk_e[2], mk_o[2];
  load_mask(2 * t0, mk_e);
  load_mask(2 * t0 + 1, mk_o);
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 x = qrow < q_end ? ld16(qb + (int64_t)qrow * p.q_sl + kk * 16 + 8 * hi) : zero16();
    qreg[kk] = __builtin_bit_cast(bf16x8, x);
  }
  wait_vmem();
  if (n_tiles > t0 + 1) load_tile((t0 + 1) * kBN, Kb[1], Vb[1]);

  // reference max (log2 units) and the sum of the fp32 weights relative to it (normalises
  // O and gives LSE), kept as two partial sums (even / odd scores) so the adds form two
  // chains.
  f32x16 oacc[D / 32];
  float mref = kNegInf, frow = 0.f, frow2 = 0.f;
  // The per-block test and offset come precomputed from the last move of mref, so a block
  // that leaves it in place spends one compare on it: mthr is the block max (raw score, or
  // natural units with a mask) past which mref moves, nmu the negated offset stage A adds
  // (0 while a row has seen no key).
  float mthr = kNegInf, nmu = 0.f;
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) oacc[mb] = f32x16{};

  const float c2 = p.scale_log2;
  const float sc = p.scale;
  // growth of the block max (raw score units; natural units with a mask) that moves mref
  const float thr = MASK ? kRescaleLog2 * kLn2 : kRescaleLog2 / c2;
  // K operand read: row kb*32 + perm_row(l32), logical chunk 2*kk + hi
  const int krow_l = perm_row(l32);
  // V^T operand (transposing read): row key_base + arow, logical chunk vchunk, half vhalf
  const int blk = lane >> 4;
  const int arow = (lane & 15) >> 2;
  const int vchunk = ((lane & 3) >> 1) + 2 * (blk & 1);
  const int vhalf = 4 * (lane & 1);

  constexpr int NS = D / 16;  // S MFMAs per block = K operand reads = PV MFMAs = V reads
  constexpr int E = 16 / NS;  // scores per lane handled in one pipeline slot
  constexpr int KPRE = 2;     // K operand reads issued ahead of their MFMA

  // K operands (row krow_l) and transposed V operands.  The K rows are read through tile
  // pointers moved back by the three V buffers (their offsets carry those bytes instead), so
  // that both K buffers lie within the read's 16-bit offset field and a read needs no add.
  OpOffsets<D> ofs;
  ofs.init(krow_l, hi, arow, vchunk, vhalf, 3 * TILE * 2);
  auto read_k1 = [&](const bf16* Kt, int kb, int kk) { return ofs.row8(Kt - 3 * TILE, kb * 32, kk); };
  // V^T operand i (half i / (D/32), d-block i % (D/32)) of the block at rows kb*32..
  auto read_v1 = [&](const bf16* Vt, int kb, int i) {
    const int half = i / (D / 32), mb = i % (D / 32);
    return ofs.tr8(Vt, kb * 32 + 8 * half, mb);  // rows kb*32 + 16 hi + 8 half + arow ..
  };

  // Scores of block bi before the max, in place in its S accumulator: raw dot products,
  // or with a mask scale * s + m in natural units; -inf where a block touching a boundary
  // hides a key.  Masked scores stay in natural units until the row max is subtracted: a
  // mask value near the bottom of the fp32 range (say the most negative bf16) times
  // log2(e) would overflow to -inf and turn a row masked that way into an empty one,
  // where the definition gives equal weights.
  // With a mask, the pairs a boundary block hides get a mask value of -inf before it is
  // added (the score itself is finite), so that the scores are written once, after the
  // branch: a branch that rewrites them makes the compiler copy all sixteen at its join.
  auto pre_scores = [&](int bi, f32x16& x, const u32x4 (&mk)[2]) {
    const int key_lo = 32 * bi;
    const int key0 = key_lo + 16 * hi;
    const bool partial = (key_lo + 32 > kv_end) || (CAUSAL && key_lo + 31 > wq_lo + coff) ||
                         (wq_lo + 32 > q_end) || (W > 0 && key_lo <= wq_hi + coff - W);
    auto visible = [&](int v) __attribute__((always_inline)) {
      const int key = key0 + v;
      return (key < kv_end) & (qrow < q_end) & (!CAUSAL | (key <= qrow + coff)) &
             ((W == 0) | (key > qrow + coff - W));
    };
    if (MASK) {
      float mv[16];
      if (mask_vec_ok(bi)) {
        const bf16x8 b0 = __builtin_bit_cast(bf16x8, mk[0]), b1 = __builtin_bit_cast(bf16x8, mk[1]);
#pragma unroll
        for (int v = 0; v < 8; ++v) { mv[v] = bf2f(b0[v]); mv[v + 8] = bf2f(b1[v]); }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          mv[v] = (qrow < q_end && key0 + v < kv_end) ? bf2f(mb_[(int64_t)qrow * p.m_si + key0 + v]) : 0.f;
      }
      if (partial) {
#pragma unroll
        for (int v = 0; v < 16; ++v) mv[v] = visible(v) ? mv[v] : kNegInf;
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) x[v] = fmaf(x[v], sc, mv[v]);
    } else if (partial) {
#pragma unroll
      for (int v = 0; v < 16; ++v) x[v] = visible(v) ? x[v] : kNegInf;
    }
  };

  // Row max of the block (partial maxima `mx` over the lane's scores) -> moves the
  // reference max if some row grew past the threshold; returns the negated offset stage A
  // adds to the scores.  mref is in log2 units, or in natural units with a mask.
  auto post_max = [&](float mx) {
    mx = xhalf_max(mx);
    const bool need = mx > mthr;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float mt = MASK ? mx : mx * c2;  // block max in mref's units (c2 > 0)
      const float mnew = need ? mt : mref;
      const float corr = need ? fast_exp2(MASK ? (mref - mnew) * kLog2e : mref - mnew) : 1.f;
      mref = mnew;
      mthr = need ? mx + thr : mthr;
      nmu = mref == kNegInf ? 0.f : -mref;
      frow *= corr;
      frow2 *= corr;
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) oacc[mb] *= corr;
    }
    return nmu;
  };

  // Weights of score pair pr (scores 2pr, 2pr+1) in three stages one pipeline slot apart,
  // so that no stage waits on the result of the one before it:
  //   A: exp2 argument;  B: exp2;  C: bf16 B operand of O^T += V^T P^T, both sums.
  auto stage_a = [&](const f32x16& x, float nm, int pr, f32x2 (&t)[8]) {
    if (MASK) {
      t[pr][0] = (x[2 * pr] + nm) * kLog2e;
      t[pr][1] = (x[2 * pr + 1] + nm) * kLog2e;
    } else {
      t[pr][0] = fmaf(x[2 * pr], c2, nm);
      t[pr][1] = fmaf(x[2 * pr + 1], c2, nm);
    }
  };
  auto stage_b = [&](int pr, f32x2 (&t)[8]) {
    t[pr][0] = fast_exp2(t[pr][0]);
    t[pr][1] = fast_exp2(t[pr][1]);
  };
  auto stage_c = [&](int pr, const f32x2 (&t)[8], bf16x8 (&pop)[2]) {
    const bf16x2 e2 = __builtin_convertvector(t[pr], bf16x2);
    frow += t[pr][0];
    frow2 += t[pr][1];
    pop[pr / 4][2 * (pr % 4)] = e2[0];
    pop[pr / 4][2 * (pr % 4) + 1] = e2[1];
  };

  // PV operands of the previous block, consumed one block late (zero before the first).
  bf16x8 pv_v[NS];
  bf16x8 pv_p[2];
#pragma unroll
  for (int i = 0; i < NS; ++i) pv_v[i] = bf16x8{};
  pv_p[0] = bf16x8{};
  pv_p[1] = bf16x8{};
  auto pv_mfma1 = [&](int i) {
    const int half = i / (D / 32), mb = i % (D / 32);
    oacc[mb] = mfma32(pv_v[i], pv_p[half], oacc[mb]);
  };

  // S of the current block and of the next one; the two phases of a tile step swap them.
  f32x16 sacc_a = f32x16{}, sacc_b = f32x16{};

  // ---- one pipeline phase for block bi (V rows kb*32.. of Vt; the next block's K rows
  // kbn*32.. of Kn).  Region 1: PV MFMAs of block bi-1 with the row max of block bi.
  // Region 2: S MFMAs of block bi+1 with the exponentials and sums of block bi, the K
  // operand reads of block bi+1 and the V operand reads of block bi.  Slots are fenced
  // with sched_barrier so each MFMA issues next to its share of vector work.
  // The S of block bi+1 is computed even past the wave's last block (from whatever the
  // buffer holds; never used), which keeps one code path.
  // With a mask, the block takes its mask values from `mk` and requests those of block
  // bi+2 into the same registers.  The load is issued before the wait ahead of the next
  // tile barrier and used only after it, so it adds no wait of its own (the compiler, which
  // cannot see the tile copies, would otherwise wait for everything in flight, the next
  // tile's copy included, before the first use of a mask value).
  auto body = [&](int bi, const bf16* Vt, int kb, const bf16* Kn, int kbn, f32x16& x,
                  f32x16& snext, u32x4 (&mk)[2]) __attribute__((always_inline)) {
    bf16x8 kop[NS];
    pre_scores(bi, x, mk);
    // region 1
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (j < KPRE) kop[j] = read_k1(Kn, kbn, j);
      if (MASK && j == 0) load_mask(bi + 2, mk);
      pv_mfma1(j);
#pragma unroll
      for (int v = j * E; v < (j + 1) * E; ++v) mx = fmaxf(mx, x[v]);
      __builtin_amdgcn_sched_barrier(0);
    }
    const float nm = post_max(mx);
    // region 2

    // At d=128 region 2 runs at raised wave priority: of the two waves on a SIMD, the one
    // in its exponential and S slots issues first, and the other's PV MFMAs and row max
    // fill in (measured: causal GQA 4k 275 -> 268 us, sliding window 149 -> 147 us; at
    // d=64 the same costs 5 %, so it is left out there).
    if constexpr (D == 128) __builtin_amdgcn_s_setprio(1);
    snext = f32x16{};
    constexpr int P = 8 / NS;  // score pairs per slot
    f32x2 t[8];
#pragma unroll
    for (int pr = 0; pr < 2 * P; ++pr) stage_a(x, nm, pr, t);
#pragma unroll
    for (int pr = 0; pr < P; ++pr) stage_b(pr, t);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + KPRE < NS) kop[i + KPRE] = read_k1(Kn, kbn, i + KPRE);
      pv_v[i] = read_v1(Vt, kb, i);
      snext = mfma32(kop[i], qreg[i], snext);
#pragma unroll
      for (int pr = (i + 2) * P; pr < (i + 3) * P && pr < 8; ++pr) stage_a(x, nm, pr, t);
#pragma unroll
      for (int pr = (i + 1) * P; pr < (i + 2) * P && pr < 8; ++pr) stage_b(pr, t);
#pragma unroll
      for (int pr = i * P; pr < (i + 1) * P; ++pr) stage_c(pr, t, pv_p);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (D == 128) __builtin_amdgcn_s_setprio(0);
    // this block's P stays computed inside this phase (see pin)
    pin(pv_p[0]);
    pin(pv_p[1]);
  };
  // `whole`: every wave works on this block (no per-wave test, so the phases join without
  // the register copies a conditional phase costs).
  auto phase = [&](int bi, const bf16* Vt, int kb, const bf16* Kn, int kbn, f32x16& sacc,
                   f32x16& snext, u32x4 (&mk)[2], bool whole) __attribute__((always_inline)) {
    if (whole || bi < nvis) body(bi, Vt, kb, Kn, kbn, sacc, snext, mk);
  };

  // One tile step; the loop below is unrolled by six (two K buffers, three V buffers) so
  // that every buffer index is a compile-time constant.
  auto step = [&](int t, const bf16* Kc, const bf16* Vc, const bf16* Kn, bf16* Kl, bf16* Vl,
                  bool whole) __attribute__((always_inline)) {
    ofs.repin();
    // block 2t: V from this tile, K of block 2t+1 from this tile
    phase(2 * t, Vc, 0, Kc, 1, sacc_a, sacc_b, mk_e, whole);
    // tile t+1 has landed for every wave, and no wave still reads K of tile t or V of
    // tile t-1.  The wait is unconditional (after the last tile only mask loads are in
    // flight) so that the compiler sees every earlier load complete on every path.
    wait_vmem();
    __syncthreads();
    if (t + 2 < n_tiles) load_tile((t + 2) * kBN, Kl, Vl);
    // block 2t+1: V from this tile, K of block 2t+2 from the next tile
    phase(2 * t + 1, Vc, 1, Kn, 0, sacc_b, sacc_a, mk_o, whole);
  };

  if (n_tiles > t0) {
    __syncthreads();  // every wave's share of the first tile has landed
    if (nvis > 2 * t0) {
#pragma unroll
      for (int kk = 0; kk < NS; ++kk) sacc_a = mfma32(read_k1(Kb[0], 0, kk), qreg[kk], sacc_a);
    }
  }
  // whole groups of six tiles that every wave works on whole, then the rest (the diagonal
  // and the lengths) with a per-wave test of each block.  With a mask the second copy of the
  // loop costs more registers than two waves per SIMD leave, so it runs the tested loop only.
  const int tl_main = !MASK && t_full > t0 ? (t_full - t0) / 6 * 6 : 0;
  for (int tl = 0; tl < tl_main; tl += 6) {
#pragma unroll
    for (int u = 0; u < 6; ++u)
      step(t0 + tl + u, Kb[u % 2], Vb[u % 3], Kb[(u + 1) % 2], Kb[u % 2], Vb[(u + 2) % 3], true);
  }
  for (int tl = tl_main; tl < n_tiles - t0; tl += 6) {
#pragma unroll
    for (int u = 0; u < 6; ++u)
      if (tl + u < n_tiles - t0)
        step(t0 + tl + u, Kb[u % 2], Vb[u % 3], Kb[(u + 1) % 2], Kb[u % 2], Vb[(u + 2) % 3], false);
  }
  // the last block's PV
#pragma unroll
  for (int j = 0; j < NS; ++j) pv_mfma1(j);

  // ---- epilogue: O = O^T / f (0 for empty rows), LSE = ln2 * mref + ln f (mref + ln f with
  // a mask).
  const float ft = xhalf_sum(frow + frow2);
  const bool rowlive = qrow < q_end && ft > 0.f;
  const float inv = rowlive ? 1.f / ft : 0.f;
  if (qrow < q_rows_out(p, q_end)) {
    bf16* orow = ob + (int64_t)qrow * p.o_sl;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(oacc[mb][v4 * 4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + mb * 32 + v4 * 8 + hi * 4) = w;
      }
    }
  }
  if (qrow < p.Lq && lseb && hi == 0) lseb[qrow] = rowlive ? ((MASK ? mref : mref * kLn2) + logf(ft)) : kNegInf;
}

template <int D, int NW, int WPE, int CM, bool MASK>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
  constexpr int BM = NW * 32;
  const int n_qt = (a.p.Lq + BM - 1) / BM;
  const int grid = n_qt * a.p.B * a.p.Hq;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, WPE, CM, MASK>), dim3(grid), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

template <int D, int CM, bool MASK>
hipError_t launch_shape(const FwdArgs& a, hipStream_t s) {
  // Two independent workgroups of 4 waves (128 query rows) per CU: two waves per SIMD hide
  // each other's LDS and MFMA latencies, and the two workgroups' barriers do not wait for
  // each other (measured faster than one 8-wave workgroup per CU on every workload here:
  // causal MHA 1k 26.3 -> 23.1 us, causal GQA 4k 318 -> 309 us, padded 2k 217 -> 205 us).
  return launch_t<D, 4, 2, CM, MASK>(a, s);
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  const bool mask = a.p.mask != nullptr;
  // the window's checks are compiled only into the windowed kernels
  if (a.p.causal && a.p.window > 0)
    return mask ? launch_shape<D, 2, true>(a, s) : launch_shape<D, 2, false>(a, s);
  if (a.p.causal) return mask ? launch_shape<D, 1, true>(a, s) : launch_shape<D, 1, false>(a, s);
  return mask ? launch_shape<D, 0, true>(a, s) : launch_shape<D, 0, false>(a, s);
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
