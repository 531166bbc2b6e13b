// decode_bf16.hip — single-query (L_q = 1) forward with split-KV, bf16, gfx950.
//
// Same operation as the prefill forward for one query position per head.  The work is
// bound by reading the KV cache from HBM ("Understanding PyTorch Scaled Dot-Product
// Attention" section 5: the KV cache dominates decode), so:
//  - the G = Hq/Hkv (at most 16) query heads that share a KV head are packed into the N
//    columns of a 16x16x32 MFMA tile (lane l%16 < G is query head g*G + l%16), so each K/V
//    byte is read once for all of them ("Understanding PyTorch Scaled Dot-Product
//    Attention" section 4 for the head map);
//  - the keys of one (batch, KV head) are cut into splits of split_keys keys; every split
//    is an independent one-wave workgroup that streams 32-key K/V tiles from HBM into
//    registers with buffer loads (rows past the split read as zeros), two tiles in flight;
//    two such waves run per SIMD; splits past the sequence length exit at once; each split
//    writes a partial (O_c normalised, lse_c);
//  - a combine kernel merges the partials exactly:  LSE = ln sum_c exp(lse_c),
//    O = sum_c exp(lse_c - LSE) O_c  (the log-sum-exp merge of split-KV partial results
//    that cuDNN "Attention", SDPA FP16/BF16 Forward, Python API describes for its stats).
#include "kern_common.h"
#include "launch.h"

namespace sdpa {
namespace {

constexpr int kDT = 32;  // keys per tile

// The KV cache is read once, so its loads carry the non-temporal cache policy (measured: 12 %
// more bandwidth than the default policy on the 8k-key GQA decode).
constexpr int kNonTemporal = 2;

// 16x16x32 MFMAs: the N columns are the (at most 16) query heads of the group, so a quarter
// of the columns do useful work where a 32-wide tile would use an eighth, and each lane holds
// 8 scores per 32-key tile instead of 16.
//   S^T (16 keys x heads) = K (16 keys x 32 d) . Q^T, twice per tile: lane (g4 = l/16,
//       i16 = l%16) ends with keys 4*g4 + v (first block) and 16 + 4*g4 + v (second) of head
//       i16.  The K operand is loaded from HBM straight into registers in the MFMA layout
//       (lane: key i16 of the block, d = 32*kk + 8*g4 .. +7).
//   O^T (16 d x heads) += V^T (16 d x 32 keys) . P^T: the 32 keys in the order lane g4
//       holds them (4*g4 + 0..3, 16 + 4*g4 + 0..3), so bf16(P) feeds the B operand as is.
//       V rows are loaded into registers whole (coalesced), written to LDS and read back
//       transposed (ds_read_b64_tr_b16).
// Two register sets of K and V rows: while tile t is computed, tile t+1 is in flight and
// tile t+2 is requested as soon as tile t's K operands and V rows have been consumed.
// PAGED: the cache lives in pages (a 32-key tile never straddles two, since the page size
// is a multiple of 32); each lane first reads the page index of one tile of the split,
// and a tile's rows are then addressed from its page like the rows of a contiguous cache.
// First key the query row sees: 0, or kv_end - W under a sliding window of W keys (the
// bottom-right diagonal of one query row ends at the last key).
__device__ __forceinline__ int decode_key_start(const Problem& p, int kv_end) {
  return (p.causal && p.window > 0) ? max(0, kv_end - p.window) : 0;
}

template <int D, bool PAGED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_split_kernel(DecodeArgs a) {
  constexpr int TILE = kDT * D;
  constexpr int NK = D / 32;          // k-steps of one S^T block
  constexpr int NM = D / 16;          // 16-row d blocks of O^T
  constexpr int LPR = D / 8;          // lanes per V row (16 bytes each)
  constexpr int RPL = 64 / LPR;       // V rows per load instruction
  constexpr int VLD = kDT / RPL;      // V load instructions per tile
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][TILE];
  const Problem& p = a.p;
  const int lane = threadIdx.x;
  const int g4 = lane >> 4;
  const int i16 = lane & 15;

  const int c = blockIdx.x / (p.B * p.Hkv);  // split-major: every live split of split c
  const int bg = blockIdx.x % (p.B * p.Hkv); // precedes the (mostly empty) higher splits
  const int b = bg / p.Hkv;
  const int g = bg % p.Hkv;
  const int kv_end = seq_len_kv(p, b);
  // a sliding window of W keys leaves the single query row the keys [klo, kv_end) with
  // klo = kv_end - W; the split's first tile starts on the 32-key boundary below klo (so a
  // tile never straddles a page) and the keys before klo are masked
  const int klo = decode_key_start(p, kv_end);
  const int k0 = max(c * a.split_keys, klo / kDT * kDT);
  const int k1 = min(c * a.split_keys + a.split_keys, kv_end);
  // the combine reads only splits that hold keys, and none of a batch whose query row is
  // past its length (an empty row)
  if (k0 >= k1 || seq_len_q(p, b) < 1) return;
  const int n_tiles = (k1 - k0 + kDT - 1) / kDT;

  const bool qvalid = i16 < p.G;
  const int h = g * p.G + (qvalid ? i16 : 0);
  const bf16* qrow = reinterpret_cast<const bf16*>(a.q) + q_base(p, b) + h * p.q_sh;
  const bf16* kbase = reinterpret_cast<const bf16*>(a.k) + (PAGED ? 0 : k_base(p, b)) + g * p.k_sh;
  const bf16* vbase = reinterpret_cast<const bf16*>(a.v) + (PAGED ? 0 : v_base(p, b)) + g * p.v_sh;
  // page index of tile `lane` of the split (the table column and the page are clamped into
  // the table row and the containers, so a length or entry out of range reads no memory
  // outside them); a split has at most 64 tiles
  int lane_page = 0;
  if (PAGED && lane < n_tiles) {
    const int col = min((k0 + kDT * lane) / a.page_size, a.max_pages - 1);
    const int pg = a.page_table[(int64_t)b * a.max_pages + col];
    lane_page = min(max(pg, 0), a.num_pages - 1);
  }

  // Per-lane byte offsets inside a tile (the tile's first row moves with the resource; the
  // whole offset is in the vector operand, which is what the range check covers): K operand
  // of block kb, k-step kk at koff[kb] + 64 * kk; V row load i at voff[i].
  uint32_t koff[2], voff[VLD];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) koff[kb] = (uint32_t)((16 * kb + i16) * p.k_sl * 2 + 16 * g4);
  const int vr = lane / LPR, vc = lane % LPR;
  // LDS element offset of V row vr + RPL*i, chunk vc, in the layout the transposing reads use
  int vlds[VLD];
#pragma unroll
  for (int i = 0; i < VLD; ++i) {
    const int r = vr + RPL * i;
    voff[i] = (uint32_t)(r * p.v_sl * 2 + 16 * vc);
    vlds[i] = r * D + ((vc ^ swz_sel<D, 2>(r)) * 8);
  }

  u32x4 kr[2][2][NK], vrg[2][VLD];
  // Tile t into register set `set`: rows of the split only (past them the loads return 0).
  auto load_tile = [&](int t, int set) __attribute__((always_inline)) {
    const int j0 = min(k0 + t * kDT, k1);
    const int n = min(kDT, k1 - j0);
    const bf16* kt = kbase;
    const bf16* vt = vbase;
    int row = j0;
    if (PAGED) {
      // tiles past the split (t >= n_tiles, empty range) read lane t's 0
      const int page = __builtin_amdgcn_readlane(lane_page, min(t, 63));
      kt += (int64_t)page * a.kp_stride;
      vt += (int64_t)page * a.vp_stride;
      row = j0 % a.page_size;
    }
    const reg_rsrc_t kr_ = reg_rsrc(kt + (int64_t)row * p.k_sl, n > 0 ? (int64_t)(n - 1) * p.k_sl * 2 + D * 2 : 0);
    const reg_rsrc_t vr_ = reg_rsrc(vt + (int64_t)row * p.v_sl, n > 0 ? (int64_t)(n - 1) * p.v_sl * 2 + D * 2 : 0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) kr[set][kb][kk] = reg_ld16<kNonTemporal>(kr_, koff[kb] + 64 * kk, 0);
#pragma unroll
    for (int i = 0; i < VLD; ++i) vrg[set][i] = reg_ld16<kNonTemporal>(vr_, voff[i], 0);
  };
  // Q^T operand (lane (g4, i16) holds d = 32*kk + 8*g4 .. +7 of head i16), loaded before
  // the tiles so that it is never the youngest load in flight at the top of the loop.
  bf16x8 qreg[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
    qreg[kk] = __builtin_bit_cast(bf16x8, qvalid ? ld16(qrow + kk * 32 + 8 * g4) : zero16());
  // The loads are unconditional: a tile past the split has an empty range and reads zeros
  // without touching memory, and every path then has the same loads in flight, so the
  // compiler's waits before each tile's first use stay exact (tile t+1 keeps streaming).
  load_tile(0, 0);
  load_tile(1, 1);

  f32x4 oacc[NM];
#pragma unroll
  for (int mb = 0; mb < NM; ++mb) oacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // reference max (log2 units; moved only when a tile's max exceeds it by more than 2^8, so
  // weights stay <= 256), rounded-weight sum, fp32-weight sum (per lane: its 8 keys)
  float mref = kNegInf, lrow = 0.f, frow = 0.f;

  const float c2 = p.scale_log2;
  const bf16x2 ones2 = {(bf16)1.f, (bf16)1.f};
  // transposing reads: lane j of a 16-lane block supplies row base + j/4, d 4*(j%4) .. +3
  const int trow = i16 >> 2;
  const int tchunk = (i16 & 3) >> 1;
  const int thalf = 4 * (i16 & 1);

  // max / sum over the four lanes l, l^16, l^32, l^48 (one head)
  auto max4 = [](float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return xhalf_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
  };
  auto sum4 = [](float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return xhalf_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
  };

  // One tile from register set `set` (unrolled by two so the set is a compile-time index).
  auto step = [&](int t, int set) __attribute__((always_inline)) {
    const int j0 = k0 + t * kDT;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      s0 = mfma16(__builtin_bit_cast(bf16x8, kr[set][0][kk]), qreg[kk], s0);
      s1 = mfma16(__builtin_bit_cast(bf16x8, kr[set][1][kk]), qreg[kk], s1);
    }
    // V rows to LDS (the same wave reads them back below; LDS operations of one wave
    // complete in order), then the register set takes tile t+2.  In the window's first
    // tile the rows before its first key are zeroed: their weight is 0, but the cache
    // there may hold anything (an evicted page), and 0 * NaN would poison O.
    bf16* vt = Vs[set];
    if (j0 < klo) {
#pragma unroll
      for (int i = 0; i < VLD; ++i)
        if (j0 + vr + RPL * i < klo) vrg[set][i] = zero16();
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) *reinterpret_cast<u32x4*>(vt + vlds[i]) = vrg[set][i];
    load_tile(t + 2, set);

    float x[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) { x[v] = s0[v]; x[4 + v] = s1[v]; }
    if (j0 + kDT > k1 || j0 < klo) {
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int key = j0 + (v < 4 ? 0 : 16) + 4 * g4 + (v & 3);
        x[v] = (key < k1 && key >= klo) ? x[v] : kNegInf;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mx = max4(mx) * c2;
    const bool need = mx > mref + 8.f;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float mnew = need ? mx : mref;
      const float corr = need ? fast_exp2(mref - mnew) : 1.f;
      mref = mnew;
      lrow *= corr;
      frow *= corr;
#pragma unroll
      for (int mb = 0; mb < NM; ++mb) oacc[mb] *= corr;
    }
    const float m_use = (mref == kNegInf) ? 0.f : mref;
    bf16x8 pop;
    float psum = lrow, fsum = frow;
#pragma unroll
    for (int t2 = 0; t2 < 4; ++t2) {
      f32x2 e;
      e[0] = fast_exp2(fmaf(x[2 * t2], c2, -m_use));
      e[1] = fast_exp2(fmaf(x[2 * t2 + 1], c2, -m_use));
      const bf16x2 e2 = __builtin_convertvector(e, bf16x2);
      psum = __builtin_amdgcn_fdot2_f32_bf16(e2, ones2, psum, false);
      fsum += e[0];
      fsum += e[1];
      pop[2 * t2] = e2[0];
      pop[2 * t2 + 1] = e2[1];
    }
    lrow = psum;
    frow = fsum;
#pragma unroll
    for (int mb = 0; mb < NM; ++mb) {
      const bf16x8 vop = join_tr(tile_tr4<D, 2>(vt, 4 * g4 + trow, 2 * mb + tchunk, thalf),
                                 tile_tr4<D, 2>(vt, 16 + 4 * g4 + trow, 2 * mb + tchunk, thalf));
      oacc[mb] = mfma16(vop, pop, oacc[mb]);
    }
  };

  // Both steps in every trip (an odd last tile after the loop), so that at the top of the
  // loop tile t's set is always the older one in flight.
  int t = 0;
  for (; t + 1 < n_tiles; t += 2) {
    step(t, 0);
    step(t + 1, 1);
  }
  if (t < n_tiles) step(t, 0);

  const float lt = sum4(lrow);
  const float ft = sum4(frow);
  if (qvalid) {
    const int64_t prow = ((int64_t)b * p.Hq + h) * a.n_split + c;  // partial row
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int mb = 0; mb < NM; ++mb) *reinterpret_cast<f32x4*>(po + 16 * mb + 4 * g4) = oacc[mb] * inv;
    if (g4 == 0) a.part_lse[prow] = lt > 0.f ? (mref * kLn2 + logf(ft)) : kNegInf;
  }
}

// One wave per (batch, query head), four per workgroup: merge the live splits.  Every
// lane reads the lse of its splits at once; the partial rows are then read 16 splits at a
// time (independent loads, so one memory latency covers up to 16 splits), each lane owning
// D/64 consecutive elements of the row.
constexpr int kCombineWaves = 4;
template <int D>
__global__ __launch_bounds__(64 * kCombineWaves) void decode_combine_kernel(DecodeArgs a) {
  constexpr int E = D / 64;  // elements per lane
  const Problem& p = a.p;
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
  if (bh >= p.B * p.Hq) return;
  const int b = bh / p.Hq;
  const int h = bh % p.Hq;
  const int kv_end = seq_len_kv(p, b);
  const bool row_live = seq_len_q(p, b) >= 1;  // else the row is empty: O = 0, LSE = -inf
  // live splits c_lo .. c_lo + n_live - 1 (those holding a key of the row's range)
  const int klo = decode_key_start(p, kv_end);
  const int c_lo = klo / a.split_keys;
  const int n_live = row_live && kv_end > klo ? (kv_end + a.split_keys - 1) / a.split_keys - c_lo : 0;
  const float* pl = a.part_lse + (int64_t)bh * a.n_split + c_lo;
  const float* po = a.part_o + ((int64_t)bh * a.n_split + c_lo) * D + E * lane;
  // M = max_c lse_c, L = sum_c exp(lse_c - M) over the live splits
  float M = kNegInf;
  for (int c = lane; c < n_live; c += 64) M = fmaxf(M, pl[c]);
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) M = fmaxf(M, __shfl_xor(M, w));
  float L = 0.f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  if (M != kNegInf) {
    for (int c0 = 0; c0 < n_live; c0 += 64) {
      const int nc = min(64, n_live - c0);
      const float wl = lane < nc ? expf(pl[c0 + lane] - M) : 0.f;  // weight of split c0 + lane
      L += wl;
      for (int c = 0; c < nc; c += 16) {
        float x[16][E];
#pragma unroll
        for (int u = 0; u < 16; ++u)
#pragma unroll
          for (int e = 0; e < E; ++e) x[u][e] = c + u < nc ? po[(int64_t)(c0 + c + u) * D + e] : 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float w = __shfl(wl, c + u);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] = fmaf(w, x[u][e], acc[e]);
        }
      }
    }
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) L += __shfl_xor(L, w);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (row_live || !p.off_q) {  // a packed batch with no query row owns no output row
    bf16* orow = reinterpret_cast<bf16*>(a.o) + o_base(p, b) + h * p.o_sh + E * lane;
#pragma unroll
    for (int e = 0; e < E; ++e) orow[e] = (bf16)(acc[e] * inv);
  }
  if (a.lse && lane == 0) a.lse[bh] = (L > 0.f) ? M + logf(L) : kNegInf;
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  const int grid = a.p.B * a.p.Hkv * a.n_split;
  if (grid > 0) {
    if (a.page_table)
      hipLaunchKernelGGL((decode_split_kernel<D, true>), dim3(grid), dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((decode_split_kernel<D, false>), dim3(grid), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int rows = a.p.B * a.p.Hq;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((rows + kCombineWaves - 1) / kCombineWaves),
                     dim3(64 * kCombineWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace

void decode_split_plan(int B, int Hkv, int Lk, int* split_keys, int* n_split) {
  // Enough splits that the (batch, KV head) pairs times splits fill the chip several
  // times over, without partial-result traffic becoming noticeable; split sizes stay whole
  // 32-key tiles (so a tile never straddles a page) and at most 64 tiles (one page index
  // per lane).  768 keys measured best on the 8k-key GQA decode (512: 2-3 % slower, 640:
  // 3 % slower, 1024 and 256: 5-7 % slower).
  int sk = 768;
  const int64_t pairs = (int64_t)B * Hkv;
  while (sk > kDT && pairs * ((Lk + sk - 1) / sk) < 2048) sk = max(kDT, sk / 2 / kDT * kDT);
  *split_keys = sk;
  *n_split = Lk > 0 ? (Lk + sk - 1) / sk : 1;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  switch (a.p.D) {
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdpa
