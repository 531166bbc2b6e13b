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
//    is an independent one-wave workgroup that streams 32-key K/V tiles HBM -> LDS with
//    buffer loads (no staging registers and no address arithmetic per copy), double
//    buffered; the small LDS and register footprint keeps two such waves per SIMD; splits
//    past the sequence length exit at once; each split writes a partial (O_c normalised,
//    lse_c);
//  - a combine kernel merges the partials exactly:  LSE = ln sum_c exp(lse_c),
//    O = sum_c exp(lse_c - LSE) O_c  (the log-sum-exp merge of split-KV partial results
//    that cuDNN "Attention", SDPA FP16/BF16 Forward, Python API describes for its stats).
#include "kern_common.h"
#include "launch.h"

namespace sdpa {
namespace {

constexpr int kDT = 32;  // keys per tile

// 16x16x32 MFMAs: the N columns are the (at most 16) query heads of the group, so a quarter
// of the columns do useful work where a 32-wide tile would use an eighth, and each lane holds
// 8 scores per 32-key tile instead of 16.
//   S^T (16 keys x heads) = K (16 keys x 32 d) . Q^T, twice per tile: lane (g4 = l/16,
//       i16 = l%16) ends with keys 4*g4 + v (first block) and 16 + 4*g4 + v (second) of head
//       i16;
//   O^T (16 d x heads) += V^T (16 d x 32 keys) . P^T: the 32 keys in the order lane g4
//       holds them (4*g4 + 0..3, 16 + 4*g4 + 0..3), so bf16(P) feeds the B operand as is and
//       V^T comes from two transposing reads per d block.
template <int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_split_kernel(DecodeArgs a) {
  constexpr int TILE = kDT * D;
  constexpr int NK = D / 32;  // k-steps of one S^T block
  constexpr int NM = D / 16;  // 16-row d blocks of O^T
  __shared__ __attribute__((aligned(16))) bf16 K0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 K1[TILE];
  __shared__ __attribute__((aligned(16))) bf16 V0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 V1[TILE];
  const Problem& p = a.p;
  const int lane = threadIdx.x;
  const int g4 = lane >> 4;
  const int i16 = lane & 15;

  const int c = blockIdx.x % a.n_split;
  const int bg = blockIdx.x / a.n_split;
  const int b = bg / p.Hkv;
  const int g = bg % p.Hkv;
  const int kv_end = p.len_kv ? min(p.len_kv[b], p.Lk) : p.Lk;
  const int k0 = c * a.split_keys;
  if (k0 >= kv_end) return;  // the combine reads only splits that hold keys
  const int k1 = min(k0 + a.split_keys, kv_end);
  const int n_tiles = (k1 - k0 + kDT - 1) / kDT;

  const bool qvalid = i16 < p.G;
  const int h = g * p.G + (qvalid ? i16 : 0);
  const bf16* qrow = reinterpret_cast<const bf16*>(a.q) + b * p.q_sb + h * p.q_sh;
  const bf16* kbase = reinterpret_cast<const bf16*>(a.k) + b * p.k_sb + g * p.k_sh;
  const bf16* vbase = reinterpret_cast<const bf16*>(a.v) + b * p.v_sb + g * p.v_sh;

  // K/V tiles HBM -> LDS, one tile ahead (rows past the split arrive as zeros), each with
  // the swizzle of the way it is read
  TileCopy<kDT, D, 1, 1> kcopy;
  TileCopy<kDT, D, 1, 2> vcopy;
  kcopy.init(p.k_sl, 0, lane);
  vcopy.init(p.v_sl, 0, lane);
  auto load_tile = [&](int t, bf16* Kd, bf16* Vd) {
    kcopy.copy(rows_rsrc<D, kDT>(kbase, p.k_sl, k0 + t * kDT, k1), Kd, 0);
    vcopy.copy(rows_rsrc<D, kDT>(vbase, p.v_sl, k0 + t * kDT, k1), Vd, 0);
  };
  load_tile(0, K0, V0);

  // Q^T operand: lane (g4, i16) holds d = 32*kk + 8*g4 .. +7 of head i16
  bf16x8 qreg[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
    qreg[kk] = __builtin_bit_cast(bf16x8, qvalid ? ld16(qrow + kk * 32 + 8 * g4) : zero16());

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

  // One tile; unrolled by two over the LDS buffers so the reads of tile t and the copies
  // into the other buffer are distinct LDS objects at compile time.  The buffer refilled
  // with tile t+1 held tile t-1, whose reads all completed before its MFMAs.  The copy is
  // unconditional: past the split every row is out of the buffer's range and the copy
  // writes zeros without touching memory.
  auto step = [&](int t, const bf16* Kt, const bf16* Vt, bf16* Kl, bf16* Vl)
                  __attribute__((always_inline)) {
    const int j0 = k0 + t * kDT;
    wait_vmem();  // tile t landed
    load_tile(t + 1, Kl, Vl);

    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      s0 = mfma16(tile_row8<D, 1>(Kt, i16, 4 * kk + g4), qreg[kk], s0);
      s1 = mfma16(tile_row8<D, 1>(Kt, 16 + i16, 4 * kk + g4), qreg[kk], s1);
    }
    float x[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) { x[v] = s0[v]; x[4 + v] = s1[v]; }
    if (j0 + kDT > k1) {
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int key = j0 + (v < 4 ? 0 : 16) + 4 * g4 + (v & 3);
        x[v] = key < k1 ? x[v] : kNegInf;
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
      const bf16x8 vop = join_tr(tile_tr4<D, 2>(Vt, 4 * g4 + trow, 2 * mb + tchunk, thalf),
                                 tile_tr4<D, 2>(Vt, 16 + 4 * g4 + trow, 2 * mb + tchunk, thalf));
      oacc[mb] = mfma16(vop, pop, oacc[mb]);
    }
  };

  for (int t = 0; t < n_tiles; t += 2) {
    step(t, K0, V0, K1, V1);
    if (t + 1 < n_tiles) step(t + 1, K1, V1, K0, V0);
  }
  wait_vmem();  // the last (empty) copy has landed before the workgroup's LDS is released

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

// One workgroup of D/4 threads per (batch, query head): merge the live splits.
template <int D>
__global__ __launch_bounds__(D / 4) void decode_combine_kernel(DecodeArgs a) {
  const Problem& p = a.p;
  const int bh = blockIdx.x;
  const int b = bh / p.Hq;
  const int h = bh % p.Hq;
  const int kv_end = p.len_kv ? min(p.len_kv[b], p.Lk) : p.Lk;
  const int n_live = (kv_end + a.split_keys - 1) / a.split_keys;
  const float* pl = a.part_lse + (int64_t)bh * a.n_split;
  const float* po = a.part_o + (int64_t)bh * a.n_split * D;
  float M = kNegInf;
  for (int c = 0; c < n_live; ++c) M = fmaxf(M, pl[c]);
  float L = 0.f;
  const int d0 = threadIdx.x * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (M != kNegInf) {
    for (int c = 0; c < n_live; ++c) {
      const float w = expf(pl[c] - M);
      L += w;
      const f32x4 x = *reinterpret_cast<const f32x4*>(po + (int64_t)c * D + d0);
      acc += w * x;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  bf16x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = (bf16)(acc[e] * inv);
  bf16* orow = reinterpret_cast<bf16*>(a.o) + b * p.o_sb + h * p.o_sh;
  *reinterpret_cast<bf16x4*>(orow + d0) = out;
  if (a.lse && threadIdx.x == 0) a.lse[bh] = (L > 0.f) ? M + logf(L) : kNegInf;
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  const int grid = a.p.B * a.p.Hkv * a.n_split;
  if (grid > 0) {
    hipLaunchKernelGGL((decode_split_kernel<D>), dim3(grid), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.p.B * a.p.Hq), dim3(D / 4), 0, s, a);
  return hipGetLastError();
}

}  // namespace

void decode_split_plan(int B, int Hkv, int Lk, int* split_keys, int* n_split) {
  // Enough splits that the (batch, KV head) pairs times splits fill the chip several
  // times over, without partial-result traffic becoming noticeable.
  int sk = 512;
  const int64_t pairs = (int64_t)B * Hkv;
  while (sk > kDT && pairs * ((Lk + sk - 1) / sk) < 2048) sk /= 2;
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
