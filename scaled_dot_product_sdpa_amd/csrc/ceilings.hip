// ceilings.hip — microbenchmarks of the gfx950 resources the attention kernels are built
// from: the bf16 MFMA rate, LDS read rates in the operand patterns the kernels use, and
// MFMA issued next to LDS reads or vector arithmetic.  Nothing here is on the attention
// path; the figures bound what the kernels can reach (the rooflines under the rooflines).
//
// Every kernel runs `iters` iterations of a fixed body on a grid that fills every SIMD with
// WPS waves (launch bounds WPS workgroups of 4 waves per CU), reads only the LDS it wrote,
// and folds its results into one float per thread so that no work is dead.
#include "kern_common.h"

namespace sdpa {
namespace {

__device__ __forceinline__ bf16x8 lane_bf16x8(int lane, int salt) {
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (bf16)(0.001f * (float)((lane * 7 + t * 3 + salt) % 17));
  return r;
}

__device__ __forceinline__ float fold16(const f32x16& x) {
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += x[v];
  return s;
}

// 1. MFMA: NCH independent 32x32x16 accumulation chains per wave.
template <int WPS, int NCH>
__global__ __launch_bounds__(256, WPS) void ceil_mfma(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  const bf16x8 a = lane_bf16x8(lane, 1), b = lane_bf16x8(lane, 2);
  f32x16 acc[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) acc[c] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) acc[c] = mfma32(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) s += fold16(acc[c]);
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// A 64 x 128 bf16 tile in LDS, in the swizzled layout of the attention kernels, filled by
// the workgroup with finite values.
constexpr int kTileRows = 64, kTileD = 128;
__device__ __forceinline__ void fill_tile(bf16* t) {
  for (int i = threadIdx.x; i < kTileRows * kTileD; i += blockDim.x) t[i] = (bf16)(0.001f * (float)(i % 29));
  __syncthreads();
}

// 2. LDS reads alone.  MODE 0: 16-byte row reads (the K operand of S^T = K Q^T, tile_row8);
// MODE 1: ds_read_b64_tr_b16 pairs (the V^T operand of O^T += V^T P^T, tile_tr8).  Each
// wave reads the whole tile per iteration (16 KB: 16 instructions of 1 KB, or 32 of 512 B).
template <int WPS, int MODE>
__global__ __launch_bounds__(256, WPS) void ceil_lds(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) bf16 tile[kTileRows * kTileD];
  fill_tile(tile);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int krow = perm_row(l32);
  const int blk = lane >> 4, arow = (lane & 15) >> 2;
  const int vchunk = ((lane & 3) >> 1) + 2 * (blk & 1), vhalf = 4 * (lane & 1);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int i = 0; i < iters; ++i) {
    asm volatile("" ::: "memory");  // LDS may have changed: every iteration reads it again
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bf16x8 x;
        if (MODE == 0) x = tile_row8<kTileD>(tile, kb * 32 + krow, 2 * j + hi);
        else x = tile_tr8<kTileD>(tile, kb * 32 + 16 * hi + 8 * (j / 4) + arow, vchunk + 4 * (j % 4), vhalf);
        acc ^= __builtin_bit_cast(u32x4, x);
      }
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

// 3. The attention forward's matrix skeleton: per 32-key block, S^T = K Q^T (NS = 8 MFMAs
// per 32-query group, K operands read from LDS with 16-byte reads) and O^T += V^T P^T
// (8 MFMAs per group, V^T operands read with ds_read_b64_tr_b16), P being the bf16 of S
// (no softmax).  GROUPS query groups of 32 rows share each operand read (1: 32 rows per
// wave, 2: 64 rows per wave).  The next block's K operands are read while this block's PV
// products run, the V operands while the S products run.
// AGPR: MFMA accumulators in the AccVGPR file instead of ordinary VGPRs.  That object is
// compiled without the flag that forces VGPR-form MFMAs (CEIL_AGPR_FORM), and an AGPR
// clobber makes the compiler select the AGPR form even where 256 VGPRs would do.
template <int WPS, int GROUPS, bool LDS, bool AGPR = false>
__global__ __launch_bounds__(256, WPS) void ceil_attn(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) bf16 tile[kTileRows * kTileD];
#if defined(__HIP_DEVICE_COMPILE__)
  if (AGPR) asm volatile("" ::: "a0");
#endif
  fill_tile(tile);
  constexpr int D = kTileD, NS = D / 16;
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int krow = perm_row(l32);
  const int blk = lane >> 4, arow = (lane & 15) >> 2;
  const int vchunk = ((lane & 3) >> 1) + 2 * (blk & 1), vhalf = 4 * (lane & 1);
  bf16x8 qreg[GROUPS][NS];
#pragma unroll
  for (int g = 0; g < GROUPS; ++g)
#pragma unroll
    for (int kk = 0; kk < NS; ++kk) qreg[g][kk] = lane_bf16x8(lane, 3 + g * NS + kk);
  f32x16 oacc[GROUPS][D / 32];
#pragma unroll
  for (int g = 0; g < GROUPS; ++g)
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[g][mb] = f32x16{};
  bf16x8 kc = lane_bf16x8(lane, 40), vc = lane_bf16x8(lane, 41);
  bf16x8 kop[NS], vop[NS];
  auto read_k = [&](int kb) {
#pragma unroll
    for (int kk = 0; kk < NS; ++kk) kop[kk] = LDS ? tile_row8<D>(tile, kb * 32 + krow, 2 * kk + hi) : kc;
  };
  auto read_v = [&](int kb) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int half = i / (D / 32), mb = i % (D / 32);
      vop[i] = LDS ? tile_tr8<D>(tile, kb * 32 + 16 * hi + 8 * half + arow, vchunk + 4 * mb, vhalf) : vc;
    }
  };
  read_k(0);
  for (int it = 0; it < iters; ++it) {
    asm volatile("" ::: "memory");  // LDS may have changed: every iteration reads it again
    if (!LDS) {  // register operands may have changed too: no product is loop-invariant
      pin(kc);
      pin(vc);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s[GROUPS];
#pragma unroll
      for (int g = 0; g < GROUPS; ++g) s[g] = f32x16{};
      read_v(kb);
#pragma unroll
      for (int kk = 0; kk < NS; ++kk)
#pragma unroll
        for (int g = 0; g < GROUPS; ++g) s[g] = mfma32(kop[kk], qreg[g][kk], s[g]);
      read_k(kb ^ 1);
      bf16x8 p[GROUPS][2];
#pragma unroll
      for (int g = 0; g < GROUPS; ++g)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          p[g][0][t] = (bf16)s[g][t];
          p[g][1][t] = (bf16)s[g][8 + t];
        }
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int half = i / (D / 32), mb = i % (D / 32);
#pragma unroll
        for (int g = 0; g < GROUPS; ++g) oacc[g][mb] = mfma32(vop[i], p[g][half], oacc[g][mb]);
      }
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int g = 0; g < GROUPS; ++g)
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) sum += fold16(oacc[g][mb]);
  out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

// 4. MFMA next to independent vector work: per MFMA, NF v_fma_f32 and NE v_exp_f32 on
// eight independent registers, in one scheduling slot per MFMA.
template <int WPS, int NF, int NE>
__global__ __launch_bounds__(256, WPS) void ceil_mfma_valu(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  const bf16x8 a = lane_bf16x8(lane, 5), b = lane_bf16x8(lane, 6);
  f32x16 acc0 = f32x16{}, acc1 = f32x16{};
  float r[8], e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) { r[j] = 0.01f * (lane + j); e[j] = -0.001f * j; }
  const float m = 0.999f, c = 1e-4f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u & 1) acc1 = mfma32(a, b, acc1);
      else acc0 = mfma32(a, b, acc0);
#pragma unroll
      for (int f = 0; f < NF; ++f) r[(u * NF + f) % 8] = fmaf(r[(u * NF + f) % 8], m, c);
#pragma unroll
      for (int x = 0; x < NE; ++x) e[(u * NE + x) % 8] = fast_exp2(e[(u * NE + x) % 8]) - 1.f;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = fold16(acc0) + fold16(acc1);
#pragma unroll
  for (int j = 0; j < 8; ++j) s += r[j] + e[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// 4b. The same vector work unevenly spread: per 16 MFMAs (two accumulation chains),
// slots 0..7 carry NF0 v_fma_f32 and NE0 v_exp_f32 each and slots 8..15 NF1 and NE1, as a
// two-region pipeline phase does (one region of MFMAs with little vector work, one with the
// exponentials).
template <int WPS, int NF0, int NE0, int NF1, int NE1>
__global__ __launch_bounds__(256, WPS) void ceil_mfma_valu2(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  const bf16x8 a = lane_bf16x8(lane, 5), b = lane_bf16x8(lane, 6);
  f32x16 acc0 = f32x16{}, acc1 = f32x16{};
  float r[8], e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) { r[j] = 0.01f * (lane + j); e[j] = -0.001f * j; }
  const float m = 0.999f, c = 1e-4f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (u & 1) acc1 = mfma32(a, b, acc1);
      else acc0 = mfma32(a, b, acc0);
      const int nf = u < 8 ? NF0 : NF1, ne = u < 8 ? NE0 : NE1;
#pragma unroll
      for (int f = 0; f < (u < 8 ? NF0 : NF1); ++f) r[(u * nf + f) % 8] = fmaf(r[(u * nf + f) % 8], m, c);
#pragma unroll
      for (int x = 0; x < (u < 8 ? NE0 : NE1); ++x) e[(u * ne + x) % 8] = fast_exp2(e[(u * ne + x) % 8]) - 1.f;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = fold16(acc0) + fold16(acc1);
#pragma unroll
  for (int j = 0; j < 8; ++j) s += r[j] + e[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// 5. Clock: four MFMA chains per wave as in probe 1; thread 0 of workgroup 0 records the
// shader-clock cycles (s_memtime) and the constant-rate wall ticks (s_memrealtime,
// 100 MHz) across its loop, as out[0] and out[1].
template <int WPS>
__global__ __launch_bounds__(256, WPS) void ceil_clock(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  const bf16x8 a = lane_bf16x8(lane, 1), b = lane_bf16x8(lane, 2);
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x16{};
  const uint64_t c0 = clock64(), w0 = wall_clock64();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = mfma32(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) s += fold16(acc[c]);
  const uint64_t c1 = clock64(), w1 = wall_clock64();
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    out[0] = (float)(c1 - c0);
    out[1] = (float)(w1 - w0);
  }
}

// 6. fp32 accumulation into global memory, as a key-stationary backward would add its dQ
// partials: thread t of the grid updates element (i * threads + t) & mask in iteration i
// (mask + 1 = buffer length, a power of two), so each wave instruction covers 256
// contiguous bytes and the grid sweeps the whole buffer every (mask + 1) / threads
// iterations.  MODE 0: atomic add without return (global_atomic_add_f32); MODE 1: plain
// store of the same addresses, for comparison.
template <int MODE>
__global__ __launch_bounds__(256) void ceil_atomic(float* buf, int64_t mask, int iters) {
  const int64_t threads = (int64_t)gridDim.x * blockDim.x;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int i = 0; i < iters; ++i) {
    float* p = buf + (((int64_t)i * threads + t) & mask);
    if constexpr (MODE == 0) unsafeAtomicAdd(p, 1.0f);
    else *p = (float)i;
  }
}

// 7. HBM streaming reads in the decode kernel's pattern: one-wave workgroups, two per SIMD,
// each reading its own contiguous chunk of every one of NSTR streams (K and V) in 8 KB
// tiles, 16 bytes per lane per load, two tiles of each stream in flight in registers
// (buffer loads with cache policy AUX).  Loads past a chunk return zeros without touching
// memory.  The loaded words are folded into one value per lane so no load is dead.
// PIN2: hold 20 KB of LDS per workgroup, so that at most two run per SIMD (as the decode
// kernel's registers allow); otherwise the registers set the occupancy.
template <int NSTR, int AUX, int TIF = 2, bool PIN2 = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
void ceil_stream(const char* buf, int64_t stream_bytes, int chunk, float* out) {
  constexpr int TILE = 8192, LD = TILE / 1024;
  const int lane = threadIdx.x;
  __shared__ float pad[PIN2 ? 5120 : 1];
  if (chunk < 0) {  // never true: keeps the allocation
    pad[lane] = 0.f;
    __syncthreads();
    out[lane] = pad[lane ^ 1];
  }
  const int64_t base = (int64_t)blockIdx.x * chunk;
  reg_rsrc_t r[NSTR];
#pragma unroll
  for (int st = 0; st < NSTR; ++st) r[st] = reg_rsrc(buf + st * stream_bytes + base, chunk);
  const int ntiles = chunk / TILE;
  u32x4 x[TIF][NSTR][LD];
  auto load = [&](int t, int set) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < NSTR; ++st)
#pragma unroll
      for (int i = 0; i < LD; ++i) x[set][st][i] = reg_ld16<AUX>(r[st], (uint32_t)(t * TILE + i * 1024 + lane * 16), 0);
  };
  u32x4 acc = zero16();
  auto fold = [&](int set) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < NSTR; ++st)
#pragma unroll
      for (int i = 0; i < LD; ++i) acc ^= x[set][st][i];
  };
#pragma unroll
  for (int k = 0; k < TIF; ++k) load(k, k);
  for (int t = 0; t < ntiles; t += TIF) {
#pragma unroll
    for (int k = 0; k < TIF; ++k) {
      fold(k);
      load(t + TIF + k, k);
    }
  }
  out[(int64_t)blockIdx.x * 64 + lane] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

template <typename K>
hipError_t launch(K kern, int wps, float* out, int iters, hipStream_t s) {
  hipLaunchKernelGGL(kern, dim3(256 * wps), dim3(256), 0, s, out, iters);
  return hipGetLastError();
}

}  // namespace
}  // namespace sdpa

using namespace sdpa;

#if defined(CEIL_AGPR_FORM)
// The AGPR-form forward skeletons (see ceil_attn).
extern "C" int ceil_probe_agpr(int id, int wps, float* out, int iters, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (wps != 1 && wps != 2) return -1;
  switch (id) {
    case 15: return wps == 1 ? launch(ceil_attn<1, 1, true, true>, 1, out, iters, s) : launch(ceil_attn<2, 1, true, true>, 2, out, iters, s);
    case 16: return wps == 1 ? launch(ceil_attn<1, 2, true, true>, 1, out, iters, s) : launch(ceil_attn<2, 2, true, true>, 2, out, iters, s);
    default: return -2;
  }
}
#else
// Runs the streaming probe (ceil_stream): nstr streams of stream_bytes each at buf, one
// workgroup per chunk (stream_bytes / chunk of them, chunk a multiple of 16 KB); out holds
// 64 floats per workgroup.  nt: non-temporal cache policy (as the decode kernel's loads);
// with two streams and the non-temporal policy, nt = 4 holds two workgroups per SIMD (two
// tiles per stream in flight, the decode kernel's occupancy) and nt = 3 also keeps three
// tiles per stream in flight.
extern "C" int ceil_stream_probe(int nstr, int nt, const void* buf, int64_t stream_bytes, int chunk,
                                 float* out, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (chunk <= 0 || chunk % 16384 != 0 || stream_bytes % chunk != 0) return -1;
  const int64_t grid = stream_bytes / chunk;
  const char* b = reinterpret_cast<const char*>(buf);
  if (nstr == 2 && nt == 3) hipLaunchKernelGGL((ceil_stream<2, 2, 3, true>), dim3(grid), dim3(64), 0, s, b, stream_bytes, chunk, out);
  else if (nstr == 2 && nt == 4) hipLaunchKernelGGL((ceil_stream<2, 2, 2, true>), dim3(grid), dim3(64), 0, s, b, stream_bytes, chunk, out);
  else if (nstr == 1 && nt) hipLaunchKernelGGL((ceil_stream<1, 2>), dim3(grid), dim3(64), 0, s, b, stream_bytes, chunk, out);
  else if (nstr == 1) hipLaunchKernelGGL((ceil_stream<1, 0>), dim3(grid), dim3(64), 0, s, b, stream_bytes, chunk, out);
  else if (nstr == 2 && nt) hipLaunchKernelGGL((ceil_stream<2, 2>), dim3(grid), dim3(64), 0, s, b, stream_bytes, chunk, out);
  else if (nstr == 2) hipLaunchKernelGGL((ceil_stream<2, 0>), dim3(grid), dim3(64), 0, s, b, stream_bytes, chunk, out);
  else return -2;
  return (int)hipGetLastError();
}

// Runs the accumulation probe (ceil_atomic) with `blocks` workgroups of 256 threads over
// buf[0 .. n), n a power of two.
extern "C" int ceil_atomic_probe(int mode, float* buf, int64_t n, int iters, int blocks, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (n <= 0 || (n & (n - 1)) != 0 || blocks <= 0 || iters < 0) return -1;
  if (mode == 0) hipLaunchKernelGGL(ceil_atomic<0>, dim3(blocks), dim3(256), 0, s, buf, n - 1, iters);
  else if (mode == 1) hipLaunchKernelGGL(ceil_atomic<1>, dim3(blocks), dim3(256), 0, s, buf, n - 1, iters);
  else return -2;
  return (int)hipGetLastError();
}

// Runs probe `id` (see the table in ceilings.py) on a grid of 256 * wps workgroups of 256
// threads (one per CU and wps resident per CU); out holds 65536 * wps floats.
extern "C" int ceil_probe_agpr(int id, int wps, float* out, int iters, void* stream);
extern "C" int ceil_probe(int id, int wps, float* out, int iters, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (wps != 1 && wps != 2) return -1;
  switch (id) {
    case 0: return wps == 1 ? launch(ceil_mfma<1, 1>, 1, out, iters, s) : launch(ceil_mfma<2, 1>, 2, out, iters, s);
    case 1: return wps == 1 ? launch(ceil_mfma<1, 4>, 1, out, iters, s) : launch(ceil_mfma<2, 4>, 2, out, iters, s);
    case 2: return wps == 1 ? launch(ceil_lds<1, 0>, 1, out, iters, s) : launch(ceil_lds<2, 0>, 2, out, iters, s);
    case 3: return wps == 1 ? launch(ceil_lds<1, 1>, 1, out, iters, s) : launch(ceil_lds<2, 1>, 2, out, iters, s);
    case 4: return wps == 1 ? launch(ceil_attn<1, 1, true>, 1, out, iters, s) : launch(ceil_attn<2, 1, true>, 2, out, iters, s);
    case 5: return wps == 1 ? launch(ceil_attn<1, 2, true>, 1, out, iters, s) : launch(ceil_attn<2, 2, true>, 2, out, iters, s);
    case 6: return wps == 1 ? launch(ceil_attn<1, 1, false>, 1, out, iters, s) : launch(ceil_attn<2, 1, false>, 2, out, iters, s);
    case 7: return wps == 1 ? launch(ceil_attn<1, 2, false>, 1, out, iters, s) : launch(ceil_attn<2, 2, false>, 2, out, iters, s);
    case 8: return wps == 1 ? launch(ceil_mfma_valu<1, 4, 0>, 1, out, iters, s) : launch(ceil_mfma_valu<2, 4, 0>, 2, out, iters, s);
    case 9: return wps == 1 ? launch(ceil_mfma_valu<1, 6, 0>, 1, out, iters, s) : launch(ceil_mfma_valu<2, 6, 0>, 2, out, iters, s);
    case 10: return wps == 1 ? launch(ceil_mfma_valu<1, 8, 0>, 1, out, iters, s) : launch(ceil_mfma_valu<2, 8, 0>, 2, out, iters, s);
    case 11: return wps == 1 ? launch(ceil_mfma_valu<1, 0, 2>, 1, out, iters, s) : launch(ceil_mfma_valu<2, 0, 2>, 2, out, iters, s);
    case 12: return wps == 1 ? launch(ceil_mfma_valu<1, 0, 4>, 1, out, iters, s) : launch(ceil_mfma_valu<2, 0, 4>, 2, out, iters, s);
    case 13: return wps == 1 ? launch(ceil_mfma_valu<1, 4, 1>, 1, out, iters, s) : launch(ceil_mfma_valu<2, 4, 1>, 2, out, iters, s);
    case 14: return wps == 1 ? launch(ceil_mfma_valu<1, 5, 1>, 1, out, iters, s) : launch(ceil_mfma_valu<2, 5, 1>, 2, out, iters, s);
    case 15:
    case 16: return ceil_probe_agpr(id, wps, out, iters, stream);
    case 17: return wps == 1 ? launch(ceil_clock<1>, 1, out, iters, s) : launch(ceil_clock<2>, 2, out, iters, s);
    case 18:
      return wps == 1 ? launch(ceil_mfma_valu2<1, 0, 0, 8, 2>, 1, out, iters, s)
                      : launch(ceil_mfma_valu2<2, 0, 0, 8, 2>, 2, out, iters, s);
    case 19:
      return wps == 1 ? launch(ceil_mfma_valu2<1, 1, 0, 7, 2>, 1, out, iters, s)
                      : launch(ceil_mfma_valu2<2, 1, 0, 7, 2>, 2, out, iters, s);
    default: return -2;
  }
}
#endif
