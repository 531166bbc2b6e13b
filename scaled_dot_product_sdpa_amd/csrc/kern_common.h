// kern_common.h — device-side building blocks shared by the gfx950 attention kernels.
//
// Matrix-core conventions (wave64, measured on gfx950 with a lane-layout probe):
//   v_mfma_f32_32x32x16_bf16  D(32x32) += A(32x16) * B(16x32)
//     A: lane l holds A[l%32][8*(l/32) + t], t = 0..7      (one row, 8 consecutive k)
//     B: lane l holds B[8*(l/32) + t][l%32], t = 0..7      (one column, 8 consecutive k)
//     D: lane l holds D[(v/4)*8 + (l/32)*4 + v%4][l%32], v = 0..15
//   ds_read_b64_tr_b16 within each 16-lane block: lane j supplies the address of a row of
//   four 16-bit elements R_j[0..3]; lane i receives { R_{4s + i/4}[i%4] : s = 0..3 }.
//
// Row permutation used by every kernel: when the 32 M-rows of an MFMA are keys (or
// queries) we place token  tok(r) = 16*((r>>2)&1) + 4*(r>>3) + (r&3)  at M-row r.  Then the
// accumulator of lane l holds tokens 16*(l/32) + v for v = 0..15 — sixteen consecutive
// tokens per lane, so a lane's half of the D tile feeds the next MFMA as a k-slice of 8
// consecutive tokens without any data movement.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16  D(16x16) += A(16x32) * B(32x16)  (measured on gfx950):
//   A: lane l holds A[l%16][8*(l/16) + t];  B: lane l holds B[8*(l/16) + t][l%16];
//   D: lane l holds D[4*(l/16) + v][l%16], v = 0..3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Token placed at M-row r of a 32-row MFMA block (see the header comment).
__device__ __forceinline__ int perm_row(int r) {
  return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of a value over lanes l and l^32 (v_permlane32_swap returns both halves).
// The max is written as the instruction itself: fmaxf would first quiet possible signalling
// NaNs in both swapped values (two extra instructions), and these values are scores.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float m;
  asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
  return m;
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// bf16 -> fp32 (exact).
__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }

// Eight fp32 -> eight bf16, round to nearest even.
__device__ __forceinline__ bf16x8 f32x8_to_bf16(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (bf16)x[t];
  return r;
}

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x4 zero16() { return u32x4{0u, 0u, 0u, 0u}; }

// LDS transposing read of four bf16 (see header comment for the lane mapping).
__device__ __forceinline__ i16x4 lds_read_tr4(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<bf16*>(p)));
}

__device__ __forceinline__ bf16x8 join_tr(i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Wait until at most N of this wave's vector-memory operations (loads, stores, copies to
// LDS) are outstanding; they complete in issue order.  The s_waitcnt builtin (not inline
// assembly) lets the compiler see the wait, so it knows its own earlier loads have landed
// and adds no waits of its own later; the empty assembly keeps memory accesses from moving
// above it.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  // gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt 6:4 (7 = no wait), lgkmcnt 11:8
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_vmem() { wait_vmem_le<0>(); }
// Wait until this wave's LDS reads have returned their data (lgkmcnt 0; vmcnt and expcnt
// fields at their maxima, i.e. no wait on those).
__device__ __forceinline__ void wait_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
}

// Keeps a register value where it is: the empty asm reads and rewrites it, so the arithmetic
// that produces the value cannot be moved below this point.  Without it the compiler sinks a
// block's softmax arithmetic across the branches between pipeline phases, next to the MFMAs
// that consume it, where it runs as one stretch of vector work with the matrix unit idle
// instead of in the MFMA slots it was written into.  The value is also opaque to the
// optimizer from here on (see OpOffsets).
template <typename T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// XOR swizzle of the 16-byte chunks inside an LDS tile row (tiles are stored unpadded).
// gfx950 LDS has 64 four-byte banks (measured: a conflict-free pattern reads ~245 B/clk per
// CU), i.e. sixteen 16-byte bank groups per 256 bytes.  Tiles are read two ways:
//  - 16 bytes per lane, in 16-lane phases on rows {r..r+3, r+16..r+19, r+4..r+7,
//    r+20..r+23} (the MFMA row permutation) at one logical chunk;
//  - ds_read_b64_tr_b16, in 32-lane phases on four consecutive rows r..r+3 (r % 4 == 0) at
//    four consecutive chunks {c..c+3} (c % 4 == 0).
// For both head dims the map below sends every phase's sixteen 16-byte accesses to
// sixteen distinct bank groups.  It depends on row bit 2, so the two row quads of one
// transposing read pair (r and r + 4) each need their own swizzle.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 4) & 1);
  else return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 4) & 1);
}

// Swizzles for the 16x16x32 MFMA operands, chosen by SW:
//  1: 16-byte reads by 16-lane phases on sixteen consecutive rows at one chunk;
//  2: ds_read_b64_tr_b16 by 32-lane phases on eight consecutive rows (r % 8 == 0) at the
//     chunk pair {2m, 2m + 1}.
// Each maps a phase onto sixteen distinct 16-byte bank groups (a D = 64 row spans half
// the banks, so its row parity is part of the bank group).
template <int D, int SW>
__device__ __forceinline__ int swz_sel(int r) {
  if constexpr (SW == 0) return swz<D>(r);
  else if constexpr (SW == 1) return D == 128 ? (r & 15) : ((r >> 1) & 7);
  else return D == 128 ? ((r & 7) << 1) : (r & 6);
}

// MFMA operand from a swizzled tile: 16 bytes (8 elements) of row r at logical chunk c.
template <int D, int SW = 0>
__device__ __forceinline__ bf16x8 tile_row8(const bf16* tile, int r, int c) {
  return *reinterpret_cast<const bf16x8*>(tile + r * D + ((c ^ swz_sel<D, SW>(r)) * 8));
}

// Transposed MFMA operand from a swizzled tile: this lane's element column of rows
// tr..tr+7 (two ds_read_b64_tr_b16 on the quads tr..tr+3 and tr+4..tr+7).  `c` and `h`
// are the lane's logical chunk and 4-element half within it (see the lane map above).
template <int D>
__device__ __forceinline__ bf16x8 tile_tr8(const bf16* tile, int tr, int c, int h) {
  const int o0 = tr * D + ((c ^ swz<D>(tr)) * 8) + h;
  const int o1 = (tr + 4) * D + ((c ^ swz<D>(tr + 4)) * 8) + h;
  return join_tr(lds_read_tr4(tile + o0), lds_read_tr4(tile + o1));
}

// A wave's operand reads of swizzled D-wide tiles by per-lane element offsets that are
// computed once and hidden from the compiler (pin): every read then adds its buffer and
// row block as a constant in the LDS instruction's offset field.  Without this the compiler
// keeps one loop-invariant address per buffer and read (tens of registers in the kernels
// with three tile buffers) and spills them.  Call repin() once per loop step, so that no
// buffer's addresses are hoisted out of the loop.  The row offsets the reads add (multiples
// of 8 rows) leave the swizzle unchanged, as it depends only on row bits 0..2 and 4.
template <int D>
struct OpOffsets {
  // byte offsets (the reads add them to byte addresses, so no shift is needed per read)
  int a[D / 16];     // tile_row8 of row `row` at logical chunk 2 kk + hi
  int t[D / 32][2];  // tile_tr8 of rows tr0 = 16 hi + arow and tr0 + 4 at chunk tchunk + 4 mb
  // abias, tbias: bytes added to the row and to the transposed offsets, for a caller that
  // reads those operands through tile pointers moved back by as much (so that tiles far into
  // the LDS array still fall within the read's 16-bit offset field and need no add)
  __device__ __forceinline__ void init(int row, int hi, int arow, int tchunk, int thalf, int abias = 0,
                                       int tbias = 0) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) a[kk] = abias + 2 * (row * D + (((2 * kk + hi) ^ swz<D>(row)) * 8));
    const int tr0 = 16 * hi + arow;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
      const int c = tchunk + 4 * mb;
      t[mb][0] = tbias + 2 * (tr0 * D + ((c ^ swz<D>(tr0)) * 8) + thalf);
      t[mb][1] = tbias + 2 * ((tr0 + 4) * D + ((c ^ swz<D>(tr0 + 4)) * 8) + thalf);
    }
    repin();
  }
  __device__ __forceinline__ void repin() {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) pin(a[kk]);
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
      pin(t[mb][0]);
      pin(t[mb][1]);
    }
  }
  // row `row` + r0 (r0 a multiple of 32), logical chunk 2 kk + hi
  __device__ __forceinline__ bf16x8 row8(const bf16* tile, int r0, int kk) const {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile + r0 * D) + a[kk]);
  }
  // transposed operand of rows r0 + tr0 .. r0 + tr0 + 7 (r0 a multiple of 8, bit 3 or 5
  // only), chunk tchunk + 4 mb
  __device__ __forceinline__ bf16x8 tr8(const bf16* tile, int r0, int mb) const {
    const char* base = reinterpret_cast<const char*>(tile + r0 * D);
    return join_tr(lds_read_tr4(reinterpret_cast<const bf16*>(base + t[mb][0])),
                   lds_read_tr4(reinterpret_cast<const bf16*>(base + t[mb][1])));
  }
};

// One transposing read (four bf16) of row r, logical chunk c, 4-element half h of a tile.
template <int D, int SW>
__device__ __forceinline__ i16x4 tile_tr4(const bf16* tile, int r, int c, int h) {
  return lds_read_tr4(tile + r * D + ((c ^ swz_sel<D, SW>(r)) * 8) + h);
}

// ---- HBM -> LDS through a buffer resource (buffer_load ... lds): the per-lane byte offset
// inside a tile is fixed, so after set-up a tile copy costs no vector instructions; the
// tile's first row moves with the (scalar) resource base.

// Raw buffer resource (stride 0, 32-bit dword format) over `bytes` bytes at `base`, as the
// four scalar registers the buffer instructions take; loads past the end return zeros.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 raw_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}


// Cache-policy bits of a buffer load or store: non-temporal (the nt bit), for data touched once.
constexpr int kNonTemporalPolicy = 2;

// Buffer resource over `bytes` bytes at `base` for loads into registers (reads past the end
// return zeros); the compiler tracks these loads like any other and inserts the wait before
// the first use of a result.  The resource type exists only for the GPU target; the host
// pass of a single-source file parses the device code with a placeholder.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t reg_rsrc_t;
__device__ __forceinline__ reg_rsrc_t reg_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes at byte offset voff + soff (AUX: cache policy bits)
template <int AUX = 0>
__device__ __forceinline__ u32x4 reg_ld16(reg_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
}
__device__ __forceinline__ float reg_ld4f(reg_rsrc_t r, uint32_t voff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}
// 16 bytes from registers to byte offset voff + soff (a vector store; stores past the end are
// dropped; AUX: cache policy bits)
template <int AUX = 0>
__device__ __forceinline__ void reg_st16(reg_rsrc_t r, uint32_t voff, uint32_t soff, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, AUX);
}
#else
struct reg_rsrc_t { uint32_t w[4]; };
__device__ __forceinline__ reg_rsrc_t reg_rsrc(const void*, int64_t) { return reg_rsrc_t{}; }
template <int AUX = 0>
__device__ __forceinline__ u32x4 reg_ld16(reg_rsrc_t, uint32_t, uint32_t) { return u32x4{0u, 0u, 0u, 0u}; }
__device__ __forceinline__ float reg_ld4f(reg_rsrc_t, uint32_t) { return 0.f; }
template <int AUX = 0>
__device__ __forceinline__ void reg_st16(reg_rsrc_t, uint32_t, uint32_t, u32x4) {}
#endif

// SIZE bytes per lane from src + voff into LDS at lds + byte_off + SIZE * lane (wave-uniform
// destination).  Written as inline assembly on purpose: the compiler then does not treat the
// copy as an LDS store that may alias the LDS reads after it, and does not make those reads
// wait for every copy in flight; each kernel instead waits for its copies (s_waitcnt vmcnt)
// before the barrier that publishes a tile.  The copy takes its LDS address from M0, and an
// SALU write of M0 needs one wait state before an LDS-DMA buffer load reads it (the CDNA
// ISA's table of manually inserted wait states), hence the s_nop; without it the load can
// see the previous copy's M0 and land in the wrong place.  M0 is a reserved register that
// cannot be named as clobbered; nothing else in these kernels uses it.
// NT: the non-temporal cache policy, for data read once (it is then the first to leave L2).
template <int SIZE, bool NT = false>
__device__ __forceinline__ void buffer_to_lds(i32x4 src, void* lds, uint32_t byte_off, uint32_t voff) {
  static_assert(SIZE == 4 || SIZE == 16, "4 or 16 bytes per lane");
  static_assert(SIZE == 16 || !NT, "non-temporal copies of 16 bytes only");
  const uint32_t addr = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lds + byte_off));
  if constexpr (SIZE == 16 && NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds" ::"s"(addr),
                 "v"(voff), "s"(src) : "memory");
  else if constexpr (SIZE == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(addr),
                 "v"(voff), "s"(src) : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(addr),
                 "v"(voff), "s"(src) : "memory");
}

// Work item of workgroup `bid` in a grid of NG groups x M items (group gi, item r).  A
// group is one (batch, KV head); its items share the K/V (or Q/dO) rows that they stream.
// Order: item-major (heavy items first where the caller numbers them so; runs of `inner`
// items of one group adjacent), or group-major (all items of a group in a row) when the
// items of a group carry equal work.  Workgroups are handed to the chip's 8 XCDs
// round-robin (workgroup i runs on XCD i % 8) and each XCD has its own L2: when the groups
// divide evenly over the XCDs, XCD x takes only the groups gi % 8 == x, in the same order,
// so the rows a group streams are fetched into one L2 and reused there.
constexpr int kNumXcd = 8;
__device__ __forceinline__ void xcd_item(int bid, int NG, int M, int inner, bool group_major,
                                         int& gi, int& r) {
  int k = bid, ng = NG, x = 0, step = 1;
  if (NG % kNumXcd == 0) {
    k = bid / kNumXcd;
    x = bid % kNumXcd;
    ng = NG / kNumXcd;
    step = kNumXcd;
  }
  if (group_major) {
    gi = (k / M) * step + x;
    r = k % M;
  } else {
    const int outer = k / (ng * inner), rem = k % (ng * inner);
    gi = (rem / inner) * step + x;
    r = outer * inner + rem % inner;
  }
}

// Offset of the causal diagonal of a batch: query i sees key j iff j <= i + offset.  0 for
// the top-left diagonal; len_kv - len_q for the bottom-right one, whose diagonal ends at
// the last (query, key) pair of the batch's actual lengths.
__device__ __forceinline__ int causal_offset(int causal, int q_end, int kv_end) {
  return causal == 2 ? kv_end - q_end : 0;
}

// Zero BYTES bytes of LDS at dst (16-byte aligned) with the NT threads of the workgroup.
// The pipelined kernels run a block's trailing MFMAs one block late, so their first block
// multiplies zero weights by the previous buffer's rows; those rows must hold finite values
// (uninitialised LDS may hold NaN or Inf bit patterns, and 0 * NaN = NaN).
template <int BYTES, int NT>
__device__ __forceinline__ void lds_zero(bf16* dst, int tid) {
  static_assert(BYTES % 16 == 0, "whole 16-byte stores");
  constexpr int N16 = BYTES / 16;
#pragma unroll
  for (int i = 0; i < (N16 + NT - 1) / NT; ++i)
    if (N16 % NT == 0 || i * NT + tid < N16) reinterpret_cast<u32x4*>(dst)[i * NT + tid] = zero16();
}

// Raw buffer over rows r0 .. min(stop, r0 + ROWS) - 1 of a row-major bf16 matrix
// (row_stride elements, rows of D elements); reads past those rows return zeros.  The
// host keeps ROWS * row_stride * 2 bytes below 2^31.
template <int D, int ROWS>
__device__ __forceinline__ i32x4 rows_rsrc(const bf16* base, int64_t row_stride, int r0, int stop) {
  const int n = min(stop - r0, ROWS);
  const int64_t bytes = n > 0 ? (int64_t)(n - 1) * row_stride * 2 + D * 2 : 0;
  return raw_rsrc(base + (int64_t)r0 * row_stride, bytes);
}

// Per-lane byte offsets of a ROWS x D tile copy by NW waves: instruction i of wave w moves
// LDS chunks (w * NBLK/NW + i) * 64 + lane, chunk ci holding logical chunk
// (ci % CPR) ^ swz_sel<D, SW>(row) of row ci / CPR (the layout tile_row8 reads).
template <int ROWS, int D, int NW, int SW = 0>
struct TileCopy {
  static constexpr int CPR = D / 8;
  static constexpr int NBLK = ROWS * CPR / 64;  // 1 KB wave-instructions per tile
  static constexpr int PER_WAVE = NBLK / NW;
  static_assert(NBLK % NW == 0, "tile must split evenly over the waves");
  uint32_t voff[PER_WAVE];
  __device__ __forceinline__ void init(int64_t row_stride, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int ci = (wave * PER_WAVE + i) * 64 + lane;
      const int r = ci / CPR;
      const int c = (ci % CPR) ^ swz_sel<D, SW>(r);
      voff[i] = (uint32_t)(r * row_stride * 2 + c * 16);
    }
  }
  __device__ __forceinline__ void copy(i32x4 src, bf16* lds_tile, int wave) const {
    if constexpr (NW > 1) wave = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform LDS destination
    else wave = 0;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) buffer_to_lds<16>(src, lds_tile, (wave * PER_WAVE + i) * 1024, voff[i]);
  }
};

}  // namespace sdpa
