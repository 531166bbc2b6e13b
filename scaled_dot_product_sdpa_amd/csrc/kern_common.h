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

// Token placed at M-row r of a 32-row MFMA block (see the header comment).
__device__ __forceinline__ int perm_row(int r) {
  return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of a value over lanes l and l^32 (v_permlane32_swap returns both halves).
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

// Global -> LDS without registers: lane L's 16 bytes from `src` land at lds_base + 16 * L
// (measured on gfx950).  lds_base must be the same for every lane of the wave.
__device__ __forceinline__ void global_to_lds16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 0);
}

// Wait until this wave's global loads (including global -> LDS copies) have landed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// ... until at most N of them are outstanding (loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

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

// MFMA operand from a swizzled tile: 16 bytes (8 elements) of row r at logical chunk c.
template <int D>
__device__ __forceinline__ bf16x8 tile_row8(const bf16* tile, int r, int c) {
  return *reinterpret_cast<const bf16x8*>(tile + r * D + ((c ^ swz<D>(r)) * 8));
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

// HBM -> LDS copy of one tile of ROWS rows x D bf16 (rows r0.. of `g`, clamped to the row
// below `stop`, so a clamped row repeats finite data whose pairs the caller masks) by the
// NW waves of the workgroup.  LDS chunk ci of the tile holds logical chunk
// (ci % CPR) ^ swz<D>(row) of row ci / CPR.
template <int ROWS, int D, int NW>
__device__ __forceinline__ void tile_to_lds_swz(const bf16* g, int64_t row_stride, int r0,
                                                int stop, bf16* lds_tile, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int NBLK = ROWS * CPR / 64;  // 1 KB wave-instructions per tile
  static_assert(NBLK % NW == 0, "tile must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < NBLK / NW; ++i) {
    const int blk = wave * (NBLK / NW) + i;
    const int ci = blk * 64 + lane;
    const int r = ci / CPR;
    const int c = (ci % CPR) ^ swz<D>(r);
    const int row = min(r0 + r, stop - 1);
    global_to_lds16(g + (int64_t)row * row_stride + c * 8, lds_tile + blk * 512);
  }
}

// ---- HBM -> LDS through a buffer resource (buffer_load ... lds): the per-lane byte offset
// inside a tile is fixed, so after set-up a tile copy costs no vector instructions; the
// tile's first row moves with the (scalar) resource base.

// The resource type exists only for the GPU target; the host pass of this single-source
// file parses the device functions with a placeholder.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t buf_rsrc_t;
#else
struct buf_rsrc_t { uint32_t w[4]; };
#endif

// Raw buffer of `bytes` bytes at `base` (stride 0, 32-bit dword format): loads past the
// end return zeros.
__device__ __forceinline__ buf_rsrc_t raw_rsrc(const void* base, int64_t bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
#else
  return buf_rsrc_t{};
#endif
}

// SIZE bytes per lane from src + voff into LDS at lds + byte_off + SIZE * lane (wave-uniform
// destination).  The offset is applied after the cast to the LDS address space, so that a
// constant destination stays a plain LDS address.
template <int SIZE>
__device__ __forceinline__ void buffer_to_lds(buf_rsrc_t src, void* lds, uint32_t byte_off, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(SIZE == 4 || SIZE == 16, "4 or 16 bytes per lane");
  auto* l = (__attribute__((address_space(3))) char*)lds + byte_off;
  if constexpr (SIZE == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(src, l, 16, voff, 0, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(src, l, 4, voff, 0, 0, 0);
#endif
}

// 16 bytes from src + voff into registers (zeros past the end of the buffer).
__device__ __forceinline__ u32x4 buffer_ld16(buf_rsrc_t src, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(src, voff, 0, 0));
#else
  return u32x4{0u, 0u, 0u, 0u};
#endif
}

// Raw buffer over rows r0 .. min(stop, r0 + ROWS) - 1 of a row-major bf16 matrix
// (row_stride elements, rows of D elements); reads past those rows return zeros.  The
// host keeps ROWS * row_stride * 2 bytes below 2^31.
template <int D, int ROWS>
__device__ __forceinline__ buf_rsrc_t rows_rsrc(const bf16* base, int64_t row_stride, int r0, int stop) {
  const int n = min(stop - r0, ROWS);
  const int64_t bytes = n > 0 ? (int64_t)(n - 1) * row_stride * 2 + D * 2 : 0;
  return raw_rsrc(base + (int64_t)r0 * row_stride, bytes);
}

// Per-lane byte offsets of a ROWS x D tile copy by NW waves: instruction i of wave w moves
// LDS chunks (w * NBLK/NW + i) * 64 + lane, chunk ci holding logical chunk
// (ci % CPR) ^ swz<D>(row) of row ci / CPR (the layout tile_to_lds_swz writes).
template <int ROWS, int D, int NW>
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
      const int c = (ci % CPR) ^ swz<D>(r);
      voff[i] = (uint32_t)(r * row_stride * 2 + c * 16);
    }
  }
  __device__ __forceinline__ void copy(buf_rsrc_t src, bf16* lds_tile, int wave) const {
    if constexpr (NW > 1) wave = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform LDS destination
    else wave = 0;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) buffer_to_lds<16>(src, lds_tile, (wave * PER_WAVE + i) * 1024, voff[i]);
  }
};

}  // namespace sdpa
