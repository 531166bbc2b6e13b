// launch.h — internal interface between the C-ABI host layer and the kernel sources.
// Not installed; the public interface is include/sdpa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

// Everything a kernel needs about one problem; strides are in elements.
struct Problem {
  int B, Hq, Hkv, G, Lq, Lk, D;  // G = Hq / Hkv; D = Dqk = Dv
  int64_t q_sb, q_sh, q_sl;
  int64_t k_sb, k_sh, k_sl;
  int64_t v_sb, v_sh, v_sl;
  int64_t o_sb, o_sh, o_sl;
  int64_t m_sb, m_sh, m_si;
  float scale;       // resolved scale
  float scale_log2;  // scale * log2(e)
  int causal;  // 0 none, 1 top-left, 2 bottom-right diagonal
  int window;  // 0 none; W > 0 (causal only): key j visible only if j > i + offset - W
  const int32_t* len_q;   // may be null
  const int32_t* len_kv;  // may be null
  // ragged (packed) sequences, may be null: batch b's query rows start at row off_q[b] of
  // q, o, dO and dq (off_kv[b] of k, v, dk, dv), and the batch stride is unused.  Without a
  // length array a batch's length is off[b+1] - off[b] (at most Lq, Lk).
  const int32_t* off_q;
  const int32_t* off_kv;
  const void* mask;       // may be null (additive, io dtype)
  int mask_vec;           // mask rows may be read with 16-byte vector loads
};

// Per-batch geometry shared by every kernel: valid lengths and the element offset of a
// batch's first row (a fixed batch stride, or the packed row of its first token).
__device__ __forceinline__ int seq_len_q(const Problem& p, int b) {
  if (p.len_q) return min(p.len_q[b], p.Lq);
  if (p.off_q) return min(max(p.off_q[b + 1] - p.off_q[b], 0), p.Lq);
  return p.Lq;
}
__device__ __forceinline__ int seq_len_kv(const Problem& p, int b) {
  if (p.len_kv) return min(p.len_kv[b], p.Lk);
  if (p.off_kv) return min(max(p.off_kv[b + 1] - p.off_kv[b], 0), p.Lk);
  return p.Lk;
}
// q, o, dO, dq (query side) and k, v, dk, dv (key side)
__device__ __forceinline__ int64_t q_base(const Problem& p, int b) {
  return p.off_q ? (int64_t)p.off_q[b] * p.q_sl : (int64_t)b * p.q_sb;
}
__device__ __forceinline__ int64_t o_base(const Problem& p, int b) {
  return p.off_q ? (int64_t)p.off_q[b] * p.o_sl : (int64_t)b * p.o_sb;
}
__device__ __forceinline__ int64_t k_base(const Problem& p, int b) {
  return p.off_kv ? (int64_t)p.off_kv[b] * p.k_sl : (int64_t)b * p.k_sb;
}
__device__ __forceinline__ int64_t v_base(const Problem& p, int b) {
  return p.off_kv ? (int64_t)p.off_kv[b] * p.v_sl : (int64_t)b * p.v_sb;
}

// The batch of rank k when batches are ordered by work, heaviest first (len_q * len_kv, ties
// by index), so that a grid dealt in group order starts the long sequences first and the
// short ones fill the tail; k itself without per-batch lengths or with more than 64
// batches.  Every lane of the calling wave must be active: lane j reads batch j's lengths.
__device__ __forceinline__ int batch_by_work(const Problem& p, int k) {
  if ((!p.len_q && !p.len_kv && !p.off_q && !p.off_kv) || p.B > 64) return k;
  const int lane = threadIdx.x & 63;
  const int64_t w = lane < p.B ? (int64_t)seq_len_q(p, lane) * seq_len_kv(p, lane) : -1;
  int rank = 0;
  for (int j = 0; j < p.B; ++j) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)w, j);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)w >> 32), j);
    const int64_t wj = (int64_t)(((uint64_t)hi << 32) | lo);
    rank += (wj > w || (wj == w && j < lane)) ? 1 : 0;
  }
  const uint64_t m = __builtin_amdgcn_ballot_w64(lane < p.B && rank == k);
  return m ? (int)__builtin_ctzll(m) : k;
}

// Output rows (o, dq; dk, dv) a batch writes: every row up to the padded length (zeros past
// the valid length), but only the valid rows of a ragged batch: the rows after them belong
// to the next batch or to a gap the caller owns.
__device__ __forceinline__ int q_rows_out(const Problem& p, int q_end) { return p.off_q ? q_end : p.Lq; }
__device__ __forceinline__ int kv_rows_out(const Problem& p, int kv_end) { return p.off_kv ? kv_end : p.Lk; }

struct FwdArgs {
  Problem p;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
};

struct BwdArgs {
  Problem p;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dsum;  // workspace: D = rowsum(dO o O), contiguous (B, Hq, Lq)
  float* lse2;  // workspace: LSE * log2(e) (LSE itself with a mask), +inf for empty rows,
                // contiguous (B, Hq, Lq)
  // workspace, may be null: bf16 dS blocks written by the paired dK/dV kernel and read by
  // the dQ-from-dS kernel when both passes run in one call.  Block (b, h, qb, kb) holds dS^T
  // of query rows 32 qb .. 32 qb + 31 and keys 32 kb .. 32 kb + 31 as 32 x 32 row-major
  // (one 64-byte row per key) at element ((((b * Hq + h) * ds_nqb + qb) * ds_nkb + kb) * 1024.
  void* ds;
  int ds_nqb;  // query blocks per head: 2 * ceil(Lq / 64) (whole 64-row dK/dV query tiles)
  int ds_nkb;  // key blocks per head: whole 128-key dK/dV workgroups
};

// Size of the dS block buffer (bytes) and its block counts; see BwdArgs::ds.
constexpr int kDsKeysPerGroup = 128;
inline void ds_blocks(int Lq, int Lk, int* nqb, int* nkb) {
  *nqb = 2 * ((Lq + 63) / 64);
  *nkb = (kDsKeysPerGroup / 32) * ((Lk + kDsKeysPerGroup - 1) / kDsKeysPerGroup);
}

struct DecodeArgs {
  Problem p;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;       // may be null
  float* part_o;    // workspace (B, Hq, n_split, D) fp32
  float* part_lse;  // workspace (B, Hq, n_split) fp32
  int split_keys;   // keys per split
  int n_split;
  // paged KV cache (page_table non-null): K of sequence b, key s is row s % page_size of
  // page page_table[b * max_pages + s / page_size] (page stride kp_stride, v: vp_stride;
  // head and row strides in p.k_sh / p.k_sl, p.v_sh / p.v_sl)
  const int32_t* page_table;
  int page_size;
  int max_pages;
  int num_pages;
  int64_t kp_stride;
  int64_t vp_stride;
};

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
// Backward stages (see sdpa_backward_prep / _dkdv / _dq in include/sdpa.h).
enum BwdStage { kBwdPrep = 1, kBwdDkdv = 2, kBwdDq = 4, kBwdAll = 7 };
hipError_t launch_bwd_bf16(const BwdArgs& a, int stages, hipStream_t s);
hipError_t launch_bwd_f32(const BwdArgs& a, int stages, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);

// Split-KV geometry used by the decode path (keys per split and number of splits).
void decode_split_plan(int B, int Hkv, int Lk, int* split_keys, int* n_split);

}  // namespace sdpa
