// sdpa_api.cpp — the C ABI declared in include/sdpa.h: argument validation, workspace
// sizing and kernel selection.  Nothing here computes attention; every step of the
// operation runs in the HIP kernels behind launch.h.
//
// Validation follows the contracts the pages state: q and k share the key width and k and
// v share the key length (Lucid ScaledDotProductAttentionBackward, forward); Hq is a
// multiple of Hkv (the GQA head map of "Understanding PyTorch Scaled Dot-Product
// Attention", section 4); a bad scale or mismatched shape fails loudly ("Scaled
// dot-product attention (forward and backward)", section 4, test_rejects_bad_arguments);
// one element type for all io tensors and rejection instead of silent resolution (cuDNN
// "Attention", SDPA PyTorch Custom Ops, Contracts and limits).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>

#include "../../include/sdpa.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

sdpa_status fail(sdpa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }
bool aligned_to(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

int elem_bytes(int dtype) { return dtype == SDPA_DTYPE_BF16 ? 2 : 4; }

// Shape / dtype / scale checks that do not involve pointers.
sdpa_status check_problem(const sdpa_problem* p) {
  if (!p) return fail(SDPA_ERR_INVALID_ARGUMENT, "problem pointer is null");
  if (p->dtype != SDPA_DTYPE_F32 && p->dtype != SDPA_DTYPE_BF16)
    return fail(SDPA_ERR_INVALID_ARGUMENT, "unknown dtype %d", p->dtype);
  if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->Lq < 0 || p->Lk < 0 || p->Dqk < 1 || p->Dv < 1)
    return fail(SDPA_ERR_INVALID_ARGUMENT,
                "sizes must satisfy B, Hq, Hkv, Dqk, Dv >= 1 and Lq, Lk >= 0 (got B=%d Hq=%d "
                "Hkv=%d Lq=%d Lk=%d Dqk=%d Dv=%d)",
                p->B, p->Hq, p->Hkv, p->Lq, p->Lk, p->Dqk, p->Dv);
  if (p->Hq % p->Hkv != 0)
    return fail(SDPA_ERR_INVALID_ARGUMENT, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (p->is_causal != SDPA_CAUSAL_NONE && p->is_causal != SDPA_CAUSAL_TOP_LEFT &&
      p->is_causal != SDPA_CAUSAL_BOTTOM_RIGHT)
    return fail(SDPA_ERR_INVALID_ARGUMENT, "is_causal must be 0, 1 (top-left) or 2 (bottom-right), got %d",
                p->is_causal);
  if (p->sliding_window < 0 || (p->sliding_window > 0 && p->is_causal == SDPA_CAUSAL_NONE))
    return fail(SDPA_ERR_INVALID_ARGUMENT,
                "sliding_window must be 0, or > 0 together with a causal diagonal (got %d, is_causal %d)",
                p->sliding_window, p->is_causal);
  if (!std::isnan(p->scale) && !(std::isfinite(p->scale) && p->scale > 0.f))
    return fail(SDPA_ERR_INVALID_ARGUMENT, "scale must be NaN (default) or finite and > 0");
  if (p->Dqk != p->Dv)
    return fail(SDPA_ERR_UNSUPPORTED, "Dqk (%d) != Dv (%d) is not supported", p->Dqk, p->Dv);
  if (p->dtype == SDPA_DTYPE_BF16 && p->Dqk != 64 && p->Dqk != 128)
    return fail(SDPA_ERR_UNSUPPORTED, "bf16 head dim %d not supported (64, 128)", p->Dqk);
  if (p->dtype == SDPA_DTYPE_F32 && p->Dqk != 32 && p->Dqk != 64 && p->Dqk != 128)
    return fail(SDPA_ERR_UNSUPPORTED, "fp32 head dim %d not supported (32, 64, 128)", p->Dqk);
  // bf16 kernels move q/k/v/o rows in 16-byte vectors; the fp32 kernels use scalar loads.
  // Mask rows of any stride are accepted (vector loads are used only when aligned).
  const int64_t vec = p->dtype == SDPA_DTYPE_BF16 ? 8 : 1;
  const int64_t* strides[5] = {p->q_stride, p->k_stride, p->v_stride, p->o_stride, p->mask_stride};
  const char* names[5] = {"q", "k", "v", "o", "mask"};
  // A stride only matters along a dimension of size > 1 (the mask may broadcast b and h).
  const int32_t dims[5][3] = {{p->B, p->Hq, p->Lq}, {p->B, p->Hkv, p->Lk}, {p->B, p->Hkv, p->Lk},
                              {p->B, p->Hq, p->Lq}, {p->B, p->Hq, p->Lq}};
  for (int t = 0; t < 5; ++t)
    for (int a = 0; a < 3; ++a) {
      if (strides[t][a] < 0)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "%s stride %d is negative", names[t], a);
      if (t < 4 && dims[t][a] > 1 && strides[t][a] % vec != 0)
        return fail(SDPA_ERR_UNSUPPORTED, "%s stride %d (%lld) is not a multiple of %lld elements",
                    names[t], a, (long long)strides[t][a], (long long)vec);
    }
  // bf16 kernels copy 64-row tiles through buffer resources whose byte range is 32-bit.
  if (p->dtype == SDPA_DTYPE_BF16)
    for (int t = 0; t < 5; ++t)
      if (strides[t][2] >= ((int64_t)1 << 24))
        return fail(SDPA_ERR_UNSUPPORTED, "%s row stride (%lld) must be below 2^24 elements", names[t],
                    (long long)strides[t][2]);
  // Rows of one (b, h) must not overlap: the row stride covers the row.
  if (p->Lq > 1 && p->q_stride[2] < p->Dqk) return fail(SDPA_ERR_INVALID_ARGUMENT, "q rows overlap");
  if (p->Lk > 1 && p->k_stride[2] < p->Dqk) return fail(SDPA_ERR_INVALID_ARGUMENT, "k rows overlap");
  if (p->Lk > 1 && p->v_stride[2] < p->Dv) return fail(SDPA_ERR_INVALID_ARGUMENT, "v rows overlap");
  if (p->Lq > 1 && p->o_stride[2] < p->Dv) return fail(SDPA_ERR_INVALID_ARGUMENT, "o rows overlap");
  return SDPA_OK;
}

// One query row per head: a bottom-right diagonal leaves every key of the row visible
// (j <= 0 + len_kv - 1), so that case is the non-causal decode too.
bool use_decode(const sdpa_problem* p, bool has_mask) {
  return p->dtype == SDPA_DTYPE_BF16 && p->Lq == 1 &&
         (p->is_causal == SDPA_CAUSAL_NONE || p->is_causal == SDPA_CAUSAL_BOTTOM_RIGHT) &&
         !has_mask && p->Hq / p->Hkv <= 16;
}

sdpa::Problem make_problem(const sdpa_problem* p, const void* mask, const int32_t* lq,
                           const int32_t* lk, const int32_t* off_q = nullptr,
                           const int32_t* off_kv = nullptr) {
  sdpa::Problem k{};
  k.B = p->B; k.Hq = p->Hq; k.Hkv = p->Hkv; k.G = p->Hq / p->Hkv;
  k.Lq = p->Lq; k.Lk = p->Lk; k.D = p->Dqk;
  k.q_sb = p->q_stride[0]; k.q_sh = p->q_stride[1]; k.q_sl = p->q_stride[2];
  k.k_sb = p->k_stride[0]; k.k_sh = p->k_stride[1]; k.k_sl = p->k_stride[2];
  k.v_sb = p->v_stride[0]; k.v_sh = p->v_stride[1]; k.v_sl = p->v_stride[2];
  k.o_sb = p->o_stride[0]; k.o_sh = p->o_stride[1]; k.o_sl = p->o_stride[2];
  k.m_sb = p->mask_stride[0]; k.m_sh = p->mask_stride[1]; k.m_si = p->mask_stride[2];
  k.scale = std::isnan(p->scale) ? 1.0f / std::sqrt((float)p->Dqk) : p->scale;
  k.scale_log2 = k.scale * 1.4426950408889634f;
  k.causal = p->is_causal;
  k.window = p->sliding_window;
  k.len_q = lq;
  k.len_kv = lk;
  k.off_q = off_q;
  k.off_kv = off_kv;
  k.mask = mask;
  // 16-byte mask vectors need every (b, h, i) row start 16-byte aligned and whole 8-key
  // chunks per row; the copies to LDS address 64 rows from one base with 32-bit offsets
  k.mask_vec = mask != nullptr && p->dtype == SDPA_DTYPE_BF16 && aligned16(mask) &&
               p->Lk % 8 == 0 &&
               (p->B == 1 || k.m_sb % 8 == 0) && (p->Hq == 1 || k.m_sh % 8 == 0) &&
               (p->Lq == 1 || k.m_si % 8 == 0) && k.m_si < (int64_t(1) << 24);
  return k;
}

sdpa_status check_ptr(const void* ptr, const char* name, bool required, uintptr_t align) {
  if (!ptr) {
    if (required) return fail(SDPA_ERR_INVALID_ARGUMENT, "%s is null", name);
    return SDPA_OK;
  }
  if (!aligned_to(ptr, align))
    return fail(SDPA_ERR_UNSUPPORTED, "%s is not %d-byte aligned", name, (int)align);
  return SDPA_OK;
}

struct IoPtr {
  const void* ptr;
  const char* name;
  bool nonempty;  // the tensor has elements, so the pointer is required
};

// io tensors: 16-byte alignment for bf16 (vector loads), 4 for fp32; an empty tensor (a
// zero length) may be null.  The mask needs only its element alignment, the length arrays
// and lse 4 bytes.
sdpa_status check_ptrs(int dtype, std::initializer_list<IoPtr> req, const void* mask,
                       const void* lq, const void* lk, const void* lse, bool lse_required) {
  const uintptr_t io = dtype == SDPA_DTYPE_BF16 ? 16 : 4;
  for (auto& x : req) {
    sdpa_status s = check_ptr(x.ptr, x.name, x.nonempty, io);
    if (s != SDPA_OK) return s;
  }
  sdpa_status s = check_ptr(mask, "mask", false, dtype == SDPA_DTYPE_BF16 ? 2 : 4);
  if (s == SDPA_OK) s = check_ptr(lq, "seq_lens_q", false, 4);
  if (s == SDPA_OK) s = check_ptr(lk, "seq_lens_kv", false, 4);
  if (s == SDPA_OK) s = check_ptr(lse, "lse", lse_required, 4);
  return s;
}

sdpa_status hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  g_last_error.clear();
  return SDPA_OK;
}

// The bf16 dS block buffer of the backward (d = 128; see sdpa_backward_workspace_bytes in
// include/sdpa.h): 2 KB per 32 x 32 block of every (batch, query head), whole dK/dV query
// tiles and key workgroups; 0 where the backward does not use one or it would exceed
// kDsBufferCap.
constexpr size_t kDsBufferCap = size_t(8) << 30;
size_t ds_buffer_bytes(const sdpa_problem* p) {
  if (p->dtype != SDPA_DTYPE_BF16 || p->Dqk != 128 || p->Dv != 128) return 0;
  int nqb = 0, nkb = 0;
  sdpa::ds_blocks(p->Lq, p->Lk, &nqb, &nkb);
  const size_t bytes = (size_t)p->B * p->Hq * nqb * nkb * 2048;
  return bytes <= kDsBufferCap ? bytes : 0;
}

}  // namespace

extern "C" {

size_t sdpa_forward_workspace_bytes(const sdpa_problem* p) {
  if (check_problem(p) != SDPA_OK) return 0;
  if (!use_decode(p, false)) return 0;
  int sk = 0, ns = 0;
  sdpa::decode_split_plan(p->B, p->Hkv, p->Lk, &sk, &ns);
  const size_t rows = (size_t)p->B * p->Hq * ns;
  return round_up(rows * p->Dv * sizeof(float)) + round_up(rows * sizeof(float));
}

size_t sdpa_backward_workspace_bytes_min(const sdpa_problem* p) {
  if (check_problem(p) != SDPA_OK) return 0;
  // D = rowsum(dO o O) and LSE * log2(e), one fp32 each per query row
  return 2 * round_up((size_t)p->B * p->Hq * p->Lq * sizeof(float));
}

size_t sdpa_backward_workspace_bytes(const sdpa_problem* p) {
  if (check_problem(p) != SDPA_OK) return 0;
  return sdpa_backward_workspace_bytes_min(p) + ds_buffer_bytes(p);
}

namespace {
sdpa_status forward_impl(const sdpa_problem* p, const void* q, const void* k, const void* v,
                         const void* mask, const int32_t* lq, const int32_t* lk,
                         const int32_t* off_q, const int32_t* off_kv, void* o, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  sdpa_status st = check_problem(p);
  if (st != SDPA_OK) return st;
  const bool hq = p->Lq > 0, hk = p->Lk > 0;
  st = check_ptrs(p->dtype, {{q, "q", hq}, {k, "k", hk}, {v, "v", hk}, {o, "o", hq}}, mask, lq,
                  lk, lse, false);
  if (st != SDPA_OK) return st;
  (void)elem_bytes;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  sdpa::Problem kp = make_problem(p, mask, lq, lk, off_q, off_kv);
  if (p->Lq == 0) {
    g_last_error.clear();
    return SDPA_OK;
  }
  if (p->dtype == SDPA_DTYPE_F32) {
    sdpa::FwdArgs a{kp, q, k, v, o, lse};
    return hip_result(sdpa::launch_fwd_f32(a, s), "fp32 forward launch");
  }
  if (use_decode(p, mask != nullptr)) {
    const size_t need = sdpa_forward_workspace_bytes(p);
    if (workspace_bytes < need || (need > 0 && workspace == nullptr))
      return fail(SDPA_ERR_WORKSPACE_TOO_SMALL, "forward (decode) needs %zu workspace bytes, got %zu",
                  need, workspace_bytes);
    if (need > 0 && !aligned16(workspace))
      return fail(SDPA_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
    sdpa::DecodeArgs a{};
    a.p = kp; a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    sdpa::decode_split_plan(p->B, p->Hkv, p->Lk, &a.split_keys, &a.n_split);
    const size_t rows = (size_t)p->B * p->Hq * a.n_split;
    a.part_o = reinterpret_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                          round_up(rows * p->Dv * sizeof(float)));
    return hip_result(sdpa::launch_decode_bf16(a, s), "decode launch");
  }
  sdpa::FwdArgs a{kp, q, k, v, o, lse};
  return hip_result(sdpa::launch_fwd_bf16(a, s), "bf16 forward launch");
}

// Ragged entry points: the offsets replace the batch strides of their side, so a copy of
// the problem with those strides zeroed goes through the common checks.
sdpa_status ragged_problem(const sdpa_problem* p, const int32_t* off_q, const int32_t* off_kv,
                           sdpa_problem* out) {
  if (!p) return fail(SDPA_ERR_INVALID_ARGUMENT, "problem pointer is null");
  if (!off_q && !off_kv)
    return fail(SDPA_ERR_INVALID_ARGUMENT, "ragged call with neither query nor key offsets");
  sdpa_status st = check_ptr(off_q, "offsets_q", false, 4);
  if (st == SDPA_OK) st = check_ptr(off_kv, "offsets_kv", false, 4);
  if (st != SDPA_OK) return st;
  *out = *p;
  if (off_q) out->q_stride[0] = out->o_stride[0] = 0;
  if (off_kv) out->k_stride[0] = out->v_stride[0] = 0;
  return SDPA_OK;
}
}  // namespace

sdpa_status sdpa_forward(const sdpa_problem* p, const void* q, const void* k, const void* v,
                         const void* mask, const int32_t* lq, const int32_t* lk, void* o,
                         float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(p, q, k, v, mask, lq, lk, nullptr, nullptr, o, lse, workspace,
                      workspace_bytes, stream);
}

// ---- The forward without a workspace argument, for callers that cannot allocate device
// memory.  The only forward path with a workspace is the split-KV decode (its partial
// results); here they live in `scratch`, a file-scope device array of kScratchBytes that
// each GPU holds for the life of the process.  Its address on a device is looked up once
// per device (with that device current) and kept; host code never passes the array's name
// itself, which on the host is only a stand-in for the device symbol.
namespace {
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

sdpa_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SDPA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch table covers", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(SDPA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SDPA_OK;
}
}  // namespace

sdpa_status sdpa_forward_noalloc(const sdpa_problem* p, const void* q, const void* k, const void* v,
                                 const void* mask, const int32_t* lq, const int32_t* lk, void* o,
                                 float* lse, void* stream) {
  sdpa_status st = check_problem(p);
  if (st != SDPA_OK) return st;
  const size_t need = use_decode(p, mask != nullptr) ? sdpa_forward_workspace_bytes(p) : 0;
  if (need > kScratchBytes)
    return fail(SDPA_ERR_UNSUPPORTED,
                "this problem needs %zu bytes of workspace; the built-in scratch holds %zu (use "
                "sdpa_forward with a workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_on_current_device(&ws);
    if (st != SDPA_OK) return st;
  }
  return forward_impl(p, q, k, v, mask, lq, lk, nullptr, nullptr, o, lse, ws, need, stream);
}

sdpa_status sdpa_forward_ragged(const sdpa_problem* p, const void* q, const void* k,
                                const void* v, const void* mask, const int32_t* lq,
                                const int32_t* lk, const int32_t* off_q, const int32_t* off_kv,
                                void* o, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream) {
  sdpa_problem r;
  sdpa_status st = ragged_problem(p, off_q, off_kv, &r);
  if (st != SDPA_OK) return st;
  return forward_impl(&r, q, k, v, mask, lq, lk, off_q, off_kv, o, lse, workspace,
                      workspace_bytes, stream);
}

namespace {
sdpa_status backward_stages(int stages, const sdpa_problem* p, const void* q, const void* k,
                            const void* v, const void* o, const void* dO, const float* lse,
                            const void* mask, const int32_t* lq, const int32_t* lk,
                            const int32_t* off_q, const int32_t* off_kv, void* dq, void* dk,
                            void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  sdpa_status st = check_problem(p);
  if (st != SDPA_OK) return st;
  const bool hq = p->Lq > 0, hk = p->Lk > 0;
  st = check_ptrs(p->dtype, {{q, "q", hq}, {k, "k", hk}, {v, "v", hk}, {o, "o", hq},
                             {dO, "dO", hq}, {dq, "dq", hq}, {dk, "dk", hk}, {dv, "dv", hk}},
                  mask, lq, lk, lse, hq);
  if (st != SDPA_OK) return st;
  // dq, dk, dv are written with the strides of q, k, v: a zero batch or head stride along a
  // dimension of size > 1 would have several gradients land on one element (the batch
  // stride of a ragged side is unused)
  {
    const int64_t* st[3] = {p->q_stride, p->k_stride, p->v_stride};
    const int32_t heads[3] = {p->Hq, p->Hkv, p->Hkv};
    const bool ragged[3] = {off_q != nullptr, off_kv != nullptr, off_kv != nullptr};
    const char* names[3] = {"q", "k", "v"};
    for (int t = 0; t < 3; ++t)
      if ((!ragged[t] && p->B > 1 && st[t][0] == 0) || (heads[t] > 1 && st[t][1] == 0))
        return fail(SDPA_ERR_INVALID_ARGUMENT,
                    "%s has a zero batch or head stride: its gradient would alias (pass a copy)",
                    names[t]);
  }
  const size_t need = sdpa_backward_workspace_bytes_min(p);
  if (workspace_bytes < need || (need > 0 && workspace == nullptr))
    return fail(SDPA_ERR_WORKSPACE_TOO_SMALL, "backward needs %zu workspace bytes, got %zu", need,
                workspace_bytes);
  if (need > 0 && !aligned16(workspace))
    return fail(SDPA_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  sdpa::BwdArgs a{};
  a.p = make_problem(p, mask, lq, lk, off_q, off_kv);
  a.q = q; a.k = k; a.v = v; a.o = o; a.dO = dO; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.dsum = reinterpret_cast<float*>(workspace);
  a.lse2 = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + need / 2);
  // room for the dS block buffer after the row values: dQ is formed from the stored dS
  const size_t dsb = ds_buffer_bytes(p);
  if (dsb > 0 && workspace_bytes - need >= dsb) {
    a.ds = reinterpret_cast<char*>(workspace) + need;
    sdpa::ds_blocks(p->Lq, p->Lk, &a.ds_nqb, &a.ds_nkb);
  }
  if (p->dtype == SDPA_DTYPE_F32)
    return hip_result(sdpa::launch_bwd_f32(a, stages, s), "fp32 backward launch");
  return hip_result(sdpa::launch_bwd_bf16(a, stages, s), "bf16 backward launch");
}
}  // namespace

#define SDPA_BWD_ARGS                                                                      \
  const sdpa_problem *p, const void *q, const void *k, const void *v, const void *o,       \
      const void *dO, const float *lse, const void *mask, const int32_t *lq,               \
      const int32_t *lk, void *dq, void *dk, void *dv, void *workspace,                    \
      size_t workspace_bytes, void *stream
#define SDPA_BWD_PASS \
  p, q, k, v, o, dO, lse, mask, lq, lk, nullptr, nullptr, dq, dk, dv, workspace, workspace_bytes, stream

sdpa_status sdpa_backward(SDPA_BWD_ARGS) { return backward_stages(sdpa::kBwdAll, SDPA_BWD_PASS); }
sdpa_status sdpa_backward_prep(SDPA_BWD_ARGS) { return backward_stages(sdpa::kBwdPrep, SDPA_BWD_PASS); }
sdpa_status sdpa_backward_dkdv(SDPA_BWD_ARGS) { return backward_stages(sdpa::kBwdDkdv, SDPA_BWD_PASS); }
sdpa_status sdpa_backward_dq(SDPA_BWD_ARGS) { return backward_stages(sdpa::kBwdDq, SDPA_BWD_PASS); }
sdpa_status sdpa_backward_main(SDPA_BWD_ARGS) {
  return backward_stages(sdpa::kBwdDkdv | sdpa::kBwdDq, SDPA_BWD_PASS);
}

sdpa_status sdpa_backward_ragged(const sdpa_problem* p, const void* q, const void* k,
                                 const void* v, const void* o, const void* dO, const float* lse,
                                 const void* mask, const int32_t* lq, const int32_t* lk,
                                 const int32_t* off_q, const int32_t* off_kv, void* dq, void* dk,
                                 void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  sdpa_problem r;
  sdpa_status st = ragged_problem(p, off_q, off_kv, &r);
  if (st != SDPA_OK) return st;
  return backward_stages(sdpa::kBwdAll, &r, q, k, v, o, dO, lse, mask, lq, lk, off_q, off_kv, dq,
                         dk, dv, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {
sdpa_status check_paged(const sdpa_paged_decode* p) {
  if (!p) return fail(SDPA_ERR_INVALID_ARGUMENT, "problem pointer is null");
  if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->num_pages < 1 || p->max_pages < 1 ||
      p->page_size < 1)
    return fail(SDPA_ERR_INVALID_ARGUMENT,
                "sizes must satisfy B, Hq, Hkv, page_size, num_pages, max_pages >= 1 (got B=%d "
                "Hq=%d Hkv=%d page_size=%d num_pages=%d max_pages=%d)",
                p->B, p->Hq, p->Hkv, p->page_size, p->num_pages, p->max_pages);
  if (p->Hq % p->Hkv != 0)
    return fail(SDPA_ERR_INVALID_ARGUMENT, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (!std::isnan(p->scale) && !(std::isfinite(p->scale) && p->scale > 0.f))
    return fail(SDPA_ERR_INVALID_ARGUMENT, "scale must be NaN (default) or finite and > 0");
  if (p->sliding_window < 0)
    return fail(SDPA_ERR_INVALID_ARGUMENT, "sliding_window must be >= 0 (got %d)", p->sliding_window);
  if (p->D != 64 && p->D != 128) return fail(SDPA_ERR_UNSUPPORTED, "head dim %d not supported (64, 128)", p->D);
  if (p->Hq / p->Hkv > 16)
    return fail(SDPA_ERR_UNSUPPORTED, "at most 16 query heads per KV head (got %d)", p->Hq / p->Hkv);
  if (p->page_size % 32 != 0)
    return fail(SDPA_ERR_UNSUPPORTED, "page_size (%d) must be a multiple of 32", p->page_size);
  if ((int64_t)p->max_pages * p->page_size > (1 << 30))
    return fail(SDPA_ERR_UNSUPPORTED, "max_pages * page_size must not exceed 2^30 keys");
  const int64_t* st[4] = {p->q_stride, p->o_stride, p->k_stride, p->v_stride};
  const int nd[4] = {2, 2, 3, 3};
  const char* names[4] = {"q", "o", "k_pages", "v_pages"};
  for (int t = 0; t < 4; ++t)
    for (int a = 0; a < nd[t]; ++a) {
      if (st[t][a] < 0) return fail(SDPA_ERR_INVALID_ARGUMENT, "%s stride %d is negative", names[t], a);
      if (st[t][a] % 8 != 0)
        return fail(SDPA_ERR_UNSUPPORTED, "%s stride %d (%lld) is not a multiple of 8 elements",
                    names[t], a, (long long)st[t][a]);
    }
  if (p->k_stride[2] >= ((int64_t)1 << 24) || p->v_stride[2] >= ((int64_t)1 << 24))
    return fail(SDPA_ERR_UNSUPPORTED, "page row strides must be below 2^24 elements");
  if (p->page_size > 1 && (p->k_stride[2] < p->D || p->v_stride[2] < p->D))
    return fail(SDPA_ERR_INVALID_ARGUMENT, "page rows overlap");
  return SDPA_OK;
}
}  // namespace

extern "C" {

size_t sdpa_decode_paged_workspace_bytes(const sdpa_paged_decode* p) {
  if (check_paged(p) != SDPA_OK) return 0;
  int sk = 0, ns = 0;
  sdpa::decode_split_plan(p->B, p->Hkv, p->max_pages * p->page_size, &sk, &ns);
  const size_t rows = (size_t)p->B * p->Hq * ns;
  return round_up(rows * p->D * sizeof(float)) + round_up(rows * sizeof(float));
}

sdpa_status sdpa_decode_paged(const sdpa_paged_decode* p, const void* q, const void* k_pages,
                              const void* v_pages, const int32_t* page_table,
                              const int32_t* seq_lens_kv, void* o, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream) {
  sdpa_status st = check_paged(p);
  if (st != SDPA_OK) return st;
  for (auto x : {std::make_pair(q, "q"), std::make_pair(k_pages, "k_pages"),
                 std::make_pair((const void*)v_pages, "v_pages"), std::make_pair((const void*)o, "o")}) {
    st = check_ptr(x.first, x.second, true, 16);
    if (st != SDPA_OK) return st;
  }
  st = check_ptr(page_table, "page_table", true, 4);
  if (st == SDPA_OK) st = check_ptr(seq_lens_kv, "seq_lens_kv", true, 4);
  if (st == SDPA_OK) st = check_ptr(lse, "lse", false, 4);
  if (st != SDPA_OK) return st;
  const size_t need = sdpa_decode_paged_workspace_bytes(p);
  if (workspace_bytes < need || workspace == nullptr)
    return fail(SDPA_ERR_WORKSPACE_TOO_SMALL, "paged decode needs %zu workspace bytes, got %zu",
                need, workspace_bytes);
  if (!aligned16(workspace)) return fail(SDPA_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");

  sdpa::DecodeArgs a{};
  sdpa::Problem& k = a.p;
  k.B = p->B; k.Hq = p->Hq; k.Hkv = p->Hkv; k.G = p->Hq / p->Hkv;
  k.Lq = 1; k.Lk = p->max_pages * p->page_size; k.D = p->D;
  k.q_sb = p->q_stride[0]; k.q_sh = p->q_stride[1]; k.q_sl = p->D;
  k.o_sb = p->o_stride[0]; k.o_sh = p->o_stride[1]; k.o_sl = p->D;
  k.k_sb = 0; k.k_sh = p->k_stride[1]; k.k_sl = p->k_stride[2];
  k.v_sb = 0; k.v_sh = p->v_stride[1]; k.v_sl = p->v_stride[2];
  k.scale = std::isnan(p->scale) ? 1.0f / std::sqrt((float)p->D) : p->scale;
  k.scale_log2 = k.scale * 1.4426950408889634f;
  // a window ends at the last key: the bottom-right diagonal of the one query row
  k.causal = p->sliding_window > 0 ? SDPA_CAUSAL_BOTTOM_RIGHT : SDPA_CAUSAL_NONE;
  k.window = p->sliding_window;
  k.len_kv = seq_lens_kv;
  a.q = q; a.k = k_pages; a.v = v_pages; a.o = o; a.lse = lse;
  a.page_table = page_table;
  a.page_size = p->page_size;
  a.max_pages = p->max_pages;
  a.num_pages = p->num_pages;
  a.kp_stride = p->k_stride[0];
  a.vp_stride = p->v_stride[0];
  sdpa::decode_split_plan(p->B, p->Hkv, k.Lk, &a.split_keys, &a.n_split);
  const size_t rows = (size_t)p->B * p->Hq * a.n_split;
  a.part_o = reinterpret_cast<float*>(workspace);
  a.part_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                        round_up(rows * p->D * sizeof(float)));
  return hip_result(sdpa::launch_decode_bf16(a, reinterpret_cast<hipStream_t>(stream)),
                    "paged decode launch");
}

const char* sdpa_status_string(sdpa_status s) {
  switch (s) {
    case SDPA_OK: return "ok";
    case SDPA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SDPA_ERR_UNSUPPORTED: return "unsupported";
    case SDPA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SDPA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* sdpa_last_error(void) { return g_last_error.c_str(); }

int sdpa_version(void) { return 200; }  // 0.2.0: sdpa_problem and sdpa_paged_decode gained sliding_window

}  // extern "C"
