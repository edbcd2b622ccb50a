// kd_api.cpp - the C ABI declared in include/kd.h: argument checks, workspace
// sizing and dispatch to the kernel launchers. Every check runs on the host
// before any HIP call.
#include "kd.h"

#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <mutex>
#include <stdio.h>
#include <string.h>

#include "kd_internal.h"

namespace {

// kd_fwd_noalloc's scratch: the forward's partial records live in this array
// instead of a caller workspace. Each GPU the library runs on holds its own
// copy until the process ends; calls on one GPU share it. In host code the
// name is only a stand-in: its device address comes from hipGetSymbolAddress.
constexpr size_t kNoAllocScratchBytes = (size_t)144 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

// Device address of `scratch` on each device, looked up once per device (with
// that device current) on the first kd_fwd_noalloc call there.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

thread_local char g_last_error[256] = "";

kd_status fail(kd_status s, const char* what) {
  snprintf(g_last_error, sizeof(g_last_error), "%s", what);
  return s;
}

kd_status hip_fail(hipError_t e, const char* where) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, hipGetErrorString(e));
  return KD_ERR_HIP;
}

constexpr int64_t kMaxTileBytes = 0x7FFFFFF0;  // largest buffer-resource extent

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

kd_status check_common(const void* h_s, const void* W_s, const void* h_t, const void* W_t, int64_t N, int64_t V,
                       int32_t d_s, int32_t d_t, kd_dtype dtype) {
  if (!h_s || !W_s || !h_t || !W_t) return fail(KD_ERR_INVALID_ARG, "null input pointer (h_s, W_s, h_t, W_t)");
  if (N <= 0) return fail(KD_ERR_INVALID_ARG, "N must be positive");
  if (V < 2) return fail(KD_ERR_INVALID_ARG, "V must be at least 2");
  if (d_s <= 0 || d_t <= 0) return fail(KD_ERR_INVALID_ARG, "d_s and d_t must be positive");
  if (dtype != KD_F32 && dtype != KD_BF16) return fail(KD_ERR_UNSUPPORTED, "unknown dtype");
  if (d_s % 8 || d_t % 8) return fail(KD_ERR_UNSUPPORTED, "d_s and d_t must be multiples of 8");
  if (!aligned16(h_s) || !aligned16(W_s) || !aligned16(h_t) || !aligned16(W_t))
    return fail(KD_ERR_UNSUPPORTED, "inputs must be 16-byte aligned");
  // token and vocabulary tile indices are 32-bit in the kernels
  if (N > ((int64_t)1 << 38) || V > ((int64_t)1 << 38)) return fail(KD_ERR_UNSUPPORTED, "N or V too large");
  // byte offsets inside a 256-row operand tile are 32-bit
  const int64_t esz = dtype == KD_BF16 ? 2 : 4;
  if (256 * (int64_t)d_s * esz >= kMaxTileBytes || 256 * (int64_t)d_t * esz >= kMaxTileBytes)
    return fail(KD_ERR_UNSUPPORTED, "hidden size too large");
  return KD_OK;
}

// Default recompute chunk: the [N, chunk] gradient tile stays within 1 GiB,
// and the vocabulary is cut into equal chunks (multiples of 256, at least
// 2048 entries unless V is smaller) so that the last one is not a sliver.
constexpr int64_t kChunkBudget = (int64_t)1 << 30;

int32_t default_chunk(int64_t N, int64_t V, int64_t esz) {
  const int64_t vr = (V + 255) / 256 * 256;
  const int64_t cap = (kMaxTileBytes - 1) / (256 * esz) / 256 * 256;  // 256 * chunk * esz < kMaxTileBytes
  int64_t cmax = N > 0 ? kChunkBudget / (N * esz) / 256 * 256 : vr;
  cmax = std::min(std::max<int64_t>(cmax, 2048), std::min(vr, cap));
  const int64_t n = (vr + cmax - 1) / cmax;
  return (int32_t)(((vr + n - 1) / n + 255) / 256 * 256);
}

// chunk_V == 0 selects the default; anything else must be a positive multiple of 256.
kd_status resolve_chunk(int32_t& chunk_V, int64_t N, int64_t V, int64_t esz) {
  if (chunk_V == 0) chunk_V = default_chunk(N, V, esz);
  if (chunk_V < 0 || chunk_V % 256) return fail(KD_ERR_INVALID_ARG, "chunk_V must be 0 or a positive multiple of 256");
  if (256 * (int64_t)chunk_V * esz >= kMaxTileBytes) return fail(KD_ERR_UNSUPPORTED, "chunk_V too large");
  return KD_OK;
}

bool bad_beta(float beta) { return !(beta >= 0.f && beta <= 1.f); }
bool bad_tau(float tau) { return !(tau > 0.f) || !isfinite(tau); }

}  // namespace

extern "C" {

const char* kd_status_string(kd_status s) {
  switch (s) {
    case KD_OK: return "KD_OK";
    case KD_ERR_INVALID_ARG: return "KD_ERR_INVALID_ARG";
    case KD_ERR_UNSUPPORTED: return "KD_ERR_UNSUPPORTED";
    case KD_ERR_WORKSPACE: return "KD_ERR_WORKSPACE";
    case KD_ERR_HIP: return "KD_ERR_HIP";
  }
  return "KD_ERR_UNKNOWN";
}

const char* kd_last_error(void) { return g_last_error; }

int32_t kd_default_chunk(int64_t N, int64_t V, kd_dtype dtype) {
  if (N < 0 || V < 1 || (dtype != KD_F32 && dtype != KD_BF16)) return 0;
  return default_chunk(N, V, dtype == KD_BF16 ? 2 : 4);
}

kd_status kd_workspace_size(kd_op op, int64_t N, int64_t V, int32_t d_s, int32_t d_t, kd_dtype dtype, float beta,
                            int32_t chunk_V, int32_t k, size_t* bytes) {
  if (!bytes) return fail(KD_ERR_INVALID_ARG, "bytes is null");
  if (N <= 0 || V < 2 || d_s <= 0 || d_t <= 0) return fail(KD_ERR_INVALID_ARG, "bad shape");
  if (dtype != KD_F32 && dtype != KD_BF16) return fail(KD_ERR_UNSUPPORTED, "unknown dtype");
  const kd::Plan p = kd::make_plan(N, V, d_s, d_t, dtype == KD_BF16);
  if (op == KD_OP_BWD || op == KD_OP_BWD_W || op == KD_OP_TOPK_BWD || op == KD_OP_TAIL_BWD) {
    const kd_status s = resolve_chunk(chunk_V, N, V, dtype == KD_BF16 ? 2 : 4);
    if (s != KD_OK) return s;
  }
  switch (op) {
    case KD_OP_FWD:
      if (bad_beta(beta)) return fail(KD_ERR_INVALID_ARG, "beta outside [0, 1]");
      *bytes = kd::fwd_workspace_bytes(p, beta > 0.f && beta < 1.f);
      return KD_OK;
    case KD_OP_BWD:
    case KD_OP_BWD_W:
      *bytes = kd::kd_bwd_workspace_bytes(p, chunk_V, op == KD_OP_BWD_W);
      return KD_OK;
    case KD_OP_TOPK:
      if (k < 1 || k > KD_TOPK_MAX || k > V) return fail(KD_ERR_INVALID_ARG, "k outside [1, min(V, KD_TOPK_MAX)]");
      *bytes = kd::topk_workspace_bytes(p, k);
      return KD_OK;
    case KD_OP_TOPK_BWD:
      if (k < 1 || k > KD_TOPK_MAX || k > V) return fail(KD_ERR_INVALID_ARG, "k outside [1, min(V, KD_TOPK_MAX)]");
      *bytes = kd::topk_bwd_workspace_bytes(p, chunk_V, k);
      return KD_OK;
    case KD_OP_TAIL:
      if (k < 1 || k > KD_TOPK_MAX || k > V) return fail(KD_ERR_INVALID_ARG, "k outside [1, min(V, KD_TOPK_MAX)]");
      *bytes = kd::tail_workspace_bytes(p, k);
      return KD_OK;
    case KD_OP_TAIL_BWD:
      if (k < 1 || k > KD_TOPK_MAX || k > V) return fail(KD_ERR_INVALID_ARG, "k outside [1, min(V, KD_TOPK_MAX)]");
      *bytes = kd::tail_bwd_workspace_bytes(p, chunk_V, k);
      return KD_OK;
  }
  return fail(KD_ERR_INVALID_ARG, "unknown op");
}

kd_status kd_fwd(const void* h_s, const void* W_s, const void* h_t, const void* W_t, int64_t N, int64_t V,
                 int32_t d_s, int32_t d_t, float beta, float tau, kd_dtype dtype, float* loss, float* lse_s,
                 float* lse_t, float* aux, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  kd_status s = check_common(h_s, W_s, h_t, W_t, N, V, d_s, d_t, dtype);
  if (s != KD_OK) return s;
  if (bad_beta(beta)) return fail(KD_ERR_INVALID_ARG, "beta outside [0, 1]");
  if (bad_tau(tau)) return fail(KD_ERR_INVALID_ARG, "tau must be positive and finite");
  if (!loss || !lse_s || !lse_t) return fail(KD_ERR_INVALID_ARG, "null output pointer (loss, lse_s, lse_t)");
  if (!aux && beta > 0.f) return fail(KD_ERR_INVALID_ARG, "aux may be null only for beta == 0");
  if (!aligned4(loss) || !aligned4(lse_s) || !aligned4(lse_t) || (aux && !aligned4(aux)))
    return fail(KD_ERR_UNSUPPORTED, "outputs must be 4-byte aligned");
  const kd::Plan p = kd::make_plan(N, V, d_s, d_t, dtype == KD_BF16);
  const size_t need = kd::fwd_workspace_bytes(p, beta > 0.f && beta < 1.f);
  if (!workspace || ws_bytes < need) return fail(KD_ERR_WORKSPACE, "workspace smaller than kd_workspace_size(FWD)");
  if (!aligned16(workspace)) return fail(KD_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  kd::FwdIO io{h_s, W_s, h_t, W_t, beta, tau, loss, lse_s, lse_t, aux, workspace};
  hipError_t e = kd::run_fwd(p, io, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KD_OK : hip_fail(e, "kd_fwd launch");
}

kd_status kd_fwd_noalloc(const void* h_s, const void* W_s, const void* h_t, const void* W_t, int64_t N, int64_t V,
                         int32_t d_s, int32_t d_t, float beta, float tau, kd_dtype dtype, float* loss, float* lse_s,
                         float* lse_t, float* aux, void* stream) {
  g_last_error[0] = 0;
  kd_status s = check_common(h_s, W_s, h_t, W_t, N, V, d_s, d_t, dtype);
  if (s != KD_OK) return s;
  if (bad_beta(beta)) return fail(KD_ERR_INVALID_ARG, "beta outside [0, 1]");
  if (bad_tau(tau)) return fail(KD_ERR_INVALID_ARG, "tau must be positive and finite");
  if (!loss || !lse_s || !lse_t) return fail(KD_ERR_INVALID_ARG, "null output pointer (loss, lse_s, lse_t)");
  if (!aux && beta > 0.f) return fail(KD_ERR_INVALID_ARG, "aux may be null only for beta == 0");
  if (!aligned4(loss) || !aligned4(lse_s) || !aligned4(lse_t) || (aux && !aligned4(aux)))
    return fail(KD_ERR_UNSUPPORTED, "outputs must be 4-byte aligned");
  const kd::Plan p = kd::make_plan(N, V, d_s, d_t, dtype == KD_BF16);
  const size_t need = kd::fwd_workspace_bytes(p, beta > 0.f && beta < 1.f);
  if (need > kNoAllocScratchBytes) {
    snprintf(g_last_error, sizeof(g_last_error),
             "kd_fwd_noalloc: this shape needs %zu bytes of scratch, above its fixed %zu (use kd_fwd with a workspace)",
             need, kNoAllocScratchBytes);
    return KD_ERR_WORKSPACE;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "kd_fwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(KD_ERR_UNSUPPORTED, "kd_fwd_noalloc: device index above 63");
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      e = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess || !g_scratch_ptr[dev]) {
        g_scratch_ptr[dev] = nullptr;
        return hip_fail(e, "kd_fwd_noalloc: hipGetSymbolAddress(scratch)");
      }
    }
    ptr = g_scratch_ptr[dev];
  }
  // every partial record the merge reads is written by the sweep first: the
  // previous call's contents need no clearing
  kd::FwdIO io{h_s, W_s, h_t, W_t, beta, tau, loss, lse_s, lse_t, aux, ptr};
  e = kd::run_fwd(p, io, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KD_OK : hip_fail(e, "kd_fwd_noalloc launch");
}

size_t kd_fwd_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

kd_status kd_bwd(const void* h_s, const void* W_s, const void* h_t, const void* W_t, int64_t N, int64_t V,
                 int32_t d_s, int32_t d_t, float beta, float tau, kd_dtype dtype, int32_t chunk_V,
                 const float* lse_s, const float* lse_t, const float* aux, const float* grad_loss, float* dh_s,
                 float* dW_s, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  kd_status s = check_common(h_s, W_s, h_t, W_t, N, V, d_s, d_t, dtype);
  if (s != KD_OK) return s;
  if (bad_beta(beta)) return fail(KD_ERR_INVALID_ARG, "beta outside [0, 1]");
  if (bad_tau(tau)) return fail(KD_ERR_INVALID_ARG, "tau must be positive and finite");
  const int64_t esz = dtype == KD_BF16 ? 2 : 4;
  if ((s = resolve_chunk(chunk_V, N, V, esz)) != KD_OK) return s;
  if (!lse_s || !lse_t) return fail(KD_ERR_INVALID_ARG, "null pointer (lse_s, lse_t)");
  if (!dh_s && !dW_s) return fail(KD_ERR_INVALID_ARG, "dh_s and dW_s are both null");
  if (!aux && beta > 0.f) return fail(KD_ERR_INVALID_ARG, "aux may be null only for beta == 0");
  if ((dh_s && !aligned4(dh_s)) || (dW_s && !aligned4(dW_s)) || !aligned4(lse_s) || !aligned4(lse_t))
    return fail(KD_ERR_UNSUPPORTED, "misaligned float arrays");
  // the weight-gradient GEMM contracts over the (padded) tokens: 256 such rows stay below 2 GiB
  if (dW_s && 256 * ((N + 127) / 128 * 128) * esz >= kMaxTileBytes)
    return fail(KD_ERR_UNSUPPORTED, "too many tokens for dW_s");
  const kd::Plan p = kd::make_plan(N, V, d_s, d_t, dtype == KD_BF16);
  const size_t need = kd::kd_bwd_workspace_bytes(p, chunk_V, dW_s != nullptr);
  if (!workspace || ws_bytes < need)
    return fail(KD_ERR_WORKSPACE, dW_s ? "workspace smaller than kd_workspace_size(BWD_W)"
                                       : "workspace smaller than kd_workspace_size(BWD)");
  if (!aligned16(workspace)) return fail(KD_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  kd::BwdIO io{h_s, W_s, h_t, W_t, beta, tau, chunk_V, lse_s, lse_t, aux, grad_loss, dh_s, dW_s, workspace};
  hipError_t e = kd::run_bwd(p, io, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KD_OK : hip_fail(e, "kd_bwd launch");
}

kd_status kd_topk_fwd(const void* h_s, const void* W_s, const void* h_t, const void* W_t, int64_t N, int64_t V,
                      int32_t d_s, int32_t d_t, int32_t k, float tau, kd_dtype dtype, const int32_t* labels,
                      int32_t* topk_idx, float* topk_val, float* topk_val_s, float* binary_kl, float* cond_kl, float* ce,
                      float* p_mass, float* q_mass, float* lse_s, float* lse_t, float* lse_s1, void* workspace,
                      size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  kd_status s = check_common(h_s, W_s, h_t, W_t, N, V, d_s, d_t, dtype);
  if (s != KD_OK) return s;
  if (dtype != KD_BF16) return fail(KD_ERR_UNSUPPORTED, "kd_topk_fwd takes bf16 inputs only");
  if (k < 1 || k > KD_TOPK_MAX || k > V) return fail(KD_ERR_INVALID_ARG, "k outside [1, min(V, KD_TOPK_MAX)]");
  if (bad_tau(tau)) return fail(KD_ERR_INVALID_ARG, "tau must be positive and finite");
  if (V > KD_TOPK_MAX_V) return fail(KD_ERR_UNSUPPORTED, "V above KD_TOPK_MAX_V for kd_topk_fwd");
  if (!topk_idx || !binary_kl || !cond_kl || !p_mass || !q_mass || !lse_s || !lse_t)
    return fail(KD_ERR_INVALID_ARG, "null output pointer");
  if (labels && !ce) return fail(KD_ERR_INVALID_ARG, "ce must be given with labels");
  const kd::Plan p = kd::make_plan(N, V, d_s, d_t, true);
  const size_t need = kd::topk_workspace_bytes(p, k);
  if (!workspace || ws_bytes < need) return fail(KD_ERR_WORKSPACE, "workspace smaller than kd_workspace_size(TOPK)");
  if (!aligned16(workspace)) return fail(KD_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  kd::TopkIO io{h_s, W_s, h_t, W_t, k, tau, labels, topk_idx, topk_val, topk_val_s, binary_kl, cond_kl, ce, p_mass,
                q_mass, lse_s, lse_t, lse_s1, workspace};
  hipError_t e = kd::run_topk(p, io, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KD_OK : hip_fail(e, "kd_topk_fwd launch");
}

kd_status kd_topk_bwd(const void* h_s, const void* W_s, int64_t N, int64_t V, int32_t d_s, int32_t k, float tau,
                      kd_dtype dtype, const int32_t* labels, const int32_t* topk_idx, const float* topk_val,
                      const float* topk_val_s, const float* p_mass, const float* q_mass, const float* lse_s,
                      const float* lse_s1, const float* grad_binary, const float* grad_cond, const float* grad_ce,
                      int32_t chunk_V, float* dh_s, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  // the teacher's arrays are not read: the student's stand in for the shape checks
  kd_status s = check_common(h_s, W_s, h_s, W_s, N, V, d_s, d_s, dtype);
  if (s != KD_OK) return s;
  if (dtype != KD_BF16) return fail(KD_ERR_UNSUPPORTED, "kd_topk_bwd takes bf16 inputs only");
  if (k < 1 || k > KD_TOPK_MAX || k > V) return fail(KD_ERR_INVALID_ARG, "k outside [1, min(V, KD_TOPK_MAX)]");
  if (bad_tau(tau)) return fail(KD_ERR_INVALID_ARG, "tau must be positive and finite");
  if ((s = resolve_chunk(chunk_V, N, V, 2)) != KD_OK) return s;
  if (!topk_idx || !topk_val || !topk_val_s || !p_mass || !q_mass || !lse_s || !dh_s)
    return fail(KD_ERR_INVALID_ARG, "null input or output pointer");
  if (grad_ce && labels && !lse_s1) return fail(KD_ERR_INVALID_ARG, "lse_s1 is needed for the CE gradient");
  if (!aligned16(dh_s)) return fail(KD_ERR_UNSUPPORTED, "dh_s must be 16-byte aligned");
  const kd::Plan p = kd::make_plan(N, V, d_s, d_s, true);
  const size_t need = kd::topk_bwd_workspace_bytes(p, chunk_V, k);
  if (!workspace || ws_bytes < need) return fail(KD_ERR_WORKSPACE, "workspace smaller than kd_workspace_size(TOPK_BWD)");
  if (!aligned16(workspace)) return fail(KD_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  kd::TopkBwdIO io{h_s, W_s, k, tau, chunk_V, labels, topk_idx, topk_val, topk_val_s, p_mass, q_mass, lse_s,
                   grad_ce && labels ? lse_s1 : nullptr, grad_binary, grad_cond, grad_ce, dh_s, workspace};
  hipError_t e = kd::run_topk_bwd(p, io, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KD_OK : hip_fail(e, "kd_topk_bwd launch");
}

kd_status kd_tail_fwd(const void* h_s, const void* W_s, const void* h_t, const void* W_t, int64_t N, int64_t V,
                      int32_t d_s, int32_t d_t, int32_t k, int32_t support, float beta, float tau, kd_dtype dtype,
                      const int32_t* labels, int32_t* sup_idx, float* sup_t, float* sup_s, float* loss, float* p_mass,
                      float* q_mass, float* lse_s, float* lse_t, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  kd_status s = check_common(h_s, W_s, h_t, W_t, N, V, d_s, d_t, dtype);
  if (s != KD_OK) return s;
  if (dtype != KD_BF16) return fail(KD_ERR_UNSUPPORTED, "kd_tail_fwd takes bf16 inputs only");
  if (k < 1 || k > KD_TOPK_MAX || k > V) return fail(KD_ERR_INVALID_ARG, "k outside [1, min(V, KD_TOPK_MAX)]");
  if (support < 1 || support > 7 || !(support & (KD_SUPPORT_TEACHER | KD_SUPPORT_STUDENT)))
    return fail(KD_ERR_INVALID_ARG, "support must include KD_SUPPORT_TEACHER or KD_SUPPORT_STUDENT");
  if ((support & KD_SUPPORT_LABEL) && !labels) return fail(KD_ERR_INVALID_ARG, "KD_SUPPORT_LABEL needs labels");
  if (bad_beta(beta)) return fail(KD_ERR_INVALID_ARG, "beta outside [0, 1]");
  if (bad_tau(tau)) return fail(KD_ERR_INVALID_ARG, "tau must be positive and finite");
  if (V > KD_TOPK_MAX_V) return fail(KD_ERR_UNSUPPORTED, "V above KD_TOPK_MAX_V for kd_tail_fwd");
  if (!sup_idx || !sup_t || !sup_s || !loss || !lse_s || !lse_t) return fail(KD_ERR_INVALID_ARG, "null output pointer");
  const kd::Plan p = kd::make_plan(N, V, d_s, d_t, true);
  const size_t need = kd::tail_workspace_bytes(p, k);
  if (!workspace || ws_bytes < need) return fail(KD_ERR_WORKSPACE, "workspace smaller than kd_workspace_size(TAIL)");
  if (!aligned16(workspace)) return fail(KD_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  kd::TailIO io{h_s,  W_s,     h_t,   W_t,  k,      support, beta,   tau,   (support & KD_SUPPORT_LABEL) ? labels : nullptr,
                sup_idx, sup_t, sup_s, loss, p_mass, q_mass,  lse_s, lse_t, workspace};
  hipError_t e = kd::run_tail(p, io, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KD_OK : hip_fail(e, "kd_tail_fwd launch");
}

kd_status kd_tail_bwd(const void* h_s, const void* W_s, int64_t N, int64_t V, int32_t d_s, int32_t k, int32_t support,
                      float beta, float tau, kd_dtype dtype, const int32_t* sup_idx, const float* sup_t,
                      const float* sup_s, const float* lse_s, const float* lse_t, const float* grad_loss,
                      int32_t chunk_V, float* dh_s, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  // the teacher's arrays are not read: the student's stand in for the shape checks
  kd_status s = check_common(h_s, W_s, h_s, W_s, N, V, d_s, d_s, dtype);
  if (s != KD_OK) return s;
  if (dtype != KD_BF16) return fail(KD_ERR_UNSUPPORTED, "kd_tail_bwd takes bf16 inputs only");
  if (k < 1 || k > KD_TOPK_MAX || k > V) return fail(KD_ERR_INVALID_ARG, "k outside [1, min(V, KD_TOPK_MAX)]");
  if (support < 1 || support > 7 || !(support & (KD_SUPPORT_TEACHER | KD_SUPPORT_STUDENT)))
    return fail(KD_ERR_INVALID_ARG, "support must include KD_SUPPORT_TEACHER or KD_SUPPORT_STUDENT");
  if (bad_beta(beta)) return fail(KD_ERR_INVALID_ARG, "beta outside [0, 1]");
  if (bad_tau(tau)) return fail(KD_ERR_INVALID_ARG, "tau must be positive and finite");
  if ((s = resolve_chunk(chunk_V, N, V, 2)) != KD_OK) return s;
  if (!sup_idx || !sup_t || !sup_s || !lse_s || !lse_t || !dh_s)
    return fail(KD_ERR_INVALID_ARG, "null input or output pointer");
  if (!aligned16(dh_s)) return fail(KD_ERR_UNSUPPORTED, "dh_s must be 16-byte aligned");
  const kd::Plan p = kd::make_plan(N, V, d_s, d_s, true);
  const size_t need = kd::tail_bwd_workspace_bytes(p, chunk_V, k);
  if (!workspace || ws_bytes < need) return fail(KD_ERR_WORKSPACE, "workspace smaller than kd_workspace_size(TAIL_BWD)");
  if (!aligned16(workspace)) return fail(KD_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  kd::TailBwdIO io{h_s, W_s, kd::tail_support_slots(k, support), beta, tau, chunk_V, sup_idx, sup_t, sup_s, lse_s,
                   lse_t, grad_loss, dh_s, workspace};
  hipError_t e = kd::run_tail_bwd(p, io, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KD_OK : hip_fail(e, "kd_tail_bwd launch");
}

kd_status kd_gather_rows(const void* src, int64_t n_src, int64_t row_bytes, const int32_t* rows, int64_t n_rows,
                         void* dst, void* stream) {
  g_last_error[0] = 0;
  if (n_rows < 0 || n_src < 0) return fail(KD_ERR_INVALID_ARG, "negative row count");
  if (n_rows == 0) return KD_OK;
  if (!src || !rows || !dst) return fail(KD_ERR_INVALID_ARG, "null pointer (src, rows, dst)");
  if (row_bytes <= 0 || row_bytes % 4) return fail(KD_ERR_INVALID_ARG, "row_bytes must be a positive multiple of 4");
  if (!aligned4(src) || !aligned4(dst) || !aligned4(rows)) return fail(KD_ERR_UNSUPPORTED, "pointers must be 4-byte aligned");
  hipError_t e = kd::run_copy_rows(src, dst, rows, n_rows, n_src, row_bytes, false, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KD_OK : hip_fail(e, "kd_gather_rows launch");
}

kd_status kd_scatter_rows(const void* src, int64_t n_rows, int64_t row_bytes, const int32_t* rows, void* dst,
                          int64_t n_dst, void* stream) {
  g_last_error[0] = 0;
  if (n_rows < 0 || n_dst < 0) return fail(KD_ERR_INVALID_ARG, "negative row count");
  if (n_rows == 0) return KD_OK;
  if (!src || !rows || !dst) return fail(KD_ERR_INVALID_ARG, "null pointer (src, rows, dst)");
  if (row_bytes <= 0 || row_bytes % 4) return fail(KD_ERR_INVALID_ARG, "row_bytes must be a positive multiple of 4");
  if (!aligned4(src) || !aligned4(dst) || !aligned4(rows)) return fail(KD_ERR_UNSUPPORTED, "pointers must be 4-byte aligned");
  hipError_t e = kd::run_copy_rows(src, dst, rows, n_rows, n_dst, row_bytes, true, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KD_OK : hip_fail(e, "kd_scatter_rows launch");
}

}  // extern "C"
