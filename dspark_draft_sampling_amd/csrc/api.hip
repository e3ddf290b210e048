// api.hip — the C ABI declared in include/dspark.h: host-side argument
// validation (no device access), workspace sizing, and dispatch to the
// per-operation launchers.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dspark.h"
#include "internal.hpp"

namespace {

using dspark::MarkovPlan;
using dspark::StatsPlan;
using dspark::VerifyPlan;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

dspark_status check_common(int dtype, int32_t gamma, int32_t V) {
  if (gamma <= 0 || V <= 0) return DSPARK_EINVAL;
  if (dtype != DSPARK_BF16 && dtype != DSPARK_F32) return DSPARK_EDTYPE;
  if (gamma > DSPARK_MAX_GAMMA || V > DSPARK_MAX_VOCAB) return DSPARK_ESHAPE;
  return DSPARK_OK;
}

// top_k and top_p are either both given or both NULL (no request truncates).
bool policy_ok(const dspark_policy& p) {
  return p.mode && p.temperature && p.request_id && p.position && (!p.top_k == !p.top_p);
}

// Scratch of dspark_verify_noalloc: one copy on every GPU the library runs
// on, held until the process ends.  In host code `scratch` only names the
// symbol; its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[DSPARK_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (looked up on the device's first call).
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Host-side checks of dspark_verify (everything but the workspace).
dspark_status verify_args(const void* target_logits, int logits_dtype, const int32_t* draft_tokens,
                          const dspark_policy& policy, int32_t B, int32_t gamma, int32_t V,
                          const int32_t* accept_len, const int32_t* out_tokens, const uint8_t* flags) {
  if (B < 0) return DSPARK_EINVAL;
  dspark_status s = check_common(logits_dtype, gamma, V);
  if (s != DSPARK_OK) return s;
  if (B > DSPARK_MAX_VERIFY_BATCH) return DSPARK_ESHAPE;
  if (B == 0) return DSPARK_OK;
  if (!target_logits || !draft_tokens || !policy_ok(policy) || !accept_len || !out_tokens || !flags)
    return DSPARK_EINVAL;
  return DSPARK_OK;
}

size_t verify_bytes(int dtype, int32_t B, int32_t gamma, int32_t V) {
  const size_t a = dspark::plan_verify(dtype, B, gamma, V, true).bytes;
  const size_t b = dspark::plan_verify(dtype, B, gamma, V, false).bytes;
  return a > b ? a : b;
}

}  // namespace

extern "C" {

size_t dspark_workspace_size(int op, int32_t B, int32_t gamma, int32_t V, int32_t r, int32_t d) {
  if (B < 0 || gamma <= 0 || V <= 0) return 0;
  switch (op) {
    case DSPARK_OP_MARKOV:
      return dspark::plan_markov(B, gamma, V, r, d).bytes;
    case DSPARK_OP_VERIFY: {
      const size_t a = verify_bytes(DSPARK_BF16, B, gamma, V);
      const size_t b = verify_bytes(DSPARK_F32, B, gamma, V);
      return a > b ? a : b;
    }
    case DSPARK_OP_STATS:
      return dspark::plan_stats(B, gamma, V).bytes;
    case DSPARK_OP_STATS_BACKWARD:
      return dspark::plan_stats_backward(B, gamma, V).bytes;
    case DSPARK_OP_STATS_MARKOV:
      return dspark::plan_stats_markov(B, gamma, V).bytes;
    default:
      return 0;
  }
}

const char* dspark_status_string(int status) {
  switch (status) {
    case DSPARK_OK:
      return "ok";
    case DSPARK_EINVAL:
      return "invalid argument (NULL pointer, non-positive size or misaligned weights)";
    case DSPARK_EDTYPE:
      return "unknown logits dtype";
    case DSPARK_ESHAPE:
      return "size outside the supported range";
    case DSPARK_EWORKSPACE:
      return "workspace missing or too small";
    case DSPARK_EDEVICE:
      return "HIP launch or runtime error";
    default:
      return "unknown status";
  }
}

int dspark_version(void) { return 100; }

dspark_status dspark_markov_sample(
    const void* backbone_logits, int logits_dtype, const int32_t* anchor,
    const uint16_t* markov_w1, const uint16_t* markov_w2, const uint16_t* hidden,
    const uint16_t* embed, const float* conf_w, dspark_policy policy, uint64_t seed, int32_t B,
    int32_t gamma, int32_t V, int32_t r, int32_t d, int32_t* draft_tokens, float* q_logits,
    float* q_lse, float* q_thr, float* q_tok, float* confidence, uint8_t* flags, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (B < 0) return DSPARK_EINVAL;
  dspark_status s = check_common(logits_dtype, gamma, V);
  if (s != DSPARK_OK) return s;
  if (r <= 0 || d <= 0) return DSPARK_EINVAL;
  if (r > DSPARK_MAX_RANK || r % 16 != 0 || d > DSPARK_MAX_HIDDEN) return DSPARK_ESHAPE;
  if (B == 0) return DSPARK_OK;
  if (!backbone_logits || !anchor || !markov_w1 || !markov_w2 || !hidden || !embed || !conf_w ||
      !policy_ok(policy) || !draft_tokens || !q_logits || !q_lse || !q_thr || !q_tok ||
      !confidence || !flags)
    return DSPARK_EINVAL;
  if (!aligned16(markov_w1) || !aligned16(markov_w2)) return DSPARK_EINVAL;
  const MarkovPlan plan = dspark::plan_markov(B, gamma, V, r, d);
  if (plan.bytes > 0 && (!workspace || workspace_bytes < plan.bytes)) return DSPARK_EWORKSPACE;
  const hipError_t e = dspark::launch_markov(
      backbone_logits, logits_dtype, anchor, markov_w1, markov_w2, hidden, embed, conf_w, policy,
      seed, B, gamma, V, r, d, draft_tokens, q_logits, q_lse, q_thr, q_tok, confidence, flags,
      workspace, plan, dspark::markov_plan_mode(), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSPARK_OK : DSPARK_EDEVICE;
}

dspark_status dspark_verify(const void* target_logits, int logits_dtype,
                            const int32_t* draft_tokens, const float* q_logits, const float* q_lse,
                            const float* q_thr, const float* q_tok, const int32_t* n_draft,
                            dspark_policy policy, uint64_t seed, int32_t B, int32_t gamma,
                            int32_t V, int32_t* accept_len, int32_t* out_tokens, uint8_t* flags,
                            void* workspace, size_t workspace_bytes, void* stream) {
  const dspark_status s = verify_args(target_logits, logits_dtype, draft_tokens, policy, B, gamma, V,
                                      accept_len, out_tokens, flags);
  if (s != DSPARK_OK || B == 0) return s;
  const VerifyPlan plan =
      dspark::plan_verify(logits_dtype, B, gamma, V, aligned16(target_logits));
  if (!workspace || workspace_bytes < plan.bytes) return DSPARK_EWORKSPACE;
  const hipError_t e = dspark::launch_verify(
      target_logits, logits_dtype, draft_tokens, q_logits, q_lse, q_thr, q_tok, n_draft, policy,
      seed, B, gamma, V, accept_len, out_tokens, flags, workspace, plan,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSPARK_OK : DSPARK_EDEVICE;
}

dspark_status dspark_verify_noalloc(const void* target_logits, int logits_dtype,
                                    const int32_t* draft_tokens, const float* q_logits,
                                    const float* q_lse, const float* q_thr, const float* q_tok,
                                    const int32_t* n_draft, dspark_policy policy, uint64_t seed,
                                    int32_t B, int32_t gamma, int32_t V, int32_t* accept_len,
                                    int32_t* out_tokens, uint8_t* flags, void* stream) {
  const dspark_status s = verify_args(target_logits, logits_dtype, draft_tokens, policy, B, gamma, V,
                                      accept_len, out_tokens, flags);
  if (s != DSPARK_OK || B == 0) return s;
  const VerifyPlan plan =
      dspark::plan_verify(logits_dtype, B, gamma, V, aligned16(target_logits));
  if (plan.bytes > DSPARK_NOALLOC_SCRATCH_BYTES) return DSPARK_EWORKSPACE;
  void* ws = nullptr;
  if (scratch_ptr(&ws) != hipSuccess) return DSPARK_EDEVICE;
  const hipError_t e = dspark::launch_verify(
      target_logits, logits_dtype, draft_tokens, q_logits, q_lse, q_thr, q_tok, n_draft, policy,
      seed, B, gamma, V, accept_len, out_tokens, flags, ws, plan, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSPARK_OK : DSPARK_EDEVICE;
}

dspark_status dspark_accept_stats(const void* draft_logits, const void* target_logits,
                                  int logits_dtype, const int32_t* teacher,
                                  const float* conf_logits, const uint8_t* block_mask, int32_t N,
                                  int32_t gamma, int32_t V, float w_ce, float w_l1, float w_conf,
                                  float* l1, float* accept_rate, float* ce, float* bce, float* tau,
                                  float* sums, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (N < 0) return DSPARK_EINVAL;
  dspark_status s = check_common(logits_dtype, gamma, V);
  if (s != DSPARK_OK) return s;
  if (!sums) return DSPARK_EINVAL;
  if (N > 0 && (!draft_logits || !target_logits || !teacher || !conf_logits || !l1 ||
                !accept_rate || !ce || !bce || !tau))
    return DSPARK_EINVAL;
  if (static_cast<int64_t>(N) * gamma > 0x7fffffffLL) return DSPARK_ESHAPE;
  const StatsPlan plan = dspark::plan_stats(N, gamma, V);
  if (plan.bytes > 0 && (!workspace || workspace_bytes < plan.bytes)) return DSPARK_EWORKSPACE;
  const hipError_t e = dspark::launch_stats(
      draft_logits, target_logits, logits_dtype, teacher, conf_logits, block_mask, N, gamma, V,
      w_ce, w_l1, w_conf, l1, accept_rate, ce, bce, tau, sums, workspace, plan,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSPARK_OK : DSPARK_EDEVICE;
}

dspark_status dspark_accept_stats_markov(const void* backbone_logits, const void* target_logits,
                                         int logits_dtype, const int32_t* anchor,
                                         const uint16_t* markov_w1, const uint16_t* markov_w2,
                                         int32_t r, const int32_t* teacher, const float* conf_logits,
                                         const uint8_t* block_mask, int32_t N, int32_t gamma,
                                         int32_t V, float w_ce, float w_l1, float w_conf, float* l1,
                                         float* accept_rate, float* ce, float* bce, float* tau,
                                         float* sums, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  if (N < 0) return DSPARK_EINVAL;
  dspark_status s = check_common(logits_dtype, gamma, V);
  if (s != DSPARK_OK) return s;
  if (r <= 0) return DSPARK_EINVAL;
  if (r > DSPARK_MAX_RANK || r % 16 != 0) return DSPARK_ESHAPE;
  if (!sums) return DSPARK_EINVAL;
  if (N > 0 && (!backbone_logits || !target_logits || !anchor || !markov_w1 || !markov_w2 ||
                !teacher || !conf_logits || !l1 || !accept_rate || !ce || !bce || !tau))
    return DSPARK_EINVAL;
  if (N > 0 && (!aligned16(markov_w1) || !aligned16(markov_w2))) return DSPARK_EINVAL;
  if (static_cast<int64_t>(N) * gamma > 0x7fffffffLL) return DSPARK_ESHAPE;
  const dspark::StatsMarkovPlan plan = dspark::plan_stats_markov(N, gamma, V);
  if (plan.bytes > 0 && (!workspace || workspace_bytes < plan.bytes)) return DSPARK_EWORKSPACE;
  const hipError_t e = dspark::launch_stats_markov(
      backbone_logits, target_logits, logits_dtype, anchor, markov_w1, markov_w2, r, teacher,
      conf_logits, block_mask, N, gamma, V, w_ce, w_l1, w_conf, l1, accept_rate, ce, bce, tau, sums,
      workspace, plan, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSPARK_OK : DSPARK_EDEVICE;
}

dspark_status dspark_accept_stats_backward(const void* draft_logits, const void* target_logits,
                                           int logits_dtype, const int32_t* teacher,
                                           const float* conf_logits, const uint8_t* block_mask,
                                           int32_t N, int32_t gamma, int32_t V, float w_ce,
                                           float w_l1, float w_conf, const float* grad_scale,
                                           void* grad_draft, float* grad_conf, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  if (N < 0) return DSPARK_EINVAL;
  dspark_status s = check_common(logits_dtype, gamma, V);
  if (s != DSPARK_OK) return s;
  if (N == 0) return DSPARK_OK;
  if (!draft_logits || !target_logits || !teacher || !conf_logits || !grad_draft || !grad_conf)
    return DSPARK_EINVAL;
  if (static_cast<int64_t>(N) * gamma > 0x7fffffffLL) return DSPARK_ESHAPE;
  const dspark::StatsGradPlan plan = dspark::plan_stats_backward(N, gamma, V);
  if (plan.bytes > 0 && (!workspace || workspace_bytes < plan.bytes)) return DSPARK_EWORKSPACE;
  const hipError_t e = dspark::launch_stats_backward(
      draft_logits, target_logits, logits_dtype, teacher, conf_logits, block_mask, N, gamma, V, w_ce,
      w_l1, w_conf, grad_scale, grad_draft, grad_conf, workspace, plan, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSPARK_OK : DSPARK_EDEVICE;
}

dspark_status dspark_select_width(const float* confidence, const float* cost, int32_t B,
                                  int32_t gamma, int32_t* n_draft, float* expected, void* stream) {
  if (B < 0 || gamma <= 0) return DSPARK_EINVAL;
  if (gamma > DSPARK_MAX_GAMMA) return DSPARK_ESHAPE;
  if (!cost) return DSPARK_EINVAL;
  if (B == 0) return DSPARK_OK;
  if (!confidence || !n_draft) return DSPARK_EINVAL;
  const hipError_t e = dspark::launch_select_width(confidence, cost, B, gamma, n_draft, expected,
                                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DSPARK_OK : DSPARK_EDEVICE;
}

}  // extern "C"
