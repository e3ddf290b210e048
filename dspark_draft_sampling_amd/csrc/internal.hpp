// internal.hpp — host-side plumbing shared by the library's translation units:
// workspace layout and the per-operation launchers behind the C ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>

#include <atomic>
#include <stdint.h>

#include "dspark.h"

namespace dspark {

// Per (row, slice) partial of the vocabulary-streaming row pass.
struct RowPart {
  float m;      // maximum logit of the slice (-inf if none)
  float s;      // sum of exp((l - m) / T) over the slice (sampled rows)
  int32_t arg;  // lowest index of the maximum (INT32_MAX if none)
  uint32_t flags;
};

// Per target row of a truncated policy: smallest kept logit and the kept
// weight sum (same base-2 shift as the row's partial sums).
struct RowTrunc {
  float thr;
  float s_kept;
};

// Per (request, slice) best chunk (level 1) of a three-level Gumbel-max draw.
struct Pick {
  float v1;     // best score
  int32_t i1;   // its chunk
  float v2;     // second-best score
  uint32_t pad;
};

// Per (request, chunk) partial of the Markov step's fused GEMM epilogue.
struct ChunkPart {
  float m;          // max of z over the chunk (-inf if none)
  float s;          // sum of exp(z - m) over the chunk
  float score;      // sampled rows: ln(chunk mass) + chunk Gumbel noise (-inf if none)
  uint32_t arg_nf;  // bits 0..30: lowest index of the max (0x7fffffff: none);
                    // bit 31: a NaN or +inf was seen
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Holds the start / stop events of one kernel launch while profiling is
// enabled (dspark_profile_enable); inactive otherwise.  The launch records the
// events at the kernel's own start and end (hipExtLaunchKernelGGL).
class ProfScope {
 public:
  explicit ProfScope(const char* name);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;
  bool active() const { return a_ != nullptr; }
  hipEvent_t start() const { return a_; }
  hipEvent_t stop() const { return b_; }

 private:
  const char* name_;
  hipEvent_t a_, b_;
};

// Launch `kernel` (parenthesise template kernels) and, while profiling, time it.
#define DSPARK_LAUNCH(name, kernel, grid, block, shmem, stream, ...)                         \
  do {                                                                                      \
    ::dspark::ProfScope dspark_ps_(name);                                                   \
    if (dspark_ps_.active())                                                                \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, dspark_ps_.start(),         \
                            dspark_ps_.stop(), 0, __VA_ARGS__);                             \
    else                                                                                    \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                  \
  } while (0)

// Vocabulary slicing of the verify row pass.
struct VerifyPlan {
  int vec;        // 1: 16-byte vector loads, 0: scalar loads
  int slice_len;  // elements per row slice
  int S;          // row slices
  int S2;         // chunk slices of the residual / bonus pass
  int cps;        // chunks per chunk slice
  size_t off_part, off_pick, off_cnt, off_trunc, off_cmax, bytes;
};
VerifyPlan plan_verify(int logits_dtype, int32_t B, int32_t gamma, int32_t V, bool aligned);

struct MarkovPlan {
  int C;  // chunks per row
  int G;  // workgroups (512-token slices) of the one-launch plans
  size_t off_part, off_xk, off_sync, bytes;
};
MarkovPlan plan_markov(int32_t B, int32_t gamma, int32_t V, int32_t r, int32_t d);

struct StatsPlan {
  int sliced;  // 1: (row pair, segment) item kernels; 0: one workgroup per row pair
  int P;       // segments per row pair
  size_t off_part, off_l1, off_pk, off_cnt, bytes;
};
StatsPlan plan_stats(int32_t N, int32_t gamma, int32_t V);

// Compute units of the current device (cached per device; stats.hip).
int device_cus();

// Grid of a kernel (workgroups of `threads`) whose waves each walk a run of
// items: every workgroup resident at once, at most one wave per item.  The
// resident count per compute unit is a property of the code object, cached
// in `cache` (stats.hip).
int resident_grid(const void* fn, int threads, int64_t items, std::atomic<int>& cache);

// Batch reduction of the per-position statistics (tau and the sums), shared by
// the statistics calls (stats.hip).
hipError_t launch_stats_reduce(const float* l1, const float* accept_rate, const float* ce, const float* bce,
                               const uint8_t* block_mask, int32_t N, int32_t gamma, float w_ce, float w_l1,
                               float w_conf, float* tau, float* sums, hipStream_t st);

// Statistics of the teacher-forced Markov draft (stats_markov.hip).
struct StatsMarkovPlan {
  int G;  // token slices (workgroups of the look kernels)
  size_t off_rec, off_norm, off_l1, off_dt, off_k1, off_k2, off_xf, bytes;
};
StatsMarkovPlan plan_stats_markov(int32_t N, int32_t gamma, int32_t V);
hipError_t launch_stats_markov(const void* backbone, const void* target, int dtype, const int32_t* anchor,
                               const uint16_t* w1, const uint16_t* w2, int32_t r, const int32_t* teacher,
                               const float* conf_logits, const uint8_t* block_mask, int32_t N, int32_t gamma,
                               int32_t V, float w_ce, float w_l1, float w_conf, float* l1, float* accept_rate,
                               float* ce, float* bce, float* tau, float* sums, void* ws,
                               const StatsMarkovPlan& pl, hipStream_t st);

// Gradient of the statistics' loss numerator (stats.hip).
struct StatsGradPlan {
  int sliced;  // 1: (row pair, segment) item kernels; 0: one workgroup per row pair
  int P;       // segments per row pair
  size_t off_part, off_l1, off_rows, off_cnt, bytes;
};
StatsGradPlan plan_stats_backward(int32_t N, int32_t gamma, int32_t V);
hipError_t launch_stats_backward(const void* draft, const void* target, int dtype, const int32_t* teacher,
                                 const float* conf_logits, const uint8_t* block_mask, int32_t N,
                                 int32_t gamma, int32_t V, float w_ce, float w_l1, float w_conf,
                                 const float* grad_scale, void* grad_draft, float* grad_conf, void* ws,
                                 const StatsGradPlan& plan, hipStream_t st);

hipError_t launch_verify(const void* target, int dtype, const int32_t* draft, const float* q_z,
                         const float* q_lse, const float* q_thr, const float* q_tok,
                         const int32_t* n_draft, dspark_policy pol, uint64_t seed, int32_t B,
                         int32_t gamma, int32_t V, int32_t* accept_len, int32_t* out_tokens,
                         uint8_t* flags, void* ws, const VerifyPlan& plan, hipStream_t st);

// Confidence-scheduled draft width (width.hip).
hipError_t launch_select_width(const float* confidence, const float* cost, int32_t B, int32_t gamma,
                               int32_t* n_draft, float* expected, hipStream_t st);

hipError_t launch_markov(const void* backbone, int dtype, const int32_t* anchor,
                         const uint16_t* w1, const uint16_t* w2, const uint16_t* hidden,
                         const uint16_t* embed, const float* conf_w, dspark_policy pol,
                         uint64_t seed, int32_t B, int32_t gamma, int32_t V, int32_t r, int32_t d,
                         int32_t* draft_tokens, float* q_z, float* q_lse, float* q_thr,
                         float* q_tok, float* confidence, uint8_t* flags, void* ws,
                         const MarkovPlan& plan, int plan_mode, hipStream_t st);

// Launch plan of the Markov sampler (DSPARK_MARKOV_AUTO / _PER_STEP).
int markov_plan_mode();
// Destroys the one-launch chain's per-device events (markov.hip).
void release_markov_chain();

hipError_t launch_stats(const void* draft, const void* target, int dtype, const int32_t* teacher,
                        const float* conf_logits, const uint8_t* block_mask, int32_t N,
                        int32_t gamma, int32_t V, float w_ce, float w_l1, float w_conf, float* l1,
                        float* accept_rate, float* ce, float* bce, float* tau, float* sums,
                        void* ws, const StatsPlan& plan, hipStream_t st);

}  // namespace dspark
