// width.hip — confidence-scheduled draft width on gfx950.
//
// Semantics ("[2/3] feat(dsv4): implement exact DSpark speculative decoding",
// scope notes and the author's reply on hardware-aware width; "DSpark
// Speculative Decoding (Draft Training) Design", "Overview"): per request,
// the number of proposals w in [0, gamma] to verify, chosen by the expected
// tokens emitted, E(w) = 1 + sum_{k<=w} prod_{j<=k} c_j, per unit of the
// measured draft-plus-verify cost D + V(w).  The full definition, with its
// tie and eligibility rules, is in include/dspark.h.
//
// One thread per request: gamma + 1 candidate widths of binary64 arithmetic
// in a fixed order, without contraction, so the choice is bit-reproducible.
// The work is a few hundred flops per request; the launch is the cost.
#include <cmath>

#include "common.hpp"
#include "internal.hpp"

namespace dspark {
namespace {

constexpr int kWidthThreads = 256;

__global__ __launch_bounds__(kWidthThreads) void select_width_kernel(
    const float* __restrict__ confidence, const float* __restrict__ cost, int32_t B, int32_t gamma,
    int32_t* __restrict__ n_draft, float* __restrict__ expected) {
#pragma clang fp contract(off)
  const int32_t b = static_cast<int32_t>(blockIdx.x) * kWidthThreads + static_cast<int32_t>(threadIdx.x);
  if (b >= B) return;
  const float* c = confidence + static_cast<size_t>(b) * gamma;
  const double D = static_cast<double>(cost[0]);
  double p = 1.0, E = 1.0;
  double best = -INFINITY, best_E = 1.0;
  int32_t best_w = 0;
  for (int32_t w = 0; w <= gamma; ++w) {
    if (w >= 1) {
      const double cj = static_cast<double>(c[w - 1]);
      p = p * (cj > 0.0 ? (cj < 1.0 ? cj : 1.0) : 0.0);  // NaN and c <= 0 count as 0
      E = E + p;
    }
    const double den = D + static_cast<double>(cost[1 + w]);
    if (!(den > 0.0) || !(den < INFINITY)) continue;  // not eligible
    const double ratio = E / den;
    if (ratio > best) {
      best = ratio;
      best_w = w;
      best_E = E;
    }
  }
  n_draft[b] = best_w;
  if (expected) expected[b] = static_cast<float>(best_E);
}

}  // namespace

hipError_t launch_select_width(const float* confidence, const float* cost, int32_t B, int32_t gamma,
                               int32_t* n_draft, float* expected, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>((B + kWidthThreads - 1) / kWidthThreads);
  DSPARK_LAUNCH("select_width", select_width_kernel, dim3(grid), dim3(kWidthThreads), 0, st, confidence,
                cost, B, gamma, n_draft, expected);
  return hipGetLastError();
}

}  // namespace dspark
