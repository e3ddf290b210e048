// stats.hip — training-side analytic acceptance statistics on gfx950.
//
// Semantics ("DSpark Speculative Decoding (Draft Training) Design", sections
// "Training objective", "Acceptance and confidence", "Loss return contract"):
// per block b and position k, with P = softmax(draft row) and T = softmax(target
// row): l1 = sum |P - T| (raw), a = clamp(1 - l1 / 2, 0, 1), ce = lse(draft) -
// draft[teacher], bce = BCE-with-logits(c, a); per block tau = 1 + sum_k
// prod_{j<=k} a_j; the position-weighted loss numerator (weights exp(-k/gamma))
// and [sum, count] report pairs are returned unnormalised.
//
// Every row pair is cut into segments of kSegIters x 64 16-byte groups per
// row (2048 bf16 or 1024 fp32 tokens), one wave each.  Look 1 forms each
// segment's normaliser part (l1norm.hpp: the maxima, and the sums under one
// power-of-two shift shared by both rows where the maxima allow it); a pair's
// parts merge exactly into its constants.  Look 2 reads the pair again and
// sums, for pairs whose L1 is at least kFarL1 by look 1's bound, the overlap
// sum min(P_v, T_v) (one exponential per element pair), and for the others
// |P_v - T_v| in the form that keeps relative accuracy when the rows nearly
// agree.
//   row path (>= 2048 pairs, or rows not 16-byte aligned): one persistent
//     workgroup of 8 waves per compute unit takes a pair at a time, its
//     waves striding over the pair's segments; the parts merge through LDS.
//   sliced path (small batches): items (pair, segment) spread over a grid
//     that is resident at once; stats_part1 writes each item's part;
//     stats_part2 gives each wave a contiguous run of items, merges a pair's
//     parts once per run, stores each item's share of L1, and at the end of
//     the run adds its item count to each pair's ticket: the wave completing
//     a pair writes the pair's outputs, the one completing the last pair tau
//     and the sums.
// stats_reduce (row path): one workgroup computes tau and the sums in fp64 in
// a fixed order, so the sums are deterministic.
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "internal.hpp"
#include "l1norm.hpp"

namespace dspark {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Row path: one workgroup of kRowThreads per compute unit, each looping over
// row pairs, so that the pairs being read at once (one per CU, 0.5 MB each at
// V = 129280 in bf16) stay within the 256 MB Infinity Cache and the later
// looks at a pair can be served from it rather than from HBM.
constexpr int kRowThreads = 512;
constexpr int kRowWaves = kRowThreads / 64;
constexpr int kItemMaxWGs = 2048;      // grid of the sliced item kernels
constexpr int kSlicedMaxPairs = 2048;  // row pairs below which the sliced path is used
constexpr int kSegIters = 4;           // 16-byte groups per lane per row per segment

template <typename T>
constexpr int stat_seg() {
  return kSegIters * 64 * (16 / static_cast<int>(sizeof(T)));
}

__device__ __forceinline__ float elem16(const uint4& u, int j, uint16_t) {
  const uint32_t w = (j >> 1) == 0 ? u.x : (j >> 1) == 1 ? u.y : (j >> 1) == 2 ? u.z : u.w;
  return (j & 1) ? bf_hi(w) : bf_lo(w);
}
__device__ __forceinline__ float elem16(const uint4& u, int j, float) {
  return __uint_as_float(j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w);
}

// Segment [lo, lo + stat_seg) of a row pair into registers, lane l holding
// the 16-byte groups it * 64 + l.  VEC (16-byte aligned rows, V a multiple of
// the group): one load per group, clamped into the row (seg_mask marks the
// groups past the row -inf before use); otherwise element loads, -inf past
// the row.
template <typename T, bool VEC>
__device__ __forceinline__ void seg_load(const T* __restrict__ dr, const T* __restrict__ tr, int32_t V, int lo,
                                         int lane, uint4* ud, uint4* ut) {
  constexpr int EPL = 16 / sizeof(T);
#pragma unroll
  for (int it = 0; it < kSegIters; ++it) {
    const int e0 = lo + (it * 64 + lane) * EPL;
    if constexpr (VEC) {
      const int e = min(e0, V - EPL);
      ud[it] = *reinterpret_cast<const uint4*>(dr + e);
      ut[it] = *reinterpret_cast<const uint4*>(tr + e);
    } else if constexpr (sizeof(T) == 2) {
      uint32_t wd[4], wt[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = e0 + 2 * q;
        const uint32_t d0 = e < V ? dr[e] : 0xFF80u, d1 = e + 1 < V ? dr[e + 1] : 0xFF80u;
        const uint32_t t0 = e < V ? tr[e] : 0xFF80u, t1 = e + 1 < V ? tr[e + 1] : 0xFF80u;
        wd[q] = d0 | (d1 << 16);
        wt[q] = t0 | (t1 << 16);
      }
      ud[it] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      ut[it] = make_uint4(wt[0], wt[1], wt[2], wt[3]);
    } else {
      uint32_t wd[4], wt[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = e0 + q;
        wd[q] = e < V ? __float_as_uint(dr[e]) : 0xFF800000u;
        wt[q] = e < V ? __float_as_uint(tr[e]) : 0xFF800000u;
      }
      ud[it] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      ut[it] = make_uint4(wt[0], wt[1], wt[2], wt[3]);
    }
  }
}

// VEC: mark the clamped groups of a partial segment -inf (the element loads
// of the other path already did).
template <typename T, bool VEC>
__device__ __forceinline__ void seg_mask(int32_t V, int lo, int lane, uint4* ud, uint4* ut) {
  constexpr int EPL = 16 / sizeof(T);
  constexpr uint32_t kNeg = sizeof(T) == 2 ? 0xFF80FF80u : 0xFF800000u;
  if constexpr (VEC) {
    if (V - lo < stat_seg<T>()) {
#pragma unroll
      for (int it = 0; it < kSegIters; ++it)
        if (lo + (it * 64 + lane) * EPL >= V) ud[it] = ut[it] = make_uint4(kNeg, kNeg, kNeg, kNeg);
    }
  }
}

// The pair's reference offset (l1norm.hpp) in two steps, so that the loads
// can travel with a segment's: pair_r5 loads t_v - d_v of token `lane` (lanes
// 0..4), pair_k5 combines them (wave-uniform).
template <typename T>
__device__ __forceinline__ float pair_r5(const T* __restrict__ dr, const T* __restrict__ tr, int32_t V, int lane) {
  return (lane < 5 && lane < V) ? load_logit(tr, lane) - load_logit(dr, lane) : pos_inf();
}
__device__ __forceinline__ float pair_k5(float r) {
  return ref_offset(lane_f(r, 0), lane_f(r, 1), lane_f(r, 2), lane_f(r, 3), lane_f(r, 4));
}

// Look 1 of a segment: its normaliser part (wave-uniform), the target values
// moved by the pair's reference offset K.
template <typename T>
__device__ __forceinline__ NormPart seg_part(const uint4* ud, const uint4* ut, float K) {
  constexpr int EPL = 16 / sizeof(T);
  float md = neg_inf(), mt = neg_inf();
#pragma unroll
  for (int it = 0; it < kSegIters; ++it)
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      md = fmaxf(md, elem16(ud[it], j, T{}));
      mt = fmaxf(mt, elem16(ut[it], j, T{}) - K);
    }
  md = wave_max(md);
  mt = wave_max(mt);
  float a2d, a2t;
  np_shifts(md, mt, a2d, a2t);
  float sd = 0.0f, x = 0.0f, ad = 0.0f;
  if (np_common(md, mt)) {
#pragma unroll
    for (int it = 0; it < kSegIters; ++it)
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        np_elem<true>(elem16(ud[it], j, T{}), elem16(ut[it], j, T{}) - K, a2d, a2t, sd, x, ad);
    ad = wave_sum(ad);
  } else {
#pragma unroll
    for (int it = 0; it < kSegIters; ++it)
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        np_elem<false>(elem16(ud[it], j, T{}), elem16(ut[it], j, T{}) - K, a2d, a2t, sd, x, ad);
  }
  return NormPart{md, mt, wave_sum(sd), wave_sum(x), ad};
}

// Look 2 of a segment: the lane's share of min(P_v, T_v) Sd (far pairs) or
// of |P_v - T_v| St (near pairs); k.far is uniform.
template <typename T>
__device__ __forceinline__ void seg_l1(const uint4* ud, const uint4* ut, const PairK& k, float& acc) {
  constexpr int EPL = 16 / sizeof(T);
  if (k.far) {
#pragma unroll
    for (int it = 0; it < kSegIters; ++it)
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        acc += l1_far(elem16(ud[it], j, T{}), elem16(ut[it], j, T{}) - k.K, k.a2d, k.a2t, k.lam2);
  } else {
#pragma unroll
    for (int it = 0; it < kSegIters; ++it)
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        acc += l1_near(elem16(ud[it], j, T{}), elem16(ut[it], j, T{}) - k.K, k.a2d, k.kappa);
  }
}

// The segments first, first + stride, ... of a pair, each handed to
// f(ud, ut, its first token) after seg_mask, the next one's loads in flight meanwhile.
template <typename T, bool VEC, class F>
__device__ __forceinline__ void seg_scan(const T* __restrict__ dr, const T* __restrict__ tr, int32_t V, int P,
                                         int first, int stride, int lane, F&& f) {
  constexpr int SEG = stat_seg<T>();
  if (first >= P) return;
  uint4 ad[kSegIters], at[kSegIters], bd[kSegIters], bt[kSegIters];
  seg_load<T, VEC>(dr, tr, V, first * SEG, lane, ad, at);
  for (int s = first;;) {
    const int n1 = s + stride;
    if (n1 < P) seg_load<T, VEC>(dr, tr, V, n1 * SEG, lane, bd, bt);
    seg_mask<T, VEC>(V, s * SEG, lane, ad, at);
    f(ad, at, s * SEG);
    if (n1 >= P) break;
    const int n2 = n1 + stride;
    if (n2 < P) seg_load<T, VEC>(dr, tr, V, n2 * SEG, lane, ad, at);
    seg_mask<T, VEC>(V, n1 * SEG, lane, bd, bt);
    f(bd, bt, n1 * SEG);
    if (n2 >= P) break;
    s = n2;
  }
}

// A pair's parts rec[0, P) merged by one wave (on every lane).
__device__ __forceinline__ NormPart pair_merge(const NormPart* __restrict__ rec, int P, int lane) {
  NormPart p = np_empty();
  for (int i = lane; i < P; i += 64) p = np_merge(p, rec[i]);
  return np_wave_merge(p);
}

__device__ __forceinline__ float bce_of(float c, float a) {
  return fmaxf(c, 0.0f) - c * a + log1pf(expf(-fabsf(c)));
}

// Row path: one persistent workgroup per compute unit, the two looks of each
// of its row pairs in turn.
template <typename T, bool VEC>
__global__ __launch_bounds__(kRowThreads) void stats_rows_kernel(
    const T* __restrict__ draft, const T* __restrict__ target, const int32_t* __restrict__ teacher,
    const float* __restrict__ conf_logits, int32_t V, int32_t npairs, float* __restrict__ l1,
    float* __restrict__ accept_rate, float* __restrict__ ce, float* __restrict__ bce) {
  constexpr int SEG = stat_seg<T>();
  __shared__ NormPart shp[kRowWaves];
  __shared__ float sha[kRowWaves];
  __shared__ PairK shk;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int P = (V + SEG - 1) / SEG;
  for (int rr = blockIdx.x; rr < npairs; rr += gridDim.x) {
    const size_t row = static_cast<size_t>(rr);
    const T* dr = draft + row * V;
    const T* tr = target + row * V;
    const float r5 = pair_r5(dr, tr, V, lane);  // issued ahead of the first segment's loads
    NormPart acc = np_empty();
    float K = 0.0f;
    bool kset = false;
    seg_scan<T, VEC>(dr, tr, V, P, wave, kRowWaves, lane, [&](const uint4* ud, const uint4* ut, int) {
      if (!kset) {  // once the first segment's loads are in flight
        K = pair_k5(r5);
        kset = true;
      }
      acc = np_merge(acc, seg_part<T>(ud, ut, K));
    });
    if (lane == 0) shp[wave] = acc;
    __syncthreads();
    if (wave == 0) {
      const NormPart m = np_wave_merge(lane < kRowWaves ? shp[lane] : np_empty());
      K = pair_k5(r5);  // wave 0 may have had no segment
      if (lane == 0) {
        shk = pair_k(m);
        shk.K = K;
      }
    }
    __syncthreads();
    const PairK k = shk;
    float a = 0.0f;
    seg_scan<T, VEC>(dr, tr, V, P, wave, kRowWaves, lane,
                     [&](const uint4* ud, const uint4* ut, int) { seg_l1<T>(ud, ut, k, a); });
    a = wave_sum(a);
    if (lane == 0) sha[wave] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
      float A = 0.0f;
#pragma unroll
      for (int w = 0; w < kRowWaves; ++w) A += sha[w];
      const float L1 = l1_final(k, A);
      const float av = fminf(1.0f, fmaxf(0.0f, 1.0f - 0.5f * L1));
      l1[row] = L1;
      accept_rate[row] = av;
      ce[row] = k.lse_d - load_logit(dr, clamp_token(teacher[row], V));
      bce[row] = bce_of(conf_logits[row], av);
    }
    __syncthreads();  // shp, sha and shk are reused by the next pair
  }
}

// ---------------------------------------------------------------------------
// Sliced path for small batches: (row pair, segment) items, one wave each, so
// that a few hundred row pairs still fill the GPU.  Both item kernels keep
// the next item's loads in flight while reducing the current one (two
// register buffers, unconditional clamped loads).

template <typename T>
__global__ __launch_bounds__(kThreads) void stats_part1_kernel(
    const T* __restrict__ draft, const T* __restrict__ target, int32_t V, int32_t P,
    int32_t items, NormPart* __restrict__ part, uint32_t* __restrict__ counters,
    int32_t ncounters) {
  constexpr int SEG = stat_seg<T>();
  const int lane = threadIdx.x & 63;
  // the ticket counters of the later kernels start at zero
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < ncounters; i += kThreads) counters[i * kTicketStride] = 0u;
  const int nwaves = gridDim.x * kWaves;
  int item = uniform_i(static_cast<int>(blockIdx.x) * kWaves + (threadIdx.x >> 6));
  if (item >= items) return;
  uint4 ad[kSegIters], at[kSegIters], bd[kSegIters], bt[kSegIters];
  float ra, rb;  // pair_r5 of the buffered items, loaded ahead of their segments
  auto load = [&](int it_, uint4* ud, uint4* ut, float& r5) {
    const int pair = it_ / P, seg = it_ - pair * P;
    const size_t off = static_cast<size_t>(pair) * V;
    r5 = pair_r5(draft + off, target + off, V, lane);
    seg_load<T, true>(draft + off, target + off, V, seg * SEG, lane, ud, ut);
  };
  auto reduce = [&](uint4* ud, uint4* ut, float r5, int it_) {
    const int seg = it_ - (it_ / P) * P;
    seg_mask<T, true>(V, seg * SEG, lane, ud, ut);
    const NormPart r = seg_part<T>(ud, ut, pair_k5(r5));
    if (lane == 0) part[it_] = r;
  };
  load(item, ad, at, ra);
  while (true) {
    const int n1 = uniform_i(item + nwaves);
    load(n1 < items ? n1 : item, bd, bt, rb);
    reduce(ad, at, ra, item);
    if (n1 >= items) break;
    const int n2 = uniform_i(n1 + nwaves);
    load(n2 < items ? n2 : n1, ad, at, ra);
    reduce(bd, bt, rb, n1);
    if (n2 >= items) break;
    item = n2;
  }
}

struct StatsOut {
  const int32_t* teacher;
  const float* conf_logits;
  const uint8_t* block_mask;
  int32_t N, gamma;
  float w_ce, w_l1, w_conf;
  float* l1;
  float* accept_rate;
  float* ce;
  float* bce;
  float* tau;
  float* sums;
  uint32_t* counters;  // per pair: items done; then pairs done (kTicketStride apart)
};

// Per-block tau and the loss / report sums by one wave, in fp64 and a fixed
// order (lane l owns blocks l, l + 64, ...; then a fixed butterfly), so the
// sums are deterministic.  The per-position values were stored by other
// waves of the same launch (device-scope loads, four positions' at a time in
// flight).
__device__ void wave_batch_reduce(const float* __restrict__ l1, const float* __restrict__ accept_rate,
                                  const float* __restrict__ ce, const float* __restrict__ bce,
                                  const uint8_t* __restrict__ block_mask, int32_t N,
                                  int32_t gamma, float w_ce, float w_l1, float w_conf,
                                  float* __restrict__ tau, float* __restrict__ sums) {
  constexpr int Q = 8;  // num, tokens, l1, accept, tau, blocks, ce, bce
  constexpr int kG = 4;  // positions per group of loads
  const int lane = threadIdx.x & 63;
  // w_k = exp(-k / gamma) (k 1-based) as powers of exp(-1 / gamma), in fp64
  const double r = exp(-1.0 / gamma);
  double acc[Q] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int b = lane; b < N; b += 64) {
    const size_t base = static_cast<size_t>(b) * gamma;
    const bool m = block_mask ? block_mask[b] != 0 : true;
    double cum = 1.0, t = 1.0, wk = 1.0;
    for (int k0 = 0; k0 < gamma; k0 += kG) {
      float a[kG], c[kG], l[kG], x[kG];
#pragma unroll
      for (int j = 0; j < kG; ++j) {
        const size_t i = base + static_cast<size_t>(min(k0 + j, gamma - 1));
        a[j] = load_coherent(accept_rate + i);
        c[j] = load_coherent(ce + i);
        l[j] = load_coherent(l1 + i);
        x[j] = load_coherent(bce + i);
      }
#pragma unroll
      for (int j = 0; j < kG; ++j) {
        if (k0 + j < gamma) {
          cum *= a[j];
          t += cum;
          wk *= r;
          if (m) {
            acc[0] += wk * (w_ce * static_cast<double>(c[j]) + w_l1 * static_cast<double>(l[j]) +
                            w_conf * static_cast<double>(x[j]));
            acc[1] += 1.0;
            acc[2] += l[j];
            acc[3] += a[j];
            acc[6] += c[j];
            acc[7] += x[j];
          }
        }
      }
    }
    tau[b] = static_cast<float>(t);
    if (m) {
      acc[4] += t;
      acc[5] += 1.0;
    }
  }
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc[q] += __shfl_xor(acc[q], o, 64);
  if (lane == 0) {
    const double n = acc[1];
    sums[0] = static_cast<float>(acc[0]);
    sums[1] = static_cast<float>(n);
    sums[2] = static_cast<float>(acc[2]);
    sums[3] = static_cast<float>(n);
    sums[4] = static_cast<float>(acc[3]);
    sums[5] = static_cast<float>(n);
    sums[6] = static_cast<float>(acc[4]);
    sums[7] = static_cast<float>(acc[5]);
    sums[8] = static_cast<float>(acc[6]);
    sums[9] = static_cast<float>(n);
    sums[10] = static_cast<float>(acc[7]);
    sums[11] = static_cast<float>(n);
  }
}

// Look 2 of the sliced path, and its outputs.  Each wave takes a contiguous
// run of items (so mostly one or two pairs), forms a pair's constants once
// per run from its part1 records, and stores each item's share of the L1
// sum; a pair's first item also stores the pair's constants.  Inside the run
// nothing waits on another wave, so the next item's loads stay in flight the
// whole time.  At the end of its run the wave adds the number of items it did
// to each pair's ticket; the wave that completes a pair writes the pair's
// outputs (stats_finish_pair), and the wave that completes the last pair
// writes tau and the sums.
template <typename T>
__device__ void stats_finish_pair(const T* __restrict__ draft, int32_t V, int32_t P, int32_t npairs, int pair,
                                  const float* __restrict__ l1part, const PairK* __restrict__ pk,
                                  const StatsOut& o) {
  const int lane = threadIdx.x & 63;
  // the pair's constants (10 words, one a lane) and the item shares were
  // stored by other waves of this launch: device-scope loads
  const uint32_t* kw = reinterpret_cast<const uint32_t*>(pk + pair);
  const uint32_t kv = lane < static_cast<int>(sizeof(PairK) / 4) ? load_coherent(kw + lane) : 0u;
  const int32_t tch = clamp_token(o.teacher[pair], V);
  const float cl = o.conf_logits[pair];
  const float xt = load_logit(draft + static_cast<size_t>(pair) * V, tch);
  float A = 0.0f;
  for (int i = lane; i < P; i += 64) A += load_coherent(l1part + static_cast<size_t>(pair) * P + i);
  A = wave_sum(A);
  PairK k;
  uint32_t* kd = reinterpret_cast<uint32_t*>(&k);
#pragma unroll
  for (int w = 0; w < static_cast<int>(sizeof(PairK) / 4); ++w) kd[w] = __builtin_amdgcn_readlane(kv, w);
  uint32_t last = 0;
  if (lane == 0) {
    const float L1 = l1_final(k, A);
    const float av = fminf(1.0f, fmaxf(0.0f, 1.0f - 0.5f * L1));
    store_coherent(o.l1 + pair, L1);
    store_coherent(o.accept_rate + pair, av);
    store_coherent(o.ce + pair, k.lse_d - xt);
    store_coherent(o.bce + pair, bce_of(cl, av));
    last = publish(o.counters + static_cast<size_t>(npairs) * kTicketStride) ==
                   static_cast<uint32_t>(npairs - 1)
               ? 1u
               : 0u;
  }
  if (uniform_i(static_cast<int>(last)))
    wave_batch_reduce(o.l1, o.accept_rate, o.ce, o.bce, o.block_mask, o.N, o.gamma, o.w_ce,
                      o.w_l1, o.w_conf, o.tau, o.sums);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void stats_part2_kernel(
    const T* __restrict__ draft, const T* __restrict__ target, int32_t V, int32_t P,
    int32_t items, const NormPart* __restrict__ part, float* __restrict__ l1part,
    PairK* __restrict__ pk, StatsOut o) {
  constexpr int SEG = stat_seg<T>();
  const int lane = threadIdx.x & 63;
  const int npairs = items / P;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWaves;
  const int64_t wv = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  const int64_t per = (items + nwaves - 1) / nwaves;
  int item = uniform_i(static_cast<int>(std::min<int64_t>(items, wv * per)));
  const int end = static_cast<int>(std::min<int64_t>(items, wv * per + per));
  if (item >= end) return;
  // two register buffers: an item's segment (and, for the first item of a
  // pair in the run, its pair_r5 and the lane's first part record) travel
  // together, one item ahead
  uint4 ad[kSegIters], at[kSegIters], bd[kSegIters], bt[kSegIters];
  float ra = 0.0f, rb = 0.0f;
  NormPart pa = np_empty(), pb = np_empty();
  const int first = item;
  auto load = [&](int it_, uint4* ud, uint4* ut, float& r5, NormPart& pr) {
    const int pair = it_ / P, seg = it_ - pair * P;
    const size_t off = static_cast<size_t>(pair) * V;
    if (seg == 0 || it_ == first) {
      r5 = pair_r5(draft + off, target + off, V, lane);
      pr = lane < P ? part[static_cast<size_t>(pair) * P + lane] : np_empty();
    }
    seg_load<T, true>(draft + off, target + off, V, seg * SEG, lane, ud, ut);
  };
  PairK k{};
  int kpair = -1;
  auto reduce = [&](uint4* ud, uint4* ut, float r5, NormPart pr, int it_) {
    const int pair = it_ / P, seg = it_ - pair * P;
    if (pair != kpair) {
      for (int i = lane + 64; i < P; i += 64) pr = np_merge(pr, part[static_cast<size_t>(pair) * P + i]);
      k = pair_k(np_wave_merge(pr));
      k.K = pair_k5(r5);
      kpair = pair;
    }
    seg_mask<T, true>(V, seg * SEG, lane, ud, ut);
    float a = 0.0f;
    seg_l1<T>(ud, ut, k, a);
    a = wave_sum(a);
    if (lane == 0) {
      store_coherent(l1part + it_, a);
      if (seg == 0) {
        const uint32_t* kd = reinterpret_cast<const uint32_t*>(&k);
        uint32_t* dst = reinterpret_cast<uint32_t*>(pk + pair);
#pragma unroll
        for (int w = 0; w < static_cast<int>(sizeof(PairK) / 4); ++w) store_coherent(dst + w, kd[w]);
      }
    }
  };
  load(item, ad, at, ra, pa);
  while (true) {
    const int n1 = item + 1;
    load(n1 < end ? n1 : item, bd, bt, rb, pb);
    reduce(ad, at, ra, pa, item);
    if (n1 >= end) break;
    const int n2 = n1 + 1;
    load(n2 < end ? n2 : n1, ad, at, ra, pa);
    reduce(bd, bt, rb, pb, n1);
    if (n2 >= end) break;
    item = n2;
  }
  // the pairs of the run: add this wave's item count to each pair's ticket
  for (int pair = first / P; pair <= (end - 1) / P; ++pair) {
    const int lo = std::max(first, pair * P), hi = std::min(end, pair * P + P);
    uint32_t done = 0;
    if (lane == 0) {
      __builtin_amdgcn_s_waitcnt(0);
      done = __hip_atomic_fetch_add(o.counters + static_cast<size_t>(pair) * kTicketStride,
                                    static_cast<uint32_t>(hi - lo), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) +
             static_cast<uint32_t>(hi - lo);
    }
    if (uniform_i(static_cast<int>(done)) == P) stats_finish_pair<T>(draft, V, P, npairs, pair, l1part, pk, o);
  }
}

// One workgroup: per-block tau and the loss / report sums, in fp64, in a fixed
// order (thread t owns blocks t, t + 256, ...; then one fixed tree over the
// eight sums at once).  Every load of a block is issued before its first use.
__global__ __launch_bounds__(kThreads) void stats_reduce_kernel(
    const float* __restrict__ l1, const float* __restrict__ accept_rate,
    const float* __restrict__ ce, const float* __restrict__ bce,
    const uint8_t* __restrict__ block_mask, int32_t N, int32_t gamma, float w_ce, float w_l1,
    float w_conf, float* __restrict__ tau, float* __restrict__ sums) {
  constexpr int Q = 8;  // num, tokens, l1, accept, tau, blocks, ce, bce
  __shared__ double sh[Q][kThreads];
  double acc[Q] = {0, 0, 0, 0, 0, 0, 0, 0};
  double wk[DSPARK_MAX_GAMMA];
#pragma unroll
  for (int k = 0; k < DSPARK_MAX_GAMMA; ++k) wk[k] = exp(-static_cast<double>(k + 1) / gamma);
  for (int b = threadIdx.x; b < N; b += kThreads) {
    float a[DSPARK_MAX_GAMMA], c[DSPARK_MAX_GAMMA], l[DSPARK_MAX_GAMMA], x[DSPARK_MAX_GAMMA];
    const size_t base = static_cast<size_t>(b) * gamma;
#pragma unroll
    for (int k = 0; k < DSPARK_MAX_GAMMA; ++k) {
      const bool in = k < gamma;
      a[k] = in ? accept_rate[base + k] : 0.0f;
      c[k] = in ? ce[base + k] : 0.0f;
      l[k] = in ? l1[base + k] : 0.0f;
      x[k] = in ? bce[base + k] : 0.0f;
    }
    const bool m = block_mask ? block_mask[b] != 0 : true;
    double cum = 1.0, t = 1.0;
#pragma unroll
    for (int k = 0; k < DSPARK_MAX_GAMMA; ++k) {
      if (k < gamma) {
        cum *= a[k];
        t += cum;
        if (m) {
          acc[0] += wk[k] * (w_ce * static_cast<double>(c[k]) + w_l1 * static_cast<double>(l[k]) +
                             w_conf * static_cast<double>(x[k]));
          acc[1] += 1.0;
          acc[2] += l[k];
          acc[3] += a[k];
          acc[6] += c[k];
          acc[7] += x[k];
        }
      }
    }
    tau[b] = static_cast<float>(t);
    if (m) {
      acc[4] += t;
      acc[5] += 1.0;
    }
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) sh[q][threadIdx.x] = acc[q];
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (static_cast<int>(threadIdx.x) < o)
#pragma unroll
      for (int q = 0; q < Q; ++q) sh[q][threadIdx.x] += sh[q][threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double n = sh[1][0];
    sums[0] = static_cast<float>(sh[0][0]);
    sums[1] = static_cast<float>(n);
    sums[2] = static_cast<float>(sh[2][0]);
    sums[3] = static_cast<float>(n);
    sums[4] = static_cast<float>(sh[3][0]);
    sums[5] = static_cast<float>(n);
    sums[6] = static_cast<float>(sh[4][0]);
    sums[7] = static_cast<float>(sh[5][0]);
    sums[8] = static_cast<float>(sh[6][0]);
    sums[9] = static_cast<float>(n);
    sums[10] = static_cast<float>(sh[7][0]);
    sums[11] = static_cast<float>(n);
  }
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);  // NaN
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------------------
// Backward: the gradient of scale x the loss numerator (definition in
// include/dspark.h).  Per row pair, three looks: the normalisers (look 1 of
// the forward); then L1 = sum |P - T| and S = sum_u sign(P_u - T_u) P_u; then
// the gradient row
//   g_v = a_ce (P_v - [v == teacher]) + a_l1 P_v (s_v - S),
// a_ce = scale m_b w_k w_ce, a_l1 = scale m_b w_k w_l1 (the only write).  For
// near pairs (l1norm.hpp) the sign s_v is that of D_v kappa - (T_v - D_v),
// exact wherever that term is, so that nearly equal rows get the oracle's
// signs; for far pairs that of log2 P_v - log2 T_v.  The sliced
// path runs the looks as item kernels (the first is stats_part1); the row
// path keeps one workgroup per pair for all three, its later looks served by
// the caches.

struct GradRow {
  PairK k;
  float S, a_ce, a_l1;
  int32_t teacher;
};

struct GradArgs {
  const int32_t* teacher;
  const float* conf_logits;
  const uint8_t* block_mask;
  const float* scale;  // device scalar or NULL (1)
  int32_t gamma;
  float w_ce, w_l1, w_conf;
  float* grad_conf;
  GradRow* rows;
  uint32_t* counters;
};

// the pair's coefficients from its constants, L1 and S; writes the
// confidence-logit gradient scale m_b w_k w_conf (sigmoid(c) - a)
__device__ __forceinline__ GradRow grad_row(const GradArgs& g, int pair, const PairK& k, float L1, float S,
                                            int32_t V) {
  const int kk = pair % g.gamma + 1, b = pair / g.gamma;
  const bool m = g.block_mask ? g.block_mask[b] != 0 : true;
  const float sc = g.scale ? *g.scale : 1.0f;
  const float alpha = m ? sc * expf(-static_cast<float>(kk) / static_cast<float>(g.gamma)) : 0.0f;
  const float a = fminf(1.0f, fmaxf(0.0f, 1.0f - 0.5f * L1));
  const float c = g.conf_logits[pair];
  g.grad_conf[pair] = alpha * g.w_conf * (1.0f / (1.0f + expf(-c)) - a);
  return GradRow{k, S, alpha * g.w_ce, alpha * g.w_l1, clamp_token(g.teacher[pair], V)};
}

// Look 2 of a segment for the gradient: the lane's share of the L1 sum (as
// seg_l1) and of sum_v sign(P_v - T_v) D_v; k.far is uniform.
template <typename T>
__device__ __forceinline__ void seg_l1s(const uint4* ud, const uint4* ut, const PairK& k, float& acc, float& s) {
  constexpr int EPL = 16 / sizeof(T);
  if (k.far) {
#pragma unroll
    for (int it = 0; it < kSegIters; ++it)
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const float u = fmaf(elem16(ud[it], j, T{}), kLog2e, -k.a2d);
        const float w = fmaf(elem16(ut[it], j, T{}) - k.K, kLog2e, -k.a2t) + k.lam2;
        const float D = __builtin_amdgcn_exp2f(u);
        acc += __builtin_amdgcn_exp2f(fminf(u, w));
        s += u > w ? D : (u < w ? -D : 0.0f);
      }
  } else {
#pragma unroll
    for (int it = 0; it < kSegIters; ++it)
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const float d = elem16(ud[it], j, T{}), t = elem16(ut[it], j, T{}) - k.K;
        const float D = __builtin_amdgcn_exp2f(fmaf(d, kLog2e, -k.a2d));
        const float Tv = __builtin_amdgcn_exp2f(fmaf(t, kLog2e, -k.a2t));
        const float e = fmaf(D, k.kappa, -np_diff<false>(d, t, D, Tv));
        acc += fabsf(e);
        s += e > 0.0f ? D : (e < 0.0f ? -D : 0.0f);
      }
  }
}

__device__ __forceinline__ float grad_elem(const GradRow& r, float x, float y0, int v) {
  const float y = y0 - r.k.K;
  const float u = fmaf(x, kLog2e, -r.k.a2d);
  const float D = __builtin_amdgcn_exp2f(u);
  float e;
  if (r.k.far) {
    e = u - (fmaf(y, kLog2e, -r.k.a2t) + r.k.lam2);
  } else {
    const float Tv = __builtin_amdgcn_exp2f(fmaf(y, kLog2e, -r.k.a2t));
    e = fmaf(D, r.k.kappa, -np_diff<false>(x, y, D, Tv));
  }
  const float sg = e > 0.0f ? 1.0f : (e < 0.0f ? -1.0f : 0.0f);
  const float P = D * r.k.isd;
  return r.a_ce * (P - (v == r.teacher ? 1.0f : 0.0f)) + r.a_l1 * P * (sg - r.S);
}

// Sliced second look: per item the pair's constants (its part1 records) and
// the item's shares of L1 and S; the pair's last item (ticket) sums the
// shares in a fixed order and stores the pair's GradRow.
template <typename T>
__global__ __launch_bounds__(kThreads) void stats_grad_part2_kernel(
    const T* __restrict__ draft, const T* __restrict__ target, int32_t V, int32_t P, int32_t items,
    const NormPart* __restrict__ part, float* __restrict__ l1part, GradArgs o) {
  constexpr int SEG = stat_seg<T>();
  const int lane = threadIdx.x & 63;
  const int nwaves = gridDim.x * kWaves;
  for (int item = static_cast<int>(blockIdx.x) * kWaves + (threadIdx.x >> 6); item < items;
       item += nwaves) {
    const int it_ = uniform_i(item);
    const int pair = it_ / P, seg = it_ - pair * P;
    const size_t off = static_cast<size_t>(pair) * V;
    uint4 ud[kSegIters], ut[kSegIters];
    const float r5 = pair_r5(draft + off, target + off, V, lane);
    seg_load<T, true>(draft + off, target + off, V, seg * SEG, lane, ud, ut);
    PairK k = pair_k(pair_merge(part + static_cast<size_t>(pair) * P, P, lane));
    k.K = pair_k5(r5);
    seg_mask<T, true>(V, seg * SEG, lane, ud, ut);
    float a = 0.0f, s = 0.0f;
    seg_l1s<T>(ud, ut, k, a, s);
    a = wave_sum(a);
    s = wave_sum(s);
    uint32_t ticket = 0;
    if (lane == 0) {
      float* q = l1part + 2 * static_cast<size_t>(it_);
      store_coherent(q, a);
      store_coherent(q + 1, s);
      ticket = publish(o.counters + static_cast<size_t>(pair) * kTicketStride);
    }
    ticket = uniform_i(static_cast<int>(ticket));
    if (ticket != static_cast<uint32_t>(P - 1)) continue;
    float A = 0.0f, S = 0.0f;
    for (int i = lane; i < P; i += 64) {
      const float* q = l1part + 2 * (static_cast<size_t>(pair) * P + i);
      A += load_coherent(q);
      S += load_coherent(q + 1);
    }
    A = wave_sum(A);
    S = wave_sum(S);
    if (lane == 0) o.rows[pair] = grad_row(o, pair, k, l1_final(k, A), S * k.isd, V);
  }
}

template <typename T>
__device__ __forceinline__ void store16(T* p, const float* g);
template <>
__device__ __forceinline__ void store16<uint16_t>(uint16_t* p, const float* g) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = static_cast<uint32_t>(bf16_rne(g[2 * i])) | (static_cast<uint32_t>(bf16_rne(g[2 * i + 1])) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}
template <>
__device__ __forceinline__ void store16<float>(float* p, const float* g) {
  *reinterpret_cast<float4*>(p) = make_float4(g[0], g[1], g[2], g[3]);
}


// The gradient of one segment (lane l: groups it * 64 + l) into row gr.
template <typename T, bool VEC>
__device__ __forceinline__ void seg_grad_store(const GradRow& r, const uint4* ud, const uint4* ut, int32_t V, int lo,
                                               int lane, T* __restrict__ gr) {
  constexpr int EPL = 16 / sizeof(T);
#pragma unroll
  for (int it = 0; it < kSegIters; ++it) {
    const int e = lo + (it * 64 + lane) * EPL;
    if (e >= V) continue;  // VEC: a clamped load past the row
    float g[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) g[j] = grad_elem(r, elem16(ud[it], j, T{}), elem16(ut[it], j, T{}), e + j);
    if constexpr (VEC) {
      store16<T>(gr + e, g);
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (e + j < V) {
          if constexpr (sizeof(T) == 2) gr[e + j] = bf16_rne(g[j]);
          else gr[e + j] = g[j];
        }
    }
  }
}

// Sliced third look: per item the gradient of its segment (the next item's
// loads in flight while the current one is computed and stored).
template <typename T>
__global__ __launch_bounds__(kThreads) void stats_grad_write_kernel(
    const T* __restrict__ draft, const T* __restrict__ target, int32_t V, int32_t P, int32_t items,
    const GradRow* __restrict__ rows, T* __restrict__ grad) {
  constexpr int SEG = stat_seg<T>();
  const int lane = threadIdx.x & 63;
  const int nwaves = gridDim.x * kWaves;
  int item = uniform_i(static_cast<int>(blockIdx.x) * kWaves + (threadIdx.x >> 6));
  if (item >= items) return;
  uint4 ad[kSegIters], at[kSegIters], bd[kSegIters], bt[kSegIters];
  auto load = [&](int it_, uint4* ud, uint4* ut) {
    const int pair = it_ / P, seg = it_ - pair * P;
    const size_t off = static_cast<size_t>(pair) * V;
    seg_load<T, true>(draft + off, target + off, V, seg * SEG, lane, ud, ut);
  };
  auto write = [&](const uint4* ud, const uint4* ut, int it_) {
    const int pair = it_ / P, seg = it_ - pair * P;
    seg_grad_store<T, true>(rows[pair], ud, ut, V, seg * SEG, lane, grad + static_cast<size_t>(pair) * V);
  };
  load(item, ad, at);
  while (true) {
    const int n1 = uniform_i(item + nwaves);
    load(n1 < items ? n1 : item, bd, bt);
    write(ad, at, item);
    if (n1 >= items) break;
    const int n2 = uniform_i(n1 + nwaves);
    load(n2 < items ? n2 : n1, ad, at);
    write(bd, bt, n1);
    if (n2 >= items) break;
    item = n2;
  }
}

// Row path: one persistent workgroup per compute unit, the three looks of
// each of its row pairs in turn.
template <typename T, bool VEC>
__global__ __launch_bounds__(kRowThreads) void stats_grad_rows_kernel(const T* __restrict__ draft,
                                                                      const T* __restrict__ target,
                                                                      int32_t V, int32_t npairs, GradArgs o,
                                                                      T* __restrict__ grad) {
  constexpr int SEG = stat_seg<T>();
  __shared__ NormPart shp[kRowWaves];
  __shared__ float sha[kRowWaves], shs[kRowWaves];
  __shared__ GradRow shr;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int P = (V + SEG - 1) / SEG;
  for (int rr = blockIdx.x; rr < npairs; rr += gridDim.x) {
    const size_t row = static_cast<size_t>(rr);
    const T* dr = draft + row * V;
    const T* tr = target + row * V;
    const float r5 = pair_r5(dr, tr, V, lane);  // issued ahead of the first segment's loads
    NormPart acc = np_empty();
    float K = 0.0f;
    bool kset = false;
    seg_scan<T, VEC>(dr, tr, V, P, wave, kRowWaves, lane, [&](const uint4* ud, const uint4* ut, int) {
      if (!kset) {  // once the first segment's loads are in flight
        K = pair_k5(r5);
        kset = true;
      }
      acc = np_merge(acc, seg_part<T>(ud, ut, K));
    });
    if (lane == 0) shp[wave] = acc;
    __syncthreads();
    if (wave == 0) {
      const NormPart m = np_wave_merge(lane < kRowWaves ? shp[lane] : np_empty());
      K = pair_k5(r5);  // wave 0 may have had no segment
      if (lane == 0) {
        shr.k = pair_k(m);
        shr.k.K = K;
      }
    }
    __syncthreads();
    const PairK k = shr.k;
    float a = 0.0f, s = 0.0f;
    seg_scan<T, VEC>(dr, tr, V, P, wave, kRowWaves, lane,
                     [&](const uint4* ud, const uint4* ut, int) { seg_l1s<T>(ud, ut, k, a, s); });
    a = wave_sum(a);
    s = wave_sum(s);
    if (lane == 0) {
      sha[wave] = a;
      shs[wave] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float A = 0.0f, S = 0.0f;
#pragma unroll
      for (int w = 0; w < kRowWaves; ++w) {
        A += sha[w];
        S += shs[w];
      }
      shr = grad_row(o, static_cast<int>(row), k, l1_final(k, A), S * k.isd, V);
    }
    __syncthreads();
    const GradRow r = shr;
    T* gr = grad + row * V;
    seg_scan<T, VEC>(dr, tr, V, P, wave, kRowWaves, lane, [&](const uint4* ud, const uint4* ut, int lo) {
      seg_grad_store<T, VEC>(r, ud, ut, V, lo, lane, gr);
    });
    __syncthreads();  // shp, sha, shs and shr are reused by the next pair
  }
}

// Compute units of the current device, cached per device.
int device_cus_cached() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDev) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev < kMaxDev) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Grid of an item kernel of kThreads: every wave resident at once (each then
// walks its items with the next one's loads in flight), no more waves than
// items.
int item_grid(int items, const void* fn, std::atomic<int>& cache) {
  return resident_grid(fn, kThreads, items, cache);
}

template <typename T>
hipError_t launch_typed(const T* draft, const T* target, const int32_t* teacher,
                        const float* conf_logits, const uint8_t* block_mask, int32_t N,
                        int32_t gamma, int32_t V, float w_ce, float w_l1, float w_conf, float* l1,
                        float* accept_rate, float* ce, float* bce, float* tau, float* sums,
                        void* ws, const StatsPlan& pl, hipStream_t st) {
  const int epl = 16 / static_cast<int>(sizeof(T));
  const bool vec = (V % epl == 0) && reinterpret_cast<uintptr_t>(draft) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(target) % 16 == 0;
  const int npairs = N * gamma;
  if (npairs > 0 && vec && pl.sliced) {
    char* w = static_cast<char*>(ws);
    NormPart* part = reinterpret_cast<NormPart*>(w + pl.off_part);
    float* l1part = reinterpret_cast<float*>(w + pl.off_l1);
    PairK* pk = reinterpret_cast<PairK*>(w + pl.off_pk);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(w + pl.off_cnt);
    const int items = npairs * pl.P;
    static std::atomic<int> occ1{0}, occ2{0};
    const int wg1 = item_grid(items, reinterpret_cast<const void*>(&stats_part1_kernel<T>), occ1);
    const int wg2 = item_grid(items, reinterpret_cast<const void*>(&stats_part2_kernel<T>), occ2);
    const StatsOut o{teacher, conf_logits, block_mask, N, gamma, w_ce, w_l1, w_conf,
                     l1, accept_rate, ce, bce, tau, sums, cnt};
    DSPARK_LAUNCH("stats_part1", (stats_part1_kernel<T>), dim3(wg1), dim3(kThreads), 0, st, draft,
                  target, V, pl.P, items, part, cnt, npairs + 1);
    DSPARK_LAUNCH("stats_part2", (stats_part2_kernel<T>), dim3(wg2), dim3(kThreads), 0, st, draft,
                  target, V, pl.P, items, part, l1part, pk, o);
    return hipGetLastError();
  } else if (npairs > 0) {
    const dim3 grid(static_cast<unsigned>(std::min(npairs, device_cus_cached())));
    if (vec)
      DSPARK_LAUNCH("stats_rows", (stats_rows_kernel<T, true>), grid, dim3(kRowThreads), 0, st, draft,
                    target, teacher, conf_logits, V, npairs, l1, accept_rate, ce, bce);
    else
      DSPARK_LAUNCH("stats_rows", (stats_rows_kernel<T, false>), grid, dim3(kRowThreads), 0, st,
                    draft, target, teacher, conf_logits, V, npairs, l1, accept_rate, ce, bce);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  DSPARK_LAUNCH("stats_reduce", stats_reduce_kernel, dim3(1), dim3(kThreads), 0, st, l1,
                accept_rate, ce, bce, block_mask, N, gamma, w_ce, w_l1, w_conf, tau, sums);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_backward_typed(const T* draft, const T* target, int32_t N, int32_t gamma, int32_t V,
                                 GradArgs o, T* grad, void* ws, const StatsGradPlan& pl,
                                 hipStream_t st) {
  const int epl = 16 / static_cast<int>(sizeof(T));
  const bool vec = (V % epl == 0) && reinterpret_cast<uintptr_t>(draft) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(target) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(grad) % 16 == 0;
  const int npairs = N * gamma;
  if (npairs == 0) return hipSuccess;
  if (vec && pl.sliced) {
    char* w = static_cast<char*>(ws);
    NormPart* part = reinterpret_cast<NormPart*>(w + pl.off_part);
    float* l1part = reinterpret_cast<float*>(w + pl.off_l1);
    o.rows = reinterpret_cast<GradRow*>(w + pl.off_rows);
    o.counters = reinterpret_cast<uint32_t*>(w + pl.off_cnt);
    const int items = npairs * pl.P;
    const int wgs = std::min(kItemMaxWGs, (items + kWaves - 1) / kWaves);
    DSPARK_LAUNCH("stats_part1", (stats_part1_kernel<T>), dim3(wgs), dim3(kThreads), 0, st, draft,
                  target, V, pl.P, items, part, o.counters, npairs);
    DSPARK_LAUNCH("stats_grad_part2", (stats_grad_part2_kernel<T>), dim3(wgs), dim3(kThreads), 0, st,
                  draft, target, V, pl.P, items, part, l1part, o);
    DSPARK_LAUNCH("stats_grad_write", (stats_grad_write_kernel<T>), dim3(wgs), dim3(kThreads), 0, st,
                  draft, target, V, pl.P, items, o.rows, grad);
  } else {
    const dim3 grid(static_cast<unsigned>(std::min(npairs, device_cus_cached())));
    if (vec)
      DSPARK_LAUNCH("stats_grad_rows", (stats_grad_rows_kernel<T, true>), grid, dim3(kRowThreads), 0, st,
                    draft, target, V, npairs, o, grad);
    else
      DSPARK_LAUNCH("stats_grad_rows", (stats_grad_rows_kernel<T, false>), grid, dim3(kRowThreads), 0,
                    st, draft, target, V, npairs, o, grad);
  }
  return hipGetLastError();
}

}  // namespace

int device_cus() { return device_cus_cached(); }

int resident_grid(const void* fn, int threads, int64_t items, std::atomic<int>& cache) {
  int nb = cache.load(std::memory_order_relaxed);
  if (nb <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, threads, 0) != hipSuccess || nb <= 0) nb = 1;
    cache.store(nb, std::memory_order_relaxed);
  }
  const int64_t res = static_cast<int64_t>(device_cus_cached()) * nb;
  const int64_t wpb = threads / 64;
  const int64_t need = (items + wpb - 1) / wpb;
  return static_cast<int>(std::max<int64_t>(1, std::min(need, res)));
}

hipError_t launch_stats_reduce(const float* l1, const float* accept_rate, const float* ce, const float* bce,
                               const uint8_t* block_mask, int32_t N, int32_t gamma, float w_ce, float w_l1,
                               float w_conf, float* tau, float* sums, hipStream_t st) {
  DSPARK_LAUNCH("stats_reduce", stats_reduce_kernel, dim3(1), dim3(kThreads), 0, st, l1, accept_rate, ce, bce,
                block_mask, N, gamma, w_ce, w_l1, w_conf, tau, sums);
  return hipGetLastError();
}

StatsGradPlan plan_stats_backward(int32_t N, int32_t gamma, int32_t V) {
  StatsGradPlan p{};
  const int64_t npairs = static_cast<int64_t>(N) * gamma;
  p.P = (V + stat_seg<uint16_t>() - 1) / stat_seg<uint16_t>();
  const int Pf = (V + stat_seg<float>() - 1) / stat_seg<float>();
  const int Pmax = p.P > Pf ? p.P : Pf;
  p.sliced = npairs > 0 && npairs < kSlicedMaxPairs;
  size_t off = 0;
  if (p.sliced) {
    const size_t items = static_cast<size_t>(npairs) * Pmax;
    p.off_part = off;
    off = align_up(off + items * sizeof(NormPart), 256);
    p.off_l1 = off;  // per item: shares of the L1 sum and of S Sd
    off = align_up(off + 2 * items * sizeof(float), 256);
    p.off_rows = off;
    off = align_up(off + static_cast<size_t>(npairs) * sizeof(GradRow), 256);
    p.off_cnt = off;
    off = align_up(off + static_cast<size_t>(npairs) * kTicketStride * sizeof(uint32_t), 256);
  }
  p.bytes = off;
  return p;
}

hipError_t launch_stats_backward(const void* draft, const void* target, int dtype, const int32_t* teacher,
                                 const float* conf_logits, const uint8_t* block_mask, int32_t N,
                                 int32_t gamma, int32_t V, float w_ce, float w_l1, float w_conf,
                                 const float* grad_scale, void* grad_draft, float* grad_conf, void* ws,
                                 const StatsGradPlan& plan, hipStream_t st) {
  GradArgs o{teacher, conf_logits, block_mask, grad_scale, gamma, w_ce, w_l1, w_conf, grad_conf,
             nullptr, nullptr};
  StatsGradPlan pl = plan;
  if (dtype == DSPARK_BF16) {
    pl.P = (V + stat_seg<uint16_t>() - 1) / stat_seg<uint16_t>();
    return launch_backward_typed(static_cast<const uint16_t*>(draft), static_cast<const uint16_t*>(target),
                                 N, gamma, V, o, static_cast<uint16_t*>(grad_draft), ws, pl, st);
  }
  pl.P = (V + stat_seg<float>() - 1) / stat_seg<float>();
  return launch_backward_typed(static_cast<const float*>(draft), static_cast<const float*>(target), N,
                               gamma, V, o, static_cast<float*>(grad_draft), ws, pl, st);
}

StatsPlan plan_stats(int32_t N, int32_t gamma, int32_t V) {
  StatsPlan p{};
  const int64_t npairs = static_cast<int64_t>(N) * gamma;
  // bf16 segments are the larger: size the workspace for them
  p.P = (V + stat_seg<uint16_t>() - 1) / stat_seg<uint16_t>();
  const int Pf = (V + stat_seg<float>() - 1) / stat_seg<float>();
  const int Pmax = p.P > Pf ? p.P : Pf;
  p.sliced = npairs > 0 && npairs < kSlicedMaxPairs;
  size_t off = 0;
  if (p.sliced) {
    const size_t items = static_cast<size_t>(npairs) * Pmax;
    p.off_part = off;
    off = align_up(off + items * sizeof(NormPart), 256);
    p.off_l1 = off;  // per item: share of the L1 sum
    off = align_up(off + items * sizeof(float), 256);
    p.off_pk = off;  // per pair: the constants of look 2 and the final
    off = align_up(off + static_cast<size_t>(npairs) * sizeof(PairK), 256);
    p.off_cnt = off;  // per pair: items done; then pairs done (cleared by stats_part1)
    off = align_up(off + (static_cast<size_t>(npairs) + 1) * kTicketStride * sizeof(uint32_t), 256);
  }
  p.bytes = off;
  return p;
}

hipError_t launch_stats(const void* draft, const void* target, int dtype, const int32_t* teacher,
                        const float* conf_logits, const uint8_t* block_mask, int32_t N,
                        int32_t gamma, int32_t V, float w_ce, float w_l1, float w_conf, float* l1,
                        float* accept_rate, float* ce, float* bce, float* tau, float* sums,
                        void* ws, const StatsPlan& plan, hipStream_t st) {
  if (dtype == DSPARK_BF16) {
    StatsPlan pl = plan;
    pl.P = (V + stat_seg<uint16_t>() - 1) / stat_seg<uint16_t>();
    return launch_typed(static_cast<const uint16_t*>(draft), static_cast<const uint16_t*>(target),
                        teacher, conf_logits, block_mask, N, gamma, V, w_ce, w_l1, w_conf, l1,
                        accept_rate, ce, bce, tau, sums, ws, pl, st);
  }
  StatsPlan pl = plan;
  pl.P = (V + stat_seg<float>() - 1) / stat_seg<float>();
  return launch_typed(static_cast<const float*>(draft), static_cast<const float*>(target), teacher,
                      conf_logits, block_mask, N, gamma, V, w_ce, w_l1, w_conf, l1, accept_rate,
                      ce, bce, tau, sums, ws, pl, st);
}

}  // namespace dspark
