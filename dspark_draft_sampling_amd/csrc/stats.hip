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
// stats_rows: one workgroup per row pair.  Pass 1 streams both rows once with
// 16-byte loads and keeps an online (max, sum exp) per thread; pass 2 streams
// them again (the pair was just read, so it is served from the caches) for
// the L1 term.  The L1 pass forms the overlap sum_v min(P_v, T_v) instead of
// sum |P_v - T_v|: both rows sum to 1, so L1 = 2 (1 - overlap) exactly, and
// min(P_v, T_v) = exp(min(d_v - lse_d, t_v - lse_t)) takes one exponential
// per element pair where |P_v - T_v| takes two.  stats_reduce: one workgroup computes tau and the sums in fp64
// in a fixed order, so the sums are deterministic.
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "internal.hpp"

namespace dspark {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Row path: one workgroup of kRowThreads per compute unit, each looping over
// row pairs, so that the pairs being read at once (one per CU, 0.5 MB each at
// V = 129280 in bf16) stay within the 256 MB Infinity Cache and the later
// looks at a pair are served from it rather than from HBM.
constexpr int kRowThreads = 1024;
constexpr int kRowWaves = kRowThreads / 64;
constexpr int kUnroll = 4;
constexpr int kItemMaxWGs = 2048;      // grid of the sliced item kernels
constexpr int kSlicedMaxPairs = 2048;  // row pairs below which the sliced path is used

template <typename T, bool VEC>
struct Vec8;

template <>
struct Vec8<uint16_t, true> {
  static constexpr int N = 8;
  __device__ static void load(const uint16_t* p, float* o) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    o[0] = bf_lo(u.x);
    o[1] = bf_hi(u.x);
    o[2] = bf_lo(u.y);
    o[3] = bf_hi(u.y);
    o[4] = bf_lo(u.z);
    o[5] = bf_hi(u.z);
    o[6] = bf_lo(u.w);
    o[7] = bf_hi(u.w);
  }
};
template <>
struct Vec8<float, true> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* o) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    o[0] = u.x;
    o[1] = u.y;
    o[2] = u.z;
    o[3] = u.w;
  }
};
template <typename T>
struct Vec8<T, false> {
  static constexpr int N = 1;
  __device__ static void load(const T* p, float* o) { o[0] = load_logit(p, 0); }
};

__device__ __forceinline__ void online(float& m, float& s, const float* x, int n) {
  float mx = x[0];
  for (int j = 1; j < n; ++j) mx = fmaxf(mx, x[j]);
  if (mx > m) {
    s = (m > neg_inf()) ? s * __builtin_amdgcn_exp2f((m - mx) * kLog2e) : 0.0f;
    m = mx;
  }
  if (m > neg_inf())
    for (int j = 0; j < n; ++j) s += __builtin_amdgcn_exp2f((x[j] - m) * kLog2e);
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kRowThreads) void stats_rows_kernel(
    const T* __restrict__ draft, const T* __restrict__ target, const int32_t* __restrict__ teacher,
    const float* __restrict__ conf_logits, int32_t V, int32_t npairs, float* __restrict__ l1,
    float* __restrict__ accept_rate, float* __restrict__ ce, float* __restrict__ bce) {
  using L = Vec8<T, VEC>;
  constexpr int EPL = L::N;
  constexpr int kThreads = kRowThreads, kWaves = kRowWaves;
  __shared__ float shv[kWaves];
  for (int rr = blockIdx.x; rr < npairs; rr += gridDim.x) {
  const size_t row = static_cast<size_t>(rr);
  const T* dr = draft + row * V;
  const T* tr = target + row * V;
  const int step = kThreads * EPL;

  // pass 1: online normalisers of both rows
  float md = neg_inf(), sd = 0.0f, mt = neg_inf(), st = 0.0f;
  int e = threadIdx.x * EPL;
  for (; e + (kUnroll - 1) * step < V; e += kUnroll * step) {
    float xd[kUnroll][EPL], xt[kUnroll][EPL];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      L::load(dr + e + u * step, xd[u]);
      L::load(tr + e + u * step, xt[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      online(md, sd, xd[u], EPL);
      online(mt, st, xt[u], EPL);
    }
  }
  for (; e < V; e += step) {
    float xd[EPL], xt[EPL];
    L::load(dr + e, xd);
    L::load(tr + e, xt);
    online(md, sd, xd, EPL);
    online(mt, st, xt, EPL);
  }
  const float Md = block_max<kWaves>(md, shv);
  const float Sd = block_sum<kWaves>(md > neg_inf() ? sd * __builtin_amdgcn_exp2f((md - Md) * kLog2e) : 0.0f, shv);
  const float Mt = block_max<kWaves>(mt, shv);
  const float St = block_sum<kWaves>(mt > neg_inf() ? st * __builtin_amdgcn_exp2f((mt - Mt) * kLog2e) : 0.0f, shv);
  // log2(Sd / St): min(P_v, T_v) = 2^min((d_v - Md) log2e, (t_v - Mt) log2e + lam) / Sd
  const float lam = __log2f(Sd) - __log2f(St);

  // pass 2: the overlap sum_v min(P_v, T_v); L1 = sum |P - T| = 2 (1 - overlap)
  // (both rows sum to 1), one exponential per element pair
  float acc = 0.0f;
  e = threadIdx.x * EPL;
  for (; e + (kUnroll - 1) * step < V; e += kUnroll * step) {
    float xd[kUnroll][EPL], xt[kUnroll][EPL];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      L::load(dr + e + u * step, xd[u]);
      L::load(tr + e + u * step, xt[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        acc += __builtin_amdgcn_exp2f(fminf((xd[u][j] - Md) * kLog2e, fmaf(xt[u][j] - Mt, kLog2e, lam)));
  }
  for (; e < V; e += step) {
    float xd[EPL], xt[EPL];
    L::load(dr + e, xd);
    L::load(tr + e, xt);
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      acc += __builtin_amdgcn_exp2f(fminf((xd[j] - Md) * kLog2e, fmaf(xt[j] - Mt, kLog2e, lam)));
  }
  const float ov = block_sum<kWaves>(acc, shv) / Sd;

  if (threadIdx.x == 0) {
    const float L1 = fmaxf(0.0f, 2.0f * (1.0f - ov));
    const float a = fminf(1.0f, fmaxf(0.0f, ov));
    const int32_t tch = clamp_token(teacher[row], V);
    const float lse_d = Md + logf(Sd);
    const float c = conf_logits[row];
    l1[row] = L1;
    accept_rate[row] = a;
    ce[row] = lse_d - load_logit(dr, tch);
    bce[row] = fmaxf(c, 0.0f) - c * a + log1pf(expf(-fabsf(c)));
  }
  }
}

// ---------------------------------------------------------------------------
// Sliced path for small batches: (row pair, 2048-token segment) items, one
// wave each, so that a few hundred row pairs still fill the GPU.
//   stats_part1  per item: (max, sum) of both rows, sums with an integer
//                base-2 shift (s = sum 2^(x log2e - floor(m log2e)))
//   stats_part2  per item: the pair's normalisers from all its part1
//                records, then the item's share of the overlap sum_v
//                min(P_v, T_v) (a second read of the pair; L1 = 2 (1 -
//                overlap)), with a ticket per pair: the pair's last
//                item writes L1, accept_rate, CE and BCE, and the wave
//                finishing the last pair writes tau and the sums
// Both item kernels keep the next item's loads in flight while reducing the
// current one (two register buffers, unconditional clamped loads).
constexpr int kSegIters = 4;  // 16-byte loads per lane per row per segment

struct StatPart {
  float md, sd, mt, st;
};

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

template <typename T>
__device__ __forceinline__ void seg_load(const T* __restrict__ draft, const T* __restrict__ target,
                                         int32_t V, int32_t P, int item, int lane, uint4* ud,
                                         uint4* ut) {
  constexpr int EPL = 16 / sizeof(T);
  constexpr int SEG = stat_seg<T>();
  const int pair = item / P, seg = item - pair * P;
  const size_t off = static_cast<size_t>(pair) * V;
  const int lo = seg * SEG;
#pragma unroll
  for (int it = 0; it < kSegIters; ++it) {
    const int e = min(lo + (it * 64 + lane) * EPL, V - EPL);
    ud[it] = *reinterpret_cast<const uint4*>(draft + off + e);
    ut[it] = *reinterpret_cast<const uint4*>(target + off + e);
  }
}

// mask the clamped loads of a partial segment with -inf
template <typename T>
__device__ __forceinline__ void seg_mask(int32_t V, int lo, int lane, uint4* ud, uint4* ut) {
  constexpr int EPL = 16 / sizeof(T);
  constexpr uint32_t kNeg = sizeof(T) == 2 ? 0xFF80FF80u : 0xFF800000u;
  if (V - lo < stat_seg<T>()) {
#pragma unroll
    for (int it = 0; it < kSegIters; ++it)
      if (lo + (it * 64 + lane) * EPL >= V) ud[it] = ut[it] = make_uint4(kNeg, kNeg, kNeg, kNeg);
  }
}

template <typename T>
__device__ __forceinline__ void seg_stats(const uint4* u, float& m, float& s) {
  constexpr int EPL = 16 / sizeof(T);
  m = neg_inf();
#pragma unroll
  for (int it = 0; it < kSegIters; ++it)
#pragma unroll
    for (int j = 0; j < EPL; ++j) m = fmaxf(m, elem16(u[it], j, T{}));
  m = wave_max(m);
  s = 0.0f;
  if (m > neg_inf()) {
    const float M2 = floorf(m * kLog2e);
#pragma unroll
    for (int it = 0; it < kSegIters; ++it)
#pragma unroll
      for (int j = 0; j < EPL; ++j) s += __builtin_amdgcn_exp2f(fmaf(elem16(u[it], j, T{}), kLog2e, -M2));
    s = wave_sum(s);
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void stats_part1_kernel(
    const T* __restrict__ draft, const T* __restrict__ target, int32_t V, int32_t P,
    int32_t items, StatPart* __restrict__ part, uint32_t* __restrict__ counters,
    int32_t ncounters) {
  constexpr int SEG = stat_seg<T>();
  const int lane = threadIdx.x & 63;
  // the ticket counters of stats_part2 start at zero
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < ncounters; i += kThreads) counters[i * kTicketStride] = 0u;
  const int nwaves = gridDim.x * kWaves;
  int item = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * kWaves +
                                            (threadIdx.x >> 6));
  if (item >= items) return;
  uint4 ad[kSegIters], at[kSegIters], bd[kSegIters], bt[kSegIters];
  auto reduce = [&](uint4* ud, uint4* ut, int it_) {
    const int seg = it_ - (it_ / P) * P;
    seg_mask<T>(V, seg * SEG, lane, ud, ut);
    StatPart r;
    seg_stats<T>(ud, r.md, r.sd);
    seg_stats<T>(ut, r.mt, r.st);
    if (lane == 0) part[it_] = r;
  };
  seg_load<T>(draft, target, V, P, item, lane, ad, at);
  while (true) {
    const int n1 = __builtin_amdgcn_readfirstlane(item + nwaves);
    seg_load<T>(draft, target, V, P, n1 < items ? n1 : item, lane, bd, bt);
    reduce(ad, at, item);
    if (n1 >= items) break;
    const int n2 = __builtin_amdgcn_readfirstlane(n1 + nwaves);
    seg_load<T>(draft, target, V, P, n2 < items ? n2 : n1, lane, ad, at);
    reduce(bd, bt, n1);
    if (n2 >= items) break;
    item = n2;
  }
}

// combine a pair's part1 records: the base-2 shift M2 of the pair and the sum
// relative to it, for the draft (d) and target (t) rows
__device__ __forceinline__ void pair_norm(const StatPart* __restrict__ rec, int P, int lane,
                                          float& M2d, float& Sd, float& M2t, float& St) {
  float md = neg_inf(), mt = neg_inf();
  for (int i = lane; i < P; i += 64) {
    md = fmaxf(md, rec[i].md);
    mt = fmaxf(mt, rec[i].mt);
  }
  md = wave_max(md);
  mt = wave_max(mt);
  M2d = md > neg_inf() ? floorf(md * kLog2e) : 0.0f;
  M2t = mt > neg_inf() ? floorf(mt * kLog2e) : 0.0f;
  float sd = 0.0f, st = 0.0f;
  for (int i = lane; i < P; i += 64) {
    const StatPart r = rec[i];
    if (r.md > neg_inf()) sd += r.sd * __builtin_amdgcn_exp2f(floorf(r.md * kLog2e) - M2d);
    if (r.mt > neg_inf()) st += r.st * __builtin_amdgcn_exp2f(floorf(r.mt * kLog2e) - M2t);
  }
  Sd = wave_sum(sd);
  St = wave_sum(st);
}

// Per-block tau and the loss / report sums by one wave, in fp64 and a fixed
// order (lane l owns blocks l, l + 64, ...; then a fixed butterfly), so the
// sums are deterministic.  The per-position values were stored by other
// waves of the same launch (device-scope loads).
__device__ void wave_batch_reduce(const float* __restrict__ l1, const float* __restrict__ accept_rate,
                                  const float* __restrict__ ce, const float* __restrict__ bce,
                                  const uint8_t* __restrict__ block_mask, int32_t N,
                                  int32_t gamma, float w_ce, float w_l1, float w_conf,
                                  float* __restrict__ tau, float* __restrict__ sums) {
  constexpr int Q = 8;  // num, tokens, l1, accept, tau, blocks, ce, bce
  const int lane = threadIdx.x & 63;
  // w_k = exp(-k / gamma) = r^k (k 1-based), r to fp32 accuracy
  const double r = static_cast<double>(expf(-1.0f / static_cast<float>(gamma)));
  double acc[Q] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int b = lane; b < N; b += 64) {
    const size_t base = static_cast<size_t>(b) * gamma;
    const bool m = block_mask ? block_mask[b] != 0 : true;
    double cum = 1.0, t = 1.0, wk = 1.0;
    for (int k = 0; k < gamma; ++k) {
      const float a = load_coherent(accept_rate + base + k);
      const float c = load_coherent(ce + base + k);
      const float l = load_coherent(l1 + base + k);
      const float x = load_coherent(bce + base + k);
      cum *= a;
      t += cum;
      wk *= r;
      if (m) {
        acc[0] += wk * (w_ce * static_cast<double>(c) + w_l1 * static_cast<double>(l) +
                        w_conf * static_cast<double>(x));
        acc[1] += 1.0;
        acc[2] += l;
        acc[3] += a;
        acc[6] += c;
        acc[7] += x;
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
  uint32_t* counters;  // per pair: segments done; then pairs done (kTicketStride apart)
};

// Per item: the pair's normalisers from all its part1 records, then the
// item's share of the overlap (times Sd), with a ticket on the pair: the pair's last
// item writes L1, accept_rate, CE and BCE, and the wave finishing the last
// pair writes tau and the sums.
template <typename T>
__global__ __launch_bounds__(kThreads) void stats_part2_kernel(
    const T* __restrict__ draft, const T* __restrict__ target, int32_t V, int32_t P,
    int32_t items, const StatPart* __restrict__ part, float* __restrict__ l1part, StatsOut o) {
  constexpr int EPL = 16 / sizeof(T);
  constexpr int SEG = stat_seg<T>();
  const int lane = threadIdx.x & 63;
  const int nwaves = gridDim.x * kWaves;
  const int npairs = items / P;
  // one item at a time per wave (its ticket waits for its own stores, so no
  // later item's loads may be in flight); the other waves of the CU cover
  // the latency
  for (int item = static_cast<int>(blockIdx.x) * kWaves + (threadIdx.x >> 6); item < items;
       item += nwaves) {
    const int it_ = __builtin_amdgcn_readfirstlane(item);
    const int pair = it_ / P, seg = it_ - pair * P;
    uint4 ud[kSegIters], ut[kSegIters];
    seg_load<T>(draft, target, V, P, it_, lane, ud, ut);
    float M2d, Sd, M2t, St;
    pair_norm(part + static_cast<size_t>(pair) * P, P, lane, M2d, Sd, M2t, St);
    seg_mask<T>(V, seg * SEG, lane, ud, ut);
    // the item's share of the overlap sum_v min(P_v, T_v), times Sd:
    // min(P_v, T_v) = 2^min(d_v log2e - M2d, t_v log2e - M2t + lam) / Sd
    const float lam = __log2f(Sd) - __log2f(St);
    float acc = 0.0f;
#pragma unroll
    for (int it = 0; it < kSegIters; ++it)
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        acc += __builtin_amdgcn_exp2f(fminf(fmaf(elem16(ud[it], j, T{}), kLog2e, -M2d),
                                            fmaf(elem16(ut[it], j, T{}), kLog2e, -M2t) + lam));
    acc = wave_sum(acc);
    uint32_t ticket = 0;
    if (lane == 0) {
      store_coherent(l1part + it_, acc);
      ticket = publish(o.counters + static_cast<size_t>(pair) * kTicketStride);
    }
    ticket = __builtin_amdgcn_readfirstlane(ticket);
    if (ticket != static_cast<uint32_t>(P - 1)) continue;
    // the pair's last item: the overlap from the item shares (fixed order);
    // L1 = sum |P - T| = 2 (1 - overlap), both rows summing to 1
    float ov = 0.0f;
    for (int i = lane; i < P; i += 64) ov += load_coherent(l1part + static_cast<size_t>(pair) * P + i);
    ov = wave_sum(ov) / Sd;
    uint32_t last = 0;
    if (lane == 0) {
      const float L1 = fmaxf(0.0f, 2.0f * (1.0f - ov));
      const float a = fminf(1.0f, fmaxf(0.0f, ov));
      const int32_t tch = clamp_token(o.teacher[pair], V);
      const float c = o.conf_logits[pair];
      const float lse_d = M2d * kLn2 + logf(Sd);
      store_coherent(o.l1 + pair, L1);
      store_coherent(o.accept_rate + pair, a);
      store_coherent(o.ce + pair, lse_d - load_logit(draft + static_cast<size_t>(pair) * V, tch));
      store_coherent(o.bce + pair, fmaxf(c, 0.0f) - c * a + log1pf(expf(-fabsf(c))));
      last = publish(o.counters + static_cast<size_t>(npairs) * kTicketStride) ==
                     static_cast<uint32_t>(npairs - 1)
                 ? 1u
                 : 0u;
    }
    if (__builtin_amdgcn_readfirstlane(last))
      wave_batch_reduce(o.l1, o.accept_rate, o.ce, o.bce, o.block_mask, o.N, o.gamma, o.w_ce,
                        o.w_l1, o.w_conf, o.tau, o.sums);
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

// ---------------------------------------------------------------------------
// Backward: the gradient of scale x the loss numerator (definition in
// include/dspark.h).  Per row pair, three looks: the normalisers; then
// L1 = sum |P - T| and S = sum_u sign(P_u - T_u) P_u; then the gradient row
//   g_v = a_ce (P_v - [v == teacher]) + a_l1 P_v (s_v - S),
// a_ce = scale m_b w_k w_ce, a_l1 = scale m_b w_k w_l1 (the only write).  The
// sliced path runs the looks as item kernels (the first is stats_part1); the
// row path keeps one workgroup per pair for all three, its second and third
// looks served by the caches.

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);  // NaN
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// A pair's coefficients: P_v = 2^(x log2e - shd) isd, and
// log2 P_v - log2 T_v = (x - y) log2e - lr (lr: the pair's log2 ratio of the
// two normalisers), so the sign of P_v - T_v needs no second exponential.
struct GradRow {
  float shd, isd, lr;
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

// the pair's coefficients from its normalisers, L1 and S; writes the
// confidence-logit gradient scale m_b w_k w_conf (sigmoid(c) - a)
__device__ __forceinline__ GradRow grad_row(const GradArgs& g, int pair, float shd, float Sd, float sht,
                                            float St, float L1, float S, int32_t V) {
  const int k = pair % g.gamma + 1, b = pair / g.gamma;
  const bool m = g.block_mask ? g.block_mask[b] != 0 : true;
  const float sc = g.scale ? *g.scale : 1.0f;
  const float alpha = m ? sc * expf(-static_cast<float>(k) / static_cast<float>(g.gamma)) : 0.0f;
  const float a = fminf(1.0f, fmaxf(0.0f, 1.0f - 0.5f * L1));
  const float c = g.conf_logits[pair];
  g.grad_conf[pair] = alpha * g.w_conf * (1.0f / (1.0f + expf(-c)) - a);
  // log2 P_v - log2 T_v = (x - y) log2e - [(shd + log2 Sd) - (sht + log2 St)]
  const float lr = (shd + __log2f(Sd)) - (sht + __log2f(St));
  return GradRow{shd, 1.0f / Sd, lr, S, alpha * g.w_ce, alpha * g.w_l1, clamp_token(g.teacher[pair], V)};
}

__device__ __forceinline__ void l1_and_s(float x, float y, float shd, float isd, float sht, float ist,
                                         float& l1, float& s) {
  const float P = __builtin_amdgcn_exp2f(fmaf(x, kLog2e, -shd)) * isd;
  const float T = __builtin_amdgcn_exp2f(fmaf(y, kLog2e, -sht)) * ist;
  l1 += fabsf(P - T);
  s += P > T ? P : (P < T ? -P : 0.0f);
}

__device__ __forceinline__ float grad_elem(const GradRow& r, float x, float y, int v) {
  const float P = __builtin_amdgcn_exp2f(fmaf(x, kLog2e, -r.shd)) * r.isd;
  const float dl = fmaf(x - y, kLog2e, -r.lr);  // NaN (both -inf: P = 0) gives sign 0
  const float sg = dl > 0.0f ? 1.0f : (dl < 0.0f ? -1.0f : 0.0f);
  return r.a_ce * (P - (v == r.teacher ? 1.0f : 0.0f)) + r.a_l1 * P * (sg - r.S);
}

// Sliced second look: per item the pair's normalisers (its part1 records)
// and the item's shares of L1 and S; the pair's last item (ticket) sums the
// shares in a fixed order and stores the pair's GradRow.
template <typename T>
__global__ __launch_bounds__(kThreads) void stats_grad_part2_kernel(
    const T* __restrict__ draft, const T* __restrict__ target, int32_t V, int32_t P, int32_t items,
    const StatPart* __restrict__ part, float* __restrict__ l1part, float* __restrict__ spart,
    GradArgs o) {
  constexpr int EPL = 16 / sizeof(T);
  constexpr int SEG = stat_seg<T>();
  const int lane = threadIdx.x & 63;
  const int nwaves = gridDim.x * kWaves;
  for (int item = static_cast<int>(blockIdx.x) * kWaves + (threadIdx.x >> 6); item < items;
       item += nwaves) {
    const int it_ = __builtin_amdgcn_readfirstlane(item);
    const int pair = it_ / P, seg = it_ - pair * P;
    uint4 ud[kSegIters], ut[kSegIters];
    seg_load<T>(draft, target, V, P, it_, lane, ud, ut);
    float M2d, Sd, M2t, St;
    pair_norm(part + static_cast<size_t>(pair) * P, P, lane, M2d, Sd, M2t, St);
    seg_mask<T>(V, seg * SEG, lane, ud, ut);
    const float isd = 1.0f / Sd, ist = 1.0f / St;
    float l1 = 0.0f, sv = 0.0f;
#pragma unroll
    for (int it = 0; it < kSegIters; ++it)
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        l1_and_s(elem16(ud[it], j, T{}), elem16(ut[it], j, T{}), M2d, isd, M2t, ist, l1, sv);
    l1 = wave_sum(l1);
    sv = wave_sum(sv);
    uint32_t ticket = 0;
    if (lane == 0) {
      store_coherent(l1part + it_, l1);
      store_coherent(spart + it_, sv);
      ticket = publish(o.counters + static_cast<size_t>(pair) * kTicketStride);
    }
    ticket = __builtin_amdgcn_readfirstlane(ticket);
    if (ticket != static_cast<uint32_t>(P - 1)) continue;
    float L1 = 0.0f, S = 0.0f;
    for (int i = lane; i < P; i += 64) {
      L1 += load_coherent(l1part + static_cast<size_t>(pair) * P + i);
      S += load_coherent(spart + static_cast<size_t>(pair) * P + i);
    }
    L1 = wave_sum(L1);
    S = wave_sum(S);
    if (lane == 0) o.rows[pair] = grad_row(o, pair, M2d, Sd, M2t, St, L1, S, V);
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

// Sliced third look: per item the gradient of its segment (the next item's
// loads in flight while the current one is computed and stored).
template <typename T>
__global__ __launch_bounds__(kThreads) void stats_grad_write_kernel(
    const T* __restrict__ draft, const T* __restrict__ target, int32_t V, int32_t P, int32_t items,
    const GradRow* __restrict__ rows, T* __restrict__ grad) {
  constexpr int EPL = 16 / sizeof(T);
  constexpr int SEG = stat_seg<T>();
  const int lane = threadIdx.x & 63;
  const int nwaves = gridDim.x * kWaves;
  int item = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * kWaves + (threadIdx.x >> 6));
  if (item >= items) return;
  uint4 ad[kSegIters], at[kSegIters], bd[kSegIters], bt[kSegIters];
  auto write = [&](const uint4* ud, const uint4* ut, int it_) {
    const int pair = it_ / P, seg = it_ - pair * P;
    const GradRow r = rows[pair];
    const size_t off = static_cast<size_t>(pair) * V;
#pragma unroll
    for (int it = 0; it < kSegIters; ++it) {
      const int e = seg * SEG + (it * 64 + lane) * EPL;
      if (e >= V) continue;  // a clamped load past the row
      float g[EPL];
#pragma unroll
      for (int j = 0; j < EPL; ++j) g[j] = grad_elem(r, elem16(ud[it], j, T{}), elem16(ut[it], j, T{}), e + j);
      store16<T>(grad + off + e, g);
    }
  };
  seg_load<T>(draft, target, V, P, item, lane, ad, at);
  while (true) {
    const int n1 = __builtin_amdgcn_readfirstlane(item + nwaves);
    seg_load<T>(draft, target, V, P, n1 < items ? n1 : item, lane, bd, bt);
    write(ad, at, item);
    if (n1 >= items) break;
    const int n2 = __builtin_amdgcn_readfirstlane(n1 + nwaves);
    seg_load<T>(draft, target, V, P, n2 < items ? n2 : n1, lane, ad, at);
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
  using L = Vec8<T, VEC>;
  constexpr int EPL = L::N;
  constexpr int kWaves = kRowWaves;
  __shared__ float shv[kWaves];
  __shared__ GradRow shr;
  const int step = kRowThreads * EPL;
  for (int rr = blockIdx.x; rr < npairs; rr += gridDim.x) {
    const size_t row = static_cast<size_t>(rr);
    const T* dr = draft + row * V;
    const T* tr = target + row * V;
    T* gr = grad + row * V;

    float md = neg_inf(), sd = 0.0f, mt = neg_inf(), st = 0.0f;
    int e = threadIdx.x * EPL;
    for (; e + (kUnroll - 1) * step < V; e += kUnroll * step) {
      float xd[kUnroll][EPL], xt[kUnroll][EPL];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        L::load(dr + e + u * step, xd[u]);
        L::load(tr + e + u * step, xt[u]);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        online(md, sd, xd[u], EPL);
        online(mt, st, xt[u], EPL);
      }
    }
    for (; e < V; e += step) {
      float xd[EPL], xt[EPL];
      L::load(dr + e, xd);
      L::load(tr + e, xt);
      online(md, sd, xd, EPL);
      online(mt, st, xt, EPL);
    }
    const float Md = block_max<kWaves>(md, shv);
    const float Sd = block_sum<kWaves>(md > neg_inf() ? sd * __builtin_amdgcn_exp2f((md - Md) * kLog2e) : 0.0f, shv);
    const float Mt = block_max<kWaves>(mt, shv);
    const float St = block_sum<kWaves>(mt > neg_inf() ? st * __builtin_amdgcn_exp2f((mt - Mt) * kLog2e) : 0.0f, shv);
    const float shd = Md > neg_inf() ? Md * kLog2e : 0.0f, sht = Mt > neg_inf() ? Mt * kLog2e : 0.0f;
    const float isd = 1.0f / Sd, ist = 1.0f / St;

    float l1 = 0.0f, sv = 0.0f;
    e = threadIdx.x * EPL;
    for (; e + (kUnroll - 1) * step < V; e += kUnroll * step) {
      float xd[kUnroll][EPL], xt[kUnroll][EPL];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        L::load(dr + e + u * step, xd[u]);
        L::load(tr + e + u * step, xt[u]);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int j = 0; j < EPL; ++j) l1_and_s(xd[u][j], xt[u][j], shd, isd, sht, ist, l1, sv);
    }
    for (; e < V; e += step) {
      float xd[EPL], xt[EPL];
      L::load(dr + e, xd);
      L::load(tr + e, xt);
#pragma unroll
      for (int j = 0; j < EPL; ++j) l1_and_s(xd[j], xt[j], shd, isd, sht, ist, l1, sv);
    }
    const float L1 = block_sum<kWaves>(l1, shv);
    const float S = block_sum<kWaves>(sv, shv);
    if (threadIdx.x == 0) shr = grad_row(o, static_cast<int>(row), shd, Sd, sht, St, L1, S, V);
    __syncthreads();
    const GradRow r = shr;

    e = threadIdx.x * EPL;
    for (; e + (kUnroll - 1) * step < V; e += kUnroll * step) {
      float xd[kUnroll][EPL], xt[kUnroll][EPL];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        L::load(dr + e + u * step, xd[u]);
        L::load(tr + e + u * step, xt[u]);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float g[EPL];
#pragma unroll
        for (int j = 0; j < EPL; ++j) g[j] = grad_elem(r, xd[u][j], xt[u][j], e + u * step + j);
        if constexpr (VEC) {
          store16<T>(gr + e + u * step, g);
        } else {
          if constexpr (sizeof(T) == 2) gr[e + u * step] = bf16_rne(g[0]);
          else gr[e + u * step] = g[0];
        }
      }
    }
    for (; e < V; e += step) {
      float xd[EPL], xt[EPL], g[EPL];
      L::load(dr + e, xd);
      L::load(tr + e, xt);
#pragma unroll
      for (int j = 0; j < EPL; ++j) g[j] = grad_elem(r, xd[j], xt[j], e + j);
      if constexpr (VEC) {
        store16<T>(gr + e, g);
      } else {
        if constexpr (sizeof(T) == 2) gr[e] = bf16_rne(g[0]);
        else gr[e] = g[0];
      }
    }
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

template <typename T>
hipError_t launch_typed(const T* draft, const T* target, const int32_t* teacher,
                        const float* conf_logits, const uint8_t* block_mask, int32_t N,
                        int32_t gamma, int32_t V, float w_ce, float w_l1, float w_conf, float* l1,
                        float* accept_rate, float* ce, float* bce, float* tau, float* sums,
                        void* ws, const StatsPlan& pl, hipStream_t st) {
  const int epl = sizeof(T) == 2 ? 8 : 4;
  const bool vec = (V % epl == 0) && reinterpret_cast<uintptr_t>(draft) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(target) % 16 == 0;
  const int npairs = N * gamma;
  if (npairs > 0 && vec && pl.sliced) {
    char* w = static_cast<char*>(ws);
    StatPart* part = reinterpret_cast<StatPart*>(w + pl.off_part);
    float* l1part = reinterpret_cast<float*>(w + pl.off_l1);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(w + pl.off_cnt);
    const int items = npairs * pl.P;
    const int wgs = std::min(kItemMaxWGs, (items + kWaves - 1) / kWaves);
    DSPARK_LAUNCH("stats_part1", (stats_part1_kernel<T>), dim3(wgs), dim3(kThreads), 0, st, draft,
                  target, V, pl.P, items, part, cnt, npairs + 1);
    const StatsOut o{teacher, conf_logits, block_mask, N, gamma, w_ce, w_l1, w_conf,
                     l1, accept_rate, ce, bce, tau, sums, cnt};
    DSPARK_LAUNCH("stats_part2", (stats_part2_kernel<T>), dim3(wgs), dim3(kThreads), 0, st, draft,
                  target, V, pl.P, items, part, l1part, o);
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
    StatPart* part = reinterpret_cast<StatPart*>(w + pl.off_part);
    float* l1part = reinterpret_cast<float*>(w + pl.off_l1);
    float* spart = reinterpret_cast<float*>(w + pl.off_s);
    o.rows = reinterpret_cast<GradRow*>(w + pl.off_rows);
    o.counters = reinterpret_cast<uint32_t*>(w + pl.off_cnt);
    const int items = npairs * pl.P;
    const int wgs = std::min(kItemMaxWGs, (items + kWaves - 1) / kWaves);
    DSPARK_LAUNCH("stats_part1", (stats_part1_kernel<T>), dim3(wgs), dim3(kThreads), 0, st, draft,
                  target, V, pl.P, items, part, o.counters, npairs);
    DSPARK_LAUNCH("stats_grad_part2", (stats_grad_part2_kernel<T>), dim3(wgs), dim3(kThreads), 0, st,
                  draft, target, V, pl.P, items, part, l1part, spart, o);
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
    off = align_up(off + items * sizeof(StatPart), 256);
    p.off_l1 = off;
    off = align_up(off + items * sizeof(float), 256);
    p.off_s = off;
    off = align_up(off + items * sizeof(float), 256);
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
    off = align_up(off + items * sizeof(StatPart), 256);
    p.off_l1 = off;
    off = align_up(off + items * sizeof(float), 256);
    p.off_cnt = off;
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
