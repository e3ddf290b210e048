// verify.hip — exact verify of DSpark proposals on gfx950.
//
// Semantics ("[2/3] feat(dsv4): implement exact DSpark speculative decoding",
// section "Exact decoding semantics"): greedy requests accept the contiguous
// prefix of proposals equal to the target argmax and emit the target token at
// the first disagreement; sampled requests accept x_k with probability
// min(1, p(x_k) / q(x_k)), draw the first rejected position from normalised
// max(p - q, 0), and draw a bonus token from the next-position target
// distribution when every proposal survives.  Target row k - 1 verifies x_k.
//
// Two launches:
//  1. verify_rows   grid-stride over (target row, 2048-token segment) items,
//     one wave per item: 16-byte loads into registers, reduced to (max, lowest
//     argmax, sum) with DPP only (no LDS, no barrier); the next item's loads
//     are in flight while the current one is reduced.
//  2. verify_decide grid (chunk slices, B).  Every workgroup of a request
//     combines the segment partials of its rows (all records loaded at once)
//     and replays the accept scan (one thread per proposal, first reject by
//     ballot), so all of them agree on the row to sample from.  Each then
//     scores its slice of 256-token chunks (level 1 of the library's
//     three-level Gumbel-max draw); the last workgroup to finish (atomic
//     ticket, armed by launch 1) picks the chunk, then the 16-token sub-chunk
//     and the token inside it (levels 2 and 3), and writes the outputs.
//
// Sums use an integer base-2 shift: s = sum 2^(l cT - M2), cT = log2(e) / T,
// M2 = floor(max(l) cT).  Partials with different shifts combine by exact
// powers of two, and p(x) = 2^(l_x cT - M2) / s uses the very expression each
// term of s used.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"
#include "truncate.hpp"

namespace dspark {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kVecIters = 4;       // 16-byte loads per lane per segment
constexpr int kScalarIters = 32;   // scalar loads per lane per segment
constexpr int kChunksPerWave = 8;  // chunks one wave scores in the decide pass
constexpr int kChunksPerWG = kChunksPerWave * kWaves;
constexpr int kRowsMaxWGs = 4096;  // grid of the row pass: up to 16 waves per SIMD
constexpr int kRowsPerWave = (DSPARK_MAX_GAMMA + 1 + kWaves - 1) / kWaves;  // decide: rows a wave combines
constexpr int kPartRegs = 2;  // decide: segment records per lane and row held in registers

// One 16-byte load per lane per iteration (vector path: 8 bf16 or 4 fp32
// logits kept packed in a uint4), or one scalar logit (scalar path).  Lanes
// past the row end hold -inf.
template <typename T, bool VEC>
struct RowLoad;

template <typename T>
struct RowLoad<T, true> {
  using Raw = uint4;
  static constexpr int EPL = 16 / sizeof(T);
  static constexpr uint32_t kNegInfBits = sizeof(T) == 2 ? 0xFF80FF80u : 0xFF800000u;
  __device__ static Raw load(const T* row, int e) { return *reinterpret_cast<const uint4*>(row + e); }
  __device__ static Raw neg() { return make_uint4(kNegInfBits, kNegInfBits, kNegInfBits, kNegInfBits); }
};

template <typename T>
struct RowLoad<T, false> {
  using Raw = float;
  static constexpr int EPL = 1;
  __device__ static Raw load(const T* row, int e) { return load_logit(row, e); }
  __device__ static Raw neg() { return neg_inf(); }
};

// element j of a packed vector
__device__ __forceinline__ float elem(const uint4& u, int j, uint16_t) {
  const uint32_t w = (j >> 1) == 0 ? u.x : (j >> 1) == 1 ? u.y : (j >> 1) == 2 ? u.z : u.w;
  return (j & 1) ? bf_hi(w) : bf_lo(w);
}
__device__ __forceinline__ float elem(const uint4& u, int j, float) {
  return __uint_as_float(j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w);
}
__device__ __forceinline__ float elem(float x, int, uint16_t) { return x; }
__device__ __forceinline__ float elem(float x, int, float) { return x; }

template <typename T, bool VEC>
constexpr int seg_len() {
  return (VEC ? kVecIters : kScalarIters) * 64 * RowLoad<T, VEC>::EPL;
}

__device__ __forceinline__ int32_t n_draft_of(const int32_t* n_draft, int b, int gamma) {
  int nd = n_draft ? n_draft[b] : gamma;
  return nd < 0 ? 0 : (nd > gamma ? gamma : nd);
}

// integer base-2 shift of a row (or segment) whose largest logit is m
__device__ __forceinline__ float shift_of(float m, float cT) { return floorf(m * cT); }

// ---------------------------------------------------------------------------
// Pass 1: per (row, segment) max, lowest argmax and sum 2^(l cT - M2).
// Grid-stride over (row, segment) items, one item per wave at a time; the
// next item's loads are issued before the current item is reduced, so memory
// and arithmetic overlap within every wave.
template <typename T, bool VEC>
__device__ __forceinline__ void rows_load(const T* __restrict__ target, int32_t V, int32_t P,
                                          int item, int lane, typename RowLoad<T, VEC>::Raw* u) {
  using L = RowLoad<T, VEC>;
  constexpr int ITERS = VEC ? kVecIters : kScalarIters;
  constexpr int EPL = L::EPL;
  constexpr int SEG = seg_len<T, VEC>();
  const int row = item / P, seg = item - row * P;
  const T* rp = target + static_cast<size_t>(row) * V;
  const int lo = seg * SEG;
  // every load is issued; past the row end the address is clamped to the
  // row's last vector and rows_reduce masks those elements
#pragma unroll
  for (int it = 0; it < ITERS; ++it)
    u[it] = L::load(rp, min(lo + (it * 64 + lane) * EPL, V - EPL));
}

// Per 256-token chunk maxima of one segment (vector paths only: a chunk is
// 32 lanes x 8 bf16 or 64 lanes x 4 fp32 of one load iteration).
template <typename T, bool VEC>
__device__ __forceinline__ void rows_chunk_max(const typename RowLoad<T, VEC>::Raw* u, int lo,
                                               int V, int C, int lane, float* __restrict__ cmax) {
  if constexpr (VEC) {
    constexpr int ITERS = kVecIters;
    constexpr int EPL = RowLoad<T, VEC>::EPL;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      float m = neg_inf();
#pragma unroll
      for (int e = 0; e < EPL; ++e) m = fmaxf(m, elem(u[it], e, T{}));
      m = fmaxf(m, dpp_f<kDppXor1>(m));
      m = fmaxf(m, dpp_f<kDppXor2>(m));
      m = fmaxf(m, dpp_f<kDppHalfMirror>(m));
      m = fmaxf(m, dpp_f<kDppMirror>(m));
      const float r0 = lane_f(m, 0), r1 = lane_f(m, 16), r2 = lane_f(m, 32), r3 = lane_f(m, 48);
      if (lane == 0) {
        const int c0 = (lo + it * 64 * EPL) >> 8;  // first chunk of this iteration
        if (EPL == 8) {
          if (c0 < C) cmax[c0] = fmaxf(r0, r1);
          if (c0 + 1 < C) cmax[c0 + 1] = fmaxf(r2, r3);
        } else {
          if (c0 < C) cmax[c0] = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
        }
      }
    }
  }
}

template <typename T, bool VEC>
__device__ __forceinline__ void rows_reduce(typename RowLoad<T, VEC>::Raw* u, int item,
                                            int32_t P, int32_t G1, int32_t vlen, int lane,
                                            const uint8_t* __restrict__ mode,
                                            const float* __restrict__ temperature,
                                            const int32_t* __restrict__ top_k,
                                            const float* __restrict__ top_p,
                                            float* __restrict__ cmax, RowPart* __restrict__ part) {
  using L = RowLoad<T, VEC>;
  constexpr int ITERS = VEC ? kVecIters : kScalarIters;
  constexpr int EPL = L::EPL;
  constexpr int SEG = seg_len<T, VEC>();
  const int row = item / P, seg = item - row * P;
  const int b = row / G1;
  const int lo = seg * SEG;
  const int V = vlen;
  if (V - lo < SEG) {  // partial segment (wave-uniform): mask the clamped loads
#pragma unroll
    for (int it = 0; it < ITERS; ++it)
      if (lo + (it * 64 + lane) * EPL >= V) u[it] = L::neg();
  }
  const float Tb = temperature[b];
  const bool sampled = load_u8_word(mode, b) != 0 && !bad_temperature(Tb);
  uint32_t fl = 0;
  float m = neg_inf();
  int32_t arg = INT32_MAX;
  float sum = 0.0f;
  if (!sampled) {
    uint32_t nan = 0;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float x = elem(u[it], e, T{});
        if (x > m) {
          m = x;
          arg = lo + (it * 64 + lane) * EPL + e;
        }
        nan |= (x != x) ? 1u : 0u;
      }
    }
    const ArgMax am = wave_argmax(ArgMax{m, arg});
    m = am.v;
    arg = am.i;
    if (wave_or(nan) || m == pos_inf()) fl |= DSPARK_FLAG_NONFINITE;
  } else {
#pragma unroll
    for (int it = 0; it < ITERS; ++it)
#pragma unroll
      for (int e = 0; e < EPL; ++e) m = fmaxf(m, elem(u[it], e, T{}));
    m = wave_max(m);
    if (m > neg_inf()) {
      const float cT = kLog2e / Tb;
      const float M2 = shift_of(m, cT);
#pragma unroll
      for (int it = 0; it < ITERS; ++it)
#pragma unroll
        for (int e = 0; e < EPL; ++e)
          sum += __builtin_amdgcn_exp2f(fmaf(elem(u[it], e, T{}), cT, -M2));
      sum = wave_sum(sum);
    }
    if (m == pos_inf() || !(sum < pos_inf())) fl |= DSPARK_FLAG_NONFINITE;
    if (truncated(top_k_of(top_k, b), top_p_of(top_p, b), V)) {
      const int C = (V + kChunk - 1) / kChunk;
      rows_chunk_max<T, VEC>(u, lo, V, C, lane, cmax + static_cast<size_t>(row) * C);
    }
  }
  if (lane == 0) part[static_cast<size_t>(row) * P + seg] = RowPart{m, sum, arg, fl};
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void verify_rows_kernel(
    const T* __restrict__ target, int32_t V, int32_t gamma, int32_t P, int32_t items,
    const uint8_t* __restrict__ mode, const float* __restrict__ temperature,
    const int32_t* __restrict__ top_k, const float* __restrict__ top_p,
    const int32_t* __restrict__ n_draft, RowPart* __restrict__ part, float* __restrict__ cmax,
    uint32_t* __restrict__ counters, int32_t B) {
  using L = RowLoad<T, VEC>;
  constexpr int ITERS = VEC ? kVecIters : kScalarIters;
  const int G1 = gamma + 1;
  const int lane = threadIdx.x & 63;
  // arm the per-request tickets of the decide pass (which starts after this
  // launch completes on the same stream)
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < B; i += kThreads) counters[i * kTicketStride] = 0u;
  const int nwaves = gridDim.x * kWaves;
  // next item at or after i whose row the decision can consult (rows past
  // n_draft are skipped); returns `items` when there is none
  auto next_live = [&](int i) {
    for (; i < items; i += nwaves) {
      const int row = i / P;
      const int b = row / G1, k = row - b * G1;
      if (k <= n_draft_of(n_draft, b, gamma)) break;
    }
    return i;
  };
  // the item index is wave-uniform: keep it (and every address derived from
  // it) in scalar registers, so per-request scalars come through the scalar
  // cache and never wait behind the vector loads in flight
  int item = next_live(
      __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * kWaves + (threadIdx.x >> 6)));
  if (item >= items) return;  // wave-uniform
  // two register buffers used alternately; the prefetch is unconditional (an
  // exhausted wave re-reads its last item), so the compiler can wait for
  // exactly the older buffer's loads
  typename L::Raw ua[ITERS], ub[ITERS];
  rows_load<T, VEC>(target, V, P, item, lane, ua);
  while (true) {
    const int n1 = __builtin_amdgcn_readfirstlane(next_live(item + nwaves));
    rows_load<T, VEC>(target, V, P, n1 < items ? n1 : item, lane, ub);
    rows_reduce<T, VEC>(ua, item, P, G1, V, lane, mode, temperature, top_k, top_p, cmax, part);
    if (n1 >= items) break;
    const int n2 = __builtin_amdgcn_readfirstlane(next_live(n1 + nwaves));
    rows_load<T, VEC>(target, V, P, n2 < items ? n2 : n1, lane, ua);
    rows_reduce<T, VEC>(ub, n1, P, G1, V, lane, mode, temperature, top_k, top_p, cmax, part);
    if (n2 >= items) break;
    item = n2;
  }
}

// ---------------------------------------------------------------------------
// Truncation pass: one workgroup per target row of a sampled request whose
// policy has top-k or top-p; every other workgroup returns at once.  Finds the
// smallest kept logit and the kept weight sum 2^(l cT - M2) (same shift M2 as
// the row pass) by radix selection.
template <typename T>
struct LogitRow {
  __amdgpu_buffer_rsrc_t rs;  // over the row (reads past it return 0)
  int V;
  bool vec4;  // 4 consecutive logits per aligned load
  __device__ LogitRow(const T* p, int V_, bool vec) : V(V_), vec4(vec) {
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(p), static_cast<short>(0),
                                           V_ * static_cast<int>(sizeof(T)), kBufferWord3);
  }
  __device__ float one(int v) const {
    if constexpr (sizeof(T) == 2)
      return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(rs, v * 2, 0, 0)) << 16);
    else
      return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, v * 4, 0, 0));
  }
  // four logits in one load (v0 a multiple of 4, the row aligned)
  __device__ void load4u(int v0, float* o) const {
    if constexpr (sizeof(T) == 2) {
      const uint2 u = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, v0 * 2, 0, 0));
      o[0] = bf_lo(u.x);
      o[1] = bf_hi(u.x);
      o[2] = bf_lo(u.y);
      o[3] = bf_hi(u.y);
    } else {
      const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(rs, v0 * 4, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = __uint_as_float(u[e]);
    }
  }
  __device__ void load4(int v0, float* o) const {
    if (vec4 && v0 + 3 < V) {
      load4u(v0, o);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = v0 + e < V ? one(v0 + e) : neg_inf();
    }
  }
};

// Workgroup w of the select grid takes the w-th row of an order that starts
// the slowest cuts first: the rows of sampled requests with top-p alone (a
// spread row takes the weight histogram), then of sampled requests with
// top-k, then the rest (which return at once); requests keep their order
// within a class.  All threads call it; returns the row.
template <int NT>
__device__ __forceinline__ int slow_first_row(int w, int B, int G1, int V, const uint8_t* __restrict__ mode,
                                              const float* __restrict__ temperature,
                                              const int32_t* __restrict__ top_k, const float* __restrict__ top_p,
                                              int* sh) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto cls = [&](int b) {
    if (mode[b] == 0 || bad_temperature(temperature[b])) return 2;
    const int tk = top_k_of(top_k, b);
    if (!truncated(tk, top_p_of(top_p, b), V)) return 2;
    return (tk > 0 && tk < V) ? 1 : 0;
  };
  const int per = (B + NT - 1) / NT, lo = min(B, tid * per), hi = min(B, lo + per);
  int cnt[3] = {0, 0, 0};
  for (int b = lo; b < hi; ++b) ++cnt[cls(b)];
  // class totals
  int n0 = wave_sum_i(cnt[0]), n1 = wave_sum_i(cnt[1]);
  if (lane == 0) {
    sh[wave] = n0;
    sh[NW + wave] = n1;
  }
  __syncthreads();
  n0 = 0;
  n1 = 0;
  for (int i = 0; i < NW; ++i) {
    n0 += sh[i];
    n1 += sh[NW + i];
  }
  __syncthreads();
  const int r = w / G1, k = w - r * G1;
  const int c = r < n0 ? 0 : (r < n0 + n1 ? 1 : 2);
  const int rank = r - (c >= 1 ? n0 : 0) - (c == 2 ? n1 : 0);
  // the rank-th request of class c: exclusive scan of the threads' counts
  const int own = cnt[c];
  int x = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int before = x - own;
  for (int i = 0; i < wave; ++i) before += sh[i];
  if (rank >= before && rank < before + own) {
    int seen = before;
    for (int b = lo; b < hi; ++b)
      if (cls(b) == c && seen++ == rank) sh[2 * NW] = b;
  }
  __syncthreads();
  const int b = sh[2 * NW];
  __syncthreads();
  return b * G1 + k;
}

template <typename T>
__global__ __launch_bounds__(kSelThreads) void verify_select_kernel(
    const T* __restrict__ target, int32_t V, int32_t gamma, int32_t P, int32_t have_cmax,
    const uint8_t* __restrict__ mode, const float* __restrict__ temperature,
    const int32_t* __restrict__ top_k, const float* __restrict__ top_p,
    const int32_t* __restrict__ n_draft, const RowPart* __restrict__ part,
    const float* __restrict__ cmax, RowTrunc* __restrict__ trunc) {
  __shared__ TruncLds<kSelThreads> U;
  __shared__ float cms[kMaxChunksBound];
  __shared__ float sh_m[kSelThreads / 64], sh_s[kSelThreads / 64];
  __shared__ int sh_o[2 * (kSelThreads / 64) + 1];
  const int G1 = gamma + 1;
  const int B = static_cast<int>(gridDim.x) / G1;
  const int row = slow_first_row<kSelThreads>(blockIdx.x, B, G1, V, mode, temperature, top_k, top_p, sh_o);
  const int b = row / G1, k = row - b * G1;
  const float Tb = temperature[b];
  const bool sampled = mode[b] != 0 && !bad_temperature(Tb);
  const int tk_raw = top_k_of(top_k, b);
  const float tp = top_p_of(top_p, b);
  if (!sampled || !truncated(tk_raw, tp, V) || k > n_draft_of(n_draft, b, gamma)) return;
  const int tk = (tk_raw > 0 && tk_raw < V) ? tk_raw : 0;
  // row maximum, its base-2 shift and the total weight, from the row pass
  const float cT = kLog2e / Tb;
  float m = neg_inf();
  for (int i = threadIdx.x; i < P; i += kSelThreads)
    m = fmaxf(m, part[static_cast<size_t>(row) * P + i].m);
  m = block_max<kSelThreads / 64>(m, sh_m);
  const float M2 = (m > neg_inf() && m < pos_inf()) ? shift_of(m, cT) : 0.0f;
  float s = 0.0f;
  for (int i = threadIdx.x; i < P; i += kSelThreads) {
    const RowPart q = part[static_cast<size_t>(row) * P + i];
    if (q.m > neg_inf()) s += q.s * __builtin_amdgcn_exp2f(shift_of(q.m, cT) - M2);
  }
  const float total = block_sum<kSelThreads / 64>(s, sh_s);
  const T* rp = target + static_cast<size_t>(row) * V;
  const LogitRow<T> lr(rp, V, (V % 4 == 0) && reinterpret_cast<uintptr_t>(target) % 16 == 0);
  const int C = (V + kChunk - 1) / kChunk;
  bool done = false;
  if (have_cmax && C <= kMaxChunksBound) {
    // candidates under the chunk-maxima bound; else, for top-p alone, the
    // weight histogram
    const float* cm = cmax + static_cast<size_t>(row) * C;
    for (int c = threadIdx.x; c < C; c += kSelThreads) cms[c] = cm[c];
    __syncthreads();
    if (chunk_bound(cms, C, tk, tp, cT, -M2, total, U.c)) {
      gather_candidates(lr, V, U.c);
      exact_cut(tk, tp, cT, -M2, total, U.c);
      if (U.c.ok) {
        if (threadIdx.x == 0) trunc[row] = RowTrunc{U.c.thr, U.c.s_kept};
        done = true;
      }
    }
    if (!done && tk == 0 && hist_cut<kSelThreads, false>(lr, V, cms, C, m, total, cT, -M2, tp, U.h)) {
      if (threadIdx.x == 0) trunc[row] = RowTrunc{U.h.thr, U.h.s_kept};
      done = true;
    }
  }
  if (!done) {  // radix selection over the whole row
    const SelResult r = select_threshold(lr, V, sizeof(T) == 2 ? 16 : 32, tk, tp, cT, -M2, U.s);
    if (threadIdx.x == 0) trunc[row] = RowTrunc{r.thr, static_cast<float>(r.s_kept)};
  }
}

// ---------------------------------------------------------------------------
// Pass 2: decision, chunk scores of the residual / bonus draw, final pick.
struct Decision {
  int kind;       // 0 greedy, 1 residual at j, 2 bonus
  int n;          // accepted proposals
  int srow;       // target row sampled from (kind 1, 2)
  uint32_t near;  // bit k: NEAR on target row k
  int32_t token;  // greedy: the emitted target token
};

__device__ __forceinline__ float draw_weight(int kind, float l, float zq, float cT, float M2,
                                             float inv_s, float lse_q, float thr_q, float thr_p) {
  if (!(l > neg_inf()) || !(l >= thr_p)) return 0.0f;
  const float e = __builtin_amdgcn_exp2f(fmaf(l, cT, -M2));
  if (kind != 1) return e;  // bonus / fallback: unnormalised p
  const float q =
      (zq >= thr_q && zq > neg_inf()) ? __builtin_amdgcn_exp2f((zq - lse_q) * kLog2e) : 0.0f;
  return fmaxf(e * inv_s - q, 0.0f);
}

// Four consecutive logits v0..v0+3 (v0 a multiple of 4) of a row, -inf past V.
template <typename T, bool VEC4>
__device__ __forceinline__ void load4(const T* row, int v0, int V, float* o) {
  if (VEC4 && v0 + 3 < V) {
    if constexpr (sizeof(T) == 2) {
      const uint2 u = *reinterpret_cast<const uint2*>(row + v0);
      o[0] = bf_lo(u.x);
      o[1] = bf_hi(u.x);
      o[2] = bf_lo(u.y);
      o[3] = bf_hi(u.y);
    } else {
      const float4 u = *reinterpret_cast<const float4*>(row + v0);
      o[0] = u.x;
      o[1] = u.y;
      o[2] = u.z;
      o[3] = u.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = v0 + e < V ? load_logit(row, v0 + e) : neg_inf();
  }
}

template <typename T, bool VEC4>
__global__ __launch_bounds__(kThreads) void verify_decide_kernel(
    const T* __restrict__ target, const int32_t* __restrict__ draft,
    const float* __restrict__ q_z, const float* __restrict__ q_lse,
    const float* __restrict__ q_thr, const float* __restrict__ q_tok,
    const int32_t* __restrict__ n_draft, const uint8_t* __restrict__ mode,
    const float* __restrict__ temperature, const int32_t* __restrict__ top_k,
    const float* __restrict__ top_p, const uint32_t* __restrict__ request_id,
    const int32_t* __restrict__ position, uint64_t seed, int32_t gamma, int32_t V, int32_t P,
    int32_t S2, const RowPart* __restrict__ part, const RowTrunc* __restrict__ trunc,
    Pick* __restrict__ picks,
    uint32_t* __restrict__ counters, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ out_tokens, uint8_t* __restrict__ flags) {
  __shared__ float rm[DSPARK_MAX_GAMMA + 1], rs[DSPARK_MAX_GAMMA + 1], rM2[DSPARK_MAX_GAMMA + 1],
      rthr[DSPARK_MAX_GAMMA + 1];
  __shared__ int32_t rarg[DSPARK_MAX_GAMMA + 1];
  __shared__ uint32_t rfl[DSPARK_MAX_GAMMA + 1];
  __shared__ Decision dec;
  __shared__ float shv[kWaves], shv2[kWaves];
  __shared__ int32_t shi[kWaves];
  __shared__ int sh_last;
  __shared__ Top2 sh_best;
  __shared__ int32_t sh_tok;
  __shared__ uint32_t sh_near;

  const int G1 = gamma + 1;
  const int b = blockIdx.y, s2 = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nd = n_draft_of(n_draft, b, gamma);
  const float Tb = temperature[b];
  const bool want_sampled = mode[b] != 0 && !bad_temperature(Tb);
  const bool sampled = want_sampled && q_z && q_lse && q_thr && q_tok;
  const float cT = sampled ? kLog2e / Tb : kLog2e;
  const int C = (V + kChunk - 1) / kChunk;
  const uint32_t req = request_id[b];
  const int32_t pos0 = position[b];
  const bool trunc_row = sampled && truncated(top_k_of(top_k, b), top_p_of(top_p, b), V);

  // proposal-side values of the accept scan, fetched up front (thread k-1
  // owns proposal k)
  int32_t xk = 0;
  float lx = neg_inf(), qk = 0.0f;
  if (tid < nd) {
    xk = clamp_token(draft[b * gamma + tid], V);
    if (sampled) {
      lx = load_logit(target, static_cast<size_t>(b * G1 + tid) * V + xk);
      qk = q_tok[b * gamma + tid];
    }
  }

  // 1. combine the segment partials of rows 0..n_d (wave w: rows w, w+4, ...).
  // With at most 64 kPartRegs segments a row, every record of the wave's rows
  // is loaded before any is reduced; longer rows loop over their records.
  auto row_out = [&](int r, ArgMax am, uint32_t fl, float M2, float s) {
    if (lane == 0) {
      if (!(am.v > neg_inf())) fl |= DSPARK_FLAG_EMPTY_ROW;
      float thr = neg_inf();
      if (trunc_row) {  // kept set of the truncated policy
        const RowTrunc t = trunc[b * G1 + r];
        thr = t.thr;
        s = t.s_kept;
      }
      rthr[r] = thr;
      rm[r] = am.v;
      rs[r] = s;
      rM2[r] = M2;
      rarg[r] = am.i;
      rfl[r] = fl;
    }
  };
  if (P <= 64 * kPartRegs) {
    RowPart q[kRowsPerWave][kPartRegs];
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      const int r = wave + kWaves * j;
#pragma unroll
      for (int h = 0; h < kPartRegs; ++h) {
        const int i = lane + 64 * h;
        q[j][h] = (r <= nd && i < P) ? part[static_cast<size_t>(b * G1 + r) * P + i]
                                     : RowPart{neg_inf(), 0.0f, INT32_MAX, 0u};
      }
    }
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
      const int r = wave + kWaves * j;
      if (r > nd) break;
      ArgMax am{neg_inf(), INT32_MAX};
      uint32_t fl = 0;
#pragma unroll
      for (int h = 0; h < kPartRegs; ++h) {
        am = better(am, ArgMax{q[j][h].m, q[j][h].arg});
        fl |= q[j][h].flags;
      }
      am = wave_argmax(am);
      fl = wave_or(fl);
      const float M2 = (am.v > neg_inf() && am.v < pos_inf()) ? shift_of(am.v, cT) : 0.0f;
      float s = 0.0f;
      if (sampled && am.v > neg_inf()) {
#pragma unroll
        for (int h = 0; h < kPartRegs; ++h)
          if (q[j][h].m > neg_inf()) s += q[j][h].s * __builtin_amdgcn_exp2f(shift_of(q[j][h].m, cT) - M2);
        s = wave_sum(s);
      }
      row_out(r, am, fl, M2, s);
    }
  } else {
    for (int r = wave; r <= nd; r += kWaves) {
      const RowPart* p = part + static_cast<size_t>(b * G1 + r) * P;
      ArgMax am{neg_inf(), INT32_MAX};
      uint32_t fl = 0;
      for (int i = lane; i < P; i += 64) {
        const RowPart q = p[i];
        am = better(am, ArgMax{q.m, q.arg});
        fl |= q.flags;
      }
      am = wave_argmax(am);
      fl = wave_or(fl);
      const float M2 = (am.v > neg_inf() && am.v < pos_inf()) ? shift_of(am.v, cT) : 0.0f;
      float s = 0.0f;
      if (sampled && am.v > neg_inf()) {
        for (int i = lane; i < P; i += 64) {
          const RowPart q = p[i];
          if (q.m > neg_inf()) s += q.s * __builtin_amdgcn_exp2f(shift_of(q.m, cT) - M2);
        }
        s = wave_sum(s);
      }
      row_out(r, am, fl, M2, s);
    }
  }
  __syncthreads();

  // 2. the decision (identical in every workgroup of the request), in wave 0
  if (wave == 0) {
    bool stop = false, near = false;
    if (lane < nd) {
      if (!sampled) {
        const int32_t t = rarg[lane] == INT32_MAX ? 0 : rarg[lane];
        stop = xk != t;
      } else {
        const float s = rs[lane];
        const float p = (lx > neg_inf() && lx >= rthr[lane] && s > 0.0f)
                            ? __builtin_amdgcn_exp2f(fmaf(lx, cT, -rM2[lane])) / s
                            : 0.0f;
        const float u = accept_uniform(seed, pos0 + lane + 1, req);
        if (qk > 0.0f) {
          const float rho = p / qk;
          stop = !(u < rho);
          near = fabsf(u - rho) <= kNearEps;
        } else {
          stop = !(p > 0.0f);
        }
      }
    }
    const uint64_t stops = __ballot(stop);
    const uint64_t nears = __ballot(near);
    if (lane == 0) {
      Decision d{};
      const int j = stops ? __builtin_ctzll(stops) + 1 : 0;  // first reject, 1-based
      // only accept tests that were reached (proposals 1..j) can be NEAR
      const uint64_t reached = j ? ((1ull << j) - 1ull) : ~0ull;
      d.near = static_cast<uint32_t>(nears & reached);
      if (!sampled) {
        d.kind = 0;
        d.n = j ? j - 1 : nd;
        d.token = rarg[d.n] == INT32_MAX ? 0 : rarg[d.n];
        d.near = 0;
      } else if (j) {
        d.kind = 1;
        d.n = j - 1;
        d.srow = j - 1;
      } else {
        d.kind = 2;
        d.n = nd;
        d.srow = nd;
      }
      dec = d;
    }
  }
  __syncthreads();
  const Decision d = dec;

  // threads 0..G1-1 write one row each
  auto write_outputs = [&](int32_t emitted, uint32_t extra_row_flags, int extra_row) {
    const int i = tid;
    if (i >= G1) return;
    int32_t t = -1;
    if (i < d.n) t = clamp_token(draft[b * gamma + i], V);
    else if (i == d.n) t = emitted;
    out_tokens[static_cast<size_t>(b) * G1 + i] = t;
    uint32_t fl = 0;
    if (i <= nd) {
      fl = rfl[i] & (DSPARK_FLAG_NONFINITE | DSPARK_FLAG_EMPTY_ROW);
      if (d.near & (1u << i)) fl |= DSPARK_FLAG_NEAR_THRESHOLD;
      if (i == extra_row) fl |= extra_row_flags;
    }
    if (i == 0 && mode[b] != 0 && !sampled) fl |= DSPARK_FLAG_BAD_POLICY;
    flags[static_cast<size_t>(b) * G1 + i] = static_cast<uint8_t>(fl);
    if (i == 0) accept_len[b] = d.n;
  };

  if (d.kind == 0) {
    if (s2 == 0) write_outputs(d.token, 0, -1);
    return;
  }

  // 3. chunk scores of this workgroup's chunk slice
  const int32_t pos = pos0 + (d.kind == 1 ? d.n + 1 : nd + 1);
  const T* trow = target + static_cast<size_t>(b * G1 + d.srow) * V;
  const size_t qoff = static_cast<size_t>(b * gamma + d.srow) * V;  // q row j-1 (kind 1)
  const float M2 = rM2[d.srow];
  const float inv_s = rs[d.srow] > 0.0f ? 1.0f / rs[d.srow] : 0.0f;
  const float lse_q = d.kind == 1 ? q_lse[b * gamma + d.srow] : 0.0f;
  const float thr_q = d.kind == 1 ? q_thr[b * gamma + d.srow] : 0.0f;
  const float thr_p = rthr[d.srow];

  // wave-level best of chunks c0 + wave + 4 i (i < kChunksPerWave)
  auto wave_chunks = [&](int kind, int c0) -> Top2 {
    float l[kChunksPerWave][4], zq[kChunksPerWave][4];
#pragma unroll
    for (int i = 0; i < kChunksPerWave; ++i) {
      const int c = c0 + wave + kWaves * i;
      const int v0 = c * kChunk + lane * 4;
      if (c < C) {
        load4<T, VEC4>(trow, v0, V, l[i]);
        if (kind == 1) load4<float, VEC4>(q_z + qoff, v0, V, zq[i]);
        else
#pragma unroll
          for (int e = 0; e < 4; ++e) zq[i][e] = neg_inf();
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) l[i][e] = zq[i][e] = neg_inf();
      }
    }
    float mine = 0.0f;
#pragma unroll
    for (int i = 0; i < kChunksPerWave; ++i) {
      float w = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w += draw_weight(kind, l[i][e], zq[i][e], cT, M2, inv_s, lse_q, thr_q, thr_p);
      w = wave_sum(w);
      if (lane == i) mine = w;  // lane i scores chunk i of this wave
    }
    Top2 t{neg_inf(), INT32_MAX, neg_inf()};
    const int c = c0 + wave + kWaves * lane;
    if (lane < kChunksPerWave && c < C && mine > 0.0f)
      t = Top2{logf(mine) + gumbel(seed, static_cast<uint32_t>(c), pos, req,
                                   DSPARK_TAG_TARGET_CHUNK),
               c, neg_inf()};
    return wave_top2(t);
  };

  Top2 mine{neg_inf(), INT32_MAX, neg_inf()};
  {
    const Top2 w = wave_chunks(d.kind, s2 * kChunksPerWG);
    if (lane == 0) {
      shv[wave] = w.v1;
      shi[wave] = w.i1;
      shv2[wave] = w.v2;
    }
    __syncthreads();
    for (int i = 0; i < kWaves; ++i) mine = top2_merge(mine, Top2{shv[i], shi[i], shv2[i]});
  }
  if (tid == 0) {
    Pick* pk = picks + static_cast<size_t>(b) * S2 + s2;
    store_coherent(&pk->v1, mine.v1);
    store_coherent(&pk->i1, mine.i1);
    store_coherent(&pk->v2, mine.v2);
    const uint32_t prev = publish(&counters[b * kTicketStride]);
    sh_last = (prev == static_cast<uint32_t>(S2 - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!sh_last) return;

  // 4. last workgroup of the request: pick the chunk, then the token
  {
    Top2 t{neg_inf(), INT32_MAX, neg_inf()};
    for (int i = tid; i < S2; i += kThreads) {
      const Pick* pk = picks + static_cast<size_t>(b) * S2 + i;
      t = top2_merge(t, Top2{load_coherent(&pk->v1), load_coherent(&pk->i1), load_coherent(&pk->v2)});
    }
    t = block_top2<kWaves>(t, shv, shi, shv2);
    if (tid == 0) sh_best = t;
  }
  __syncthreads();
  Top2 best = sh_best;
  int kind = d.kind;
  uint32_t row_flags = 0;
  if (best.i1 == INT32_MAX && kind == 1) {
    // max(p - q, 0) has no mass (only reachable by rounding): draw from p
    kind = 3;
    row_flags |= DSPARK_FLAG_RESIDUAL_ZERO;
    Top2 t{neg_inf(), INT32_MAX, neg_inf()};
    for (int c0 = 0; c0 < C; c0 += kChunksPerWG) t = top2_merge(t, wave_chunks(3, c0));
    best = block_top2<kWaves>(t, shv, shi, shv2);
  }
  if (best.i1 != INT32_MAX && best.v2 > neg_inf() && near_gap(best.v1, best.v2))
    row_flags |= DSPARK_FLAG_NEAR_THRESHOLD;

  // levels 2 and 3 inside the chosen chunk, by wave 0 (lane l: tokens 4l..4l+3)
  if (wave == 0) {
    InChunk dr{-1, neg_inf(), false};
    if (best.i1 != INT32_MAX) {
      const int v0 = best.i1 * kChunk + 4 * lane;
      float l[4], zq[4], lw[4];
      load4<T, VEC4>(trow, v0, V, l);
      if (kind == 1) load4<float, VEC4>(q_z + qoff, v0, V, zq);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lw[e] = neg_inf();
        if (kind == 1) {
          const float w = draw_weight(1, l[e], zq[e], cT, M2, inv_s, lse_q, thr_q, thr_p);
          lw[e] = w > 0.0f ? logf(w) : neg_inf();
        } else if (l[e] > neg_inf() && l[e] >= thr_p) {
          lw[e] = (l[e] - rm[d.srow]) / Tb;
        }
      }
      dr = draw_in_chunk(lw, best.i1, seed, pos, req, DSPARK_TAG_TARGET_SUB, DSPARK_TAG_TARGET_TOKEN);
    }
    if (lane == 0) {
      sh_tok = dr.tok;
      sh_near = dr.near ? 1u : 0u;
    }
  }
  __syncthreads();
  if (sh_near) row_flags |= DSPARK_FLAG_NEAR_THRESHOLD;
  write_outputs(sh_tok < 0 ? 0 : sh_tok, row_flags, d.srow);
}

template <typename T>
hipError_t launch_typed(const T* target, const int32_t* draft, const float* q_z,
                        const float* q_lse, const float* q_thr, const float* q_tok,
                        const int32_t* n_draft, dspark_policy pol, uint64_t seed, int32_t B,
                        int32_t gamma, int32_t V, int32_t* accept_len, int32_t* out_tokens,
                        uint8_t* flags, void* ws, const VerifyPlan& pl, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  RowPart* part = reinterpret_cast<RowPart*>(w + pl.off_part);
  Pick* picks = reinterpret_cast<Pick*>(w + pl.off_pick);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(w + pl.off_cnt);
  const int items = B * (gamma + 1) * pl.S;
  const int wgs = std::min(kRowsMaxWGs, (items + kWaves - 1) / kWaves);
  float* cmax = reinterpret_cast<float*>(w + pl.off_cmax);
  if (pl.vec)
    DSPARK_LAUNCH("verify_rows", (verify_rows_kernel<T, true>), dim3(wgs), dim3(kThreads), 0, st,
                  target, V, gamma, pl.S, items, pol.mode, pol.temperature, pol.top_k, pol.top_p,
                  n_draft, part, cmax, cnt, B);
  else
    DSPARK_LAUNCH("verify_rows", (verify_rows_kernel<T, false>), dim3(wgs), dim3(kThreads), 0, st,
                  target, V, gamma, pl.S, items, pol.mode, pol.temperature, pol.top_k, pol.top_p,
                  n_draft, part, cmax, cnt, B);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  RowTrunc* trunc = reinterpret_cast<RowTrunc*>(w + pl.off_trunc);
  // truncation thresholds, unless the caller passed no truncation arrays (no
  // request truncates)
  if (pol.top_k || pol.top_p) {
    DSPARK_LAUNCH("verify_select", (verify_select_kernel<T>), dim3(B * (gamma + 1)),
                  dim3(kSelThreads), 0, st, target, V, gamma, pl.S, pl.vec, pol.mode,
                  pol.temperature, pol.top_k, pol.top_p, n_draft, part, cmax, trunc);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool vec4 = V % 4 == 0 && reinterpret_cast<uintptr_t>(target) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(q_z) % 16 == 0;
  if (vec4)
    DSPARK_LAUNCH("verify_decide", (verify_decide_kernel<T, true>), dim3(pl.S2, B),
                  dim3(kThreads), 0, st, target, draft, q_z, q_lse, q_thr, q_tok, n_draft,
                  pol.mode, pol.temperature, pol.top_k, pol.top_p, pol.request_id, pol.position,
                  seed, gamma, V, pl.S, pl.S2, part, trunc, picks, cnt, accept_len, out_tokens,
                  flags);
  else
    DSPARK_LAUNCH("verify_decide", (verify_decide_kernel<T, false>), dim3(pl.S2, B),
                  dim3(kThreads), 0, st, target, draft, q_z, q_lse, q_thr, q_tok, n_draft,
                  pol.mode, pol.temperature, pol.top_k, pol.top_p, pol.request_id, pol.position,
                  seed, gamma, V, pl.S, pl.S2, part, trunc, picks, cnt, accept_len, out_tokens,
                  flags);
  return hipGetLastError();
}

}  // namespace

VerifyPlan plan_verify(int dtype, int32_t B, int32_t gamma, int32_t V, bool aligned) {
  VerifyPlan p{};
  const bool bf = dtype == DSPARK_BF16;
  p.vec = (aligned && V % (bf ? 8 : 4) == 0) ? 1 : 0;
  p.slice_len = bf ? (p.vec ? seg_len<uint16_t, true>() : seg_len<uint16_t, false>())
                   : (p.vec ? seg_len<float, true>() : seg_len<float, false>());
  p.S = (V + p.slice_len - 1) / p.slice_len;  // row segments (one wave each)
  const int C = (V + kChunk - 1) / kChunk;
  p.cps = kChunksPerWG;
  p.S2 = (C + p.cps - 1) / p.cps;
  size_t off = 0;
  p.off_part = off;
  off = align_up(off + static_cast<size_t>(B) * (gamma + 1) * p.S * sizeof(RowPart), 256);
  p.off_pick = off;
  off = align_up(off + static_cast<size_t>(B) * p.S2 * sizeof(Pick), 256);
  p.off_cnt = off;
  off = align_up(off + static_cast<size_t>(B) * kTicketStride * sizeof(uint32_t), 256);
  p.off_trunc = off;
  off = align_up(off + static_cast<size_t>(B) * (gamma + 1) * sizeof(RowTrunc), 256);
  p.off_cmax = off;
  off = align_up(off + static_cast<size_t>(B) * (gamma + 1) * C * sizeof(float), 256);
  p.bytes = off;
  return p;
}

hipError_t launch_verify(const void* target, int dtype, const int32_t* draft, const float* q_z,
                         const float* q_lse, const float* q_thr, const float* q_tok,
                         const int32_t* n_draft, dspark_policy pol, uint64_t seed, int32_t B,
                         int32_t gamma, int32_t V, int32_t* accept_len, int32_t* out_tokens,
                         uint8_t* flags, void* ws, const VerifyPlan& plan, hipStream_t st) {
  if (dtype == DSPARK_BF16)
    return launch_typed(static_cast<const uint16_t*>(target), draft, q_z, q_lse, q_thr, q_tok,
                        n_draft, pol, seed, B, gamma, V, accept_len, out_tokens, flags, ws, plan,
                        st);
  return launch_typed(static_cast<const float*>(target), draft, q_z, q_lse, q_thr, q_tok, n_draft,
                      pol, seed, B, gamma, V, accept_len, out_tokens, flags, ws, plan, st);
}

}  // namespace dspark
