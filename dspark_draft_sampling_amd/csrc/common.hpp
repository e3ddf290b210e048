// common.hpp — device helpers shared by the gfx950 kernels of the DSpark
// sampling / verification library: bf16 unpacking, Philox4x32-10, the uniform
// and Gumbel maps, wave64 and workgroup reductions.
//
// Random numbers follow the library's documented convention: Philox4x32-10
// (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
// SC'11) keyed by the 64-bit seed, counter (i / 4, position, request, tag),
// output word i % 4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dspark.h"

namespace dspark {

constexpr int kChunk = DSPARK_CHUNK;  // tokens per level-1 chunk of the sampler
constexpr int kSub = DSPARK_SUB;      // tokens per level-2 sub-chunk of the sampler
constexpr float kNearEps = 1e-6f;     // margin of the NEAR_THRESHOLD diagnostic
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Words between ticket counters: each on its own 256-byte line, because
// device-scope atomics to one line are performed one at a time.
constexpr int kTicketStride = 64;

// Raw buffer resources (loads bounds-checked against the resource's size:
// reads past it return 0).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format

// Index of the calling wave in its workgroup, as a scalar (the compiler
// cannot tell that threadIdx.x / 64 is uniform across the wave).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)); }
// A value the caller knows to be the same on every lane, as a scalar.
__device__ __forceinline__ int uniform_i(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float pos_inf() { return __builtin_inff(); }

// bf16 halves of a packed 32-bit word (element 2i in the low half).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T>
__device__ __forceinline__ float load_logit(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_logit<uint16_t>(const uint16_t* p, size_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
template <>
__device__ __forceinline__ float load_logit<float>(const float* p, size_t i) {
  return p[i];
}

// ---- Philox4x32-10 ----------------------------------------------------------
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                              uint32_t& c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

__device__ __forceinline__ uint32_t philox_word(uint64_t seed, uint32_t i, int32_t position,
                                                uint32_t request, uint32_t tag) {
  uint32_t c0 = i >> 2, c1 = static_cast<uint32_t>(position), c2 = request, c3 = tag;
  philox4x32_10(c0, c1, c2, c3, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
  const uint32_t s = i & 3u;
  return s == 0 ? c0 : s == 1 ? c1 : s == 2 ? c2 : c3;
}

// Gumbel noise from a 32-bit word: u = ((w >> 9) + 1/2) 2^-23 in (0, 1) is
// exact in fp32; g = -ln(-ln u) with the accurate logf.
__device__ __forceinline__ float gumbel_of(uint32_t w) {
  const float u = (static_cast<float>(w >> 9) + 0.5f) * 0x1.0p-23f;
  const float e = -logf(u);
  return -logf(e);
}

__device__ __forceinline__ float gumbel(uint64_t seed, uint32_t i, int32_t position,
                                        uint32_t request, uint32_t tag) {
  return gumbel_of(philox_word(seed, i, position, request, tag));
}

// Accept-test uniform u' = (w >> 8) 2^-24 in [0, 1).
__device__ __forceinline__ float accept_uniform(uint64_t seed, int32_t position,
                                                uint32_t request) {
  const uint32_t w = philox_word(seed, 0, position, request, DSPARK_TAG_ACCEPT);
  return static_cast<float>(w >> 8) * 0x1.0p-24f;
}

__device__ __forceinline__ bool near_gap(float best, float second) {
  return (best - second) <= kNearEps * fmaxf(1.0f, fabsf(best));
}

// ---- wave64 reductions --------------------------------------------------------
// Butterfly inside each row of 16 lanes with DPP (quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_half_mirror, row_mirror), then the four row results
// are read with v_readlane and combined in a fixed order, so every lane gets
// the same, deterministic result.  All 64 lanes must be active.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ int lane_i(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  int x = static_cast<int>(v);
  x |= dpp_i<kDppXor1>(x);
  x |= dpp_i<kDppXor2>(x);
  x |= dpp_i<kDppHalfMirror>(x);
  x |= dpp_i<kDppMirror>(x);
  return static_cast<uint32_t>(lane_i(x, 0) | lane_i(x, 16) | lane_i(x, 32) | lane_i(x, 48));
}

// (value, index) maximum: larger value wins, the lower index on equal values.
// An index of INT32_MAX marks "nothing".
struct ArgMax {
  float v;
  int32_t i;
};
__device__ __forceinline__ ArgMax better(ArgMax a, ArgMax b) {
  return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}
template <int CTRL>
__device__ __forceinline__ ArgMax dpp_step(ArgMax a) {
  return better(a, ArgMax{dpp_f<CTRL>(a.v), dpp_i<CTRL>(a.i)});
}
__device__ __forceinline__ ArgMax wave_argmax(ArgMax a) {
  a = dpp_step<kDppXor1>(a);
  a = dpp_step<kDppXor2>(a);
  a = dpp_step<kDppHalfMirror>(a);
  a = dpp_step<kDppMirror>(a);
  ArgMax r{lane_f(a.v, 0), lane_i(a.i, 0)};
  r = better(r, ArgMax{lane_f(a.v, 16), lane_i(a.i, 16)});
  r = better(r, ArgMax{lane_f(a.v, 32), lane_i(a.i, 32)});
  r = better(r, ArgMax{lane_f(a.v, 48), lane_i(a.i, 48)});
  return r;
}

// ArgMax over the four 16-lane rows (see rows_combine).
__device__ __forceinline__ ArgMax rows_argmax(ArgMax a) {
  const auto v1 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a.v), __float_as_uint(a.v), false, false);
  const auto i1 = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(a.i), static_cast<uint32_t>(a.i), false, false);
  a = better(ArgMax{__uint_as_float(v1[0]), static_cast<int32_t>(i1[0])},
             ArgMax{__uint_as_float(v1[1]), static_cast<int32_t>(i1[1])});
  const auto v2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a.v), __float_as_uint(a.v), false, false);
  const auto i2 = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(a.i), static_cast<uint32_t>(a.i), false, false);
  return better(ArgMax{__uint_as_float(v2[0]), static_cast<int32_t>(i2[0])},
                ArgMax{__uint_as_float(v2[1]), static_cast<int32_t>(i2[1])});
}

// ---- reductions over the four 16-lane rows of a wave -------------------------
// Lanes l, l^16, l^32, l^48 combined in registers with the gfx950 lane swaps
// (v_permlane16_swap: rows 1 and 3 of the first operand trade places with
// rows 0 and 2 of the second; v_permlane32_swap: the upper half of the first
// with the lower half of the second).  Swapping a value with itself leaves a
// lane holding its own value and its partner row's (or half's) in the two
// results, so op(r0, r1) is the pairwise combination on every lane.
template <class Op>
__device__ __forceinline__ uint32_t rows_combine(uint32_t x, Op op) {
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(b[0], b[1]);
}
__device__ __forceinline__ float rows_sum(float v) {
  return __uint_as_float(rows_combine(__float_as_uint(v), [](uint32_t p, uint32_t q) {
    return __float_as_uint(__uint_as_float(p) + __uint_as_float(q));
  }));
}
__device__ __forceinline__ uint32_t rows_or(uint32_t v) {
  return rows_combine(v, [](uint32_t p, uint32_t q) { return p | q; });
}

__device__ __forceinline__ float rows_max(float v) {
  return __uint_as_float(rows_combine(__float_as_uint(v), [](uint32_t p, uint32_t q) {
    return __float_as_uint(fmaxf(__uint_as_float(p), __uint_as_float(q)));
  }));
}

// Top-2 scores with the argmax: (best, index, second best).
struct Top2 {
  float v1;
  int32_t i1;
  float v2;
};
__device__ __forceinline__ Top2 top2_merge(Top2 a, Top2 b) {
  Top2 r;
  if (b.v1 > a.v1 || (b.v1 == a.v1 && b.i1 < a.i1)) {
    r.v1 = b.v1;
    r.i1 = b.i1;
    r.v2 = fmaxf(a.v1, b.v2);
  } else {
    r.v1 = a.v1;
    r.i1 = a.i1;
    r.v2 = fmaxf(b.v1, a.v2);
  }
  return r;
}
template <int CTRL>
__device__ __forceinline__ Top2 dpp_step(Top2 a) {
  return top2_merge(a, Top2{dpp_f<CTRL>(a.v1), dpp_i<CTRL>(a.i1), dpp_f<CTRL>(a.v2)});
}
__device__ __forceinline__ Top2 wave_top2(Top2 a) {
  a = dpp_step<kDppXor1>(a);
  a = dpp_step<kDppXor2>(a);
  a = dpp_step<kDppHalfMirror>(a);
  a = dpp_step<kDppMirror>(a);
  Top2 r{lane_f(a.v1, 0), lane_i(a.i1, 0), lane_f(a.v2, 0)};
#pragma unroll
  for (int l = 16; l < 64; l += 16) r = top2_merge(r, Top2{lane_f(a.v1, l), lane_i(a.i1, l), lane_f(a.v2, l)});
  return r;
}

// Top2 over each group of four consecutive lanes (DPP quad_perm).
__device__ __forceinline__ Top2 quad_top2(Top2 a) {
  a = dpp_step<kDppXor1>(a);
  return dpp_step<kDppXor2>(a);
}

// Top2 over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ Top2 rows_top2(Top2 a) {
  const auto v1 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a.v1), __float_as_uint(a.v1), false, false);
  const auto i1 = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(a.i1), static_cast<uint32_t>(a.i1), false, false);
  const auto v2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a.v2), __float_as_uint(a.v2), false, false);
  a = top2_merge(Top2{__uint_as_float(v1[0]), static_cast<int32_t>(i1[0]), __uint_as_float(v2[0])},
                 Top2{__uint_as_float(v1[1]), static_cast<int32_t>(i1[1]), __uint_as_float(v2[1])});
  const auto w1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a.v1), __float_as_uint(a.v1), false, false);
  const auto j1 = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(a.i1), static_cast<uint32_t>(a.i1), false, false);
  const auto w2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a.v2), __float_as_uint(a.v2), false, false);
  return top2_merge(Top2{__uint_as_float(w1[0]), static_cast<int32_t>(j1[0]), __uint_as_float(w2[0])},
                    Top2{__uint_as_float(w1[1]), static_cast<int32_t>(j1[1]), __uint_as_float(w2[1])});
}

// Cross-workgroup hand-off without whole-cache maintenance: values are written
// through to the device-coherent level (agent-scope relaxed atomic stores, sc1)
// and read from it (agent-scope relaxed atomic loads); publish() waits for the
// writer's stores to complete before its ticket increment is issued.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_coherent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait for every outstanding memory operation of this wave (s_waitcnt 0),
// then increment the ticket; returns the ticket's previous value.
__device__ __forceinline__ uint32_t publish(uint32_t* ticket) {
  __builtin_amdgcn_s_waitcnt(0);
  return __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge of log-sum-exp partials (m, s) meaning s * exp(m): returns the pair
// relative to the larger maximum.  exp here is exp(x) via exp2.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 > m) {
    s = s * __builtin_amdgcn_exp2f((m - m2) * kLog2e) + s2;
    m = m2;
  } else if (m2 == m) {
    s += s2;
  } else if (m2 > neg_inf()) {
    s += s2 * __builtin_amdgcn_exp2f((m2 - m) * kLog2e);
  }
}

// Workgroup-wide reductions through a small LDS array (one slot per wave).
template <int NW>
__device__ __forceinline__ float block_max(float v, float* sh) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxf(r, sh[i]);
  return r;
}
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r += sh[i];
  return r;
}
template <int NW>
__device__ __forceinline__ uint32_t block_or(uint32_t v, uint32_t* sh) {
  v = wave_or(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  uint32_t r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r |= sh[i];
  return r;
}
template <int NW>
__device__ __forceinline__ ArgMax block_argmax(ArgMax a, float* shv, int32_t* shi) {
  a = wave_argmax(a);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    shv[w] = a.v;
    shi[w] = a.i;
  }
  __syncthreads();
  ArgMax r{shv[0], shi[0]};
#pragma unroll
  for (int i = 1; i < NW; ++i) r = better(r, ArgMax{shv[i], shi[i]});
  return r;
}
template <int NW>
__device__ __forceinline__ Top2 block_top2(Top2 a, float* shv, int32_t* shi, float* shv2) {
  a = wave_top2(a);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    shv[w] = a.v1;
    shi[w] = a.i1;
    shv2[w] = a.v2;
  }
  __syncthreads();
  Top2 r{shv[0], shi[0], shv2[0]};
#pragma unroll
  for (int i = 1; i < NW; ++i) r = top2_merge(r, Top2{shv[i], shi[i], shv2[i]});
  return r;
}

// Reductions over each group of four consecutive lanes (DPP quad_perm); the
// result is the same on the four lanes.
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  return fmaxf(v, dpp_f<kDppXor2>(v));
}
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  return v + dpp_f<kDppXor2>(v);
}

// Levels 2 and 3 of the library's three-level Gumbel-max draw, inside the
// chosen 256-token chunk c, by one whole wave.  Lane l holds the log-weights
// lw[e] of tokens 256 c + 4 l + e (-inf: excluded or past the row), so lanes
// 4 j .. 4 j + 3 hold sub-chunk j of the chunk.
//  * level 2: sub-chunk j* = argmax_j (ln W_j + g_j), W_j its total weight,
//    g_j the sub-chunk noise of global sub-chunk index 16 c + j;
//  * level 3: token v* = argmax_{v in j*} (lw_v + g_v), token noise of v.
// Ties go to the lowest index.  Returns the token (-1 if the chunk has no
// weight), its log-weight, and whether a level's top-2 gap is within the
// NEAR margin.  Every lane gets the same result.
struct InChunk {
  int32_t tok;
  float lw;
  bool near;
};
__device__ __forceinline__ InChunk draw_in_chunk(const float (&lw)[4], int c, uint64_t seed, int32_t pos,
                                                 uint32_t req, uint32_t tag_sub, uint32_t tag_tok) {
  const int lane = threadIdx.x & 63;
  // sub-chunk masses relative to the maximum m64 of the sub-chunk's 64-token
  // group (lanes 16 w .. 16 w + 15), exactly as the one-launch Markov kernel
  // forms them from the values it holds: per lane the sum of
  // 2^(lw log2e - m64 log2e) over its four tokens, then over the four lanes
  // of the sub-chunk as (l0 + l1) + (l2 + l3)
  float m = fmaxf(fmaxf(lw[0], lw[1]), fmaxf(lw[2], lw[3]));
  m = fmaxf(m, dpp_f<kDppXor1>(m));
  m = fmaxf(m, dpp_f<kDppXor2>(m));
  m = fmaxf(m, dpp_f<kDppHalfMirror>(m));
  m = fmaxf(m, dpp_f<kDppMirror>(m));
  float s = 0.0f;
  const float mb = (m > neg_inf() && m < pos_inf()) ? m * kLog2e : 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s += __builtin_amdgcn_exp2f(fmaf(lw[e], kLog2e, -mb));
  s = quad_sum(s);
  const uint32_t j = static_cast<uint32_t>(c) * (kChunk / kSub) + static_cast<uint32_t>(lane >> 2);
  const float g2 = gumbel(seed, j, pos, req, tag_sub);
  Top2 t2{neg_inf(), INT32_MAX, neg_inf()};
  if ((lane & 3) == 0 && m > neg_inf() && m < pos_inf() && s > 0.0f)
    t2 = Top2{m + logf(s) + g2, static_cast<int32_t>(j), neg_inf()};
  t2 = wave_top2(t2);
  InChunk r{-1, neg_inf(), false};
  if (t2.i1 == INT32_MAX) return r;
  r.near = t2.v2 > neg_inf() && near_gap(t2.v1, t2.v2);
  // tokens 4 l .. 4 l + 3 of the chunk share Philox counter (64 c + l, pos, req, tag)
  uint32_t c0 = static_cast<uint32_t>(c) * (kChunk / 4) + static_cast<uint32_t>(lane), c1 = static_cast<uint32_t>(pos),
           c2 = req, c3 = tag_tok;
  philox4x32_10(c0, c1, c2, c3, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
  const uint32_t w[4] = {c0, c1, c2, c3};
  Top2 t3{neg_inf(), INT32_MAX, neg_inf()};
  if (static_cast<uint32_t>(lane >> 2) == static_cast<uint32_t>(t2.i1) - static_cast<uint32_t>(c) * (kChunk / kSub)) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (lw[e] > neg_inf()) t3 = top2_merge(t3, Top2{lw[e] + gumbel_of(w[e]), c * kChunk + 4 * lane + e, neg_inf()});
  }
  t3 = wave_top2(t3);
  if (t3.i1 == INT32_MAX) return r;
  r.tok = t3.i1;
  if (t3.v2 > neg_inf() && near_gap(t3.v1, t3.v2)) r.near = true;
  const int e = r.tok & 3;
  const float mine = e == 0 ? lw[0] : e == 1 ? lw[1] : e == 2 ? lw[2] : lw[3];
  r.lw = __shfl(mine, (r.tok - c * kChunk) >> 2, 64);
  return r;
}

// Byte i of a byte array, read through the aligned 32-bit word that holds it,
// so that a wave-uniform index becomes a scalar (SMEM) load.  The word never
// leaves the 4-byte-aligned block of the byte itself.
__device__ __forceinline__ uint32_t load_u8_word(const uint8_t* __restrict__ p, int i) {
  const int off = static_cast<int>(reinterpret_cast<uintptr_t>(p + i) & 3u);
  const uint32_t w = *reinterpret_cast<const uint32_t*>(p + (i - off));
  return (w >> (8 * off)) & 0xffu;
}

__device__ __forceinline__ bool bad_temperature(float T) {
  return !(T > 0.0f) || !(T < pos_inf());
}

__device__ __forceinline__ int32_t clamp_token(int32_t x, int32_t V) {
  return x < 0 ? 0 : (x >= V ? V - 1 : x);
}

}  // namespace dspark
