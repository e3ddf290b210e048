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

constexpr int kChunk = DSPARK_CHUNK;  // tokens per chunk of two-level Gumbel-max
constexpr float kNearEps = 1e-6f;     // margin of the NEAR_THRESHOLD diagnostic
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, 64);
  return v;
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
__device__ __forceinline__ ArgMax wave_argmax(ArgMax a) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ArgMax b{__shfl_xor(a.v, o, 64), __shfl_xor(a.i, o, 64)};
    a = better(a, b);
  }
  return a;
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
__device__ __forceinline__ Top2 wave_top2(Top2 a) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Top2 b{__shfl_xor(a.v1, o, 64), __shfl_xor(a.i1, o, 64), __shfl_xor(a.v2, o, 64)};
    a = top2_merge(a, b);
  }
  return a;
}

// Merge of log-sum-exp partials (m, s) meaning s * exp(m): returns the pair
// relative to the larger maximum.  exp here is exp(x) via exp2.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 > m) {
    s = s * exp2f((m - m2) * kLog2e) + s2;
    m = m2;
  } else if (m2 == m) {
    s += s2;
  } else if (m2 > neg_inf()) {
    s += s2 * exp2f((m2 - m) * kLog2e);
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

__device__ __forceinline__ bool bad_temperature(float T) {
  return !(T > 0.0f) || !(T < pos_inf());
}

__device__ __forceinline__ int32_t clamp_token(int32_t x, int32_t V) {
  return x < 0 ? 0 : (x >= V ? V - 1 : x);
}

}  // namespace dspark
