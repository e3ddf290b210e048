// truncate.hpp — top-k / top-p thresholds of one logits row, computed by one
// workgroup of NT threads (a multiple of 64 dividing 2048): an exact cut on
// candidates bounded by chunk maxima, and a radix select over order-preserving
// float keys as the fallback.
//
// Policy ("[2/3] feat(dsv4): implement exact DSpark speculative decoding",
// "Exact decoding semantics", "Probabilistic": temperature, top-k and top-p
// shape both p and q), with the library's reading of order and ties:
//   top-k keeps every token whose value is >= the k-th largest value (ties
//   with it kept); top-p then keeps, on the renormalised top-k set, every
//   value group whose strictly-larger groups hold less than top_p of the mass
//   (top_p <= 0 keeps the largest group).
//
// Keys: a float maps to a 32-bit key whose unsigned order is the float order.
// Each histogram level bins the keys that share the bits chosen so far by the
// next 11 (or 10 / 5) bits, counting elements (top-k) or summing their
// weights in fp64 (top-p).  bf16 rows resolve in two levels (16 key bits),
// fp32 rows in three.
#pragma once

#include "common.hpp"

namespace dspark {

constexpr int kSelThreads = 512;  // workgroup size of the verify select
constexpr int kSelBins = 2048;

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <int NT>
struct SelLds {
  uint32_t cnt[kSelBins];
  double mass[kSelBins];
  uint32_t tc[NT];
  double tm[NT];
  int bin;
  uint32_t above_c;
  double above_m;
  double total_m;
  uint32_t total_c;
};

struct SelResult {
  float thr;      // smallest kept value
  double s_kept;  // total weight of the kept tokens
};

// One histogram level over the row: tokens with key >= kmin whose key bits at
// and above `top` equal `prefix` are binned by key bits [shift, top).  The row
// functor provides load4(v0, x[4]) for v0 a multiple of 4 (-inf past V).
template <int NT, class Row>
__device__ __forceinline__ void sel_level(const Row& row, int V, uint32_t prefix, int top, int shift, uint32_t kmin,
                          float wa, float wb, SelLds<NT>& S) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kSelBins; i += NT) {
    S.cnt[i] = 0u;
    S.mass[i] = 0.0;
  }
  if (tid == 0) S.total_m = 0.0;
  __syncthreads();
  const uint32_t mask = (1u << (top - shift)) - 1u;
  double local = 0.0;
  // eight groups of four tokens per thread per round, all loads issued first
  constexpr int U = 8;
  for (int base = tid * 4; base < V; base += NT * 4 * U) {
    float x[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) row.load4(base + u * NT * 4, x[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xv = x[u][e];  // -inf past the row end
        if (!(xv > neg_inf()) || xv != xv) continue;
        const uint32_t k = order_key(xv);
        if (k < kmin) continue;
        if (top < 32 && (k >> top) != prefix) continue;
        const int bin = static_cast<int>((k >> shift) & mask);
        const double w = static_cast<double>(__builtin_amdgcn_exp2f(fmaf(xv, wa, wb)));
        atomicAdd(&S.cnt[bin], 1u);
        atomicAdd(&S.mass[bin], w);
        local += w;
      }
  }
  atomicAdd(&S.total_m, local);  // the level's total weight
  __syncthreads();
}

// First bin, scanning from the largest keys down, at which the running count
// (by_mass = false) or weight (true) including the bin reaches `target`; if
// the whole level holds less, the smallest non-empty bin.  Leaves the bin and
// the count / weight strictly above it in S.
template <int NT>
__device__ __forceinline__ void sel_find(SelLds<NT>& S, int nbins, bool by_mass, double target) {
  const int tid = threadIdx.x;
  constexpr int per = kSelBins / NT;  // bins per thread, descending
  uint32_t c = 0;
  double m = 0.0;
  for (int j = 0; j < per; ++j) {
    const int bin = nbins - 1 - (tid * per + j);
    if (bin >= 0) {
      c += S.cnt[bin];
      m += S.mass[bin];
    }
  }
  S.tc[tid] = c;
  S.tm[tid] = m;
  __syncthreads();
  if (tid == 0) {
    // exclusive scan in descending-key order
    uint32_t ac = 0;
    double am = 0.0;
    for (int t = 0; t < NT; ++t) {
      const uint32_t xc = S.tc[t];
      const double xm = S.tm[t];
      S.tc[t] = ac;
      S.tm[t] = am;
      ac += xc;
      am += xm;
    }
    S.total_c = ac;
    S.total_m = am;
    S.bin = -1;
  }
  __syncthreads();
  const double total = by_mass ? S.total_m : static_cast<double>(S.total_c);
  const double tgt = target < total ? target : total;
  uint32_t ac = S.tc[tid];
  double am = S.tm[tid];
  for (int j = 0; j < per; ++j) {
    const int bin = nbins - 1 - (tid * per + j);
    if (bin < 0) break;
    const uint32_t bc = S.cnt[bin];
    const double bm = S.mass[bin];
    const double before = by_mass ? am : static_cast<double>(ac);
    const double incl = by_mass ? am + bm : static_cast<double>(ac + bc);
    if (bc > 0 && before < tgt && incl >= tgt) {
      S.bin = bin;
      S.above_c = ac;
      S.above_m = am;
    }
    ac += bc;
    am += bm;
  }
  __syncthreads();
}

// Thresholds of a row.  `row(v)` returns the value the policy orders by
// (logit or scaled logit); the weight of a token is exp2(value * wa + wb).
// keybits = 16 for bf16 rows (their key's low 16 bits are determined by the
// sign), 32 otherwise.
template <int NT, class Row>
__device__ __forceinline__ SelResult select_threshold(const Row& row, int V, int keybits, int top_k, float top_p,
                                      float wa, float wb, SelLds<NT>& S) {
  const int nlev = keybits == 16 ? 2 : 3;
  const int tops[3] = {32, 21, 10};
  const int shifts16[2] = {21, 16};
  const int shifts32[3] = {21, 10, 0};
  uint32_t kmin = 0u;
  uint32_t key = 0u;
  double s_kept = 0.0;
  const bool use_k = top_k > 0 && top_k < V;
  if (use_k) {
    uint32_t prefix = 0u;
    double need = static_cast<double>(top_k);
    for (int l = 0; l < nlev; ++l) {
      const int top = tops[l];
      const int shift = keybits == 16 ? shifts16[l] : shifts32[l];
      sel_level(row, V, prefix, top, shift, 0u, wa, wb, S);
      sel_find(S, 1 << (top - shift), false, need);
      const int bin = S.bin < 0 ? 0 : S.bin;
      need -= static_cast<double>(S.above_c);
      s_kept += S.above_m;
      if (l == nlev - 1) s_kept += S.mass[bin];
      prefix = (prefix << (top - shift)) | static_cast<uint32_t>(bin);
      __syncthreads();
    }
    key = keybits == 16 ? ((prefix << 16) | ((prefix & 0x8000u) ? 0u : 0xffffu)) : prefix;
    kmin = key;
  }
  if (top_p < 1.0f) {
    uint32_t prefix = 0u;
    double target = 0.0;
    s_kept = 0.0;
    for (int l = 0; l < nlev; ++l) {
      const int top = tops[l];
      const int shift = keybits == 16 ? shifts16[l] : shifts32[l];
      sel_level(row, V, prefix, top, shift, kmin, wa, wb, S);
      if (l == 0) {
        // top_p applies to the renormalised (top-k) set; top_p <= 0 keeps
        // only the largest group: the first bin with weight
        target = top_p > 0.0f ? static_cast<double>(top_p) * S.total_m : 1e-300;
      }
      sel_find(S, 1 << (top - shift), true, target);
      const int bin = S.bin < 0 ? 0 : S.bin;
      target -= S.above_m;
      s_kept += S.above_m;
      if (l == nlev - 1) s_kept += S.mass[bin];
      prefix = (prefix << (top - shift)) | static_cast<uint32_t>(bin);
      __syncthreads();
    }
    key = keybits == 16 ? ((prefix << 16) | ((prefix & 0x8000u) ? 0u : 0xffffu)) : prefix;
  }
  return SelResult{key_value(key), s_kept};
}

// Truncation settings of request b; the two arrays are both NULL when no
// request of the call truncates.
__device__ __forceinline__ int top_k_of(const int32_t* top_k, int b) { return top_k ? top_k[b] : 0; }
__device__ __forceinline__ float top_p_of(const float* top_p, int b) { return top_p ? top_p[b] : 1.0f; }

__device__ __forceinline__ bool truncated(int top_k, float top_p, int V) {
  return (top_k > 0 && top_k < V) || top_p < 1.0f;
}

// ---------------------------------------------------------------------------
// Candidate path.  Per 256-token chunk maxima bound the kept set from below:
//  * top-k: the k-th largest chunk maximum is <= the k-th largest value (the
//    maxima of the k best chunks are k distinct tokens);
//  * top-p: any tau whose chunks' maxima alone carry top_p of the weight has
//    mass(x >= tau) >= top_p * total, so the cut lies at or above tau.
// Tokens of the chunks whose maximum reaches tau are gathered into LDS,
// sorted, and the exact cut is taken there.  The caller falls back when the
// bound cannot be formed or the candidates overflow.
constexpr int kMaxChunksBound = 1024;  // chunk maxima a bound looks at
constexpr int kCandCap = 4096;         // candidate tokens held in LDS

template <int NT>
struct CandLds {
  int ci[kMaxChunksBound];  // chunks whose maximum reaches tau (any order)
  float cv[kCandCap];       // candidate values, sorted descending
  float tmp[kCandCap];      // sort scratch
  unsigned long long wt[NT / 64];
  uint32_t key;  // order key of tau (0: no bound)
  int n;         // candidates gathered (> kCandCap: overflow)
  int nchunks;   // chunks whose maximum reaches tau
  int idx;       // scratch index
  int cnt;       // scratch count
  float tau;
  float thr;
  float s_kept;
  int nkept;
  int ok;  // the cut lies inside the candidates
};

// Weight-histogram path for top-p without top-k (its state is HistLds below).
// Weights are summed in fixed point, units of 2^-40 of the row's shifted
// frame (the maximum weighs [1, 2)): integer sums are exact and independent
// of order.
using fix_t = unsigned long long;
constexpr float kFix = 1099511627776.0f;  // 2^40

// w * 2^40 truncated to an integer, for w in [0, 2) with w >= 2^-64 or 0:
// w = m 2^(E - 150) (m the 24-bit significand, E the biased exponent), so
// w 2^40 = (m 2^24) >> (134 - E); shifts past 63 leave less than one unit.
__device__ __forceinline__ fix_t to_fix(float w) {
  const uint32_t b = __float_as_uint(w);
  const uint32_t sh = min(134u - (b >> 23), 63u);
  const fix_t m = static_cast<fix_t>((b & 0x7fffffu) | 0x800000u) << 24;
  return m >> sh;
}

constexpr int kHistBins = 2048;
constexpr int kHistCap = 512;  // tokens of the cut's bin range held in LDS

template <int NT>
struct HistLds {
  fix_t hw[kHistBins];        // weight per bin
  fix_t cw[kMaxChunksBound];  // per chunk: its kept weight
  int cl[kMaxChunksBound];    // chunks whose maximum lies in the window
  float cv[kHistCap];         // tokens of the cut's bin: values, sorted descending,
  int ct[kHistCap];           // their token indices,
  fix_t pw[kHistCap];         // and the running weight from the row's top (inclusive)
  fix_t wt[NT / 64];
  fix_t above;  // weight of the bins before the cut's bin
  int nl;       // listed chunks
  int n;        // tokens of the cut's bin (> kHistCap: overflow)
  int jc;       // the cut's bin
  int cs;       // start of the cut group in cv
  float thr;
  float s_kept;
};

// Either the candidate, the histogram or the radix-select state: never live
// at the same time.
template <int NT>
union TruncLds {
  CandLds<NT> c;
  HistLds<NT> h;
  SelLds<NT> s;
};

__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<kDppXor1>(v);
  v += dpp_i<kDppXor2>(v);
  v += dpp_i<kDppHalfMirror>(v);
  v += dpp_i<kDppMirror>(v);
  return (lane_i(v, 0) + lane_i(v, 16)) + (lane_i(v, 32) + lane_i(v, 48));
}

// Integer sum over the wave (same butterfly as wave_sum, on both halves).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(dpp_i<CTRL>(static_cast<int>(static_cast<uint32_t>(v))));
  const uint32_t hi = static_cast<uint32_t>(dpp_i<CTRL>(static_cast<int>(static_cast<uint32_t>(v >> 32))));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l) {
  const uint32_t lo = static_cast<uint32_t>(lane_i(static_cast<int>(static_cast<uint32_t>(v)), l));
  const uint32_t hi = static_cast<uint32_t>(lane_i(static_cast<int>(static_cast<uint32_t>(v >> 32)), l));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  v += dpp_u64<kDppXor1>(v);
  v += dpp_u64<kDppXor2>(v);
  v += dpp_u64<kDppHalfMirror>(v);
  v += dpp_u64<kDppMirror>(v);
  return (lane_u64(v, 0) + lane_u64(v, 16)) + (lane_u64(v, 32) + lane_u64(v, 48));
}

// Rank sort of v[0 .. n) descending (LDS, n <= NT), ties by ascending ix
// (IX) or by position; tv / ti: scratch of n entries.  For the small sets
// where a bitonic network would spend most of its time in barriers.
template <int NT, bool IX>
__device__ __forceinline__ void rank_sort_desc(float* v, int* ix, int n, float* tv, int* ti) {
  const int i = threadIdx.x;
  float x = 0.0f;
  int id = 0, r = 0;
  if (i < n) {
    x = v[i];
    if constexpr (IX) id = ix[i];
#pragma unroll 4
    for (int j = 0; j < n; ++j) {
      const float y = v[j];
      bool before = y > x;
      if constexpr (IX) before = before || (y == x && ix[j] < id);
      else before = before || (y == x && j < i);
      r += before ? 1 : 0;
    }
  }
  __syncthreads();
  if (i < n) {
    tv[r] = x;
    if constexpr (IX) ti[r] = id;
  }
  __syncthreads();
  if (i < n) {
    v[i] = tv[i];
    if constexpr (IX) ix[i] = ti[i];
  }
  __syncthreads();
}

// Bitonic sort of n2 (a power of two) values, descending; with IX the
// indices travel along (ascending index among equal values).  All threads of
// the workgroup take part.
template <int NT, bool IX>
__device__ __forceinline__ void sort_desc(float* v, int* ix, int n2) {
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n2; i += NT) {
        const int l = i ^ j;
        if (l > i) {
          const bool desc = (i & k) == 0;
          const float a = v[i], b = v[l];
          bool a_first = a > b;
          if constexpr (IX) a_first = a_first || (a == b && ix[i] < ix[l]);
          else a_first = a_first || a == b;
          if (desc != a_first) {
            v[i] = b;
            v[l] = a;
            if constexpr (IX) {
              const int t = ix[i];
              ix[i] = ix[l];
              ix[l] = t;
            }
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Number of v[0 .. n) that are >= t (v sorted descending), all threads.
template <int NT>
__device__ __forceinline__ int count_at_least(const float* v, int n, float t, int& slot) {
  if (threadIdx.x == 0) slot = 0;
  __syncthreads();
  int c = 0;
  for (int i = threadIdx.x; i < n; i += NT) c += v[i] >= t ? 1 : 0;
  c = static_cast<int>(wave_sum(static_cast<float>(c)));
  if ((threadIdx.x & 63) == 0 && c) atomicAdd(&slot, c);
  __syncthreads();
  const int r = slot;
  __syncthreads();
  return r;
}

// tau of the chunk-maxima bound and the chunks whose maximum reaches it.
// cm: the C chunk maxima (LDS; -inf or NaN: no finite token).  Wave 0 finds
// tau by bisection over the maxima's order keys: top-k, the largest key with
// at least top_k maxima at or above it (the k-th largest maximum); top-p, the
// largest key whose maxima at or above it weigh top_p * total (with a margin
// against rounding).  Sets L.tau, L.ci / L.nchunks (any order) and L.n = 0;
// returns false when there is no bound.  wa, wb: a value x weighs
// exp2(x wa + wb); total: the row's weight.
template <int NT>
__device__ __forceinline__ bool chunk_bound(const float* cm, int C, int top_k, float top_p, float wa, float wb,
                            float total, CandLds<NT>& L) {
  if (C > kMaxChunksBound) return false;
  if (threadIdx.x < 64) {
    constexpr int PER = kMaxChunksBound / 64;
    const int lane = threadIdx.x;
    const bool byk = top_k > 0;
    uint32_t key[PER];
    float w[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int c = lane + 64 * j;
      const float x = c < C ? cm[c] : neg_inf();
      const bool fin = x > neg_inf();  // false for NaN
      key[j] = fin ? order_key(x) : 0u;
      w[j] = (!byk && fin) ? __builtin_amdgcn_exp2f(fmaf(x, wa, wb)) : 0.0f;
    }
    uint32_t t = 0u;
    if (byk) {
      if (top_k <= C && top_k <= kCandCap) {
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t cand = t | (1u << bit);
          int cnt = 0;
#pragma unroll
          for (int j = 0; j < PER; ++j) cnt += key[j] >= cand ? 1 : 0;
          if (wave_sum_i(cnt) >= top_k) t = cand;
        }
      }
    } else if (top_p < 1.0f) {
      const float target = (top_p > 0.0f ? top_p : 0.0f) * total * 1.0009765625f;
      float all = 0.0f;
#pragma unroll
      for (int j = 0; j < PER; ++j) all += w[j];
      if (wave_sum(all) >= target) {
        // the masked sums only grow as the key falls (rounding is monotone)
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t cand = t | (1u << bit);
          float ws = 0.0f;
#pragma unroll
          for (int j = 0; j < PER; ++j) ws += key[j] >= cand ? w[j] : 0.0f;
          if (wave_sum(ws) >= target) t = cand;
        }
      }
    }
    if (lane == 0) {
      L.key = t;
      L.tau = t ? key_value(t) : neg_inf();
      L.nchunks = 0;
      L.n = 0;
    }
  }
  __syncthreads();
  if (L.key == 0u) {
    __syncthreads();
    return false;
  }
  const float tau = L.tau;
  for (int c0 = 0; c0 < C; c0 += NT) {
    const int c = c0 + static_cast<int>(threadIdx.x);
    const bool take = c < C && cm[c] >= tau;
    const uint64_t mask = __ballot(take);
    int base = 0;
    if ((threadIdx.x & 63) == 0 && mask) base = atomicAdd(&L.nchunks, __popcll(mask));
    base = __shfl(base, 0, 64);
    if (take) L.ci[base + __popcll(mask & ((1ull << (threadIdx.x & 63)) - 1ull))] = c;
  }
  __syncthreads();
  return true;
}

// Four tokens v0 .. v0+3 of a listed chunk (v0 a multiple of 4, -inf past
// V): VL rows (V a multiple of 4, aligned) take one vector load, masked as a
// whole; others the row's checked path.
template <bool VL, class Row>
__device__ __forceinline__ void hist_load(const Row& row, int v0, int V, float* x) {
  if constexpr (VL) {
    row.load4u(v0, x);
    const bool in = v0 < V;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = in ? x[e] : neg_inf();
  } else {
    row.load4(v0, x);
  }
}

// Gather every token >= tau of the chunks L.ci[0 .. L.nchunks): wave w
// takes groups of CU chunks, the group's loads issued together (lane l the
// tokens 4l .. 4l+3 of each chunk); one LDS atomic reserves the group's
// slots, and each token's slot follows from the ballots before it.  Sets
// L.n (possibly above kCandCap: overflow, nothing beyond the cap is stored).
template <int NT, bool VL, class Row>
__device__ __forceinline__ void gather_group(const Row& row, int V, CandLds<NT>& L) {
  constexpr int NW = NT / 64;
  constexpr int CU = 8;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const uint64_t below = (1ull << lane) - 1ull;
  const float tau = L.tau;
  const int nch = uniform_i(L.nchunks);
  for (int j0 = wave * CU; j0 < nch; j0 += NW * CU) {
    float x[CU][4];
    int v0[CU];
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int j = j0 + u;
      v0[u] = j < nch ? uniform_i(L.ci[j]) * kChunk + lane * 4 : V;  // V: nothing to load
      hist_load<VL>(row, v0[u], V, x[u]);
    }
    int total = 0;
#pragma unroll
    for (int u = 0; u < CU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) total += __popcll(__ballot(x[u][e] >= tau));
    if (total == 0) continue;  // wave-uniform
    int base = 0;
    if (lane == 0) base = atomicAdd(&L.n, total);
    base = uniform_i(base);
#pragma unroll
    for (int u = 0; u < CU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool take = x[u][e] >= tau;  // -inf past V never passes
        const uint64_t m = __ballot(take);
        const int slot = base + __popcll(m & below);
        if (take && slot < kCandCap) L.cv[slot] = x[u][e];
        base += __popcll(m);
      }
  }
}

template <int NT, class Row>
__device__ __forceinline__ void gather_candidates(const Row& row, int V, CandLds<NT>& L) {
  if (row.vec4) gather_group<NT, true>(row, V, L);
  else gather_group<NT, false>(row, V, L);
  __syncthreads();
}

// Sum of one fixed-point value per thread over the workgroup (all threads).
template <int NT>
__device__ __forceinline__ fix_t block_sum_fix(fix_t v, fix_t* wt) {
  v = wave_sum_u64(v);
  if ((threadIdx.x & 63) == 0) wt[threadIdx.x >> 6] = v;
  __syncthreads();
  fix_t all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) all += wt[w];
  __syncthreads();
  return all;
}

// Exclusive prefix of one fixed-point value per thread in thread order, and
// the total (all threads).
template <int NT>
__device__ __forceinline__ fix_t block_excl_scan_fix(fix_t own, fix_t* wt, fix_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  fix_t x = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const fix_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wt[wave] = x;
  __syncthreads();
  fix_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const fix_t t = wt[w];
    if (w < wave) before += t;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + x - own;
}

// Exact cut on the gathered candidates: sorts them, applies top-k (ties
// kept) and then top-p on the renormalised set (the first value group always
// kept, a later group kept iff the weight strictly above it is below top_p of
// the set's weight).  Weights are summed in 2^-40 fixed point (exact, in any
// order): thread t owns a contiguous stretch of the sorted candidates and the
// running weight at each of them is its stretch's prefix plus the weight of
// the stretches before.  total: the row's total weight (the set's weight
// when top-k is off).  Sets L.thr (smallest kept value), L.s_kept (kept
// weight), L.nkept and L.ok (0: the cut is not decided by the candidates).
template <int NT>
__device__ __forceinline__ void exact_cut(int top_k, float top_p, float wa, float wb, float total, CandLds<NT>& L) {
  const int n = L.n;
  if (n > kCandCap || n < 1 || (top_k > 0 && top_k > n)) {
    __syncthreads();
    if (threadIdx.x == 0) L.ok = 0;
    __syncthreads();
    return;
  }
  if (n <= NT) {
    rank_sort_desc<NT, false>(L.cv, nullptr, n, L.tmp, nullptr);
  } else {
    const int n2 = pow2_at_least(n);
    for (int i = n + static_cast<int>(threadIdx.x); i < n2; i += NT) L.cv[i] = neg_inf();
    __syncthreads();
    sort_desc<NT, false>(L.cv, nullptr, n2);
  }
  const int tid = threadIdx.x;
  const int per = (n + NT - 1) / NT, lo = min(n, tid * per), hi = min(n, lo + per);
  auto wfix = [&](int i) { return to_fix(__builtin_amdgcn_exp2f(fmaf(L.cv[i], wa, wb))); };
  // weight of this thread's share of the first m candidates
  auto share = [&](int m) {
    fix_t v = 0;
    for (int i = lo; i < hi && i < m; ++i) v += wfix(i);
    return v;
  };
  fix_t own = share(n), all;
  const fix_t before = block_excl_scan_fix<NT>(own, L.wt, all);
  int nk = n;
  fix_t set_w = 0;
  if (top_k > 0) {
    nk = count_at_least<NT>(L.cv, n, L.cv[top_k - 1], L.cnt);
    set_w = block_sum_fix<NT>(share(nk), L.wt);
  }
  int cut = nk;
  bool ok = true;
  if (top_p < 1.0f) {
    // a group is kept iff the weight above it is < p * (set weight): for
    // the integer sums, iff it is < T = ceil(p * set weight)
    const double p = top_p > 0.0f ? static_cast<double>(top_p) : 0.0;
    const double set_d = top_k > 0 ? static_cast<double>(set_w) : static_cast<double>(total) * static_cast<double>(kFix);
    const fix_t T = static_cast<fix_t>(ceil(p * set_d));
    if (tid == 0) L.idx = 0;
    __syncthreads();
    // the last group start whose strictly-larger weight is below T
    int best = 0;
    fix_t run = before;
    for (int i = lo; i < hi; ++i) {
      if (i > 0 && i < nk && L.cv[i] != L.cv[i - 1] && run < T) best = i;
      run += wfix(i);
    }
    if (best > 0) atomicMax(&L.idx, best);
    __syncthreads();
    cut = count_at_least<NT>(L.cv, nk, L.cv[L.idx], L.cnt);
    // top-p alone: the candidates must carry the target, else the cut may
    // lie below tau
    if (top_k <= 0) ok = all >= T;
  }
  const fix_t kept = block_sum_fix<NT>(share(cut), L.wt);
  if (tid == 0) {
    L.nkept = cut;
    L.thr = L.cv[cut - 1];
    L.s_kept = static_cast<float>(kept) * (1.0f / kFix);
    L.ok = ok ? 1 : 0;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Histogram path: top-p without top-k, for rows whose kept set spreads over
// too many chunks for the maxima bound.  A value x weighs 2^u, u = x wa + wb
// (the row maximum M has u in [0, 1)), taken in fixed point.
//
// Window: the smallest kept value thr has w(thr) > (1 - top_p) total / V (the
// tokens at or below thr weigh more than (1 - top_p) of the total and number
// at most V), so no token with u below ulo = log2 of that bound, less one for
// rounding, is kept; ulo is also held within 64 of umax (the bound itself
// lies within 55 of it).  The window [ulo, umax] is cut into kHistBins bins
// of equal width by (umax - u), a non-increasing function of x: equal values
// share a bin and a larger value never lies in a later bin.
//  pass A: the weight of every bin, over the chunks whose maximum lies in
//    the window (their list kept);
//  the cut's bin jc: the first non-empty bin at which the running weight
//    reaches top_p * total.  The running sums are exact, so every group
//    before jc is kept (its weight from the top stays below the target),
//    every group after jc is not, and jc's first group is kept;
//  pass B: per listed chunk reaching jc, the weight of its tokens before jc;
//    jc's tokens into LDS;
//  cut: jc's tokens sorted, their running weight from the weight before jc,
//    the top-p rule group by group.
// Leaves H.thr, H.s_kept (kept weight, 2^u units) and H.cw[c] = chunk c's
// kept weight (fixed point) for the chunks H.cl[0 .. H.nl) (the others hold
// no kept token).  Returns false when jc's tokens overflow LDS or the window
// does not reach the target (then nothing is decided).
struct HistMap {
  float wa, wb, umax, ulo, inv;
  // bin of u = x wa + wb, for u >= ulo (u <= umax: the row maximum's)
  __device__ __forceinline__ int bin_of(float u) const {
    const int j = static_cast<int>((umax - u) * inv);
    return j < 0 ? 0 : (j < kHistBins ? j : kHistBins - 1);
  }
  // bin of value x (-1 below the window, NaN and -inf included) and its weight
  __device__ __forceinline__ int bin(float x, float& w) const {
    const float u = fmaf(x, wa, wb);
    if (!(u >= ulo)) return -1;
    w = __builtin_amdgcn_exp2f(u);
    const int j = static_cast<int>((umax - u) * inv);
    return j < 0 ? 0 : (j < kHistBins ? j : kHistBins - 1);
  }
};

// In-place inclusive prefix sum of a[0 .. n) (LDS) plus base, all threads.
template <int NT>
__device__ __forceinline__ void block_scan_fix(fix_t* a, int n, fix_t base, fix_t* wt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + NT - 1) / NT;
  const int lo = tid * per, hi = min(n, lo + per);
  fix_t s = 0;
  for (int i = lo; i < hi; ++i) s += a[i];
  fix_t x = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const fix_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wt[wave] = x;
  __syncthreads();
  fix_t run = base + x - s;
  for (int w = 0; w < wave; ++w) run += wt[w];
  for (int i = lo; i < hi; ++i) {
    run += a[i];
    a[i] = run;
  }
  __syncthreads();
}

// Pass A: the weight of every bin over the listed chunks (wave w takes groups
// of CU chunks, the group's loads issued together; lane l the tokens 4l ..
// 4l+3 of each chunk).
template <int NT, int CU, bool VL, class Row>
__device__ __forceinline__ void hist_pass_a(const Row& row, int V, const HistMap& hm, const int* cl, int nl,
                                            fix_t* hw) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = wave_id();
  for (int j0 = wave * CU; j0 < nl; j0 += NW * CU) {
    float x[CU][4];
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int j = j0 + u;
      const int cc = j < nl ? uniform_i(cl[j]) : -1;
      hist_load<VL>(row, cc >= 0 ? cc * kChunk + 4 * lane : V, V, x[u]);
    }
#pragma unroll
    for (int u = 0; u < CU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float uu = fmaf(x[u][e], hm.wa, hm.wb);
        const int b = hm.bin_of(uu);
        const fix_t f = to_fix(__builtin_amdgcn_exp2f(uu));
        if (uu >= hm.ulo) atomicAdd(&hw[b], f);
      }
  }
}

// Appends the lanes' token (value xv, index tok) where take holds to jc's
// tokens (H.cv / H.ct; H.n counts past the cap).  All lanes call it.
template <int NT>
__device__ __forceinline__ void hist_append(bool take, float xv, int tok, HistLds<NT>& H) {
  const int lane = threadIdx.x & 63;
  const uint64_t mask = __ballot(take);
  if (!mask) return;
  int base = 0;
  if (lane == 0) base = atomicAdd(&H.n, __popcll(mask));
  base = __shfl(base, 0, 64);
  const int slot = base + __popcll(mask & ((1ull << lane) - 1ull));
  if (take && slot < kHistCap) {
    H.cv[slot] = xv;
    H.ct[slot] = tok;
  }
}

// Pass B over the listed chunks reaching the cut's bin jc: jc's tokens into
// H.cv / H.ct and, with CW, each chunk's weight of tokens before jc added to
// H.cw (integer LDS atomics: few tokens lie before jc, and the sums do not
// depend on order).
template <int NT, int CU, bool VL, bool CW, class Row>
__device__ __forceinline__ void hist_pass_b(const Row& row, int V, const HistMap& hm, int jc, const float* cm,
                                            HistLds<NT>& H) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int nl = uniform_i(H.nl);
  for (int j0 = wave * CU; j0 < nl; j0 += NW * CU) {
    float x[CU][4];
    int c[CU];
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int j = j0 + u;
      int cc = -1;
      if (j < nl) {
        cc = uniform_i(H.cl[j]);
        float w;
        if (uniform_i(hm.bin(cm[cc], w)) > jc) cc = -1;  // every token of the chunk lies past jc
      }
      c[u] = cc;
      hist_load<VL>(row, cc >= 0 ? cc * kChunk + 4 * lane : V, V, x[u]);
    }
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      if (c[u] < 0) continue;  // wave-uniform
      uint32_t at = 0;  // bit e: token 4 lane + e lies in jc
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float uu = fmaf(x[u][e], hm.wa, hm.wb);
        const bool inw = uu >= hm.ulo;
        const int b = hm.bin_of(uu);
        if constexpr (CW) {
          if (inw && b < jc) atomicAdd(&H.cw[c[u]], to_fix(__builtin_amdgcn_exp2f(uu)));
        }
        at |= (inw && b == jc) ? (1u << e) : 0u;
      }
      if (__ballot(at != 0)) {  // rare: the chunk holds tokens of jc
#pragma unroll
        for (int e = 0; e < 4; ++e) hist_append((at >> e) & 1u, x[u][e], c[u] * kChunk + 4 * lane + e, H);
      }
    }
  }
}

template <int NT, bool CW, class Row>
__device__ __forceinline__ bool hist_cut(const Row& row, int V, const float* cm, int C, float M, float total,
                         float wa, float wb, float top_p, HistLds<NT>& H) {
  constexpr int CU = 8, PB = kHistBins / NT;
  static_assert(kHistBins % NT == 0, "bins per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (C > kMaxChunksBound || !(total > 0.0f) || !(total < pos_inf())) return false;
  const float p = top_p > 0.0f ? top_p : 0.0f;
  HistMap hm;
  hm.wa = wa;
  hm.wb = wb;
  hm.umax = fmaf(M, wa, wb);
  hm.ulo = fmaxf(__log2f((1.0f - p) * total / static_cast<float>(V)) - 1.0f, hm.umax - 64.0f);
  hm.inv = static_cast<float>(kHistBins) / (hm.umax - hm.ulo);
  // a group is kept iff the weight above it is < p * total: for the integer
  // sums, iff it is < T = ceil(p * total * 2^40)
  const fix_t T = static_cast<fix_t>(ceil(static_cast<double>(p) * static_cast<double>(total) *
                                          static_cast<double>(kFix)));
  for (int i = tid; i < kHistBins; i += NT) H.hw[i] = 0;
  for (int c = tid; c < C; c += NT) H.cw[c] = 0;
  if (tid == 0) {
    H.nl = 0;
    H.n = 0;
    H.jc = INT32_MAX;
  }
  __syncthreads();
  for (int c0 = 0; c0 < C; c0 += NT) {
    const int c = c0 + tid;
    float w;
    const bool take = c < C && hm.bin(cm[c], w) >= 0;
    const uint64_t mask = __ballot(take);
    int base = 0;
    if (lane == 0 && mask) base = atomicAdd(&H.nl, __popcll(mask));
    base = __shfl(base, 0, 64);
    if (take) H.cl[base + __popcll(mask & ((1ull << lane) - 1ull))] = c;
  }
  __syncthreads();
  const int nl = uniform_i(H.nl);
  if (row.vec4) hist_pass_a<NT, CU, true>(row, V, hm, H.cl, nl, H.hw);
  else hist_pass_a<NT, CU, false>(row, V, hm, H.cl, nl, H.hw);
  __syncthreads();
  // the cut's bin: thread t owns bins t*PB .. t*PB+PB-1
  fix_t own = 0;
#pragma unroll
  for (int i = 0; i < PB; ++i) own += H.hw[tid * PB + i];
  fix_t incl = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const fix_t y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) H.wt[wave] = incl;
  __syncthreads();
  fix_t run = incl - own;
  for (int w = 0; w < wave; ++w) run += H.wt[w];
#pragma unroll
  for (int i = 0; i < PB; ++i) {
    const int j = tid * PB + i;
    const fix_t h = H.hw[j];
    if (h && run + h >= T) {  // this thread's first such bin; the smallest wins
      atomicMin(&H.jc, j);
      break;
    }
    run += h;
  }
  __syncthreads();
  const int jc = uniform_i(H.jc);
  if (jc == INT32_MAX) {  // the window holds less than the target
    __syncthreads();
    return false;
  }
  // weight before jc: the owner of jc knows it
  {
    fix_t r = incl - own;
    for (int w = 0; w < wave; ++w) r += H.wt[w];
    if (jc / PB == tid) {
      for (int j = tid * PB; j < jc; ++j) r += H.hw[j];
      H.above = r;
    }
  }
  __syncthreads();  // H.hw is read above; H.cw is added to below
  if (row.vec4) hist_pass_b<NT, CU, true, CW>(row, V, hm, jc, cm, H);
  else hist_pass_b<NT, CU, false, CW>(row, V, hm, jc, cm, H);
  __syncthreads();
  const int n = H.n;
  if (n > kHistCap || n < 1) {
    __syncthreads();
    return false;
  }
  // the cut inside jc (the bins are no longer needed: sort scratch)
  if (n <= NT) {
    rank_sort_desc<NT, true>(H.cv, H.ct, n, reinterpret_cast<float*>(H.hw),
                             reinterpret_cast<int*>(H.hw) + kHistCap);
  } else {
    const int n2 = pow2_at_least(n);
    for (int i = n + tid; i < n2; i += NT) {
      H.cv[i] = neg_inf();
      H.ct[i] = INT32_MAX;
    }
    __syncthreads();
    sort_desc<NT, true>(H.cv, H.ct, n2);
  }
  for (int i = tid; i < n; i += NT) H.pw[i] = to_fix(__builtin_amdgcn_exp2f(fmaf(H.cv[i], wa, wb)));
  if (tid == 0) H.cs = 0;  // jc's first group is kept
  __syncthreads();
  block_scan_fix<NT>(H.pw, n, H.above, H.wt);
  int best = 0;
  for (int i = tid; i < n; i += NT)
    if (i > 0 && H.cv[i] != H.cv[i - 1] && H.pw[i - 1] < T) best = i;
  if (best > 0) atomicMax(&H.cs, best);
  __syncthreads();
  const float thr = H.cv[H.cs];
  // the cut group ends where the values fall below thr; its kept tokens add
  // to their chunks' weight
  for (int i = tid; i < n; i += NT)
    if (H.cv[i] >= thr) {
      if constexpr (CW) atomicAdd(&H.cw[H.ct[i] / kChunk], to_fix(__builtin_amdgcn_exp2f(fmaf(H.cv[i], wa, wb))));
      if (i + 1 == n || H.cv[i + 1] < thr) {
        H.thr = thr;
        H.s_kept = static_cast<float>(H.pw[i]) * (1.0f / kFix);
      }
    }
  __syncthreads();
  return true;
}

}  // namespace dspark
