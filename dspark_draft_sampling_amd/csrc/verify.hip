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
//  1. verify_rows   grid (row slices, B (gamma+1) rows).  Each workgroup pulls
//     one slice of one target row into registers with 16-byte loads, then
//     reduces max / lowest argmax / sum exp((l - max) / T) over it.
//  2. verify_decide grid (chunk slices, B).  Every workgroup of a request
//     combines the row partials and replays the (cheap, deterministic) accept
//     scan, so all of them agree on the row to sample from.  Each then scores
//     its slice of 256-token chunks for the two-level Gumbel-max draw; the last
//     workgroup to finish (atomic ticket) picks the chunk and the token inside
//     it and writes the outputs.  The tickets are armed by the first launch.
#include "common.hpp"
#include "internal.hpp"

namespace dspark {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kVecIters = 8;      // 16-byte loads per thread per row slice
constexpr int kScalarIters = 32;  // scalar loads per thread per row slice
constexpr int kMaxSlices2 = 8;    // chunk slices per request in the decide pass

template <typename T, bool VEC>
struct RowLoad;

template <>
struct RowLoad<uint16_t, true> {
  static constexpr int EPL = 8;
  __device__ static void load(const uint16_t* row, int e, int hi, float* o) {
    if (e < hi) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + e);
      o[0] = bf_lo(u.x);
      o[1] = bf_hi(u.x);
      o[2] = bf_lo(u.y);
      o[3] = bf_hi(u.y);
      o[4] = bf_lo(u.z);
      o[5] = bf_hi(u.z);
      o[6] = bf_lo(u.w);
      o[7] = bf_hi(u.w);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = neg_inf();
    }
  }
};

template <>
struct RowLoad<float, true> {
  static constexpr int EPL = 4;
  __device__ static void load(const float* row, int e, int hi, float* o) {
    if (e < hi) {
      const float4 u = *reinterpret_cast<const float4*>(row + e);
      o[0] = u.x;
      o[1] = u.y;
      o[2] = u.z;
      o[3] = u.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = neg_inf();
    }
  }
};

template <typename T>
struct RowLoad<T, false> {
  static constexpr int EPL = 1;
  __device__ static void load(const T* row, int e, int hi, float* o) {
    o[0] = e < hi ? load_logit(row, e) : neg_inf();
  }
};

__device__ __forceinline__ int32_t n_draft_of(const int32_t* n_draft, int b, int gamma) {
  int nd = n_draft ? n_draft[b] : gamma;
  return nd < 0 ? 0 : (nd > gamma ? gamma : nd);
}

// ---------------------------------------------------------------------------
// Pass 1: per (row, slice) max, lowest argmax and sum of exp((l - max) / T).
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void verify_rows_kernel(
    const T* __restrict__ target, int32_t V, int32_t gamma, int32_t slice_len, int32_t S,
    const uint8_t* __restrict__ mode, const float* __restrict__ temperature,
    const int32_t* __restrict__ n_draft, RowPart* __restrict__ part,
    uint32_t* __restrict__ counters, int32_t B) {
  using L = RowLoad<T, VEC>;
  constexpr int ITERS = VEC ? kVecIters : kScalarIters;
  constexpr int EPL = L::EPL;
  constexpr int N = ITERS * EPL;
  __shared__ float shv[kWaves];
  __shared__ int32_t shi[kWaves];
  __shared__ uint32_t shu[kWaves];

  const int G1 = gamma + 1;
  const int s = blockIdx.x, row = blockIdx.y;
  // arm the per-request tickets of the decide pass (which starts after this
  // launch completes on the same stream)
  if (s == 0 && row == 0)
    for (int i = threadIdx.x; i < B; i += kThreads) counters[i] = 0u;
  const int b = row / G1, k = row - b * G1;
  if (k > n_draft_of(n_draft, b, gamma)) return;  // never consulted
  const T* rp = target + static_cast<size_t>(row) * V;
  const int lo = s * slice_len;
  const int hi = min(V, lo + slice_len);

  float v[N];
#pragma unroll
  for (int it = 0; it < ITERS; ++it)
    L::load(rp, lo + (it * kThreads + static_cast<int>(threadIdx.x)) * EPL, hi, v + it * EPL);

  const float Tb = temperature[b];
  const bool sampled = mode[b] != 0 && !bad_temperature(Tb);

  float m = neg_inf();
  int32_t arg = INT32_MAX;
  uint32_t nan = 0;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float x = v[it * EPL + e];
      if (x > m) {
        m = x;
        arg = lo + (it * kThreads + static_cast<int>(threadIdx.x)) * EPL + e;
      }
      if (!sampled) nan |= (x != x) ? 1u : 0u;
    }
  }
  const ArgMax am = block_argmax<kWaves>(ArgMax{m, arg}, shv, shi);

  float sum = 0.0f;
  if (sampled && am.v > neg_inf()) {
    const float cT = kLog2e / Tb;
#pragma unroll
    for (int j = 0; j < N; ++j) sum += __builtin_amdgcn_exp2f((v[j] - am.v) * cT);
    sum = block_sum<kWaves>(sum, shv);
  }
  if (!sampled) nan = block_or<kWaves>(nan, shu);
  if (threadIdx.x == 0) {
    uint32_t fl = 0;
    if (nan || am.v == pos_inf() || (sampled && !(sum < pos_inf()))) fl |= DSPARK_FLAG_NONFINITE;
    part[static_cast<size_t>(row) * S + s] = RowPart{am.v, sum, am.i, fl};
  }
}

// ---------------------------------------------------------------------------
// Pass 2: decision, chunk scores of the residual / bonus draw, final pick.
struct Decision {
  int kind;      // 0 greedy, 1 residual at j, 2 bonus
  int n;         // accepted proposals
  int srow;      // target row sampled from (kind 1, 2)
  int qrow;      // proposal row of the residual (kind 1)
  uint32_t near; // bit k: NEAR on target row k
  int32_t token; // greedy: the emitted target token
};

template <typename T>
__device__ __forceinline__ float draw_weight(int kind, const T* trow, const float* qrow, int v,
                                             float m, float cT, float inv_s, float lse_q,
                                             float thr_q) {
  const float l = load_logit(trow, v);
  const float e = __builtin_amdgcn_exp2f((l - m) * cT);
  if (kind != 1) return e;  // bonus / fallback: unnormalised p
  const float zq = qrow[v];
  const float q = (zq >= thr_q && zq > neg_inf()) ? __builtin_amdgcn_exp2f((zq - lse_q) * kLog2e) : 0.0f;
  return fmaxf(e * inv_s - q, 0.0f);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void verify_decide_kernel(
    const T* __restrict__ target, const int32_t* __restrict__ draft,
    const float* __restrict__ q_z, const float* __restrict__ q_lse,
    const float* __restrict__ q_thr, const float* __restrict__ q_tok,
    const int32_t* __restrict__ n_draft, const uint8_t* __restrict__ mode,
    const float* __restrict__ temperature, const uint32_t* __restrict__ request_id,
    const int32_t* __restrict__ position, uint64_t seed, int32_t gamma, int32_t V, int32_t S,
    int32_t S2, int32_t cps, const RowPart* __restrict__ part, Pick* __restrict__ picks,
    uint32_t* __restrict__ counters, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ out_tokens, uint8_t* __restrict__ flags) {
  __shared__ float rm[DSPARK_MAX_GAMMA + 1], rs[DSPARK_MAX_GAMMA + 1];
  __shared__ int32_t rarg[DSPARK_MAX_GAMMA + 1];
  __shared__ uint32_t rfl[DSPARK_MAX_GAMMA + 1];
  __shared__ Decision dec;
  __shared__ float shv[kWaves], shv2[kWaves];
  __shared__ int32_t shi[kWaves];
  __shared__ int sh_last;
  __shared__ Top2 sh_best;

  const int G1 = gamma + 1;
  const int b = blockIdx.y, s2 = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nd = n_draft_of(n_draft, b, gamma);
  const float Tb = temperature[b];
  const bool want_sampled = mode[b] != 0 && !bad_temperature(Tb);
  const bool sampled = want_sampled && q_z && q_lse && q_thr && q_tok;
  const float cT = sampled ? kLog2e / Tb : kLog2e;
  const int C = (V + kChunk - 1) / kChunk;

  // 1. combine the row partials of rows 0..n_d
  if (tid <= nd) {
    const RowPart* p = part + static_cast<size_t>(b * G1 + tid) * S;
    float m = neg_inf(), s = 0.0f;
    int32_t arg = INT32_MAX;
    uint32_t fl = 0;
    for (int i = 0; i < S; ++i) {
      const RowPart q = p[i];
      fl |= q.flags;
      const ArgMax a = better(ArgMax{m, arg}, ArgMax{q.m, q.arg});
      if (sampled) {
        if (q.m > m) {
          s = s * __builtin_amdgcn_exp2f((m - q.m) * cT) + q.s;
        } else if (q.m > neg_inf()) {
          s += q.s * __builtin_amdgcn_exp2f((q.m - m) * cT);
        }
      }
      m = a.v;
      arg = a.i;
    }
    if (!(m > neg_inf())) fl |= DSPARK_FLAG_EMPTY_ROW;
    rm[tid] = m;
    rs[tid] = s;
    rarg[tid] = arg;
    rfl[tid] = fl;
  }
  __syncthreads();

  // 2. the decision (identical in every workgroup of the request)
  if (tid == 0) {
    Decision d{};
    d.near = 0;
    if (!sampled) {
      int n = nd;
      for (int k = 1; k <= nd; ++k) {
        const int32_t x = clamp_token(draft[b * gamma + k - 1], V);
        const int32_t t = rarg[k - 1] == INT32_MAX ? 0 : rarg[k - 1];
        if (x != t) {
          n = k - 1;
          break;
        }
      }
      d.kind = 0;
      d.n = n;
      d.token = rarg[n] == INT32_MAX ? 0 : rarg[n];
    } else {
      const uint32_t req = request_id[b];
      const int32_t pos0 = position[b];
      int j = 0;
      for (int k = 1; k <= nd; ++k) {
        const int32_t x = clamp_token(draft[b * gamma + k - 1], V);
        const float lx = load_logit(target, static_cast<size_t>(b * G1 + k - 1) * V + x);
        const float p = (lx > neg_inf() && rs[k - 1] > 0.0f)
                            ? expf((lx - rm[k - 1]) / Tb) / rs[k - 1]
                            : 0.0f;
        const float q = q_tok[b * gamma + k - 1];
        const float u = accept_uniform(seed, pos0 + k, req);
        bool acc;
        if (q > 0.0f) {
          const float rho = p / q;
          acc = u < rho;
          if (fabsf(u - rho) <= kNearEps) d.near |= 1u << (k - 1);
        } else {
          acc = p > 0.0f;
        }
        if (!acc) {
          j = k;
          break;
        }
      }
      if (j > 0) {
        d.kind = 1;
        d.n = j - 1;
        d.srow = j - 1;
        d.qrow = j - 1;
      } else {
        d.kind = 2;
        d.n = nd;
        d.srow = nd;
        d.qrow = 0;
      }
      d.token = 0;
    }
    dec = d;
  }
  __syncthreads();
  const Decision d = dec;

  auto write_outputs = [&](int32_t emitted, uint32_t extra_row_flags, int extra_row) {
    // thread 0 only
    int32_t* out = out_tokens + static_cast<size_t>(b) * G1;
    for (int i = 0; i < G1; ++i) {
      int32_t t = -1;
      if (i < d.n) t = clamp_token(draft[b * gamma + i], V);
      else if (i == d.n) t = emitted;
      out[i] = t;
      uint32_t fl = 0;
      if (i <= nd) {
        fl = rfl[i] & (DSPARK_FLAG_NONFINITE | DSPARK_FLAG_EMPTY_ROW);
        if (d.near & (1u << i)) fl |= DSPARK_FLAG_NEAR_THRESHOLD;
        if (i == extra_row) fl |= extra_row_flags;
      }
      if (i == 0 && mode[b] != 0 && !sampled) fl |= DSPARK_FLAG_BAD_POLICY;
      flags[static_cast<size_t>(b) * G1 + i] = static_cast<uint8_t>(fl);
    }
    accept_len[b] = d.n;
  };

  if (d.kind == 0) {
    if (s2 == 0 && tid == 0) write_outputs(d.token, 0, -1);
    return;
  }

  // 3. chunk scores of this workgroup's chunk slice
  const uint32_t req = request_id[b];
  const int32_t pos = position[b] + (d.kind == 1 ? d.n + 1 : nd + 1);
  const T* trow = target + static_cast<size_t>(b * G1 + d.srow) * V;
  const float* qrow = d.kind == 1 ? q_z + static_cast<size_t>(b * gamma + d.qrow) * V : nullptr;
  const float m = rm[d.srow];
  const float inv_s = rs[d.srow] > 0.0f ? 1.0f / rs[d.srow] : 0.0f;
  const float lse_q = d.kind == 1 ? q_lse[b * gamma + d.qrow] : 0.0f;
  const float thr_q = d.kind == 1 ? q_thr[b * gamma + d.qrow] : 0.0f;

  auto chunk_scores = [&](int kind, int c_lo, int c_hi) -> Top2 {
    Top2 best{neg_inf(), INT32_MAX, neg_inf()};
    for (int c = c_lo + wave; c < c_hi; c += kWaves) {
      float w = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = c * kChunk + lane * 4 + e;
        if (v < V) w += draw_weight(kind, trow, qrow, v, m, cT, inv_s, lse_q, thr_q);
      }
      w = wave_sum(w);
      const float sc = w > 0.0f ? logf(w) + gumbel(seed, static_cast<uint32_t>(c), pos, req,
                                                   DSPARK_TAG_TARGET_CHUNK)
                                : neg_inf();
      best = top2_merge(best, Top2{sc, w > 0.0f ? c : INT32_MAX, neg_inf()});
    }
    return block_top2<kWaves>(best, shv, shi, shv2);
  };

  const int c_lo = s2 * cps, c_hi = min(C, c_lo + cps);
  const Top2 mine = chunk_scores(d.kind, c_lo, c_hi);
  if (tid == 0) {
    picks[static_cast<size_t>(b) * S2 + s2] = Pick{mine.v1, mine.i1, mine.v2, 0u};
    __threadfence();
    const uint32_t prev = atomicAdd(&counters[b], 1u);
    sh_last = (prev == static_cast<uint32_t>(S2 - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!sh_last) return;

  // 4. last workgroup of the request: pick the chunk, then the token
  __threadfence();
  if (tid == 0) {
    Top2 best{neg_inf(), INT32_MAX, neg_inf()};
    for (int i = 0; i < S2; ++i) {
      const Pick p = picks[static_cast<size_t>(b) * S2 + i];
      best = top2_merge(best, Top2{p.v1, p.i1, p.v2});
    }
    sh_best = best;
  }
  __syncthreads();
  Top2 best = sh_best;
  int kind = d.kind;
  uint32_t row_flags = 0;
  if (best.i1 == INT32_MAX && kind == 1) {
    // max(p - q, 0) has no mass (only reachable by rounding): draw from p
    kind = 3;
    row_flags |= DSPARK_FLAG_RESIDUAL_ZERO;
    best = chunk_scores(3, 0, C);
  }
  if (best.i1 != INT32_MAX && best.v2 > neg_inf() && near_gap(best.v1, best.v2))
    row_flags |= DSPARK_FLAG_NEAR_THRESHOLD;

  Top2 tok{neg_inf(), INT32_MAX, neg_inf()};
  if (best.i1 != INT32_MAX) {
    const int v = best.i1 * kChunk + tid;
    if (v < V) {
      float lw;
      if (kind == 1) {
        const float w = draw_weight(1, trow, qrow, v, m, cT, inv_s, lse_q, thr_q);
        lw = w > 0.0f ? logf(w) : neg_inf();
      } else {
        const float l = load_logit(trow, v);
        lw = l > neg_inf() ? (l - m) / Tb : neg_inf();
      }
      if (lw > neg_inf())
        tok = Top2{lw + gumbel(seed, static_cast<uint32_t>(v), pos, req, DSPARK_TAG_TARGET_TOKEN),
                   v, neg_inf()};
    }
  }
  tok = block_top2<kWaves>(tok, shv, shi, shv2);
  if (tid == 0) {
    if (tok.i1 != INT32_MAX && tok.v2 > neg_inf() && near_gap(tok.v1, tok.v2))
      row_flags |= DSPARK_FLAG_NEAR_THRESHOLD;
    const int32_t emitted = tok.i1 == INT32_MAX ? 0 : tok.i1;
    write_outputs(emitted, row_flags, d.srow);
  }
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
  const dim3 g1(pl.S, B * (gamma + 1));
  {
  ProfScope ps("verify_rows", st);
  if (pl.vec)
    hipLaunchKernelGGL((verify_rows_kernel<T, true>), g1, dim3(kThreads), 0, st, target, V, gamma,
                       pl.slice_len, pl.S, pol.mode, pol.temperature, n_draft, part, cnt, B);
  else
    hipLaunchKernelGGL((verify_rows_kernel<T, false>), g1, dim3(kThreads), 0, st, target, V,
                       gamma, pl.slice_len, pl.S, pol.mode, pol.temperature, n_draft, part, cnt,
                       B);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ProfScope ps("verify_decide", st);
  hipLaunchKernelGGL((verify_decide_kernel<T>), dim3(pl.S2, B), dim3(kThreads), 0, st, target,
                     draft, q_z, q_lse, q_thr, q_tok, n_draft, pol.mode, pol.temperature,
                     pol.request_id, pol.position, seed, gamma, V, pl.S, pl.S2, pl.cps, part,
                     picks, cnt, accept_len, out_tokens, flags);
  return hipGetLastError();
}

}  // namespace

VerifyPlan plan_verify(int dtype, int32_t B, int32_t gamma, int32_t V, bool aligned) {
  VerifyPlan p{};
  const int epl16 = dtype == DSPARK_BF16 ? 8 : 4;
  p.vec = (aligned && V % epl16 == 0) ? 1 : 0;
  const int epl = p.vec ? epl16 : 1;
  p.slice_len = (p.vec ? kVecIters : kScalarIters) * kThreads * epl;
  p.S = (V + p.slice_len - 1) / p.slice_len;
  const int C = (V + kChunk - 1) / kChunk;
  const int S2 = C < kMaxSlices2 ? C : kMaxSlices2;
  p.cps = (C + S2 - 1) / S2;
  p.S2 = (C + p.cps - 1) / p.cps;
  size_t off = 0;
  p.off_part = off;
  off = align_up(off + static_cast<size_t>(B) * (gamma + 1) * p.S * sizeof(RowPart), 256);
  p.off_pick = off;
  off = align_up(off + static_cast<size_t>(B) * p.S2 * sizeof(Pick), 256);
  p.off_cnt = off;
  off = align_up(off + static_cast<size_t>(B) * sizeof(uint32_t), 256);
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
