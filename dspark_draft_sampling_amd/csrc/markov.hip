// markov.hip — left-to-right Markov draft sampling on gfx950.
//
// Semantics ("[2/3] feat(dsv4): implement exact DSpark speculative decoding",
// "Checkpoint-faithful DSpark architecture"; "DSpark Speculative Decoding
// (Draft Training) Design", "Semi-autoregressive draft"): for k = 1..gamma in
// order, y_k = backbone row k-1 + A[x_{k-1}] . B (a rank-r additive bias, x_0 the
// anchor), q_k = policy(y_k), x_k ~ q_k (argmax for greedy requests); the full
// q_k and the confidence c_k = sigmoid(w . [h_k ; embed(x_{k-1})]) are kept.
//
// Each step k is two launches:
//  * markov_step: one workgroup per (256-token chunk, 64-request tile).  The
//    bias tile bias[v, b] = sum_i W2[v, i] W1[x_{k-1}(b), i] is a bf16 MFMA
//    product (v_mfma_f32_16x16x32_bf16) with the vocabulary as the M side, so
//    each lane's accumulators hold 4 consecutive tokens of one request and the
//    epilogue reads the backbone with 8-byte loads and writes z = y / T with
//    16-byte stores.  The epilogue also reduces each request's chunk to
//    (max z, lowest argmax, sum exp(z - max)) for the sampler.
//  * markov_finalize: one workgroup per request.  Combines the chunk partials
//    into the log-normaliser, picks the chunk by Gumbel-max over the chunk
//    log-masses and the token inside it by Gumbel-max over its 256 z values
//    (two-level Gumbel-max: exact, no prefix sum over the vocabulary), and
//    evaluates the confidence head.
#include "common.hpp"
#include "internal.hpp"

namespace dspark {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;          // requests per workgroup tile (MFMA N side)
constexpr int kStepThreads = 512;  // 8 waves, 32 tokens each
constexpr int kStepWaves = kStepThreads / 64;
constexpr int kMaxR = DSPARK_MAX_RANK;
constexpr int kPad = 8;            // bf16 padding per staged W1 row (bank spread)
constexpr int kFinThreads = 256;
constexpr int kFinWaves = kFinThreads / 64;

template <typename T, bool VEC>
struct Quad;  // four consecutive logits starting at a multiple of 4

template <>
struct Quad<uint16_t, true> {
  __device__ static void load(const uint16_t* p, float* o) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    o[0] = bf_lo(u.x);
    o[1] = bf_hi(u.x);
    o[2] = bf_lo(u.y);
    o[3] = bf_hi(u.y);
  }
};
template <>
struct Quad<float, true> {
  __device__ static void load(const float* p, float* o) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    o[0] = u.x;
    o[1] = u.y;
    o[2] = u.z;
    o[3] = u.w;
  }
};
template <typename T>
struct Quad<T, false> {
  __device__ static void load(const T* p, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = load_logit(p, i);
  }
};

__device__ __forceinline__ bf16x8 load_frag(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kStepThreads) void markov_step_kernel(
    const T* __restrict__ backbone, const int32_t* __restrict__ xprev, int32_t xstride,
    const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w2,
    const uint8_t* __restrict__ mode, const float* __restrict__ temperature, int32_t B,
    int32_t gamma, int32_t k, int32_t V, int32_t r, int32_t C, float* __restrict__ q_z,
    ChunkPart* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t a_lds[kTile * (kMaxR + kPad)];
  __shared__ float red_m[kStepWaves][kTile], red_s[kStepWaves][kTile];
  __shared__ int32_t red_i[kStepWaves][kTile];
  __shared__ uint32_t red_f[kStepWaves][kTile];

  const int c = blockIdx.x;
  const int b0 = blockIdx.y * kTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kpad = (r + 31) & ~31;
  const int ld = kpad + kPad;
  const int ksteps = kpad / 32;

  // W2 fragments of this wave's 32 tokens (MFMA A operand: token rows, K slices)
  const int vb = c * kChunk + wave * 32;
  bf16x8 af[2][kMaxR / 32];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) {
    const int v = vb + ms * 16 + (lane & 15);
#pragma unroll
    for (int ks = 0; ks < kMaxR / 32; ++ks) {
      const int k0 = ks * 32 + (lane >> 4) * 8;
      bf16x8 f = {};
      if (ks < ksteps && v < V && k0 < r) f = load_frag(w2 + static_cast<size_t>(v) * r + k0);
      af[ms][ks] = f;
    }
  }

  // stage the gathered W1 rows of the tile's requests (MFMA B operand)
  const int pieces = kpad / 8;
  for (int idx = tid; idx < kTile * pieces; idx += kStepThreads) {
    const int row = idx / pieces, pc = idx - row * pieces;
    const int b = b0 + row;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (b < B && pc * 8 < r) {
      const int32_t x = clamp_token(xprev[static_cast<size_t>(b) * xstride], V);
      val = *reinterpret_cast<const uint4*>(w1 + static_cast<size_t>(x) * r + pc * 8);
    }
    *reinterpret_cast<uint4*>(a_lds + row * ld + pc * 8) = val;
  }
  __syncthreads();

  f32x4 acc[2][4];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kMaxR / 32; ++ks) {
    if (ks < ksteps) {
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        const bf16x8 bfr =
            load_frag(a_lds + (ns * 16 + (lane & 15)) * ld + ks * 32 + (lane >> 4) * 8);
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
          acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ms][ks], bfr, acc[ms][ns], 0, 0, 0);
      }
    }
  }

  // epilogue: lane holds tokens vb + ms*16 + 4*(lane>>4) + i of request ns*16 + (lane&15)
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    const int n = ns * 16 + (lane & 15);
    const int b = b0 + n;
    const bool bvalid = b < B;
    float invT = 1.0f;
    bool sampled = false;
    if (bvalid) {
      const float Tb = temperature[b];
      sampled = mode[b] != 0 && !bad_temperature(Tb);
      if (sampled) invT = 1.0f / Tb;
    }
    const size_t rowoff = (static_cast<size_t>(bvalid ? b : 0) * gamma + (k - 1)) * V;
    float z[8];
    int32_t zi[8];
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
      const int v0 = vb + ms * 16 + 4 * (lane >> 4);
      float bb[4] = {0.f, 0.f, 0.f, 0.f};
      const bool full = bvalid && v0 + 3 < V;
      if (full) {
        Quad<T, VEC>::load(backbone + rowoff + v0, bb);
      } else if (bvalid) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (v0 + i < V) bb[i] = load_logit(backbone, rowoff + v0 + i);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool in = bvalid && v0 + i < V;
        z[ms * 4 + i] = in ? (acc[ms][ns][i] + bb[i]) * invT : neg_inf();
        zi[ms * 4 + i] = v0 + i;
      }
      if (sampled) {
        float* dst = q_z + rowoff + v0;
        if (VEC && full) {
          *reinterpret_cast<float4*>(dst) =
              make_float4(z[ms * 4], z[ms * 4 + 1], z[ms * 4 + 2], z[ms * 4 + 3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (v0 + i < V) dst[i] = z[ms * 4 + i];
        }
      }
    }
    // reduce over this lane's 8 tokens, then over the 4 lane groups sharing n
    float m = neg_inf();
    int32_t arg = INT32_MAX;
    uint32_t bad = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (z[j] > m) {
        m = z[j];
        arg = zi[j];
      }
      bad |= (z[j] != z[j] || z[j] == pos_inf()) ? 1u : 0u;
    }
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      const ArgMax other{__shfl_xor(m, o, 64), __shfl_xor(arg, o, 64)};
      const ArgMax a = better(ArgMax{m, arg}, other);
      m = a.v;
      arg = a.i;
      bad |= __shfl_xor(bad, o, 64);
    }
    float s = 0.0f;
    if (m > neg_inf() && m < pos_inf()) {
#pragma unroll
      for (int j = 0; j < 8; ++j) s += __builtin_amdgcn_exp2f((z[j] - m) * kLog2e);
    }
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) s += __shfl_xor(s, o, 64);
    if (lane < 16) {
      red_m[wave][n] = m;
      red_s[wave][n] = s;
      red_i[wave][n] = arg;
      red_f[wave][n] = bad;
    }
  }
  __syncthreads();
  if (tid < kTile && b0 + tid < B) {
    float m = red_m[0][tid], s = red_s[0][tid];
    ArgMax a{red_m[0][tid], red_i[0][tid]};
    uint32_t bad = red_f[0][tid];
#pragma unroll
    for (int w = 1; w < kStepWaves; ++w) {
      lse_merge(m, s, red_m[w][tid], red_s[w][tid]);
      a = better(a, ArgMax{red_m[w][tid], red_i[w][tid]});
      bad |= red_f[w][tid];
    }
    part[static_cast<size_t>(b0 + tid) * C + c] =
        ChunkPart{m, s, a.i, bad ? static_cast<uint32_t>(DSPARK_FLAG_NONFINITE) : 0u};
  }
}

__global__ __launch_bounds__(kFinThreads) void markov_finalize_kernel(
    const int32_t* __restrict__ xprev, int32_t xstride, const uint16_t* __restrict__ hidden,
    const uint16_t* __restrict__ embed, const float* __restrict__ conf_w,
    const uint8_t* __restrict__ mode, const float* __restrict__ temperature,
    const uint32_t* __restrict__ request_id, const int32_t* __restrict__ position,
    uint64_t seed, int32_t gamma, int32_t k, int32_t V, int32_t d, int32_t C,
    const ChunkPart* __restrict__ part, const float* __restrict__ q_z,
    int32_t* __restrict__ draft_tokens, float* __restrict__ q_lse, float* __restrict__ q_thr,
    float* __restrict__ q_tok, float* __restrict__ confidence, uint8_t* __restrict__ flags) {
  __shared__ float shv[kFinWaves], shv2[kFinWaves];
  __shared__ int32_t shi[kFinWaves];
  __shared__ uint32_t shu[kFinWaves];
  __shared__ float sh_zx;

  const int b = blockIdx.x, tid = threadIdx.x;
  const size_t row = static_cast<size_t>(b) * gamma + (k - 1);
  const float Tb = temperature[b];
  const bool sampled = mode[b] != 0 && !bad_temperature(Tb);
  const uint32_t req = request_id[b];
  const int32_t pos = position[b] + k;

  float m = neg_inf(), s = 0.0f;
  ArgMax am{neg_inf(), INT32_MAX};
  uint32_t fl = 0;
  Top2 best{neg_inf(), INT32_MAX, neg_inf()};
  for (int c = tid; c < C; c += kFinThreads) {
    const ChunkPart p = part[static_cast<size_t>(b) * C + c];
    fl |= p.flags;
    am = better(am, ArgMax{p.m, p.arg});
    lse_merge(m, s, p.m, p.s);
    if (sampled && p.m > neg_inf() && p.s > 0.0f) {
      const float sc = p.m + logf(p.s) +
                       gumbel(seed, static_cast<uint32_t>(c), pos, req, DSPARK_TAG_DRAFT_CHUNK);
      best = top2_merge(best, Top2{sc, c, neg_inf()});
    }
  }
  am = block_argmax<kFinWaves>(am, shv, shi);
  const float M = block_max<kFinWaves>(m, shv);
  const float S = block_sum<kFinWaves>(
      (m > neg_inf() && M < pos_inf()) ? s * __builtin_amdgcn_exp2f((m - M) * kLog2e) : 0.0f, shv);
  fl = block_or<kFinWaves>(fl, shu);

  int32_t x = 0;
  uint32_t near = 0;
  if (!sampled) {
    if (am.i == INT32_MAX) fl |= DSPARK_FLAG_EMPTY_ROW;
    else x = am.i;
  } else {
    best = block_top2<kFinWaves>(best, shv, shi, shv2);
    if (best.i1 == INT32_MAX) {
      fl |= DSPARK_FLAG_EMPTY_ROW;
    } else {
      if (best.v2 > neg_inf() && near_gap(best.v1, best.v2)) near = 1;
      const int v = best.i1 * kChunk + tid;
      Top2 tok{neg_inf(), INT32_MAX, neg_inf()};
      if (v < V) {
        const float z = q_z[row * V + v];
        if (z > neg_inf())
          tok = Top2{z + gumbel(seed, static_cast<uint32_t>(v), pos, req, DSPARK_TAG_DRAFT_TOKEN),
                     v, neg_inf()};
      }
      tok = block_top2<kFinWaves>(tok, shv, shi, shv2);
      if (tok.i1 == INT32_MAX) {
        fl |= DSPARK_FLAG_EMPTY_ROW;
      } else {
        x = tok.i1;
        if (tok.v2 > neg_inf() && near_gap(tok.v1, tok.v2)) near = 1;
      }
    }
  }

  // confidence head on [h_k ; embed(x_{k-1})]
  const int32_t xp = clamp_token(xprev[static_cast<size_t>(b) * xstride], V);
  const uint16_t* h = hidden + row * d;
  const uint16_t* e = embed + static_cast<size_t>(xp) * d;
  float dot = 0.0f;
  for (int i = tid; i < d; i += kFinThreads)
    dot += conf_w[i] * load_logit(h, i) + conf_w[d + i] * load_logit(e, i);
  dot = block_sum<kFinWaves>(dot, shv);

  if (tid == 0) {
    draft_tokens[row] = x;
    if (sampled) {
      const float zx = q_z[row * V + x];
      q_lse[row] = M + logf(S);
      q_thr[row] = neg_inf();
      q_tok[row] = (zx > neg_inf() && S > 0.0f) ? expf(zx - M) / S : 0.0f;
    } else {
      q_lse[row] = 0.0f;
      q_thr[row] = 0.0f;
      q_tok[row] = 1.0f;
    }
    confidence[row] = 1.0f / (1.0f + expf(-dot));
    if (near) fl |= DSPARK_FLAG_NEAR_THRESHOLD;
    if (mode[b] != 0 && !sampled) fl |= DSPARK_FLAG_BAD_POLICY;
    flags[row] = static_cast<uint8_t>(fl);
  }
  (void)sh_zx;
}

template <typename T>
hipError_t launch_typed(const T* backbone, const int32_t* anchor, const uint16_t* w1,
                        const uint16_t* w2, const uint16_t* hidden, const uint16_t* embed,
                        const float* conf_w, dspark_policy pol, uint64_t seed, int32_t B,
                        int32_t gamma, int32_t V, int32_t r, int32_t d, int32_t* draft_tokens,
                        float* q_z, float* q_lse, float* q_thr, float* q_tok, float* confidence,
                        uint8_t* flags, void* ws, const MarkovPlan& pl, hipStream_t st) {
  ChunkPart* part = reinterpret_cast<ChunkPart*>(static_cast<char*>(ws) + pl.off_part);
  const bool vec = (V % 4 == 0) && (reinterpret_cast<uintptr_t>(backbone) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(q_z) % 16 == 0);
  const dim3 g_step(pl.C, (B + kTile - 1) / kTile);
  for (int k = 1; k <= gamma; ++k) {
    const int32_t* xp = k == 1 ? anchor : draft_tokens + (k - 2);
    const int32_t xs = k == 1 ? 1 : gamma;
    if (vec)
      DSPARK_LAUNCH("markov_step", (markov_step_kernel<T, true>), g_step, dim3(kStepThreads), 0,
                    st, backbone, xp, xs, w1, w2, pol.mode, pol.temperature, B, gamma, k, V, r,
                    pl.C, q_z, part);
    else
      DSPARK_LAUNCH("markov_step", (markov_step_kernel<T, false>), g_step, dim3(kStepThreads), 0,
                    st, backbone, xp, xs, w1, w2, pol.mode, pol.temperature, B, gamma, k, V, r,
                    pl.C, q_z, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    DSPARK_LAUNCH("markov_finalize", markov_finalize_kernel, dim3(B), dim3(kFinThreads), 0, st, xp,
                  xs, hidden, embed, conf_w, pol.mode, pol.temperature, pol.request_id,
                  pol.position, seed, gamma, k, V, d, pl.C, part, q_z, draft_tokens, q_lse, q_thr,
                  q_tok, confidence, flags);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

MarkovPlan plan_markov(int32_t B, int32_t gamma, int32_t V, int32_t r, int32_t d) {
  (void)gamma;
  (void)r;
  (void)d;
  MarkovPlan p{};
  p.C = (V + kChunk - 1) / kChunk;
  p.off_part = 0;
  p.bytes = align_up(static_cast<size_t>(B) * p.C * sizeof(ChunkPart), 256);
  return p;
}

hipError_t launch_markov(const void* backbone, int dtype, const int32_t* anchor,
                         const uint16_t* w1, const uint16_t* w2, const uint16_t* hidden,
                         const uint16_t* embed, const float* conf_w, dspark_policy pol,
                         uint64_t seed, int32_t B, int32_t gamma, int32_t V, int32_t r, int32_t d,
                         int32_t* draft_tokens, float* q_z, float* q_lse, float* q_thr,
                         float* q_tok, float* confidence, uint8_t* flags, void* ws,
                         const MarkovPlan& plan, hipStream_t st) {
  if (dtype == DSPARK_BF16)
    return launch_typed(static_cast<const uint16_t*>(backbone), anchor, w1, w2, hidden, embed,
                        conf_w, pol, seed, B, gamma, V, r, d, draft_tokens, q_z, q_lse, q_thr,
                        q_tok, confidence, flags, ws, plan, st);
  return launch_typed(static_cast<const float*>(backbone), anchor, w1, w2, hidden, embed, conf_w,
                      pol, seed, B, gamma, V, r, d, draft_tokens, q_z, q_lse, q_thr, q_tok,
                      confidence, flags, ws, plan, st);
}

}  // namespace dspark
