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
#include "truncate.hpp"

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

// Four consecutive logits starting at a multiple of 4, kept packed (bf16:
// 8 bytes, fp32: 16 bytes) until the epilogue unpacks them.
template <typename T>
struct QuadRaw;
template <>
struct QuadRaw<uint16_t> {
  uint2 u;
  __device__ void load(const uint16_t* p, bool vec, int n) {
    if (vec && n >= 4) {
      u = *reinterpret_cast<const uint2*>(p);
    } else {
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = i < n ? p[i] : 0u;
      u = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    }
  }
  __device__ float at(int i) const {
    const uint32_t w = i < 2 ? u.x : u.y;
    return (i & 1) ? bf_hi(w) : bf_lo(w);
  }
};
template <>
struct QuadRaw<float> {
  float4 u;
  __device__ void load(const float* p, bool vec, int n) {
    if (vec && n >= 4) {
      u = *reinterpret_cast<const float4*>(p);
    } else {
      u = make_float4(n > 0 ? p[0] : 0.f, n > 1 ? p[1] : 0.f, n > 2 ? p[2] : 0.f, n > 3 ? p[3] : 0.f);
    }
  }
  __device__ float at(int i) const { return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w; }
};

__device__ __forceinline__ bf16x8 load_frag(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kStepThreads) void markov_step_kernel(
    const T* __restrict__ backbone, const int32_t* __restrict__ xprev, int32_t xstride,
    const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w2,
    const uint8_t* __restrict__ mode, const float* __restrict__ temperature,
    const uint32_t* __restrict__ request_id, const int32_t* __restrict__ position, uint64_t seed,
    int32_t B, int32_t gamma, int32_t k, int32_t V, int32_t r, int32_t C, float* __restrict__ q_z,
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

  // prefetch this lane's backbone values (tokens vb + ms*16 + 4*(lane>>4) + i of
  // request ns*16 + (lane&15)) so their latency overlaps the product
  QuadRaw<T> bbv[4][2];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    const int b = b0 + ns * 16 + (lane & 15);
    const size_t rowoff = (static_cast<size_t>(b < B ? b : 0) * gamma + (k - 1)) * V;
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
      const int v0 = vb + ms * 16 + 4 * (lane >> 4);
      const int n = b < B ? (V - v0 < 4 ? (V - v0 > 0 ? V - v0 : 0) : 4) : 0;
      bbv[ns][ms].load(backbone + rowoff + (n > 0 ? v0 : 0), VEC, n);
    }
  }

  // stage the gathered W1 rows of the tile's requests (MFMA B operand): the
  // 64 tokens first, then every 16-byte piece load issued back to back
  __shared__ int32_t xs_lds[kTile];
  if (tid < kTile) {
    const int b = b0 + tid;
    xs_lds[tid] = b < B ? clamp_token(xprev[static_cast<size_t>(b) * xstride], V) : -1;
  }
  __syncthreads();
  const int pieces = kpad / 8;
  constexpr int kMaxPieces = kTile * (kMaxR / 8) / kStepThreads;  // 4
  uint4 stage[kMaxPieces];
#pragma unroll
  for (int j = 0; j < kMaxPieces; ++j) {
    const int idx = tid + j * kStepThreads;
    const int row = idx / pieces, pc = idx - row * pieces;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (row < kTile && pc * 8 < r) {
      const int32_t x = xs_lds[row];
      if (x >= 0) val = *reinterpret_cast<const uint4*>(w1 + static_cast<size_t>(x) * r + pc * 8);
    }
    stage[j] = val;
  }
#pragma unroll
  for (int j = 0; j < kMaxPieces; ++j) {
    const int idx = tid + j * kStepThreads;
    const int row = idx / pieces, pc = idx - row * pieces;
    if (row < kTile) *reinterpret_cast<uint4*>(a_lds + row * ld + pc * 8) = stage[j];
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
      const QuadRaw<T>& bb = bbv[ns][ms];
      const bool full = bvalid && v0 + 3 < V;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool in = bvalid && v0 + i < V;
        z[ms * 4 + i] = in ? (acc[ms][ns][i] + bb.at(i)) * invT : neg_inf();
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
    const int b = b0 + tid;
    float m = red_m[0][tid], s = red_s[0][tid];
    ArgMax a{red_m[0][tid], red_i[0][tid]};
    uint32_t bad = red_f[0][tid];
#pragma unroll
    for (int w = 1; w < kStepWaves; ++w) {
      lse_merge(m, s, red_m[w][tid], red_s[w][tid]);
      a = better(a, ArgMax{red_m[w][tid], red_i[w][tid]});
      bad |= red_f[w][tid];
    }
    // chunk level of the two-level Gumbel-max draw: ln(mass) + chunk noise
    float score = neg_inf();
    const float Tb = temperature[b];
    if (mode[b] != 0 && !bad_temperature(Tb) && m > neg_inf() && m < pos_inf() && s > 0.0f)
      score = m + logf(s) + gumbel(seed, static_cast<uint32_t>(c), position[b] + k, request_id[b],
                                   DSPARK_TAG_DRAFT_CHUNK);
    part[static_cast<size_t>(b) * C + c] =
        ChunkPart{m, s, score, (static_cast<uint32_t>(a.i) & 0x7fffffffu) | (bad ? 0x80000000u : 0u)};
  }
}

// One workgroup per request.  All waves combine the chunk partials; then wave
// 0 draws the token inside the chosen chunk (lane l scores tokens 4l..4l+3 with
// one Philox block) while waves 1-3 evaluate the confidence head.
// One proposal row of scaled logits z (fp32), 4 tokens per load.
struct QzRow {
  const float* p;
  int V;
  bool vec4;
  __device__ float operator()(int v) const { return p[v]; }
  __device__ void load4(int v0, float* o) const {
    if (vec4 && v0 + 3 < V) {
      const float4 u = *reinterpret_cast<const float4*>(p + v0);
      o[0] = u.x;
      o[1] = u.y;
      o[2] = u.z;
      o[3] = u.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = v0 + e < V ? p[v0 + e] : neg_inf();
    }
  }
};

// Level-1 scores of the two-level draw restricted to the kept set
// (z >= thr): for each listed chunk (list[j], or j itself without a list)
// holding kept tokens, log of its kept mass plus the chunk's Gumbel.  Wave w
// takes entries w, w + 4, ...; four chunks' loads are issued together.
// Returns the wave's best two (score, chunk).
__device__ Top2 kept_chunk_scores(const QzRow& qr, int n, const int* list, float thr,
                                  uint64_t seed, int32_t pos, uint32_t req) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  Top2 best{neg_inf(), INT32_MAX, neg_inf()};
  constexpr int kU = 4;
  for (int j0 = wave * kU; j0 < n; j0 += kFinWaves * kU) {
    float z[kU][4];
    int cs[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = j0 + u;
      cs[u] = j < n ? (list ? list[j] : j) : -1;
      if (cs[u] >= 0) {
        qr.load4(cs[u] * kChunk + 4 * lane, z[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) z[u][e] = neg_inf();
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (cs[u] < 0) continue;  // wave-uniform
      float mc = neg_inf();
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (z[u][e] >= thr) mc = fmaxf(mc, z[u][e]);
      mc = wave_max(mc);
      if (!(mc > neg_inf())) continue;
      float w = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (z[u][e] >= thr) w += __builtin_amdgcn_exp2f((z[u][e] - mc) * kLog2e);
      w = wave_sum(w);
      const float score = mc + logf(w) +
                          gumbel(seed, static_cast<uint32_t>(cs[u]), pos, req, DSPARK_TAG_DRAFT_CHUNK);
      best = top2_merge(best, Top2{score, cs[u], neg_inf()});
    }
  }
  return best;
}

template <bool VEC>
__global__ __launch_bounds__(kFinThreads) void markov_finalize_kernel(
    const int32_t* __restrict__ xprev, int32_t xstride, const uint16_t* __restrict__ hidden,
    const uint16_t* __restrict__ embed, const float* __restrict__ conf_w,
    const uint8_t* __restrict__ mode, const float* __restrict__ temperature,
    const int32_t* __restrict__ top_k, const float* __restrict__ top_p,
    const uint32_t* __restrict__ request_id, const int32_t* __restrict__ position,
    uint64_t seed, int32_t gamma, int32_t k, int32_t V, int32_t d, int32_t C, int32_t cvec,
    const ChunkPart* __restrict__ part, const float* __restrict__ q_z,
    int32_t* __restrict__ draft_tokens, float* __restrict__ q_lse, float* __restrict__ q_thr,
    float* __restrict__ q_tok, float* __restrict__ confidence, uint8_t* __restrict__ flags) {
  __shared__ float sh_m[kFinWaves], sh_s[kFinWaves], sh_am[kFinWaves], sh_v1[kFinWaves],
      sh_v2[kFinWaves], sh_dot[kFinWaves];
  __shared__ int32_t sh_ai[kFinWaves], sh_i1[kFinWaves];
  __shared__ uint32_t sh_bad[kFinWaves];
  __shared__ float fin_M, fin_S, fin_zx;
  __shared__ int32_t fin_x;
  __shared__ uint32_t fin_fl;
  __shared__ TruncLds U;

  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t row = static_cast<size_t>(b) * gamma + (k - 1);
  const float Tb = temperature[b];
  const bool sampled = mode[b] != 0 && !bad_temperature(Tb);
  const uint32_t req = request_id[b];
  const int32_t pos = position[b] + k;

  // 1. combine the chunk partials
  float m = neg_inf(), s = 0.0f;
  ArgMax am{neg_inf(), INT32_MAX};
  Top2 best{neg_inf(), INT32_MAX, neg_inf()};
  uint32_t bad = 0;
  for (int c = tid; c < C; c += kFinThreads) {
    const ChunkPart p = part[static_cast<size_t>(b) * C + c];
    const int32_t arg = static_cast<int32_t>(p.arg_nf & 0x7fffffffu);
    bad |= p.arg_nf >> 31;
    am = better(am, ArgMax{p.m, arg == 0x7fffffff ? INT32_MAX : arg});
    lse_merge(m, s, p.m, p.s);
    if (p.score > neg_inf()) best = top2_merge(best, Top2{p.score, c, neg_inf()});
  }
  {
    const float wm = wave_max(m);
    const float ws = wave_sum((m > neg_inf() && wm < pos_inf()) ? s * __builtin_amdgcn_exp2f((m - wm) * kLog2e) : 0.0f);
    const ArgMax wa = wave_argmax(am);
    const Top2 wb = wave_top2(best);
    const uint32_t wbad = wave_or(bad);
    if (lane == 0) {
      sh_m[wave] = wm;
      sh_s[wave] = ws;
      sh_am[wave] = wa.v;
      sh_ai[wave] = wa.i;
      sh_v1[wave] = wb.v1;
      sh_i1[wave] = wb.i1;
      sh_v2[wave] = wb.v2;
      sh_bad[wave] = wbad;
    }
  }
  __syncthreads();
  float M = sh_m[0], S = sh_s[0];
  ArgMax A{sh_am[0], sh_ai[0]};
  Top2 Bst{sh_v1[0], sh_i1[0], sh_v2[0]};
  uint32_t fl = sh_bad[0] ? DSPARK_FLAG_NONFINITE : 0u;
#pragma unroll
  for (int w = 1; w < kFinWaves; ++w) {
    lse_merge(M, S, sh_m[w], sh_s[w]);
    A = better(A, ArgMax{sh_am[w], sh_ai[w]});
    Bst = top2_merge(Bst, Top2{sh_v1[w], sh_i1[w], sh_v2[w]});
    if (sh_bad[w]) fl |= DSPARK_FLAG_NONFINITE;
  }

  // 1b. truncated rows (top-k / top-p on z): the kept set's smallest value
  // thr and weight, then the level-1 choice over kept chunks only
  // Kept weights are 2^(z log2e - M2) with the integer shift M2, so that the
  // drawn token's weight and the kept sum round alike (one kept token: q = 1).
  float thr = neg_inf(), s_kept = 0.0f, M2 = 0.0f;
  const int tk_raw = top_k[b];
  const float tp = top_p[b];
  const bool trunc_row = sampled && truncated(tk_raw, tp, V) && M > neg_inf() && M < pos_inf();
  if (trunc_row) {
    const int tk = (tk_raw > 0 && tk_raw < V) ? tk_raw : 0;
    M2 = floorf(M * kLog2e);
    const float wa = kLog2e, wb = -M2;
    const float total = S * __builtin_amdgcn_exp2f(fmaf(M, kLog2e, -M2));
    const QzRow qr{q_z + row * V, V, VEC};
    const ChunkPart* pb = part + static_cast<size_t>(b) * C;
    auto chunk_max = [pb](int c) { return pb[c].m; };
    bool cand = false;
    if (chunk_bound(chunk_max, C, tk, tp, wa, wb, total, U.c)) {
      gather_candidates(qr, V, U.c);
      exact_cut(tk, tp, wa, wb, total, U.c);
      cand = U.c.ok != 0;
    }
    int nlist = C;
    const int* list = nullptr;
    if (cand) {
      thr = U.c.thr;
      s_kept = U.c.s_kept;
      // the kept tokens lie in the chunks whose maximum reaches thr: a
      // prefix of the sorted chunk list
      nlist = count_at_least(U.c.cm, U.c.nchunks, thr, U.c.cnt);
      list = U.c.ci;
    } else {
      const SelResult r = select_threshold(qr, V, 32, tk, tp, wa, wb, U.s);
      thr = r.thr;
      s_kept = static_cast<float>(r.s_kept);
    }
    const Top2 tb = wave_top2(kept_chunk_scores(qr, nlist, list, thr, seed, pos, req));
    __syncthreads();
    if (lane == 0) {
      sh_v1[wave] = tb.v1;
      sh_i1[wave] = tb.i1;
      sh_v2[wave] = tb.v2;
    }
    __syncthreads();
    Bst = Top2{sh_v1[0], sh_i1[0], sh_v2[0]};
#pragma unroll
    for (int w = 1; w < kFinWaves; ++w) Bst = top2_merge(Bst, Top2{sh_v1[w], sh_i1[w], sh_v2[w]});
  }

  if (wave == 0) {
    // 2a. the draw
    int32_t x = 0;
    float zx = neg_inf();
    uint32_t near = 0;
    if (!sampled) {
      if (A.i == INT32_MAX) fl |= DSPARK_FLAG_EMPTY_ROW;
      else x = A.i;
    } else if (Bst.i1 == INT32_MAX) {
      fl |= DSPARK_FLAG_EMPTY_ROW;
    } else {
      if (Bst.v2 > neg_inf() && near_gap(Bst.v1, Bst.v2)) near = 1;
      const int v0 = Bst.i1 * kChunk + 4 * lane;
      float z[4];
      if (VEC && v0 + 3 < V) {
        const float4 u = *reinterpret_cast<const float4*>(q_z + row * V + v0);
        z[0] = u.x;
        z[1] = u.y;
        z[2] = u.z;
        z[3] = u.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] = v0 + e < V ? q_z[row * V + v0 + e] : neg_inf();
      }
      // tokens v0..v0+3 share Philox counter (v0 / 4, pos, req, tag)
      uint32_t c0 = static_cast<uint32_t>(v0) >> 2, c1 = static_cast<uint32_t>(pos), c2 = req,
               c3 = DSPARK_TAG_DRAFT_TOKEN;
      philox4x32_10(c0, c1, c2, c3, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
      const uint32_t wv[4] = {c0, c1, c2, c3};
      Top2 t{neg_inf(), INT32_MAX, neg_inf()};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (z[e] > neg_inf() && z[e] >= thr)
          t = top2_merge(t, Top2{z[e] + gumbel_of(wv[e]), v0 + e, neg_inf()});
      t = wave_top2(t);
      if (t.i1 == INT32_MAX) {
        fl |= DSPARK_FLAG_EMPTY_ROW;
      } else {
        x = t.i1;
        if (t.v2 > neg_inf() && near_gap(t.v1, t.v2)) near = 1;
        zx = q_z[row * V + x];
      }
    }
    if (near) fl |= DSPARK_FLAG_NEAR_THRESHOLD;
    if (lane == 0) {
      fin_x = x;
      fin_zx = zx;
      fin_M = M;
      fin_S = S;
      fin_fl = fl;
    }
  } else {
    // 2b. confidence head on [h_k ; embed(x_{k-1})]: 8 elements per 16-byte
    // load, every load of a thread issued before the first use
    const int32_t xp = clamp_token(xprev[static_cast<size_t>(b) * xstride], V);
    const uint16_t* h = hidden + row * d;
    const uint16_t* e = embed + static_cast<size_t>(xp) * d;
    const int t = tid - 64;
    constexpr int kConfThreads = kFinThreads - 64;
    float dot = 0.0f;
    if (cvec) {
      constexpr int kU = 4;  // vectors per thread per round
      for (int base = 0; base < d; base += kConfThreads * 8 * kU) {
        uint4 hv[kU], ev[kU];
        float4 wh[kU][2], we[kU][2];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i = base + (t + u * kConfThreads) * 8;
          if (i < d) {
            hv[u] = *reinterpret_cast<const uint4*>(h + i);
            ev[u] = *reinterpret_cast<const uint4*>(e + i);
            wh[u][0] = *reinterpret_cast<const float4*>(conf_w + i);
            wh[u][1] = *reinterpret_cast<const float4*>(conf_w + i + 4);
            we[u][0] = *reinterpret_cast<const float4*>(conf_w + d + i);
            we[u][1] = *reinterpret_cast<const float4*>(conf_w + d + i + 4);
          } else {
            hv[u] = ev[u] = make_uint4(0u, 0u, 0u, 0u);
            wh[u][0] = wh[u][1] = we[u][0] = we[u][1] = make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const float hx[8] = {bf_lo(hv[u].x), bf_hi(hv[u].x), bf_lo(hv[u].y), bf_hi(hv[u].y),
                               bf_lo(hv[u].z), bf_hi(hv[u].z), bf_lo(hv[u].w), bf_hi(hv[u].w)};
          const float ex[8] = {bf_lo(ev[u].x), bf_hi(ev[u].x), bf_lo(ev[u].y), bf_hi(ev[u].y),
                               bf_lo(ev[u].z), bf_hi(ev[u].z), bf_lo(ev[u].w), bf_hi(ev[u].w)};
          const float whx[8] = {wh[u][0].x, wh[u][0].y, wh[u][0].z, wh[u][0].w,
                                wh[u][1].x, wh[u][1].y, wh[u][1].z, wh[u][1].w};
          const float wex[8] = {we[u][0].x, we[u][0].y, we[u][0].z, we[u][0].w,
                                we[u][1].x, we[u][1].y, we[u][1].z, we[u][1].w};
#pragma unroll
          for (int j = 0; j < 8; ++j) dot += whx[j] * hx[j] + wex[j] * ex[j];
        }
      }
    } else {
      for (int i = t; i < d; i += kConfThreads)
        dot += conf_w[i] * load_logit(h, i) + conf_w[d + i] * load_logit(e, i);
    }
    dot = wave_sum(dot);
    if (lane == 0) sh_dot[wave] = dot;
  }
  __syncthreads();
  if (tid == 0) {
    float dot = 0.0f;
#pragma unroll
    for (int w = 1; w < kFinWaves; ++w) dot += sh_dot[w];
    const int32_t x = fin_x;
    draft_tokens[row] = x;
    if (sampled) {
      if (trunc_row) {
        q_lse[row] = M2 * kLn2 + logf(s_kept);
        q_thr[row] = thr;
        q_tok[row] = (fin_zx > neg_inf() && fin_zx >= thr && s_kept > 0.0f)
                         ? __builtin_amdgcn_exp2f(fmaf(fin_zx, kLog2e, -M2)) / s_kept
                         : 0.0f;
      } else {
        q_lse[row] = fin_M + logf(fin_S);
        q_thr[row] = neg_inf();
        q_tok[row] = (fin_zx > neg_inf() && fin_S > 0.0f) ? expf(fin_zx - fin_M) / fin_S : 0.0f;
      }
    } else {
      q_lse[row] = 0.0f;
      q_thr[row] = 0.0f;
      q_tok[row] = 1.0f;
    }
    confidence[row] = 1.0f / (1.0f + expf(-dot));
    uint32_t f = fin_fl;
    if (mode[b] != 0 && !sampled) f |= DSPARK_FLAG_BAD_POLICY;
    flags[row] = static_cast<uint8_t>(f);
  }
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
  // 16-byte loads of the confidence head's rows and weights
  const int32_t cvec = (d % 8 == 0) && reinterpret_cast<uintptr_t>(hidden) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(embed) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(conf_w) % 16 == 0;
  for (int k = 1; k <= gamma; ++k) {
    const int32_t* xp = k == 1 ? anchor : draft_tokens + (k - 2);
    const int32_t xs = k == 1 ? 1 : gamma;
    if (vec)
      DSPARK_LAUNCH("markov_step", (markov_step_kernel<T, true>), g_step, dim3(kStepThreads), 0,
                    st, backbone, xp, xs, w1, w2, pol.mode, pol.temperature, pol.request_id,
                    pol.position, seed, B, gamma, k, V, r, pl.C, q_z, part);
    else
      DSPARK_LAUNCH("markov_step", (markov_step_kernel<T, false>), g_step, dim3(kStepThreads), 0,
                    st, backbone, xp, xs, w1, w2, pol.mode, pol.temperature, pol.request_id,
                    pol.position, seed, B, gamma, k, V, r, pl.C, q_z, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (vec)
      DSPARK_LAUNCH("markov_finalize", markov_finalize_kernel<true>, dim3(B), dim3(kFinThreads), 0,
                    st, xp, xs, hidden, embed, conf_w, pol.mode, pol.temperature, pol.top_k,
                    pol.top_p, pol.request_id,
                    pol.position, seed, gamma, k, V, d, pl.C, cvec, part, q_z, draft_tokens,
                    q_lse, q_thr, q_tok, confidence, flags);
    else
      DSPARK_LAUNCH("markov_finalize", markov_finalize_kernel<false>, dim3(B), dim3(kFinThreads), 0,
                    st, xp, xs, hidden, embed, conf_w, pol.mode, pol.temperature, pol.top_k,
                    pol.top_p, pol.request_id,
                    pol.position, seed, gamma, k, V, d, pl.C, cvec, part, q_z, draft_tokens,
                    q_lse, q_thr, q_tok, confidence, flags);
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
