// markov.hip — left-to-right Markov draft sampling on gfx950.
//
// Semantics ("[2/3] feat(dsv4): implement exact DSpark speculative decoding",
// "Checkpoint-faithful DSpark architecture"; "DSpark Speculative Decoding
// (Draft Training) Design", "Semi-autoregressive draft"): for k = 1..gamma in
// order, y_k = backbone row k-1 + A[x_{k-1}] . B (a rank-r additive bias, x_0 the
// anchor), q_k = policy(y_k), x_k ~ q_k (argmax for greedy requests); the full
// q_k and the confidence c_k = sigmoid(w . [h_k ; embed(x_{k-1})]) are kept.
//
// Every step has two phases:
//  * stream: per (16 MS-token group, 64-request tile) of one wave, the bias tile
//    bias[v, b] = sum_i W2[v, i] W1[x_{k-1}(b), i] is a bf16 MFMA product
//    (v_mfma_f32_16x16x32_bf16) with the vocabulary as the M side, so each
//    lane's accumulators hold 4 consecutive tokens of one request and the
//    epilogue reads the backbone with 8-byte loads and writes z = y / T with
//    16-byte stores.  The epilogue reduces each request's 256-token chunk to
//    (max z, lowest argmax, sum exp(z - max), ln mass + chunk Gumbel).
//  * finalize, per request: combines the chunk partials into the
//    log-normaliser, picks the chunk by Gumbel-max over the chunk log-masses,
//    then a 16-token sub-chunk inside it and the token inside that (the
//    library's three-level Gumbel-max: exact, no prefix sum over the
//    vocabulary), and applies top-k / top-p when the request truncates.
// The confidence head needs only x_{k-1}, so one kernel evaluates it for every
// row after the last step.
//
// Two launch plans run these phases:
//  * fused: one launch for all gamma steps (its whole grid resident at once).
//    Workgroup g owns the 512 tokens [512 g, 512 g + 512) and keeps their W2
//    rows in registers (the MFMA A fragments) for the whole call, so the
//    rank-r factor is read from HBM once per call rather than once per step.
//    A finalize starts when its request's chunk records of the step are all
//    stored (polled, no grid barrier) and hands x_k to the next stream phase
//    through draft_tokens (both cleared before the launch).  Everything that
//    crosses workgroups inside the launch (chunk records, z rows read by the
//    draw, x_k) is stored and loaded at device scope (sc1), so no L2
//    writeback or invalidate is needed.
//  * per step: 2 gamma launches (stream kernel over all chunks, finalize
//    kernel over all requests), used when the fused grid cannot be resident
//    at once (V above 512 tokens per compute unit).
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "internal.hpp"
#include "truncate.hpp"

namespace dspark {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;           // requests per tile (MFMA N side)
constexpr int kStepThreads = 512;   // per-step stream kernel: 8 waves x 32 tokens, one chunk
constexpr int kFusedThreads = 512;  // fused kernel: 8 waves x 64 tokens, two chunks
constexpr int kStepMS = 2;          // 16-token MFMA row blocks per wave (per-step kernel)
constexpr int kFusedMS = 4;         // 16-token MFMA row blocks per wave (fused kernel)
constexpr int kFusedTokens = kFusedThreads / 64 * 16 * kFusedMS;
constexpr int kMaxR = DSPARK_MAX_RANK;
constexpr int kPad = 8;             // bf16 padding per staged W1 row (bank spread)
constexpr int kFinThreads = 256;    // per-step finalize kernel
constexpr uint32_t kSpinLimit = 1u << 22;  // polls (~1 us each) of one wait before giving up

// The one-launch plan's synchronisation area: the timeout word, alone on its
// 256-byte line.
constexpr int kSyncTimeout = 0;
constexpr int kSyncWords = 64;

// Everything one Markov call reads and writes.
struct MarkovArgs {
  const void* backbone;
  const int32_t* anchor;
  const uint16_t* w1;
  const uint16_t* w2;
  const uint16_t* hidden;
  const uint16_t* embed;
  const float* conf_w;
  dspark_policy pol;
  uint64_t seed;
  int32_t B, gamma, V, r, d, C, cvec;
  int32_t* draft_tokens;
  float* q_z;
  float* q_lse;
  float* q_thr;
  float* q_tok;
  float* confidence;
  uint8_t* flags;
  ChunkPart* part;
  uint32_t* sync;  // fused plan: timeout word (kSyncWords)
};

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

// Device-scope 16-byte store (written through to memory): z values that a
// workgroup of the same launch reads later.
__device__ __forceinline__ void store4_coherent(float* p, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}

// Device-scope 16-byte load (bypassing stale cached copies); the wait for its
// data is part of the instruction sequence.
__device__ __forceinline__ f32x4 load4_coherent(const void* p) {
  f32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off sc1\n\ts_waitcnt vmcnt(0)"
               : "=v"(v)
               : "v"(p)
               : "memory");
  return v;
}

template <bool COH>
__device__ __forceinline__ ChunkPart load_part(const ChunkPart* p) {
  if constexpr (COH) {
    const f32x4 v = load4_coherent(p);
    return ChunkPart{v[0], v[1], v[2], __float_as_uint(v[3])};
  } else {
    return *p;
  }
}
template <bool COH>
__device__ __forceinline__ void store_part(ChunkPart* p, ChunkPart v) {
  if constexpr (COH) {
    store4_coherent(reinterpret_cast<float*>(p), f32x4{v.m, v.s, v.score, __uint_as_float(v.arg_nf)});
  } else {
    *p = v;
  }
}
template <bool COH>
__device__ __forceinline__ void store_flag(uint8_t* p, uint8_t v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

// The thread index, opaque to the optimiser: the phases of the one-launch plan
// recompute their lane-derived addresses instead of keeping them live (in
// registers) across the whole step loop.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// ---------------------------------------------------------------------------
// Stream phase.

template <int NT>
struct StreamLds {
  static constexpr int NW = NT / 64;
  __attribute__((aligned(16))) uint16_t a[kTile * (kMaxR + kPad)];  // staged W1 rows
  float red_m[NW][kTile], red_s[NW][kTile];  // per (wave, request)
  int32_t red_i[NW][kTile];
  uint32_t red_f[NW][kTile];
  int32_t xs[kTile];
};

// W2 fragments of the 16 MS tokens [vb, vb + 16 MS) (MFMA A operand: token
// rows, K slices of 32).
template <int MS>
__device__ __forceinline__ void load_w2(bf16x8 (&af)[MS][kMaxR / 32], const uint16_t* w2, int vb,
                                        int V, int r, int lane) {
  const int ksteps = ((r + 31) & ~31) / 32;
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int v = vb + ms * 16 + (lane & 15);
#pragma unroll
    for (int ks = 0; ks < kMaxR / 32; ++ks) {
      const int k0 = ks * 32 + (lane >> 4) * 8;
      bf16x8 f = {};
      if (ks < ksteps && v < V && k0 < r) f = load_frag(w2 + static_cast<size_t>(v) * r + k0);
      af[ms][ks] = f;
    }
  }
}

// Backbone values of this lane for the request blocks [ns0, ns0 + NSP) of the
// tile: tokens vb + ms*16 + 4*(lane>>4) + i of request b0 + ns*16 + (lane&15).
template <typename T, bool VEC, int MS, int NSP>
__device__ __forceinline__ void load_backbone(QuadRaw<T> (&bbv)[NSP][MS], const T* backbone,
                                              int B, int gamma, int V, int k, int b0, int ns0,
                                              int vb, int lane) {
#pragma unroll
  for (int j = 0; j < NSP; ++j) {
    const int b = b0 + (ns0 + j) * 16 + (lane & 15);
    const size_t rowoff = (static_cast<size_t>(b < B ? b : 0) * gamma + (k - 1)) * V;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int v0 = vb + ms * 16 + 4 * (lane >> 4);
      const int n = b < B ? (V - v0 < 4 ? (V - v0 > 0 ? V - v0 : 0) : 4) : 0;
      bbv[j][ms].load(backbone + rowoff + (n > 0 ? v0 : 0), VEC, n);
    }
  }
}

// Step k for requests [b0, b0 + 64) over the workgroup's tokens [tok0, tok0 +
// 16 MS NW): wave w takes the 16 MS tokens at vb = tok0 + 16 MS w with its W2
// fragments af, and the 64 requests in NH passes of 64 / NH.  Writes z of
// sampled requests and one ChunkPart per (request, chunk of the workgroup).
// COH: z and the partials are read by other workgroups of the same launch.
template <typename T, bool VEC, int NT, int MS, int NH, bool COH>
__device__ __forceinline__ void stream_tile(const MarkovArgs& a, const bf16x8 (&af)[MS][kMaxR / 32], int tok0,
                            int b0, int k, StreamLds<NT>& L) {
  constexpr int NW = NT / 64;
  constexpr int NSP = 4 / NH;         // 16-request blocks per pass
  constexpr int TPW = 16 * MS;        // tokens per wave
  constexpr int WPC = kChunk / TPW;   // waves per chunk
  const T* __restrict__ backbone = static_cast<const T*>(a.backbone);
  const int B = a.B, gamma = a.gamma, V = a.V, r = a.r;
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int vb = tok0 + wave * TPW;
  const int kpad = (r + 31) & ~31;
  const int ld = kpad + kPad;
  const int ksteps = kpad / 32;

  // every pass's backbone values are requested first (they do not depend on
  // x_{k-1}), so that their transfer overlaps the wait for the tile's tokens
  // x_{k-1}, the W1 staging and the products
  QuadRaw<T> bbv[NH][NSP][MS];
#pragma unroll
  for (int h = 0; h < NH; ++h)
    load_backbone<T, VEC, MS, NSP>(bbv[h], backbone, B, gamma, V, k, b0, h * NSP, vb, lane);

  int32_t xv = -1;
  if (tid < kTile) {
    const int b = b0 + tid;
    if (b < B) {
      if (k == 1) {
        xv = a.anchor[b];
      } else if constexpr (COH) {
        // one-launch plan: x_{k-1} is -1 until its finalize stores it
        const int32_t* xp = a.draft_tokens + static_cast<size_t>(b) * gamma + (k - 2);
        uint32_t polls = 0;
        while ((xv = load_coherent(xp)) < 0) {
          __builtin_amdgcn_s_sleep(2);
          if (++polls > kSpinLimit) {
            __hip_atomic_store(a.sync + kSyncTimeout, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
      } else {
        xv = a.draft_tokens[static_cast<size_t>(b) * gamma + (k - 2)];
      }
      xv = clamp_token(xv, V);
    }
  }

  // stage the gathered W1 rows of the tile's requests (MFMA B operand): every
  // 16-byte piece load issued back to back
  if (tid < kTile) L.xs[tid] = xv;
  __syncthreads();
  const int pieces = kpad / 8;
  constexpr int kMaxPieces = kTile * (kMaxR / 8) / NT;
  uint4 stage[kMaxPieces];
#pragma unroll
  for (int j = 0; j < kMaxPieces; ++j) {
    const int idx = tid + j * NT;
    const int row = idx / pieces, pc = idx - row * pieces;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (row < kTile && pc * 8 < r) {
      const int32_t x = L.xs[row];
      if (x >= 0) val = *reinterpret_cast<const uint4*>(a.w1 + static_cast<size_t>(x) * r + pc * 8);
    }
    stage[j] = val;
  }
#pragma unroll
  for (int j = 0; j < kMaxPieces; ++j) {
    const int idx = tid + j * NT;
    const int row = idx / pieces, pc = idx - row * pieces;
    if (row < kTile) *reinterpret_cast<uint4*>(L.a + row * ld + pc * 8) = stage[j];
  }
  __syncthreads();

#pragma unroll
  for (int h = 0; h < NH; ++h) {
  f32x4 acc[MS][NSP];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int j = 0; j < NSP; ++j) acc[ms][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kMaxR / 32; ++ks) {
    if (ks < ksteps) {
#pragma unroll
      for (int j = 0; j < NSP; ++j) {
        const int ns = h * NSP + j;
        const bf16x8 bfr =
            load_frag(L.a + (ns * 16 + (lane & 15)) * ld + ks * 32 + (lane >> 4) * 8);
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
          acc[ms][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ms][ks], bfr, acc[ms][j], 0, 0, 0);
      }
    }
  }

  // epilogue: lane holds tokens vb + ms*16 + 4*(lane>>4) + i of request ns*16 + (lane&15)
#pragma unroll
  for (int j = 0; j < NSP; ++j) {
    const int ns = h * NSP + j;
    const int n = ns * 16 + (lane & 15);
    const int b = b0 + n;
    const bool bvalid = b < B;
    float invT = 1.0f;
    bool sampled = false;
    if (bvalid) {
      const float Tb = a.pol.temperature[b];
      sampled = a.pol.mode[b] != 0 && !bad_temperature(Tb);
      if (sampled) invT = 1.0f / Tb;
    }
    const size_t rowoff = (static_cast<size_t>(bvalid ? b : 0) * gamma + (k - 1)) * V;
    float z[4 * MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int v0 = vb + ms * 16 + 4 * (lane >> 4);
      const QuadRaw<T>& bb = bbv[h][j][ms];
      const bool full = bvalid && v0 + 3 < V;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool in = bvalid && v0 + i < V;
        z[ms * 4 + i] = in ? (acc[ms][j][i] + bb.at(i)) * invT : neg_inf();
      }
      if (sampled) {
        float* dst = a.q_z + rowoff + v0;
        if (VEC && full) {
          const f32x4 zv{z[ms * 4], z[ms * 4 + 1], z[ms * 4 + 2], z[ms * 4 + 3]};
          if constexpr (COH) store4_coherent(dst, zv);
          else *reinterpret_cast<f32x4*>(dst) = zv;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (v0 + i < V) {
              if constexpr (COH) store_coherent(dst + i, z[ms * 4 + i]);
              else dst[i] = z[ms * 4 + i];
            }
        }
      }
    }
    // reduce over this lane's 4 MS tokens, then over the 4 lane groups
    // sharing n: max, lowest argmax, and a NaN / +inf detector (the sum of z
    // is NaN iff some z is NaN or +inf meets -inf; +inf alone shows as max)
    float m = neg_inf(), zsum = 0.0f;
    int32_t ej = -1;  // element of the lane's first maximum
#pragma unroll
    for (int e = 0; e < 4 * MS; ++e) {
      if (z[e] > m) {
        m = z[e];
        ej = e;
      }
      zsum += z[e];
    }
    int32_t arg = ej < 0 ? INT32_MAX : vb + (ej >> 2) * 16 + 4 * (lane >> 4) + (ej & 3);
    const uint32_t bad = rows_or((zsum != zsum || m == pos_inf()) ? 1u : 0u);
    {
      const ArgMax am = rows_argmax(ArgMax{m, arg});
      m = am.v;
      arg = am.i;
    }
    // sum of 2^(z log2e - m log2e) relative to the 4 lanes' maximum
    float s = 0.0f;
    if (m > neg_inf() && m < pos_inf()) {
      const float mb = m * kLog2e;
#pragma unroll
      for (int e = 0; e < 4 * MS; ++e) s += __builtin_amdgcn_exp2f(fmaf(z[e], kLog2e, -mb));
    }
    s = rows_sum(s);
    if (lane < 16) {
      L.red_m[wave][n] = m;
      L.red_s[wave][n] = s;
      L.red_i[wave][n] = arg;
      L.red_f[wave][n] = bad;
    }
  }
  }
  __syncthreads();
  // one ChunkPart per (request, chunk): the chunk's waves combined
  constexpr int kChunksPerWG = NW / WPC;
  constexpr int kRecPerThread = (kChunksPerWG * kTile + NT - 1) / NT;
  ChunkPart rec[kRecPerThread];
  ChunkPart* dst[kRecPerThread];
#pragma unroll
  for (int j = 0; j < kRecPerThread; ++j) {
    dst[j] = nullptr;
    const int idx = tid + j * NT;
    const int h = idx / kTile, n = idx - h * kTile;
    const int c = tok0 / kChunk + h;
    const int b = b0 + n;
    if (idx >= kChunksPerWG * kTile || c >= a.C || b >= B) continue;
    const int w0 = h * WPC;
    float m = L.red_m[w0][n], s = L.red_s[w0][n];
    ArgMax am{L.red_m[w0][n], L.red_i[w0][n]};
    uint32_t bad = L.red_f[w0][n];
#pragma unroll
    for (int w = 1; w < WPC; ++w) {
      lse_merge(m, s, L.red_m[w0 + w][n], L.red_s[w0 + w][n]);
      am = better(am, ArgMax{L.red_m[w0 + w][n], L.red_i[w0 + w][n]});
      bad |= L.red_f[w0 + w][n];
    }
    // level 1 of the three-level Gumbel-max draw: ln(chunk mass) + chunk noise
    float score = neg_inf();
    const float Tb = a.pol.temperature[b];
    if (a.pol.mode[b] != 0 && !bad_temperature(Tb) && m > neg_inf() && m < pos_inf() && s > 0.0f)
      score = m + logf(s) + gumbel(a.seed, static_cast<uint32_t>(c), a.pol.position[b] + k,
                                   a.pol.request_id[b], DSPARK_TAG_DRAFT_CHUNK);
    rec[j] = ChunkPart{m, s, score, (static_cast<uint32_t>(am.i) & 0x7fffffffu) | (bad ? 0x80000000u : 0u)};
    dst[j] = a.part + (static_cast<size_t>(k - 1) * B + b) * a.C + c;
  }
  if constexpr (COH) {
    // a record, once visible, vouches for every z of the step this
    // workgroup stored: all waves' stores complete before any record is
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < kRecPerThread; ++j)
    if (dst[j]) store_part<COH>(dst[j], rec[j]);
  __syncthreads();  // the LDS tile is reused by the next call
}

// ---------------------------------------------------------------------------
// Finalize phase.

// One proposal row of scaled logits z (fp32), 4 tokens per load, read through
// a buffer resource over the row (reads past the row return 0, never fault).
// COH: the row was written by other workgroups of the same launch, so every
// load carries the sc1 policy (served by the device-coherent level, not a
// possibly stale cache line); the compiler still batches them.
template <bool COH>
struct QzRow {
  static constexpr int kPolicy = COH ? 16 : 0;  // cache policy bits: sc1
  __amdgpu_buffer_rsrc_t rs;
  int V;
  bool vec4;
  __device__ QzRow(const float* p, int V_, bool vec) : V(V_), vec4(vec) {
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), static_cast<short>(0), V_ * 4,
                                           kBufferWord3);
  }
  // one 16-byte load (row 16-byte aligned, v0 a multiple of 4; 0 past V)
  __device__ void load4u(int v0, float* o) const {
    const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(rs, v0 * 4, 0, kPolicy);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __uint_as_float(u[e]);
  }
  __device__ void load4(int v0, float* o) const {
    if (vec4 && v0 + 3 < V) {
      load4u(v0, o);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = v0 + e < V ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (v0 + e) * 4, 0, kPolicy))
                          : neg_inf();
    }
  }
};

// Level-1 scores of the three-level draw restricted to the kept set
// (z >= thr): for each listed chunk (list[j], or j itself without a list)
// holding kept tokens, log of its kept mass plus the chunk's Gumbel.  Wave w
// takes entries w, w + NW, ...; four chunks' loads are issued together.
// Returns the wave's best two (score, chunk).
template <int NT, bool COH>
__device__ __forceinline__ Top2 kept_chunk_scores(const QzRow<COH>& qr, int n, const int* list, float thr,
                                  uint64_t seed, int32_t pos, uint32_t req) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = wave_id();
  Top2 best{neg_inf(), INT32_MAX, neg_inf()};
  constexpr int kU = 4;
  for (int j0 = wave * kU; j0 < n; j0 += NW * kU) {
    float z[kU][4];
    int cs[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = j0 + u;
      cs[u] = j < n ? (list ? uniform_i(list[j]) : j) : -1;
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

// Level-1 scores over the listed chunks list[0 .. n) (n <= kMaxChunksBound)
// for the kept set z >= thr, as kept_chunk_scores computes them, in two
// stages: the waves reduce eight chunks at a time (their loads issued
// together) to each chunk's kept maximum and weight in smc / sw (LDS, n
// entries each); then thread t scores the chunks t, t + NT, ... (one Philox
// noise per thread rather than per wave).  Returns the thread's best two.
template <int NT, bool COH>
__device__ __forceinline__ Top2 kept_list_scores(const QzRow<COH>& qr, int n, const int* list, float thr,
                                                 uint64_t seed, int32_t pos, uint32_t req, float* smc, float* sw) {
  constexpr int NW = NT / 64;
  constexpr int kU = 8;
  const int lane = threadIdx.x & 63, wave = wave_id();
  for (int j0 = wave * kU; j0 < n; j0 += NW * kU) {
    float z[kU][4];
    int cs[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = j0 + u;
      cs[u] = j < n ? uniform_i(list[j]) : -1;
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
      float w = 0.0f;
      if (mc > neg_inf()) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (z[u][e] >= thr) w += __builtin_amdgcn_exp2f((z[u][e] - mc) * kLog2e);
        w = wave_sum(w);
      }
      if (lane == 0) {
        smc[j0 + u] = mc;
        sw[j0 + u] = w;
      }
    }
  }
  __syncthreads();
  Top2 best{neg_inf(), INT32_MAX, neg_inf()};
  for (int j = threadIdx.x; j < n; j += NT) {
    const float mc = smc[j];
    if (!(mc > neg_inf())) continue;
    const int c = list[j];
    const float score = mc + logf(sw[j]) + gumbel(seed, static_cast<uint32_t>(c), pos, req, DSPARK_TAG_DRAFT_CHUNK);
    best = top2_merge(best, Top2{score, c, neg_inf()});
  }
  return best;
}

// Level-1 scores from the histogram cut's kept chunk weights (fixed point,
// 2^-40 units of the shifted frame 2^(z log2e - M2)): ln of the chunk's kept
// mass plus the chunk's Gumbel.  Returns the thread's best two.
template <int NT>
__device__ __forceinline__ Top2 hist_chunk_scores(const HistLds<NT>& H, float M2, uint64_t seed,
                                                  int32_t pos, uint32_t req) {
  Top2 best{neg_inf(), INT32_MAX, neg_inf()};
  const float off = (M2 - 40.0f) * kLn2;
  for (int j = threadIdx.x; j < H.nl; j += NT) {
    const int c = H.cl[j];
    const fix_t w = H.cw[c];
    if (w == 0) continue;
    const float score = logf(static_cast<float>(w)) + off +
                        gumbel(seed, static_cast<uint32_t>(c), pos, req, DSPARK_TAG_DRAFT_CHUNK);
    best = top2_merge(best, Top2{score, c, neg_inf()});
  }
  return best;
}

template <int NT>
struct FinLds {
  static constexpr int NW = NT / 64;
  float sh_m[NW], sh_s[NW], sh_am[NW], sh_v1[NW], sh_v2[NW];
  int32_t sh_ai[NW], sh_i1[NW];
  uint32_t sh_bad[NW];
  float cm[kMaxChunksBound];  // chunk maxima of the row (truncated rows)
  TruncLds<NT> U;
};

// Kept set of a truncated row (smallest kept z, kept weight in units of
// 2^(z log2e - M2)) and the level-1 choice over its chunks: candidates under
// the chunk-maxima bound; else, for top-p alone, the weight histogram; else
// radix selection over the row.  Kept out of line: only truncated rows pay
// for its registers.  All threads of the workgroup call it.
struct TruncOut {
  float thr, s_kept;
  Top2 best;
};

template <int NT, bool COH>
__device__ __noinline__ TruncOut truncate_row(const float* zrow, int V, int vec, int C, int tk, float tp,
                                              float M, float M2, float total, uint64_t seed, int32_t pos,
                                              uint32_t req, FinLds<NT>& F) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // every argument is uniform: keep the row's buffer resource scalar
  const uint64_t pz = reinterpret_cast<uint64_t>(zrow);
  const float* zr = reinterpret_cast<const float*>(
      (static_cast<uint64_t>(static_cast<uint32_t>(uniform_i(static_cast<int>(pz >> 32)))) << 32) |
      static_cast<uint32_t>(uniform_i(static_cast<int>(pz))));
  V = uniform_i(V);
  C = uniform_i(C);
  const QzRow<COH> qr(zr, V, uniform_i(vec) != 0);
  const float wa = kLog2e, wb = -M2;
  int path = 0;
  if (C <= kMaxChunksBound && chunk_bound(F.cm, C, tk, tp, wa, wb, total, F.U.c)) {
    gather_candidates(qr, V, F.U.c);
    exact_cut(tk, tp, wa, wb, total, F.U.c);
    if (F.U.c.ok) path = 1;
  }
  if (path == 0 && tk == 0 && C <= kMaxChunksBound && hist_cut<NT, true>(qr, V, F.cm, C, M, total, wa, wb, tp, F.U.h))
    path = 2;
  TruncOut o;
  Top2 tb;
  if (path == 1) {
    o.thr = F.U.c.thr;
    o.s_kept = F.U.c.s_kept;
    // the sort scratch is free once the cut is taken
    tb = kept_list_scores<NT, COH>(qr, F.U.c.nchunks, F.U.c.ci, o.thr, seed, pos, req, F.U.c.tmp,
                                   F.U.c.tmp + kMaxChunksBound);
  } else if (path == 2) {
    o.thr = F.U.h.thr;
    o.s_kept = F.U.h.s_kept;
    tb = hist_chunk_scores<NT>(F.U.h, M2, seed, pos, req);
  } else {
    const SelResult sr = select_threshold(qr, V, 32, tk, tp, wa, wb, F.U.s);
    o.thr = sr.thr;
    o.s_kept = static_cast<float>(sr.s_kept);
    tb = kept_chunk_scores<NT, COH>(qr, C, nullptr, o.thr, seed, pos, req);
  }
  tb = wave_top2(tb);
  __syncthreads();
  if (lane == 0) {
    F.sh_v1[wave] = tb.v1;
    F.sh_i1[wave] = tb.i1;
    F.sh_v2[wave] = tb.v2;
  }
  __syncthreads();
  o.best = Top2{F.sh_v1[0], F.sh_i1[0], F.sh_v2[0]};
#pragma unroll
  for (int w = 1; w < NW; ++w) o.best = top2_merge(o.best, Top2{F.sh_v1[w], F.sh_i1[w], F.sh_v2[w]});
  return o;
}

// Finalize step k of request b with the whole workgroup.  All waves combine
// the chunk partials (and cut the kept set of a truncating request); then
// wave 0 draws the token inside the chosen chunk (lane l scores tokens
// 4l..4l+3 with one Philox block).  COH: the partials and z were written by
// other workgroups of the same launch, and x_k is read by them.
template <int NT, bool VEC, bool COH>
__device__ __forceinline__ void finalize_request(const MarkovArgs& a, int b, int k, FinLds<NT>& F) {
  constexpr int NW = NT / 64;
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int V = a.V, C = a.C, gamma = a.gamma;
  const size_t row = static_cast<size_t>(b) * gamma + (k - 1);
  const float Tb = a.pol.temperature[b];
  const bool sampled = a.pol.mode[b] != 0 && !bad_temperature(Tb);
  const uint32_t req = a.pol.request_id[b];
  const int32_t pos = a.pol.position[b] + k;
  const ChunkPart* pb = a.part + (static_cast<size_t>(k - 1) * a.B + b) * C;

  // 1. combine the chunk partials
  float m = neg_inf(), s = 0.0f;
  ArgMax am{neg_inf(), INT32_MAX};
  Top2 best{neg_inf(), INT32_MAX, neg_inf()};
  uint32_t bad = 0;
  const float tp = a.pol.top_p[b];
  const int tk_raw = a.pol.top_k[b];
  const bool want_cm = sampled && truncated(tk_raw, tp, V) && C <= kMaxChunksBound;
  // a sampled row without truncation draws inside its best-scoring chunk:
  // each wave fetches its own best chunk while the waves' results merge, and
  // the wave holding the row's best draws from registers
  const bool spec = sampled && !truncated(tk_raw, tp, V);
  const QzRow<COH> qr(a.q_z + row * V, V, VEC);
  Top2 wbest;
  float zpre[4];
  for (int c = tid; c < C; c += NT) {
    ChunkPart p = load_part<COH>(pb + c);
    if constexpr (COH) {
      // the fused plan's records start as s = -1 (a stored s is >= 0 or NaN)
      uint32_t polls = 0;
      while (p.s < 0.0f) {
        __builtin_amdgcn_s_sleep(2);
        if (++polls > kSpinLimit) {
          __hip_atomic_store(a.sync + kSyncTimeout, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          p = ChunkPart{neg_inf(), 0.0f, neg_inf(), 0x7fffffffu};
          break;
        }
        p = load_part<COH>(pb + c);
      }
    }
    if (want_cm) F.cm[c] = p.m;
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
    wbest = wb;
    const uint32_t wbad = wave_or(bad);
    if (lane == 0) {
      F.sh_m[wave] = wm;
      F.sh_s[wave] = ws;
      F.sh_am[wave] = wa.v;
      F.sh_ai[wave] = wa.i;
      F.sh_v1[wave] = wb.v1;
      F.sh_i1[wave] = wb.i1;
      F.sh_v2[wave] = wb.v2;
      F.sh_bad[wave] = wbad;
    }
  }
  if (spec && wbest.i1 != INT32_MAX) qr.load4(wbest.i1 * kChunk + 4 * lane, zpre);
  __syncthreads();
  float M = F.sh_m[0], S = F.sh_s[0];
  ArgMax A{F.sh_am[0], F.sh_ai[0]};
  Top2 Bst{F.sh_v1[0], F.sh_i1[0], F.sh_v2[0]};
  uint32_t fl = F.sh_bad[0] ? DSPARK_FLAG_NONFINITE : 0u;
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    lse_merge(M, S, F.sh_m[w], F.sh_s[w]);
    A = better(A, ArgMax{F.sh_am[w], F.sh_ai[w]});
    Bst = top2_merge(Bst, Top2{F.sh_v1[w], F.sh_i1[w], F.sh_v2[w]});
    if (F.sh_bad[w]) fl |= DSPARK_FLAG_NONFINITE;
  }

  // 1b. truncated rows (top-k / top-p on z): the kept set's smallest value
  // thr and weight, then the level-1 choice over kept chunks only.  Kept
  // weights are 2^(z log2e - M2) with the integer shift M2, so that the drawn
  // token's weight and the kept sum round alike (one kept token: q = 1).
  float thr = neg_inf(), s_kept = 0.0f, M2 = 0.0f;
  const bool trunc_row = sampled && truncated(tk_raw, tp, V) && M > neg_inf() && M < pos_inf();
  if (trunc_row) {
    const int tk = (tk_raw > 0 && tk_raw < V) ? tk_raw : 0;
    M2 = floorf(M * kLog2e);
    const float total = S * __builtin_amdgcn_exp2f(fmaf(M, kLog2e, -M2));
    const TruncOut o = truncate_row<NT, COH>(a.q_z + row * V, V, VEC ? 1 : 0, C, tk, tp, M, M2, total,
                                              a.seed, pos, req, F);
    thr = o.thr;
    s_kept = o.s_kept;
    Bst = o.best;
  }

  // the drawing wave: the holder of the best chunk's prefetched z, else wave 0
  const bool pre = spec && Bst.i1 != INT32_MAX && wbest.i1 == Bst.i1;
  if (spec && Bst.i1 != INT32_MAX ? pre : wave == 0) {
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
      if (pre) {
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] = zpre[e];
      } else {
        qr.load4(v0, z);
      }
      // levels 2 and 3 of the draw over the chunk's kept tokens
      float lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) lw[e] = (z[e] > neg_inf() && z[e] >= thr) ? z[e] : neg_inf();
      const InChunk dr =
          draw_in_chunk(lw, Bst.i1, a.seed, pos, req, DSPARK_TAG_DRAFT_SUB, DSPARK_TAG_DRAFT_TOKEN);
      if (dr.tok < 0) {
        fl |= DSPARK_FLAG_EMPTY_ROW;
      } else {
        x = dr.tok;
        zx = dr.lw;
        if (dr.near) near = 1;
      }
    }
    if (near) fl |= DSPARK_FLAG_NEAR_THRESHOLD;
    // the drawing wave writes the row's outputs, x_k first: the next step's
    // workgroups wait for it
    if (lane == 0) {
      if constexpr (COH) store_coherent(a.draft_tokens + row, x);
      else a.draft_tokens[row] = x;
      if (!sampled) {
        a.q_lse[row] = 0.0f;
        a.q_thr[row] = 0.0f;
        a.q_tok[row] = 1.0f;
      } else if (trunc_row) {
        a.q_lse[row] = M2 * kLn2 + logf(s_kept);
        a.q_thr[row] = thr;
        a.q_tok[row] = (zx > neg_inf() && zx >= thr && s_kept > 0.0f)
                           ? __builtin_amdgcn_exp2f(fmaf(zx, kLog2e, -M2)) / s_kept
                           : 0.0f;
      } else {
        a.q_lse[row] = M + logf(S);
        a.q_thr[row] = neg_inf();
        a.q_tok[row] = (zx > neg_inf() && S > 0.0f) ? expf(zx - M) / S : 0.0f;
      }
      if (a.pol.mode[b] != 0 && !sampled) fl |= DSPARK_FLAG_BAD_POLICY;
      store_flag<COH>(a.flags + row, static_cast<uint8_t>(fl));
    }
  }
  __syncthreads();  // F is reused by the next request
}

// Confidence head of every draft row (b, k): c = sigmoid(w . [h_k ;
// embed(x_{k-1})]), one workgroup per row, run after the last step (x_{k-1}
// is the anchor for k = 1, else draft token k-1).  8 elements per 16-byte
// load, every load of a thread issued before the first use.
constexpr int kConfThreads = 256;

__global__ __launch_bounds__(kConfThreads) void markov_confidence_kernel(MarkovArgs a) {
  __shared__ float sh[kConfThreads / 64];
  const int row = blockIdx.x;
  const int b = row / a.gamma, k = row - b * a.gamma + 1;
  const int d = a.d, V = a.V, t = threadIdx.x;
  const int32_t xp =
      clamp_token(k == 1 ? a.anchor[b] : a.draft_tokens[static_cast<size_t>(b) * a.gamma + (k - 2)], V);
  const uint16_t* h = a.hidden + static_cast<size_t>(row) * d;
  const uint16_t* e = a.embed + static_cast<size_t>(xp) * d;
  const float* cw = a.conf_w;
  float dot = 0.0f;
  if (a.cvec) {
    constexpr int kU = 2;  // vectors per thread per round
    for (int base = 0; base < d; base += kConfThreads * 8 * kU) {
      uint4 hv[kU], ev[kU];
      float4 wh[kU][2], we[kU][2];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = base + (t + u * kConfThreads) * 8;
        if (i < d) {
          hv[u] = *reinterpret_cast<const uint4*>(h + i);
          ev[u] = *reinterpret_cast<const uint4*>(e + i);
          wh[u][0] = *reinterpret_cast<const float4*>(cw + i);
          wh[u][1] = *reinterpret_cast<const float4*>(cw + i + 4);
          we[u][0] = *reinterpret_cast<const float4*>(cw + d + i);
          we[u][1] = *reinterpret_cast<const float4*>(cw + d + i + 4);
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
      dot += cw[i] * load_logit(h, i) + cw[d + i] * load_logit(e, i);
  }
  dot = block_sum<kConfThreads / 64>(dot, sh);
  if (t == 0) a.confidence[row] = 1.0f / (1.0f + expf(-dot));
}

// ---------------------------------------------------------------------------
// Kernels.

template <typename T, bool VEC>
__global__ __launch_bounds__(kStepThreads) void markov_step_kernel(MarkovArgs a, int32_t k) {
  __shared__ StreamLds<kStepThreads> L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok0 = blockIdx.x * kChunk;
  bf16x8 af[kStepMS][kMaxR / 32];
  load_w2<kStepMS>(af, a.w2, tok0 + wave * 16 * kStepMS, a.V, a.r, lane);
  stream_tile<T, VEC, kStepThreads, kStepMS, 1, false>(a, af, tok0, blockIdx.y * kTile, k, L);
}

template <bool VEC>
__global__ __launch_bounds__(kFinThreads) void markov_finalize_kernel(MarkovArgs a, int32_t k) {
  __shared__ FinLds<kFinThreads> F;
  finalize_request<kFinThreads, VEC, false>(a, blockIdx.x, k, F);
}

// One-launch plan.  Every workgroup streams its vocabulary slice for every
// request and step; workgroup g also finalizes requests g, g + G, ...  The
// steps meet through the data itself, without a grid-wide barrier:
//  * each step's chunk records have their own slice of the workspace, reset
//    to s = -1 before the launch; a workgroup stores its records of step k
//    only after all of its waves' stores of step k completed, so a record
//    that is visible vouches for the z values behind it, and a finalizer
//    polls its request's records until none is -1;
//  * x_k reaches the next step's stream phase through draft_tokens (-1
//    until its finalizer stores it).
// A poll limit bounds every wait; on expiry the timeout word is set and the
// launch runs on to its end (its rows are then flagged).

// Clears the timeout word, marks every draft token as not yet drawn and every
// chunk record (nrec of them) as not yet stored.
__global__ void markov_sync_reset_kernel(uint32_t* sync, int32_t* draft_tokens, size_t n, ChunkPart* part,
                                         size_t nrec) {
  const size_t i0 = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t step = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = i0; i < kSyncWords; i += step) sync[i] = 0u;
  for (size_t i = i0; i < n; i += step) draft_tokens[i] = -1;
  for (size_t i = i0; i < nrec; i += step) part[i] = ChunkPart{neg_inf(), -1.0f, neg_inf(), 0x7fffffffu};
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kFusedThreads) void markov_fused_kernel(MarkovArgs a) {
  __shared__ StreamLds<kFusedThreads> SL;
  __shared__ FinLds<kFusedThreads> FL;
  const int g = blockIdx.x, G = gridDim.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok0 = g * kFusedTokens;
  bf16x8 af[kFusedMS][kMaxR / 32];  // resident for the whole call
  load_w2<kFusedMS>(af, a.w2, tok0 + wave * 16 * kFusedMS, a.V, a.r, lane);
  for (int k = 1; k <= a.gamma; ++k) {
    for (int b0 = 0; b0 < a.B; b0 += kTile)
      stream_tile<T, VEC, kFusedThreads, kFusedMS, 4, true>(a, af, tok0, b0, k, SL);
    for (int b = g; b < a.B; b += G) finalize_request<kFusedThreads, VEC, true>(a, b, k, FL);
  }
  // after a timed-out wait, mark the rows this workgroup finalized
  if (threadIdx.x == 0 &&
      __hip_atomic_load(a.sync + kSyncTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    for (int b = g; b < a.B; b += G)
      for (int k = 0; k < a.gamma; ++k) {
        uint8_t* f = a.flags + static_cast<size_t>(b) * a.gamma + k;
        *f = static_cast<uint8_t>(*f | DSPARK_FLAG_SYNC_TIMEOUT);
      }
  }
}

// Resident workgroups per compute unit of a fused instantiation, the
// device's compute units and whether it offers cooperative launch, cached per
// device: a property of the device and the code object only.
struct FusedFit {
  int blocks_per_cu;
  int cus;
  bool coop;
};

template <typename T, bool VEC>
FusedFit fused_fit() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];  // (coop << 30 | blocks << 16 | cus) + 1; 0 = unknown
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FusedFit{0, 0, false};
  if (dev < kMaxDev) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c) return FusedFit{((c - 1) >> 16) & 0x3fff, (c - 1) & 0xffff, ((c - 1) >> 30) != 0};
  }
  int coop = 0, cus = 0, nb = 0;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess) coop = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, markov_fused_kernel<T, VEC>, kFusedThreads,
                                                   0) != hipSuccess)
    nb = 0;
  FusedFit f{nb, cus, coop != 0};
  if (f.blocks_per_cu < 0 || f.blocks_per_cu > 0x3fff || cus < 0 || cus > 0xffff) f = FusedFit{0, 0, false};
  if (dev < kMaxDev)
    cache[dev].store(((f.coop ? 1 << 30 : 0) | (f.blocks_per_cu << 16) | f.cus) + 1, std::memory_order_relaxed);
  return f;
}

// Compute units the stream's queue may use (its CU mask), or all of them.
int stream_cus(hipStream_t st, int cus) {
  uint32_t mask[32] = {};
  const int words = (cus + 31) / 32;
  if (words > 32 || hipExtStreamGetCUMask(st, static_cast<uint32_t>(words), mask) != hipSuccess) return cus;
  int n = 0;
  for (int w = 0; w < words; ++w) n += __builtin_popcount(mask[w]);
  return n > 0 && n < cus ? n : cus;
}

// An ordinary launch of the fused grid relies on all of it being resident at
// once, which an occupancy-sized grid is unless another such grid holds part
// of the device: fused launches on one device are therefore chained, each
// waiting for the previous one's completion event when that one went to
// another stream (one stream orders its own launches), not inside a stream
// capture (where the caller orders the work).
struct FusedChain {
  std::mutex mu;
  hipEvent_t ev[64] = {};
  hipStream_t last[64] = {};
};
FusedChain g_chain;

// fused: 0 per-step kernels, 1 one ordinary launch, 2 one cooperative launch
template <typename T, bool VEC>
hipError_t launch_plan(const MarkovArgs& a, int fused, hipStream_t st) {
  if (fused) {
    const size_t ntok = static_cast<size_t>(a.B) * a.gamma;
    const size_t nrec = ntok * static_cast<size_t>(a.C);
    const size_t most = std::max({ntok, nrec, static_cast<size_t>(kSyncWords)});
    DSPARK_LAUNCH("markov_sync_reset", markov_sync_reset_kernel,
                  dim3(static_cast<unsigned>(std::min<size_t>(1024, (most + 255) / 256))), dim3(256), 0, st,
                  a.sync, a.draft_tokens, ntok, a.part, nrec);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int G = (a.V + kFusedTokens - 1) / kFusedTokens;
    MarkovArgs arg = a;
    if (fused == 2) {
      void* params[] = {&arg};
      ProfScope ps("markov_fused");
      if (ps.active()) (void)hipEventRecord(ps.start(), st);
      e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(markov_fused_kernel<T, VEC>),
                                     dim3(G), dim3(kFusedThreads), params, 0, st);
      if (ps.active()) (void)hipEventRecord(ps.stop(), st);
      if (e != hipSuccess) return e;
    } else {
      int dev = 0;
      e = hipGetDevice(&dev);
      if (e != hipSuccess) return e;
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(st, &cs) != hipSuccess) cs = hipStreamCaptureStatusNone;
      const bool chain = cs == hipStreamCaptureStatusNone && dev >= 0 && dev < 64;
      std::unique_lock<std::mutex> lk(g_chain.mu, std::defer_lock);
      if (chain) {
        lk.lock();
        hipEvent_t& ev = g_chain.ev[dev];
        if (!ev) {
          e = hipEventCreate(&ev);
          if (e != hipSuccess) return e;
        } else if (g_chain.last[dev] != st) {
          e = hipStreamWaitEvent(st, ev, 0);
          if (e != hipSuccess) return e;
        }
      }
      // the chain's event rides on the kernel's own dispatch (no marker
      // packet between it and the next kernel of the stream)
      ProfScope ps("markov_fused");
      if (ps.active()) {
        hipExtLaunchKernelGGL((markov_fused_kernel<T, VEC>), dim3(G), dim3(kFusedThreads), 0, st, ps.start(),
                              ps.stop(), 0, arg);
        if (chain) (void)hipEventRecord(g_chain.ev[dev], st);
      } else if (chain) {
        hipExtLaunchKernelGGL((markov_fused_kernel<T, VEC>), dim3(G), dim3(kFusedThreads), 0, st, nullptr,
                              g_chain.ev[dev], 0, arg);
      } else {
        hipLaunchKernelGGL((markov_fused_kernel<T, VEC>), dim3(G), dim3(kFusedThreads), 0, st, arg);
      }
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (chain) g_chain.last[dev] = st;
    }
  } else {
    const dim3 g_step(a.C, (a.B + kTile - 1) / kTile);
    for (int k = 1; k <= a.gamma; ++k) {
      DSPARK_LAUNCH("markov_step", (markov_step_kernel<T, VEC>), g_step, dim3(kStepThreads), 0, st,
                    a, k);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      DSPARK_LAUNCH("markov_finalize", markov_finalize_kernel<VEC>, dim3(a.B), dim3(kFinThreads),
                    0, st, a, k);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  DSPARK_LAUNCH("markov_confidence", markov_confidence_kernel, dim3(a.B * a.gamma),
                dim3(kConfThreads), 0, st, a);
  return hipGetLastError();
}

template <typename T, bool VEC>
hipError_t launch_typed(const MarkovArgs& a, int plan_mode, hipStream_t st) {
  // fused when its grid (one workgroup per 512 tokens) is resident at once
  const int G = (a.V + kFusedTokens - 1) / kFusedTokens;
  int fused = 0;
  if (plan_mode == DSPARK_MARKOV_AUTO) {
    const FusedFit f = fused_fit<T, VEC>();
    if (f.blocks_per_cu > 0 && G <= f.blocks_per_cu * stream_cus(st, f.cus)) fused = 1;
  } else if (plan_mode == DSPARK_MARKOV_COOPERATIVE) {
    const FusedFit f = fused_fit<T, VEC>();
    if (f.coop && f.blocks_per_cu > 0 && G <= f.blocks_per_cu * f.cus) fused = 2;
  }
  return launch_plan<T, VEC>(a, fused, st);
}

}  // namespace

MarkovPlan plan_markov(int32_t B, int32_t gamma, int32_t V, int32_t r, int32_t d) {
  (void)r;
  (void)d;
  MarkovPlan p{};
  p.C = (V + kChunk - 1) / kChunk;
  p.off_part = 0;  // one slice of B x C records per step
  size_t off = align_up(static_cast<size_t>(gamma) * B * p.C * sizeof(ChunkPart), 256);
  p.off_sync = off;
  off += align_up(kSyncWords * sizeof(uint32_t), 256);
  p.bytes = off;
  return p;
}

hipError_t launch_markov(const void* backbone, int dtype, const int32_t* anchor,
                         const uint16_t* w1, const uint16_t* w2, const uint16_t* hidden,
                         const uint16_t* embed, const float* conf_w, dspark_policy pol,
                         uint64_t seed, int32_t B, int32_t gamma, int32_t V, int32_t r, int32_t d,
                         int32_t* draft_tokens, float* q_z, float* q_lse, float* q_thr,
                         float* q_tok, float* confidence, uint8_t* flags, void* ws,
                         const MarkovPlan& plan, int plan_mode, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  MarkovArgs a{};
  a.backbone = backbone;
  a.anchor = anchor;
  a.w1 = w1;
  a.w2 = w2;
  a.hidden = hidden;
  a.embed = embed;
  a.conf_w = conf_w;
  a.pol = pol;
  a.seed = seed;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.r = r;
  a.d = d;
  a.C = plan.C;
  // 16-byte loads of the confidence head's rows and weights
  a.cvec = (d % 8 == 0) && reinterpret_cast<uintptr_t>(hidden) % 16 == 0 &&
           reinterpret_cast<uintptr_t>(embed) % 16 == 0 &&
           reinterpret_cast<uintptr_t>(conf_w) % 16 == 0;
  a.draft_tokens = draft_tokens;
  a.q_z = q_z;
  a.q_lse = q_lse;
  a.q_thr = q_thr;
  a.q_tok = q_tok;
  a.confidence = confidence;
  a.flags = flags;
  a.part = reinterpret_cast<ChunkPart*>(w + plan.off_part);
  a.sync = reinterpret_cast<uint32_t*>(w + plan.off_sync);
  const bool vec = (V % 4 == 0) && (reinterpret_cast<uintptr_t>(backbone) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(q_z) % 16 == 0);
  if (dtype == DSPARK_BF16)
    return vec ? launch_typed<uint16_t, true>(a, plan_mode, st)
               : launch_typed<uint16_t, false>(a, plan_mode, st);
  return vec ? launch_typed<float, true>(a, plan_mode, st) : launch_typed<float, false>(a, plan_mode, st);
}

}  // namespace dspark
