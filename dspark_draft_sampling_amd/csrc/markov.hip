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
// Three launch plans run these phases:
//  * fused: one launch for all gamma steps (its whole grid resident at once).
//    Workgroup g owns the 512 tokens [512 g, 512 g + 512) and keeps their W2
//    rows in registers (the MFMA A fragments) for the whole call, so the
//    rank-r factor is read from HBM once per call rather than once per step.
//    A finalize starts when its request's records of the step are all
//    stored (polled, no grid barrier) and hands x_k to the next stream phase
//    through tagged words in the workspace: every word that crosses
//    workgroups carries the call's epoch, so nothing is cleared before the
//    launch (a captured call derives its epoch from the workspace:
//    dev_epoch_begin).  Everything that crosses workgroups inside the launch (records,
//    z rows read by the draw, x_k) is stored and loaded at device scope
//    (sc1), so no L2 writeback or invalidate is needed.  Without truncation
//    arrays the untruncated kernel (markov_fast) draws a candidate in every
//    workgroup and the finalize only compares records.
//  * per step: 2 gamma launches (stream kernel over all chunks, finalize
//    kernel over all requests), used when the fused grid cannot be resident
//    at once (V above 512 tokens per compute unit).
//  * request groups (on request, untruncated): the one-launch grid walks
//    16-request groups step by step, so one group's hand-off overlaps the
//    other groups' streaming; extra workgroups finalize (markov_pipe).
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
// Every wait of the one-launch plans for another workgroup's data gives up
// after this many ticks of the 100 MHz real-time counter (20 ms; a whole call
// takes well under 1 ms when its grid is resident).
constexpr uint64_t kWaitTicks = 2000000;
// Second-word patterns of the tagged two-word values (x_k, the timeout mark).
constexpr uint32_t kTokenCheck = 0x5A5A5A5Au;
constexpr uint32_t kTimeoutMark = 0x7113007Du;

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
  ChunkPart* part;  // per-step plan: chunk records [gamma][B][C]
  // one-launch plans: everything that crosses workgroups is a 64-bit word
  // (epoch << 32 | payload), so a reader accepts a word only from this call
  // and never depends on more than 64-bit single-copy atomicity
  uint32_t epoch;   // this call's tag (never 0); eager calls keep the top bit clear
  int32_t dev_epoch;  // captured call: the kernels derive the tag from the workspace
  int32_t G;        // workgroups of the one-launch plans (512-token slices)
  int32_t F;        // pipelined plan: finalizing workgroups after the G streaming ones (else 0)
  uint64_t* tpart;  // truncating plan: chunk records [gamma][B][C][4]
  uint64_t* frec;   // untruncated plan: workgroup records [gamma][B][7][G] (word-major)
  uint64_t* xk;     // x_k hand-off [gamma][B][2]
  uint64_t* sync;   // timeout mark [2], then the captured calls' epoch word
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

// The thread index, opaque to the optimiser: the phases of the one-launch plan
// recompute their lane-derived addresses instead of keeping them live (in
// registers) across the whole step loop.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// ---------------------------------------------------------------------------
// Tagged hand-off of the one-launch plans.  A 64-bit word carries the call's
// epoch in its upper half; it is stored and loaded as one agent-scope atomic
// (single-copy atomic at 64 bits, write-through to the device-coherent level),
// so a reader that sees the epoch sees the payload stored with it, and a word
// left by an earlier call (another epoch) is never taken for this call's.

__device__ __forceinline__ void st_tagged(uint64_t* p, uint32_t epoch, uint32_t v) {
  __hip_atomic_store(p, (static_cast<uint64_t>(epoch) << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tagged(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_is(uint64_t w, uint32_t epoch) { return static_cast<uint32_t>(w >> 32) == epoch; }
__device__ __forceinline__ uint32_t payload(uint64_t w) { return static_cast<uint32_t>(w); }
__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// The call's timeout mark: set by any wait that gave up; read by the waits
// (to give up at once) and by the confidence kernel (to flag every row).
__device__ __forceinline__ void mark_timeout(const MarkovArgs& a) {
  st_tagged(a.sync, a.epoch, kTimeoutMark);
  st_tagged(a.sync + 1, a.epoch, ~kTimeoutMark);
}
__device__ __forceinline__ bool timed_out(const MarkovArgs& a) {
  const uint64_t w0 = ld_tagged(a.sync), w1 = ld_tagged(a.sync + 1);
  return tag_is(w0, a.epoch) && tag_is(w1, a.epoch) && payload(w0) == kTimeoutMark &&
         payload(w1) == ~kTimeoutMark;
}
// A captured call cannot take its tag from the host (a graph replays its
// launch arguments), so the one-launch kernels derive it from the
// workspace's epoch word: the word + 1, with the top bit set (host tags keep
// it clear, so the two never meet).  Workgroup 0 stores the tag back at its
// end, once every workgroup has read the word: in the whole-step and
// truncating kernels its last finalize needs records of every workgroup; in
// the request-group kernel it first waits for the last step's x of every
// request, which needs every streaming and finalizing workgroup.  (A ticket
// counted by every workgroup would need no such argument, but 250-odd
// workgroups ending together on one compare-and-swap word cost about 250 us.)
// The kernels that follow in the call read the stored tag.
constexpr uint32_t kDevEpochBit = 0x80000000u;
__device__ __forceinline__ void dev_epoch_begin(MarkovArgs& a) {
  if (a.dev_epoch)
    a.epoch = ((static_cast<uint32_t>(ld_tagged(a.sync + 2)) + 1u) & ~kDevEpochBit) | kDevEpochBit;
}
__device__ __forceinline__ void dev_epoch_end(const MarkovArgs& a) {
  if (a.dev_epoch && blockIdx.x == 0 && threadIdx.x == 0) st_tagged(a.sync + 2, 0u, a.epoch & ~kDevEpochBit);
}
__device__ __forceinline__ void dev_epoch_after(MarkovArgs& a) {
  if (a.dev_epoch) a.epoch = (static_cast<uint32_t>(ld_tagged(a.sync + 2)) & ~kDevEpochBit) | kDevEpochBit;
}

// True (after marking the timeout) once a wait begun at t0 should give up.
__device__ __forceinline__ bool give_up(const MarkovArgs& a, uint64_t t0) {
  if (now_ticks() - t0 > kWaitTicks || timed_out(a)) {
    mark_timeout(a);
    return true;
  }
  return false;
}

// x_k of request b (step k) as two tagged words: the token and the token
// xor a fixed pattern.
__device__ __forceinline__ void put_token(const MarkovArgs& a, int k, int b, int32_t x) {
  uint64_t* p = a.xk + (static_cast<size_t>(k - 1) * a.B + b) * 2;
  st_tagged(p, a.epoch, static_cast<uint32_t>(x));
  st_tagged(p + 1, a.epoch, static_cast<uint32_t>(x) ^ kTokenCheck);
}
// Waits for x_k of request b; -1 if the wait gave up.
__device__ __forceinline__ int32_t wait_token(const MarkovArgs& a, int k, int b) {
  const uint64_t* p = a.xk + (static_cast<size_t>(k - 1) * a.B + b) * 2;
  const uint64_t t0 = now_ticks();
  for (uint32_t it = 1;; ++it) {
    const uint64_t w0 = ld_tagged(p), w1 = ld_tagged(p + 1);
    if (tag_is(w0, a.epoch) && tag_is(w1, a.epoch) && (payload(w0) ^ kTokenCheck) == payload(w1))
      return static_cast<int32_t>(payload(w0));
    if ((it & 31) == 0 && give_up(a, t0)) return -1;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Waits for the tagged chunk record idx of the truncating one-launch plan; a
// placeholder (no mass, no maximum) if the wait gave up.
__device__ __forceinline__ ChunkPart wait_part(const MarkovArgs& a, size_t idx) {
  const uint64_t* t = a.tpart + idx * 4;
  const uint64_t t0 = now_ticks();
  for (uint32_t it = 1;; ++it) {
    const uint64_t w0 = ld_tagged(t), w1 = ld_tagged(t + 1), w2 = ld_tagged(t + 2), w3 = ld_tagged(t + 3);
    if (tag_is(w0, a.epoch) && tag_is(w1, a.epoch) && tag_is(w2, a.epoch) && tag_is(w3, a.epoch))
      return ChunkPart{__uint_as_float(payload(w0)), __uint_as_float(payload(w1)), __uint_as_float(payload(w2)),
                       payload(w3)};
    if ((it & 31) == 0 && give_up(a, t0)) return ChunkPart{neg_inf(), 0.0f, neg_inf(), 0x7fffffffu};
    __builtin_amdgcn_s_sleep(1);
  }
}

// Partials of one request over a wave's 16 MS tokens, from the lane's 4 MS
// values z[4 ms + i] (token vb + 16 ms + 4 (lane >> 4) + i; the lanes l,
// l ^ 16, l ^ 32, l ^ 48 hold the request) and the wave's maximum m over
// them: sj[ms] = the sum of 2^(z log2e - m log2e) over 16-token sub-chunk ms
// (per lane over its four tokens in order, then (l0 + l1) + (l2 + l3) over
// the lanes), and s = the sum of the sj in a fixed order.  Every lane of the
// wave must call it; the results are equal on the four lanes of a request.
// The level-2 mass of sub-chunk ms relative to m is sj[ms] (the three-level
// draw inside a chunk forms the same sums from the same values).
template <int MS>
__device__ __forceinline__ void sub_partials(const float (&z)[4 * MS], float m, float (&sj)[MS], float& s) {
  // branch-free: with no finite maximum every z is -inf (or the row is
  // flagged), so a zero shift gives the empty sums 0
  const float mb = (m > neg_inf() && m < pos_inf()) ? m * kLog2e : 0.0f;
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) t += __builtin_amdgcn_exp2f(fmaf(z[4 * ms + i], kLog2e, -mb));
    sj[ms] = rows_sum(t);
  }
  if constexpr (MS == 4) {
    s = (sj[0] + sj[1]) + (sj[2] + sj[3]);
  } else {
    s = 0.0f;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) s += sj[ms];
  }
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
        // one-launch plan: x_{k-1} from its finalize's tagged hand-off
        xv = wait_token(a, k - 1, b);
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
          else __builtin_nontemporal_store(zv, reinterpret_cast<f32x4*>(dst));
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
    // sum of 2^((z - m) log2e) over the wave's tokens, through the
    // 16-token sub-chunk sums (the same arithmetic as the untruncated
    // one-launch kernel)
    float sj[MS], s;
    sub_partials<MS>(z, m, sj, s);
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
  size_t dst[kRecPerThread];  // record index, or kNoRec
  constexpr size_t kNoRec = ~static_cast<size_t>(0);
#pragma unroll
  for (int j = 0; j < kRecPerThread; ++j) {
    dst[j] = kNoRec;
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
    dst[j] = (static_cast<size_t>(k - 1) * B + b) * a.C + c;
  }
  if constexpr (COH) {
    // a record, once visible, vouches for every z of the step this
    // workgroup stored: all waves' stores complete before any record is
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < kRecPerThread; ++j)
    if (dst[j] != kNoRec) {
      const size_t idx = dst[j];
      if constexpr (COH) {
        uint64_t* t = a.tpart + idx * 4;
        st_tagged(t, a.epoch, __float_as_uint(rec[j].m));
        st_tagged(t + 1, a.epoch, __float_as_uint(rec[j].s));
        st_tagged(t + 2, a.epoch, __float_as_uint(rec[j].score));
        st_tagged(t + 3, a.epoch, rec[j].arg_nf);
      } else {
        a.part[idx] = rec[j];
      }
    }
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
  const float tp = top_p_of(a.pol.top_p, b);
  const int tk_raw = top_k_of(a.pol.top_k, b);
  const bool want_cm = sampled && truncated(tk_raw, tp, V) && C <= kMaxChunksBound;
  // a sampled row without truncation draws inside its best-scoring chunk:
  // each wave fetches its own best chunk while the waves' results merge, and
  // the wave holding the row's best draws from registers
  const bool spec = sampled && !truncated(tk_raw, tp, V);
  const QzRow<COH> qr(a.q_z + row * V, V, VEC);
  Top2 wbest;
  float zpre[4];
  for (int c = tid; c < C; c += NT) {
    ChunkPart p;
    if constexpr (COH) p = wait_part(a, (static_cast<size_t>(k - 1) * a.B + b) * C + c);
    else p = pb[c];
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
      if constexpr (COH) put_token(a, k, b, x);
      a.draft_tokens[row] = x;
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
      a.flags[row] = static_cast<uint8_t>(fl);
    }
  }
  __syncthreads();  // F is reused by the next request
}

// ---------------------------------------------------------------------------
// Untruncated one-launch plan (no request of the call truncates).
//
// Workgroup g owns the 512 tokens [512 g, 512 g + 512) (chunks 2g, 2g + 1)
// and keeps their W2 rows in registers, as in the truncating plan.  Nothing
// is read back across workgroups except small tagged records:
//  * in the stream phase each wave keeps, per request, the best two level-2
//    scores of its four 16-token sub-chunks and stashes the best one's 16 z
//    values in LDS;
//  * the workgroup then takes, per request, level 1 over its two chunks, level
//    2 over the chosen chunk's sub-chunks and level 3 over the chosen
//    sub-chunk's tokens: the token the draw would pick if the chunk choice
//    fell on this workgroup's best chunk;
//  * wave 0 stores one record per request (the slice's maximum and sum, its
//    argmax, its best and second chunk scores, the candidate and its z), and
//    one wave of workgroup b mod G finalizes request b: the record with the
//    best chunk score holds x_k.
// The q stores of a step are streaming (non-temporal) stores that drain while
// the hand-off runs: no record depends on them, and no dirty lines are left
// for the following kernels to write back.  Wave 0 does all the waiting (x_{k-1}, records),
// so its loads never queue behind the other waves' stores.

constexpr int kZ0Ld = 68;  // floats per row of wave 0's z tile (64 + 4: bank spread)
constexpr int kW1Slots = (kMaxR + kPad) / 8;  // 16-byte slots per staged W1 row (the last: padding)

struct FastLds {
  __attribute__((aligned(16))) uint16_t a[kTile * (kMaxR + kPad)];  // staged W1 rows (kW1Slots slots each)
  // per (wave, request): partials of the wave's 64 tokens
  float red_m[kFusedThreads / 64][kTile], red_s[kFusedThreads / 64][kTile];
  uint32_t red_i[kFusedThreads / 64][kTile];  // lowest argmax (bits 0..30); bit 31: NaN / +inf seen
  float sub_v1[kFusedThreads / 64][kTile], sub_v2[kFusedThreads / 64][kTile];  // best two level-2 scores
  int32_t sub_i1[kFusedThreads / 64][kTile];  // global sub-chunk index of the best
  __attribute__((aligned(16))) float stash[kFusedThreads / 64][kTile][kSub];   // its z values
  int32_t xs[kTile];
  uint32_t rec[kTile][8];  // the workgroup's record per request
  // Gumbel noise of the step (it does not depend on x_{k-1}): level 2 per
  // (wave, request, sub-chunk of the wave), level 1 per (request, chunk)
  __attribute__((aligned(16))) float g2[kFusedThreads / 64][kTile][4];
  float g1[kTile][2];
  // the tile's policy: 1 / T for sampled requests (0 for greedy, -1 absent),
  // request ids and the step's positions
  float invT[kTile];
  uint32_t req[kTile];
  int32_t pos[kTile];
  // wave 0's z tiles (stored to q by waves 4..7 one step later, so that no
  // barrier waits for those stores): by step parity, rows of 64 tokens, padded
  __attribute__((aligned(16))) float z0[2][kTile][kZ0Ld];
  float z0_invT[2][kTile];  // the tile's policy of that step (> 0: sampled)
};

// Waves 4..7: wave 0's z tile of step k (tile b0, workgroup tokens from tok0)
// to q, for the sampled requests; 16 lanes per 64-token row.
template <bool VEC>
__device__ __forceinline__ void store_z0(const MarkovArgs& a, const FastLds& L, int tok0, int b0, int k) {
  const int t = static_cast<int>(threadIdx.x) - 4 * kTile;
  const int par = k & 1;
#pragma unroll
  for (int i = 0; i < kTile * 16 / (4 * kTile); ++i) {
    const int f = t + i * 4 * kTile;
    const int n = f >> 4, col = (f & 15) * 4;
    if (!(L.z0_invT[par][n] > 0.0f)) continue;  // absent or greedy request
    const int v0 = tok0 + col;
    const f32x4 zz = *reinterpret_cast<const f32x4*>(&L.z0[par][n][col]);
    float* dst = a.q_z + (static_cast<size_t>(b0 + n) * a.gamma + (k - 1)) * a.V + v0;
    if (VEC && v0 + 3 < a.V) {
      __builtin_nontemporal_store(zz, reinterpret_cast<f32x4*>(dst));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (v0 + e < a.V) dst[e] = zz[e];
    }
  }
}

// Step k of the requests [b0, b0 + 64) over workgroup g's tokens.  EDGE: the
// tile holds absent requests or the workgroup tokens past the vocabulary
// (element-wise checks); otherwise every value is in range.
template <typename T, bool VEC, bool EDGE>
__device__ __forceinline__ void fast_tile(const MarkovArgs& a, const bf16x8 (&af)[kFusedMS][kMaxR / 32], int g,
                                          int b0, int k, FastLds& L) {
  constexpr int MS = kFusedMS, NH = 4, NSP = 1, TPW = 16 * MS;
  const T* __restrict__ backbone = static_cast<const T*>(a.backbone);
  const int B = a.B, gamma = a.gamma, V = a.V, r = a.r;
  const int tid = opaque_tid(), lane = tid & 63, wave = wave_id();
  const int tok0 = g * kFusedTokens;
  const int vb = tok0 + wave * TPW;
  const int kpad = (r + 31) & ~31;
  constexpr int ld = kMaxR + kPad;  // fixed row stride of the DMA-staged W1 rows
  const int ksteps = kpad / 32;

  typedef __attribute__((address_space(3))) void lds_void;
  // the backbone values do not depend on x_{k-1}: waves 1..7 request them
  // first (behind their previous q stores); wave 0, which does the waiting,
  // requests its own after x_{k-1} arrived, so that no poll queues behind them
  QuadRaw<T> bbv[NH][NSP][MS];
  if (wave != 0) {
#pragma unroll
    for (int h = 0; h < NH; ++h)
      load_backbone<T, VEC, MS, NSP>(bbv[h], backbone, B, gamma, V, k, b0, h * NSP, vb, lane);
  }

  // the step's level-2 noise (thread (w, n): sub-chunks 4w .. 4w+3 of the
  // workgroup for request n, one Philox block) and level-1 noise (wave 1:
  // chunks 2g, 2g+1), while wave 0 waits for x_{k-1}
  {
    const int n = lane;
    const int b = b0 + n;
    uint32_t req = 0;
    int32_t pos = 0;
    if (b < B) {
      req = a.pol.request_id[b];
      pos = a.pol.position[b] + k;
    }
    if (wave == 2) {
      float it = -1.0f;
      if (b < B) {
        const float Tb = a.pol.temperature[b];
        it = (a.pol.mode[b] != 0 && !bad_temperature(Tb)) ? 1.0f / Tb : 0.0f;
      }
      L.invT[n] = it;
      L.req[n] = req;
      L.pos[n] = pos;
    }
    uint32_t c0 = (static_cast<uint32_t>(tok0) >> 6) + static_cast<uint32_t>(wave), c1 = static_cast<uint32_t>(pos),
             c2 = req, c3 = DSPARK_TAG_DRAFT_SUB;
    philox4x32_10(c0, c1, c2, c3, static_cast<uint32_t>(a.seed), static_cast<uint32_t>(a.seed >> 32));
    *reinterpret_cast<f32x4*>(&L.g2[wave][n][0]) = f32x4{gumbel_of(c0), gumbel_of(c1), gumbel_of(c2), gumbel_of(c3)};
    if (wave == 1) {
      uint32_t d0 = static_cast<uint32_t>(2 * g) >> 2, d1 = static_cast<uint32_t>(pos), d2 = req,
               d3 = DSPARK_TAG_DRAFT_CHUNK;
      philox4x32_10(d0, d1, d2, d3, static_cast<uint32_t>(a.seed), static_cast<uint32_t>(a.seed >> 32));
      const uint32_t cw[4] = {d0, d1, d2, d3};
      L.g1[n][0] = gumbel_of(cw[(2 * g) & 3]);
      L.g1[n][1] = gumbel_of(cw[(2 * g + 1) & 3]);
    }
  }
  if (wave == 0) {
    int32_t xv = -1;
    const int b = b0 + lane;
    if (b < B) {
      xv = k == 1 ? a.anchor[b] : wait_token(a, k - 1, b);
      xv = clamp_token(xv, V);
    }
    L.xs[lane] = xv;
#pragma unroll
    for (int h = 0; h < NH; ++h)
      load_backbone<T, VEC, MS, NSP>(bbv[h], backbone, B, gamma, V, k, b0, h * NSP, vb, lane);
    // the tile's W1 rows (MFMA B operand) by LDS DMA: instruction q fills the
    // 16-byte slots 64 q .. 64 q + 63 (row n = slot / kW1Slots); padding
    // slots, pieces past the rank and absent rows read past the buffer (0)
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.w1), static_cast<short>(0), V * r * 2, kBufferWord3);
#pragma unroll
    for (int q = 0; q < kTile * kW1Slots / 64; ++q) {
      const int sl = q * 64 + lane, n = sl / kW1Slots, c = sl - n * kW1Slots;
      const int32_t x = L.xs[n];
      const bool ok = c < kW1Slots - 1 && c * 8 < r && x >= 0;
      const uint32_t off = ok ? static_cast<uint32_t>((x * r + c * 8) * 2) : 0xfffffff0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(L.a + q * 64 * 8), 16, off, 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the DMA (and the backbone loads) landed
  }
  if (wave == 2) L.z0_invT[k & 1][lane] = L.invT[lane];
  __syncthreads();
  // waves 4..7: wave 0's z tile of the previous step (a one-tile batch; a
  // batch of several tiles stores each tile's right after its draw)
  if (tid >= 4 * kTile && B <= kTile && k > 1) store_z0<VEC>(a, L, tok0, b0, k - 1);

  const uint32_t jbase = static_cast<uint32_t>(vb) >> 4;  // global index of the wave's first sub-chunk
  const int q = lane >> 4;                                // this lane's sub-chunk for level 2
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    f32x4 acc[MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) acc[ms] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kMaxR / 32; ++ks) {
      if (ks < ksteps) {
        const bf16x8 bfr = load_frag(L.a + (h * 16 + (lane & 15)) * ld + ks * 32 + (lane >> 4) * 8);
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
          acc[ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ms][ks], bfr, acc[ms], 0, 0, 0);
      }
    }
    // epilogue: lane holds tokens vb + ms*16 + 4*(lane>>4) + i of request n
    const int n = h * 16 + (lane & 15);
    const int b = b0 + n;
    const float pit = L.invT[n];  // 1 / T (sampled), 0 (greedy), -1 (absent)
    const bool bvalid = pit >= 0.0f;
    const bool sampled = pit > 0.0f;
    const float invT = sampled ? pit : 1.0f;
    const size_t rowoff = (static_cast<size_t>(bvalid ? b : 0) * gamma + (k - 1)) * V;
    float z[4 * MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int v0 = vb + ms * 16 + 4 * (lane >> 4);
      const QuadRaw<T>& bb = bbv[h][0][ms];
      const bool full = bvalid && v0 + 3 < V;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y = (acc[ms][i] + bb.at(i)) * invT;
        if constexpr (EDGE) z[ms * 4 + i] = (bvalid && v0 + i < V) ? y : neg_inf();
        else z[ms * 4 + i] = y;
      }
      if (wave == 0) {
        // wave 0 keeps its memory queue free for the hand-off: its z go to
        // LDS and waves 4..7 store them
        *reinterpret_cast<f32x4*>(&L.z0[k & 1][n][ms * 16 + 4 * (lane >> 4)]) =
            f32x4{z[ms * 4], z[ms * 4 + 1], z[ms * 4 + 2], z[ms * 4 + 3]};
      } else if (VEC && !EDGE) {
        if (sampled)
          __builtin_nontemporal_store(f32x4{z[ms * 4], z[ms * 4 + 1], z[ms * 4 + 2], z[ms * 4 + 3]},
                                      reinterpret_cast<f32x4*>(a.q_z + rowoff + v0));
      } else if (sampled) {
        float* dst = a.q_z + rowoff + v0;
        if (VEC && full) {
          __builtin_nontemporal_store(f32x4{z[ms * 4], z[ms * 4 + 1], z[ms * 4 + 2], z[ms * 4 + 3]},
                                      reinterpret_cast<f32x4*>(dst));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (v0 + i < V) dst[i] = z[ms * 4 + i];
        }
      }
    }
    // the wave's maximum over its 64 tokens
    float lm = z[0];
#pragma unroll
    for (int e = 1; e < 4 * MS; ++e) lm = fmaxf(lm, z[e]);
    const float m = rows_max(lm);
    // lowest argmax, only when the pass holds a greedy request
    int32_t arg = INT32_MAX;
    if (__builtin_amdgcn_ballot_w64(bvalid && !sampled)) {
#pragma unroll
      for (int e = 4 * MS - 1; e >= 0; --e)
        if (z[e] == m && m > neg_inf()) arg = vb + (e >> 2) * 16 + 4 * (lane >> 4) + (e & 3);
      arg = static_cast<int32_t>(rows_combine(static_cast<uint32_t>(arg), [](uint32_t p, uint32_t q) {
        return p < q ? p : q;
      }));
    }
    // sub-chunk sums relative to m (the level-2 masses) and the wave's sum;
    // a NaN, or +inf, in the row shows as a NaN sum or an infinite maximum
    float sj[MS], s;
    sub_partials<MS>(z, m, sj, s);
    const bool bad = s != s || m == pos_inf();
    // level 2 inside the wave: lane row q scores sub-chunk jbase + q
    const float sq = q == 0 ? sj[0] : q == 1 ? sj[1] : q == 2 ? sj[2] : sj[3];
    Top2 t2{neg_inf(), INT32_MAX, neg_inf()};
    if (sampled && m > neg_inf() && !bad && sq > 0.0f)
      t2 = Top2{m + logf(sq) + L.g2[wave][n][q], static_cast<int32_t>(jbase + q), neg_inf()};
    t2 = rows_top2(t2);
    if (t2.i1 != INT32_MAX) {
      const int m1 = t2.i1 - static_cast<int32_t>(jbase);
      const f32x4 zz = m1 == 0   ? f32x4{z[0], z[1], z[2], z[3]}
                       : m1 == 1 ? f32x4{z[4], z[5], z[6], z[7]}
                       : m1 == 2 ? f32x4{z[8], z[9], z[10], z[11]}
                                 : f32x4{z[12], z[13], z[14], z[15]};
      *reinterpret_cast<f32x4*>(&L.stash[wave][n][4 * q]) = zz;
    }
    if (q == 0) {
      L.red_m[wave][n] = m;
      L.red_s[wave][n] = s;
      L.red_i[wave][n] = (static_cast<uint32_t>(arg) & 0x7fffffffu) | (bad ? 0x80000000u : 0u);
      L.sub_v1[wave][n] = t2.v1;
      L.sub_i1[wave][n] = t2.i1;
      L.sub_v2[wave][n] = t2.v2;
    }
  }
  __syncthreads();  // every wave's partials, stash and wave 0's z tile are in LDS
  if (tid >= 4 * kTile && B > kTile) store_z0<VEC>(a, L, tok0, b0, k);

  // the workgroup's candidate per request: 4 threads per request (waves 0-3,
  // one per SIMD)
  if (tid < 4 * kTile) {
    const int n = tid >> 2, p = tid & 3;
    float wm[8], wsum[8];
    uint32_t wi[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      wm[w] = L.red_m[w][n];
      wsum[w] = L.red_s[w][n];
      wi[w] = L.red_i[w][n];
    }
    ArgMax am{wm[0], static_cast<int32_t>(wi[0] & 0x7fffffffu)};
    uint32_t bad = wi[0] >> 31;
#pragma unroll
    for (int w = 1; w < 8; ++w) {
      am = better(am, ArgMax{wm[w], static_cast<int32_t>(wi[w] & 0x7fffffffu)});
      bad |= wi[w] >> 31;
    }
    const bool sampled = L.invT[n] > 0.0f;
    const uint32_t req = L.req[n];
    const int32_t pos = L.pos[n];
    // level 1 over the workgroup's chunks 2g, 2g + 1 (their partials merged
    // wave by wave, as the chunk records of the truncating kernel); the
    // workgroup's partials are the two chunks' merged
    float sc[2], cmv[2], csv[2];
#pragma unroll
    for (int hc = 0; hc < 2; ++hc) {
      const int c = 2 * g + hc;
      float cm = wm[4 * hc], cs = wsum[4 * hc];
#pragma unroll
      for (int w = 1; w < 4; ++w) lse_merge(cm, cs, wm[4 * hc + w], wsum[4 * hc + w]);
      cmv[hc] = cm;
      csv[hc] = cs;
      sc[hc] = (sampled && c < a.C && cm > neg_inf() && cm < pos_inf() && cs > 0.0f)
                   ? cm + logf(cs) + L.g1[n][hc]
                   : neg_inf();
    }
    float m = cmv[0], s = csv[0];
    lse_merge(m, s, cmv[1], csv[1]);
    const int hb = sc[1] > sc[0] ? 1 : 0;
    // level 2 over the chosen chunk's sub-chunks (its waves' best two)
    Top2 t2{neg_inf(), INT32_MAX, neg_inf()};
#pragma unroll
    for (int w = 0; w < 4; ++w)
      t2 = top2_merge(t2, Top2{L.sub_v1[4 * hb + w][n], L.sub_i1[4 * hb + w][n], L.sub_v2[4 * hb + w][n]});
    // level 3 over the chosen sub-chunk's tokens: thread p takes 4p .. 4p+3
    const bool draw = sampled && sc[hb] > neg_inf() && t2.i1 != INT32_MAX;
    Top2 t3{neg_inf(), INT32_MAX, neg_inf()};
    f32x4 zz = f32x4{neg_inf(), neg_inf(), neg_inf(), neg_inf()};
    if (draw) {
      const int wj = (t2.i1 - (tok0 >> 4)) >> 2;  // wave holding the sub-chunk
      zz = *reinterpret_cast<const f32x4*>(&L.stash[wj][n][4 * p]);
      uint32_t d0 = static_cast<uint32_t>(t2.i1) * 4u + static_cast<uint32_t>(p), d1 = static_cast<uint32_t>(pos),
               d2 = req, d3 = DSPARK_TAG_DRAFT_TOKEN;
      philox4x32_10(d0, d1, d2, d3, static_cast<uint32_t>(a.seed), static_cast<uint32_t>(a.seed >> 32));
      const uint32_t tw[4] = {d0, d1, d2, d3};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (zz[e] > neg_inf())
          t3 = top2_merge(t3, Top2{zz[e] + gumbel_of(tw[e]), t2.i1 * kSub + 4 * p + e, neg_inf()});
    }
    t3 = quad_top2(t3);
    float zmine = neg_inf();
    if (draw && t3.i1 != INT32_MAX && ((t3.i1 - t2.i1 * kSub) >> 2) == p) {
      const int e = t3.i1 & 3;
      zmine = e == 0 ? zz[0] : e == 1 ? zz[1] : e == 2 ? zz[2] : zz[3];
    }
    const float zc = quad_max(zmine);
    const bool near23 = (t2.v2 > neg_inf() && near_gap(t2.v1, t2.v2)) ||
                        (t3.i1 != INT32_MAX && t3.v2 > neg_inf() && near_gap(t3.v1, t3.v2));
    if (p == 0) {
      L.rec[n][0] = __float_as_uint(m);
      L.rec[n][1] = __float_as_uint(s);
      L.rec[n][2] = __float_as_uint(sc[hb]);
      L.rec[n][3] = __float_as_uint(sc[1 - hb]);
      L.rec[n][4] = (static_cast<uint32_t>(am.i) & 0x7fffffffu) | (bad ? 0x80000000u : 0u);
      L.rec[n][5] = (draw && t3.i1 != INT32_MAX)
                        ? (0x80000000u | (near23 ? 0x40000000u : 0u) | static_cast<uint32_t>(t3.i1))
                        : 0u;
      L.rec[n][6] = __float_as_uint(zc);
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int b = b0 + lane;
    if (b < B) {
      // word i of every workgroup's record sits side by side: the finalize
      // reads each word of 64 records with one contiguous 512-byte load
      uint64_t* R = a.frec + (static_cast<size_t>(k - 1) * B + b) * 7 * a.G + g;
#pragma unroll
      for (int i = 0; i < 7; ++i) st_tagged(R + static_cast<size_t>(i) * a.G, a.epoch, L.rec[lane][i]);
    }
  }
}

// Finalize step k of request b from the G workgroup records, by one wave.
constexpr int kFastMaxG = 256;
__device__ __forceinline__ void fast_finalize(const MarkovArgs& a, int b, int k) {
  constexpr int kPer = kFastMaxG / 64;  // records per lane
  const int lane = threadIdx.x & 63;
  const int G = a.G;
  const uint64_t* R = a.frec + (static_cast<size_t>(k - 1) * a.B + b) * 7 * G;
  // the request's policy, read before the wait
  const float Tb = a.pol.temperature[b];
  const bool req_sampled = a.pol.mode[b] != 0;
  // every poll issues the loads of all of the lane's records at once (absent
  // records read record 0 and are ignored); a record once whole stays whole
  const uint64_t* rp[kPer];
#pragma unroll
  for (int t = 0; t < kPer; ++t) rp[t] = R + (lane + 64 * t < G ? lane + 64 * t : 0);
  uint64_t w[kPer][7];
  uint32_t have = 0;  // bit t: record lane + 64 t read whole (or absent)
  const uint64_t t0 = now_ticks();
  for (uint32_t it = 1;; ++it) {
#pragma unroll
    for (int t = 0; t < kPer; ++t)
#pragma unroll
      for (int i = 0; i < 7; ++i) w[t][i] = ld_tagged(rp[t] + static_cast<size_t>(i) * G);
    have = 0;
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      bool ok = lane + 64 * t >= G;
      if (!ok) {
        ok = true;
#pragma unroll
        for (int i = 0; i < 7; ++i) ok = ok && tag_is(w[t][i], a.epoch);
      }
      if (ok) have |= 1u << t;
    }
    if (have == (1u << kPer) - 1) break;
    if ((it & 31) == 0 && give_up(a, t0)) break;
    __builtin_amdgcn_s_sleep(1);
  }
  float m = neg_inf(), s = 0.0f;
  ArgMax am{neg_inf(), INT32_MAX};
  Top2 best{neg_inf(), INT32_MAX, neg_inf()};
  uint32_t bad = 0;
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    if (lane + 64 * t >= G || !(have & (1u << t))) continue;
    const float rm = __uint_as_float(payload(w[t][0])), rs = __uint_as_float(payload(w[t][1]));
    const float s1 = __uint_as_float(payload(w[t][2])), s2 = __uint_as_float(payload(w[t][3]));
    const uint32_t ai = payload(w[t][4]), cand = payload(w[t][5]);
    lse_merge(m, s, rm, rs);
    am = better(am, ArgMax{rm, static_cast<int32_t>(ai & 0x7fffffffu)});
    bad |= ai >> 31;
    if ((cand >> 31) && s1 > neg_inf())
      best = top2_merge(best, Top2{s1, static_cast<int32_t>(cand & 0x3fffffffu), s2});
  }
  const float M = wave_max(m);
  const float S = wave_sum((m > neg_inf() && M < pos_inf()) ? s * __builtin_amdgcn_exp2f((m - M) * kLog2e) : 0.0f);
  const ArgMax A = wave_argmax(am);
  const Top2 Bst = wave_top2(best);
  const uint32_t anybad = wave_or(bad);
  // the winning record's candidate z and its level-2 / level-3 margin bit
  float zw = neg_inf();
  uint32_t nw = 0;
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    if (lane + 64 * t >= G || !(have & (1u << t))) continue;
    const uint32_t cand = payload(w[t][5]);
    if ((cand >> 31) && static_cast<int32_t>(cand & 0x3fffffffu) == Bst.i1) {
      zw = __uint_as_float(payload(w[t][6]));
      nw = (cand >> 30) & 1u;
    }
  }
  zw = wave_max(zw);
  nw = wave_or(nw);
  if (lane == 0) {
    const size_t row = static_cast<size_t>(b) * a.gamma + (k - 1);
    const bool sampled = req_sampled && !bad_temperature(Tb);
    uint32_t fl = anybad ? DSPARK_FLAG_NONFINITE : 0u;
    int32_t x = 0;
    if (!sampled) {
      if (A.i == INT32_MAX) fl |= DSPARK_FLAG_EMPTY_ROW;
      else x = A.i;
    } else if (Bst.i1 == INT32_MAX) {
      fl |= DSPARK_FLAG_EMPTY_ROW;
    } else {
      x = Bst.i1;
      if ((Bst.v2 > neg_inf() && near_gap(Bst.v1, Bst.v2)) || nw) fl |= DSPARK_FLAG_NEAR_THRESHOLD;
    }
    // x_k first: the next step's workgroups wait for it
    put_token(a, k, b, x);
    a.draft_tokens[row] = x;
    if (!sampled) {
      a.q_lse[row] = 0.0f;
      a.q_thr[row] = 0.0f;
      a.q_tok[row] = 1.0f;
    } else {
      a.q_lse[row] = M + logf(S);
      a.q_thr[row] = neg_inf();
      a.q_tok[row] = (zw > neg_inf() && S > 0.0f) ? expf(zw - M) / S : 0.0f;
    }
    if (req_sampled && !sampled) fl |= DSPARK_FLAG_BAD_POLICY;
    a.flags[row] = static_cast<uint8_t>(fl);
  }
}

// ---------------------------------------------------------------------------
// Pipelined untruncated one-launch plan.
//
// Request b's step k depends on nothing but its own x_{k-1}, so the batch is
// cut into groups of 16 requests (one MFMA N block) and each streaming
// workgroup walks the passes (step k, group j) in step-major order: pass
// p = (k - 1) NG + j.  A group's hand-off (records, finalize, x_k, its W1
// rows) then runs while the other NG - 1 groups of the step stream, instead
// of stalling the whole batch once per step.
//  * Workgroups 0 .. G-1 stream (512 tokens each, W2 rows in registers, as in
//    markov_fast); workgroups G .. G+F-1 hold no W2 and only finalize
//    (fast_finalize: one wave per request).
//  * One barrier per pass.  Two waves have a duty besides their tokens and
//    issue no q stores (their z go to LDS and waves 2, 3, 6, 7 store them one
//    pass later), so their polls and record stores never queue behind
//    streaming stores:
//    - wave 0 polls the next pass's x words before the products, takes them
//      after, and stages the next pass's W1 rows by LDS DMA into the other
//      buffer while the epilogue runs;
//    - wave 1 draws the previous pass's candidates from the LDS partials
//      (markov_fast's three-level draw, with the level-1 noise of every
//      request and step drawn once, at the start of the call) and stores the
//      records.
//  * Every other wave requests the backbone values of pass p+1 before pass
//    p's products, so they arrive while pass p runs.
// The partials (lanes, tokens, reduction orders, noise), the draw and the
// records are markov_fast's, so every output is equal bit for bit.
constexpr int kGrp = 16;          // requests per pass (MFMA N block)
constexpr int kPipeMaxB = 256;    // requests per call (policy held in LDS)
constexpr int kPipeFin = 2;       // finalizing workgroups, at most
constexpr int kPipeDma = 9;       // DMA instructions per pass (kGrp rows x kW1Slots slots, rounded up)

struct PipeLds {
  // W1 rows of a pass by pass parity (kW1Slots 16-byte slots per row, the
  // last DMA instruction's excess slots land in the padding)
  __attribute__((aligned(16))) uint16_t a[2][kPipeDma * 64 * 8];
  float red_m[2][8][kGrp], red_s[2][8][kGrp];
  uint32_t red_i[2][8][kGrp];
  float sub_v1[2][8][kGrp], sub_v2[2][8][kGrp];
  int32_t sub_i1[2][8][kGrp];
  __attribute__((aligned(16))) float stash[2][8][kGrp][kSub];
  // waves 0 and 1: z tiles by pass parity, rows of 64 tokens, padded
  __attribute__((aligned(16))) float z01[2][2][kGrp][kZ0Ld];
  // level-2 noise of each wave's four sub-chunks for four consecutive groups
  __attribute__((aligned(16))) float g2[8][4][kGrp][4];
  // level-1 noise of the workgroup's two chunks per (request, step)
  float g1[kPipeMaxB][DSPARK_MAX_GAMMA][2];
  // the batch's policy: 1 / T (sampled), 0 (greedy), -1 (absent); request
  // ids; positions of the anchors
  float invT[kPipeMaxB];
  uint32_t req[kPipeMaxB];
  int32_t pos0[kPipeMaxB];
  int32_t xs[kGrp];
};

// Backbone values of this lane for pass (k, j): tokens vb + 16 ms + 4 (lane >> 4)
// + i of request 16 j + (lane & 15).
template <typename T, bool VEC>
__device__ __forceinline__ void pipe_backbone(QuadRaw<T> (&bb)[kFusedMS], const MarkovArgs& a, int k, int j,
                                              int vb, int lane) {
  QuadRaw<T> t[1][kFusedMS];
  load_backbone<T, VEC, kFusedMS, 1>(t, static_cast<const T*>(a.backbone), a.B, a.gamma, a.V, k, j * kGrp, 0, vb,
                                     lane);
#pragma unroll
  for (int ms = 0; ms < kFusedMS; ++ms) bb[ms] = t[0][ms];
}

// Waves 2, 3, 6, 7: the z tiles of waves 0 and 1 of pass (k, j) to q, for the
// sampled requests (thread t of the four waves: one 16-byte piece of each tile).
template <bool VEC>
__device__ __forceinline__ void pipe_store_z01(const MarkovArgs& a, const PipeLds& L, int tok0, int k, int j,
                                               int par, int t) {
  const int n = t >> 4, col = (t & 15) * 4;
  const int b = j * kGrp + n;
  if (!(L.invT[b] > 0.0f)) return;  // absent or greedy request
  float* row = a.q_z + (static_cast<size_t>(b) * a.gamma + (k - 1)) * a.V;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const int v0 = tok0 + w * 64 + col;
    const f32x4 zz = *reinterpret_cast<const f32x4*>(&L.z01[par][w][n][col]);
    if (VEC && v0 + 3 < a.V) {
      __builtin_nontemporal_store(zz, reinterpret_cast<f32x4*>(row + v0));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (v0 + e < a.V) row[v0 + e] = zz[e];
    }
  }
}

// Wave 1: the workgroup's candidate of every request of pass (k, j) (four
// lanes per request, as markov_fast's draw, with the level-1 noise drawn at
// the start of the call) and its tagged record, word-major
// [gamma][B][7][G] as markov_fast's.
__device__ __forceinline__ void pipe_draw(const MarkovArgs& a, const PipeLds& L, int g, int k, int j, int par) {
  const int lane = threadIdx.x & 63;
  const int n = lane >> 2, p = lane & 3;
  const int b = j * kGrp + n;
  const int tok0 = g * kFusedTokens;
  float wm[8], wsum[8];
  uint32_t wi[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    wm[w] = L.red_m[par][w][n];
    wsum[w] = L.red_s[par][w][n];
    wi[w] = L.red_i[par][w][n];
  }
  ArgMax am{wm[0], static_cast<int32_t>(wi[0] & 0x7fffffffu)};
  uint32_t bad = wi[0] >> 31;
#pragma unroll
  for (int w = 1; w < 8; ++w) {
    am = better(am, ArgMax{wm[w], static_cast<int32_t>(wi[w] & 0x7fffffffu)});
    bad |= wi[w] >> 31;
  }
  const bool sampled = L.invT[b] > 0.0f;
  const uint32_t req = L.req[b];
  const int32_t pos = L.pos0[b] + k;
  float sc[2], cmv[2], csv[2];
#pragma unroll
  for (int hc = 0; hc < 2; ++hc) {
    const int c = 2 * g + hc;
    float cm = wm[4 * hc], cs = wsum[4 * hc];
#pragma unroll
    for (int w = 1; w < 4; ++w) lse_merge(cm, cs, wm[4 * hc + w], wsum[4 * hc + w]);
    cmv[hc] = cm;
    csv[hc] = cs;
    sc[hc] = (sampled && c < a.C && cm > neg_inf() && cm < pos_inf() && cs > 0.0f)
                 ? cm + logf(cs) + L.g1[b][k - 1][hc]
                 : neg_inf();
  }
  float m = cmv[0], s = csv[0];
  lse_merge(m, s, cmv[1], csv[1]);
  const int hb = sc[1] > sc[0] ? 1 : 0;
  Top2 t2{neg_inf(), INT32_MAX, neg_inf()};
#pragma unroll
  for (int w = 0; w < 4; ++w)
    t2 = top2_merge(t2, Top2{L.sub_v1[par][4 * hb + w][n], L.sub_i1[par][4 * hb + w][n], L.sub_v2[par][4 * hb + w][n]});
  // level 3 over the chosen sub-chunk's tokens: lane p takes 4p .. 4p+3
  const bool draw = sampled && sc[hb] > neg_inf() && t2.i1 != INT32_MAX;
  Top2 t3{neg_inf(), INT32_MAX, neg_inf()};
  f32x4 zz = f32x4{neg_inf(), neg_inf(), neg_inf(), neg_inf()};
  if (draw) {
    const int wj = (t2.i1 - (tok0 >> 4)) >> 2;  // wave holding the sub-chunk
    zz = *reinterpret_cast<const f32x4*>(&L.stash[par][wj][n][4 * p]);
    uint32_t d0 = static_cast<uint32_t>(t2.i1) * 4u + static_cast<uint32_t>(p), d1 = static_cast<uint32_t>(pos),
             d2 = req, d3 = DSPARK_TAG_DRAFT_TOKEN;
    philox4x32_10(d0, d1, d2, d3, static_cast<uint32_t>(a.seed), static_cast<uint32_t>(a.seed >> 32));
    const uint32_t tw[4] = {d0, d1, d2, d3};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (zz[e] > neg_inf()) t3 = top2_merge(t3, Top2{zz[e] + gumbel_of(tw[e]), t2.i1 * kSub + 4 * p + e, neg_inf()});
  }
  t3 = quad_top2(t3);
  float zmine = neg_inf();
  if (draw && t3.i1 != INT32_MAX && ((t3.i1 - t2.i1 * kSub) >> 2) == p) {
    const int e = t3.i1 & 3;
    zmine = e == 0 ? zz[0] : e == 1 ? zz[1] : e == 2 ? zz[2] : zz[3];
  }
  const float zc = quad_max(zmine);
  const bool near23 = (t2.v2 > neg_inf() && near_gap(t2.v1, t2.v2)) ||
                      (t3.i1 != INT32_MAX && t3.v2 > neg_inf() && near_gap(t3.v1, t3.v2));
  if (b < a.B) {
    // the four lanes of a request hold the same record: lane p stores words
    // p and p + 4
    uint64_t* R = a.frec + (static_cast<size_t>(k - 1) * a.B + b) * 7 * a.G + g;
    const uint32_t w0 = p == 0 ? __float_as_uint(m) : p == 1 ? __float_as_uint(s)
                        : p == 2 ? __float_as_uint(sc[hb]) : __float_as_uint(sc[1 - hb]);
    const uint32_t w1 = p == 0 ? ((static_cast<uint32_t>(am.i) & 0x7fffffffu) | (bad ? 0x80000000u : 0u))
                        : p == 1 ? ((draw && t3.i1 != INT32_MAX)
                                        ? (0x80000000u | (near23 ? 0x40000000u : 0u) | static_cast<uint32_t>(t3.i1))
                                        : 0u)
                                 : __float_as_uint(zc);
    st_tagged(R + static_cast<size_t>(p) * a.G, a.epoch, w0);
    if (p < 3) st_tagged(R + static_cast<size_t>(p + 4) * a.G, a.epoch, w1);
  }
}

// Wave 0: x_{k-1} of pass (k, j)'s requests (lanes 0..15; anchors at k = 1),
// after a first poll issued earlier (w0, w1: its words).  -1 for absent
// requests and waits that gave up.
__device__ __forceinline__ int32_t pipe_x(const MarkovArgs& a, int k, int j, uint64_t w0, uint64_t w1) {
  const int lane = threadIdx.x & 63;
  const int b = j * kGrp + lane;
  if (lane >= kGrp || b >= a.B) return -1;
  if (k == 1) return clamp_token(a.anchor[b], a.V);
  if (tag_is(w0, a.epoch) && tag_is(w1, a.epoch) && (payload(w0) ^ kTokenCheck) == payload(w1))
    return clamp_token(static_cast<int32_t>(payload(w0)), a.V);
  return clamp_token(wait_token(a, k - 1, b), a.V);
}

// Wave 0: the W1 rows of the pass whose x values are in L.xs into buffer par
// (LDS DMA; slot sl = 64 q + lane holds 8 rank elements of row sl / kW1Slots;
// padding slots, pieces past the rank and absent rows read past the buffer: 0).
__device__ __forceinline__ void pipe_dma(const MarkovArgs& a, PipeLds& L, int par) {
  typedef __attribute__((address_space(3))) void lds_void;
  const int lane = threadIdx.x & 63;
  const int r = a.r;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.w1), static_cast<short>(0), a.V * r * 2, kBufferWord3);
#pragma unroll
  for (int q = 0; q < kPipeDma; ++q) {
    const int sl = q * 64 + lane, n = sl / kW1Slots, c = sl - n * kW1Slots;
    const int32_t x = n < kGrp ? L.xs[n] : -1;
    const bool ok = n < kGrp && c < kW1Slots - 1 && c * 8 < r && x >= 0;
    const uint32_t off = ok ? static_cast<uint32_t>((x * r + c * 8) * 2) : 0xfffffff0u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(L.a[par] + q * 64 * 8), 16, off, 0, 0, 0);
  }
}

// Level-2 noise of this wave's four sub-chunks for groups j .. j+3 of step k
// (lane (n, q): request 16 (j + q) + n, one Philox block).
__device__ __forceinline__ void pipe_noise2(const MarkovArgs& a, PipeLds& L, int tok0, int wave, int k, int j) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, q = lane >> 4;
  const int b = (j + q) * kGrp + n;  // < kPipeMaxB (j <= 12 when B <= kPipeMaxB)
  uint32_t c0 = (static_cast<uint32_t>(tok0) >> 6) + static_cast<uint32_t>(wave),
           c1 = static_cast<uint32_t>(L.pos0[b] + k), c2 = L.req[b], c3 = DSPARK_TAG_DRAFT_SUB;
  philox4x32_10(c0, c1, c2, c3, static_cast<uint32_t>(a.seed), static_cast<uint32_t>(a.seed >> 32));
  *reinterpret_cast<f32x4*>(&L.g2[wave][q][n][0]) = f32x4{gumbel_of(c0), gumbel_of(c1), gumbel_of(c2), gumbel_of(c3)};
}

// Pass p = (k - 1) NG + j of a streaming workgroup.  bb holds this pass's
// backbone values (requested during the previous pass); bbn receives the next
// pass's.  On entry buffer p & 1 holds this pass's W1 rows; on exit (after
// the barrier) buffer (p + 1) & 1 holds the next pass's, and this pass's
// partials, stash and z tiles are in LDS for the next pass's draw and stores.
template <typename T, bool VEC, bool EDGE>
__device__ __forceinline__ void pipe_pass(const MarkovArgs& a, const bf16x8 (&af)[kFusedMS][kMaxR / 32], int g,
                                          int p, int P, int NG, PipeLds& L, const QuadRaw<T> (&bb)[kFusedMS],
                                          QuadRaw<T> (&bbn)[kFusedMS]) {
  constexpr int MS = kFusedMS;
  const int tid = opaque_tid(), lane = tid & 63, wave = wave_id();
  const int gamma = a.gamma, V = a.V;
  const int k = p / NG + 1, j = p - (k - 1) * NG;
  const int par = p & 1;
  const int tok0 = g * kFusedTokens;
  const int vb = tok0 + wave * 16 * MS;
  const int ksteps = ((a.r + 31) & ~31) / 32;
  const bool more = p + 1 < P;
  const int k1 = (p + 1) / NG + 1, j1 = p + 1 - (k1 - 1) * NG;

  uint64_t w0 = 0, w1 = 0;  // wave 0: the first poll of the next pass's x words
  if (wave == 0) {
    if (more && k1 > 1 && lane < kGrp && j1 * kGrp + lane < a.B) {
      const uint64_t* xp = a.xk + (static_cast<size_t>(k1 - 2) * a.B + j1 * kGrp + lane) * 2;
      w0 = ld_tagged(xp);
      w1 = ld_tagged(xp + 1);
    }
    if (more) pipe_backbone<T, VEC>(bbn, a, k1, j1, vb, lane);
  } else if (wave == 1) {
    if (p > 0) {
      const int kp = (p - 1) / NG + 1, jp = p - 1 - (kp - 1) * NG;
      pipe_draw(a, L, g, kp, jp, par ^ 1);
    }
    if (more) pipe_backbone<T, VEC>(bbn, a, k1, j1, vb, lane);
  }
  if ((j & 3) == 0) pipe_noise2(a, L, tok0, wave, k, j);

  // the bias tile of this pass: W2 rows (A) times the staged W1 rows (B)
  f32x4 acc[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) acc[ms] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int ld = kMaxR + kPad;
#pragma unroll
  for (int ks = 0; ks < kMaxR / 32; ++ks) {
    if (ks < ksteps) {
      const bf16x8 bfr = load_frag(L.a[par] + (lane & 15) * ld + ks * 32 + (lane >> 4) * 8);
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
        acc[ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ms][ks], bfr, acc[ms], 0, 0, 0);
    }
  }
  if (wave == 0 && more) {
    // the next pass's x (the poll issued above is back by now, unless the
    // finalize is late) and its W1 rows, landing while the epilogue runs
    const int32_t x = pipe_x(a, k1, j1, w0, w1);
    if (lane < kGrp) L.xs[lane] = x;
    pipe_dma(a, L, par ^ 1);
  } else if (wave >= 2) {
    // the streaming waves' bulk traffic goes out after the duty waves' polls
    // and record stores of this pass, so those do not queue behind it
    if (more) pipe_backbone<T, VEC>(bbn, a, k1, j1, vb, lane);
    if (p > 0 && (wave & 2)) {
      const int kp = (p - 1) / NG + 1, jp = p - 1 - (kp - 1) * NG;
      pipe_store_z01<VEC>(a, L, tok0, kp, jp, par ^ 1, ((wave >> 1) & 2 | (wave & 1)) * 64 + lane);
    }
  }
  // epilogue: lane holds tokens vb + ms*16 + 4*(lane>>4) + i of request n
  const int n = lane & 15;
  const int b = j * kGrp + n;
  const int q = lane >> 4;
  const float pit = L.invT[b];  // 1 / T (sampled), 0 (greedy), -1 (absent)
  const bool bvalid = pit >= 0.0f;
  const bool sampled = pit > 0.0f;
  const float invT = sampled ? pit : 1.0f;
  const size_t rowoff = (static_cast<size_t>(bvalid ? b : 0) * gamma + (k - 1)) * V;
  float z[4 * MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int v0 = vb + ms * 16 + 4 * (lane >> 4);
    const bool full = bvalid && v0 + 3 < V;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y = (acc[ms][i] + bb[ms].at(i)) * invT;
      if constexpr (EDGE) z[ms * 4 + i] = (bvalid && v0 + i < V) ? y : neg_inf();
      else z[ms * 4 + i] = y;
    }
    if (wave < 2) {
      *reinterpret_cast<f32x4*>(&L.z01[par][wave][n][ms * 16 + 4 * (lane >> 4)]) =
          f32x4{z[ms * 4], z[ms * 4 + 1], z[ms * 4 + 2], z[ms * 4 + 3]};
    } else if (VEC && !EDGE) {
      if (sampled)
        __builtin_nontemporal_store(f32x4{z[ms * 4], z[ms * 4 + 1], z[ms * 4 + 2], z[ms * 4 + 3]},
                                    reinterpret_cast<f32x4*>(a.q_z + rowoff + v0));
    } else if (sampled) {
      float* dst = a.q_z + rowoff + v0;
      if (VEC && full) {
        __builtin_nontemporal_store(f32x4{z[ms * 4], z[ms * 4 + 1], z[ms * 4 + 2], z[ms * 4 + 3]},
                                    reinterpret_cast<f32x4*>(dst));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (v0 + i < V) dst[i] = z[ms * 4 + i];
      }
    }
  }
  float lm = z[0];
#pragma unroll
  for (int e = 1; e < 4 * MS; ++e) lm = fmaxf(lm, z[e]);
  const float m = rows_max(lm);
  int32_t arg = INT32_MAX;
  if (__builtin_amdgcn_ballot_w64(bvalid && !sampled)) {
#pragma unroll
    for (int e = 4 * MS - 1; e >= 0; --e)
      if (z[e] == m && m > neg_inf()) arg = vb + (e >> 2) * 16 + 4 * (lane >> 4) + (e & 3);
    arg = static_cast<int32_t>(rows_combine(static_cast<uint32_t>(arg), [](uint32_t u, uint32_t v) {
      return u < v ? u : v;
    }));
  }
  float sj[MS], s;
  sub_partials<MS>(z, m, sj, s);
  const bool bad = s != s || m == pos_inf();
  const uint32_t jbase = static_cast<uint32_t>(vb) >> 4;
  const float sq = q == 0 ? sj[0] : q == 1 ? sj[1] : q == 2 ? sj[2] : sj[3];
  Top2 t2{neg_inf(), INT32_MAX, neg_inf()};
  if (sampled && m > neg_inf() && !bad && sq > 0.0f)
    t2 = Top2{m + logf(sq) + L.g2[wave][j & 3][n][q], static_cast<int32_t>(jbase + q), neg_inf()};
  t2 = rows_top2(t2);
  if (t2.i1 != INT32_MAX) {
    const int m1 = t2.i1 - static_cast<int32_t>(jbase);
    const f32x4 zz = m1 == 0   ? f32x4{z[0], z[1], z[2], z[3]}
                     : m1 == 1 ? f32x4{z[4], z[5], z[6], z[7]}
                     : m1 == 2 ? f32x4{z[8], z[9], z[10], z[11]}
                               : f32x4{z[12], z[13], z[14], z[15]};
    *reinterpret_cast<f32x4*>(&L.stash[par][wave][n][4 * q]) = zz;
  }
  if (q == 0) {
    L.red_m[par][wave][n] = m;
    L.red_s[par][wave][n] = s;
    L.red_i[par][wave][n] = (static_cast<uint32_t>(arg) & 0x7fffffffu) | (bad ? 0x80000000u : 0u);
    L.sub_v1[par][wave][n] = t2.v1;
    L.sub_i1[par][wave][n] = t2.i1;
    L.sub_v2[par][wave][n] = t2.v2;
  }
  if (wave == 0) __builtin_amdgcn_s_waitcnt(0);  // the next pass's W1 rows landed
  __syncthreads();
}

// Streaming workgroup g: every pass, then the last pass's draw and z tiles.
template <typename T, bool VEC, bool EDGE>
__device__ __forceinline__ void pipe_stream(const MarkovArgs& a, const bf16x8 (&af)[kFusedMS][kMaxR / 32], int g,
                                            PipeLds& L) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int NG = (a.B + kGrp - 1) / kGrp, P = a.gamma * NG;
  const int vb = g * kFusedTokens + wave * 16 * kFusedMS;
  QuadRaw<T> bbA[kFusedMS], bbB[kFusedMS];
  // pass 0: x_0 = the anchors, its W1 rows and backbone values
  if (wave == 0) {
    const int32_t x = pipe_x(a, 1, 0, 0, 0);
    if (lane < kGrp) L.xs[lane] = x;
    pipe_dma(a, L, 0);
  }
  pipe_backbone<T, VEC>(bbA, a, 1, 0, vb, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int p = 0; p < P; p += 2) {
    pipe_pass<T, VEC, EDGE>(a, af, g, p, P, NG, L, bbA, bbB);
    if (p + 1 < P) pipe_pass<T, VEC, EDGE>(a, af, g, p + 1, P, NG, L, bbB, bbA);
  }
  const int kp = (P - 1) / NG + 1, jp = P - 1 - (kp - 1) * NG;
  if (wave == 1) pipe_draw(a, L, g, kp, jp, (P - 1) & 1);
  if (wave & 2)
    pipe_store_z01<VEC>(a, L, g * kFusedTokens, kp, jp, (P - 1) & 1, ((wave >> 1) & 2 | (wave & 1)) * 64 + lane);
}

// Confidence head of every draft row (b, k): c = sigmoid(w . [h_k ;
// embed(x_{k-1})]), one workgroup per row, run after the last step (x_{k-1}
// is the anchor for k = 1, else draft token k-1).  8 elements per 16-byte
// load, every load of a thread issued before the first use.
constexpr int kConfThreads = 256;

__global__ __launch_bounds__(kConfThreads) void markov_confidence_kernel(MarkovArgs a) {
  dev_epoch_after(a);
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
  if (t == 0) {
    a.confidence[row] = 1.0f / (1.0f + expf(-dot));
    // a one-launch call whose waits gave up: every row is unspecified
    if (a.epoch && timed_out(a)) a.flags[row] = static_cast<uint8_t>(a.flags[row] | DSPARK_FLAG_SYNC_TIMEOUT);
  }
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

// Truncating one-launch plan.  Every workgroup streams its vocabulary slice
// for every request and step; workgroup g also finalizes requests g, g + G,
// ...  The steps meet through tagged data, without a grid-wide barrier:
//  * a workgroup stores its chunk records of step k only after all of its
//    waves' z stores of step k completed, so a record that carries this
//    call's epoch vouches for the z values behind it (a truncated row's
//    finalize reads its whole z row);
//  * x_k reaches the next step's stream phase through the tagged hand-off.
// Every wait gives up after kWaitTicks; the call's rows are then flagged by
// the confidence kernel.
template <typename T, bool VEC>
__global__ __launch_bounds__(kFusedThreads) void markov_fused_kernel(MarkovArgs a) {
  dev_epoch_begin(a);
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
  dev_epoch_end(a);
}

// Untruncated one-launch plan (see fast_tile / fast_finalize).
template <typename T, bool VEC>
__global__ __launch_bounds__(kFusedThreads) void markov_fast_kernel(MarkovArgs a) {
  dev_epoch_begin(a);
  __shared__ FastLds L;
  const int g = blockIdx.x, G = gridDim.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  bf16x8 af[kFusedMS][kMaxR / 32];  // resident for the whole call
  load_w2<kFusedMS>(af, a.w2, g * kFusedTokens + wave * 16 * kFusedMS, a.V, a.r, lane);
  const bool edge_wg = (g + 1) * kFusedTokens > a.V;  // the slice runs past the vocabulary
  for (int k = 1; k <= a.gamma; ++k) {
    for (int b0 = 0; b0 < a.B; b0 += kTile) {
      if (edge_wg || b0 + kTile > a.B) fast_tile<T, VEC, true>(a, af, g, b0, k, L);
      else fast_tile<T, VEC, false>(a, af, g, b0, k, L);
    }
    if (wave == 0)
      for (int b = g; b < a.B; b += G) fast_finalize(a, b, k);
  }
  // a one-tile batch's last wave-0 z tile (the barrier after the last draw
  // ordered its LDS writes)
  if (threadIdx.x >= 4 * kTile && a.B <= kTile) store_z0<VEC>(a, L, g * kFusedTokens, 0, a.gamma);
  dev_epoch_end(a);
}

// Pipelined untruncated one-launch plan (see pipe_pass): G streaming
// workgroups, then F finalizing ones.
template <typename T, bool VEC>
__global__ __launch_bounds__(kFusedThreads) void markov_pipe_kernel(MarkovArgs a) {
  dev_epoch_begin(a);
  __shared__ PipeLds L;
  const int g = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int NG = (a.B + kGrp - 1) / kGrp, P = a.gamma * NG;
  if (g >= a.G) {
    // finalizing workgroup: wave fw takes requests fw, fw + FW, ... of every
    // group, pass by pass (the order in which their records complete)
    const int FW = a.F * 8, fw = (g - a.G) * 8 + wave;
    for (int p = 0; p < P; ++p) {
      const int k = p / NG + 1, j = p - (k - 1) * NG;
      for (int i = fw; i < kGrp; i += FW) {
        const int b = j * kGrp + i;
        if (b < a.B) fast_finalize(a, b, k);
      }
    }
    return;
  }
  for (int t = threadIdx.x; t < kPipeMaxB; t += kFusedThreads) {
    float it = -1.0f;
    uint32_t req = 0;
    int32_t pos = 0;
    if (t < a.B) {
      const float Tb = a.pol.temperature[t];
      it = (a.pol.mode[t] != 0 && !bad_temperature(Tb)) ? 1.0f / Tb : 0.0f;
      req = a.pol.request_id[t];
      pos = a.pol.position[t];
    }
    L.invT[t] = it;
    L.req[t] = req;
    L.pos0[t] = pos;
  }
  bf16x8 af[kFusedMS][kMaxR / 32];  // resident for the whole call
  load_w2<kFusedMS>(af, a.w2, g * kFusedTokens + wave * 16 * kFusedMS, a.V, a.r, lane);
  // the level-1 noise of chunks 2g, 2g + 1 for every (request, step): one
  // Philox block each, while the W2 rows arrive
  __syncthreads();
  for (int t = threadIdx.x; t < a.B * a.gamma; t += kFusedThreads) {
    const int b = t / a.gamma, k = t - b * a.gamma + 1;
    uint32_t d0 = static_cast<uint32_t>(2 * g) >> 2, d1 = static_cast<uint32_t>(L.pos0[b] + k), d2 = L.req[b],
             d3 = DSPARK_TAG_DRAFT_CHUNK;
    philox4x32_10(d0, d1, d2, d3, static_cast<uint32_t>(a.seed), static_cast<uint32_t>(a.seed >> 32));
    const uint32_t cw[4] = {d0, d1, d2, d3};
    L.g1[b][k - 1][0] = gumbel_of(cw[(2 * g) & 3]);
    L.g1[b][k - 1][1] = gumbel_of(cw[(2 * g + 1) & 3]);
  }
  // element-wise checks only where the slice runs past the vocabulary or the
  // last group is partly absent
  if ((g + 1) * kFusedTokens > a.V || a.B % kGrp != 0) pipe_stream<T, VEC, true>(a, af, g, L);
  else pipe_stream<T, VEC, false>(a, af, g, L);
  if (a.dev_epoch && g == 0 && wave == 0) {
    // the last step's x of every request: every workgroup has run
    for (int b = lane; b < a.B; b += 64) (void)wait_token(a, a.gamma, b);
    dev_epoch_end(a);
  }
}

// Resident workgroups per compute unit of a one-launch kernel, the device's
// compute units and whether it offers cooperative launch, cached per device
// and kernel: a property of the device and the code object only.
struct FusedFit {
  int blocks_per_cu;
  int cus;
  bool coop;
};

// Kernels of the one-launch plans.
enum { kKindFused = 0, kKindFast = 1, kKindPipe = 2 };
template <typename T, bool VEC, int KIND>
const void* one_launch_fn() {
  return KIND == kKindPipe   ? reinterpret_cast<const void*>(markov_pipe_kernel<T, VEC>)
         : KIND == kKindFast ? reinterpret_cast<const void*>(markov_fast_kernel<T, VEC>)
                             : reinterpret_cast<const void*>(markov_fused_kernel<T, VEC>);
}
constexpr const char* kKindName[3] = {"markov_fused", "markov_fast", "markov_pipe"};

template <typename T, bool VEC, int KIND>
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
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, one_launch_fn<T, VEC, KIND>(), kFusedThreads, 0) !=
      hipSuccess)
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

// An ordinary launch of a one-launch grid relies on all of it being resident
// at once, which an occupancy-sized grid is unless another such grid holds
// part of the device: one-launch grids of this library on one device are
// therefore chained, each waiting for the previous one's completion event when
// that one went to another stream (one stream orders its own launches), not
// inside a stream capture (where the caller orders the work).  The events are
// the library's only HIP objects besides the profiler's; dspark_release
// destroys them.
struct FusedChain {
  std::mutex mu;
  hipEvent_t ev[64] = {};
  hipStream_t last[64] = {};
};
FusedChain g_chain;

// The epoch of an eager one-launch call: a process-wide counter, never 0,
// top bit clear (captured calls' tags have it set).
std::atomic<uint32_t> g_epoch{0};
uint32_t next_epoch() {
  uint32_t e;
  do e = (g_epoch.fetch_add(1, std::memory_order_relaxed) + 1) & ~kDevEpochBit;
  while (e == 0);
  return e;
}

// One ordinary (or cooperative) launch of a one-launch kernel, chained.
hipError_t launch_one(const void* fn, const char* name, const MarkovArgs& a, bool coop, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.G + a.F)), block(kFusedThreads);
  MarkovArgs arg = a;
  void* params[] = {&arg};
  if (coop) {
    ProfScope ps(name);
    if (ps.active()) (void)hipEventRecord(ps.start(), st);
    hipError_t e = hipLaunchCooperativeKernel(fn, grid, block, params, 0, st);
    if (ps.active()) (void)hipEventRecord(ps.stop(), st);
    return e;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) cs = hipStreamCaptureStatusNone;
  const bool chain = cs == hipStreamCaptureStatusNone && dev >= 0 && dev < 64;
  std::unique_lock<std::mutex> lk(g_chain.mu, std::defer_lock);
  if (chain) {
    lk.lock();
    hipEvent_t& ev = g_chain.ev[dev];
    if (!ev) {
      e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
      if (e != hipSuccess) return e;
    } else if (g_chain.last[dev] != st) {
      e = hipStreamWaitEvent(st, ev, 0);
      if (e != hipSuccess) return e;
    }
  }
  // the chain's event rides on the kernel's own dispatch (no marker packet
  // between it and the next kernel of the stream)
  ProfScope ps(name);
  if (ps.active()) {
    e = hipExtLaunchKernel(fn, grid, block, params, 0, st, ps.start(), ps.stop(), 0);
    if (e == hipSuccess && chain) e = hipEventRecord(g_chain.ev[dev], st);
  } else if (chain) {
    e = hipExtLaunchKernel(fn, grid, block, params, 0, st, nullptr, g_chain.ev[dev], 0);
  } else {
    e = hipLaunchKernel(fn, grid, block, params, 0, st);
  }
  if (e != hipSuccess) return e;
  if (chain) g_chain.last[dev] = st;
  return hipSuccess;
}

// plan: 0 per-step kernels, 1 one ordinary launch, 2 one cooperative launch
// of the one-launch kernel KIND
template <typename T, bool VEC>
hipError_t launch_plan(MarkovArgs a, int plan, int kind, hipStream_t st) {
  if (plan) {
    a.epoch = a.dev_epoch ? 0u : next_epoch();
    const void* fn = kind == kKindPipe   ? one_launch_fn<T, VEC, kKindPipe>()
                     : kind == kKindFast ? one_launch_fn<T, VEC, kKindFast>()
                                         : one_launch_fn<T, VEC, kKindFused>();
    hipError_t e = launch_one(fn, kKindName[kind], a, plan == 2, st);
    if (e != hipSuccess) return e;
  } else {
    a.epoch = 0;
    a.dev_epoch = 0;
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
hipError_t launch_typed(MarkovArgs a, int plan_mode, hipStream_t st) {
  // the untruncated kernels when the call passes no truncation arrays; a
  // one-launch plan when its grid (one workgroup per 512 tokens, plus the
  // pipelined plan's finalizing workgroups) is resident at once
  const bool fast = !a.pol.top_k && !a.pol.top_p;
  a.F = 0;
  if (fast && a.G > kFastMaxG) {
    // the untruncated finalize reads at most kFastMaxG records per request
    return launch_plan<T, VEC>(a, 0, kKindFast, st);
  }
  // a graph replays its launch arguments, so a captured one-launch kernel
  // takes its hand-off tag from the workspace (dev_epoch_begin); the
  // cross-stream chaining of one-launch grids is not recorded, and the
  // cooperative plan runs as an ordinary launch
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) cs = hipStreamCaptureStatusNone;
  const bool captured = cs != hipStreamCaptureStatusNone;
  a.dev_epoch = captured ? 1 : 0;
  if (captured && plan_mode == DSPARK_MARKOV_COOPERATIVE) plan_mode = DSPARK_MARKOV_AUTO;
  // the request-group plan on request (with fewer than three groups a
  // group's hand-off has no other group's streaming to hide behind)
  if (plan_mode == DSPARK_MARKOV_REQUEST_GROUPS && fast && a.B > 2 * kGrp && a.B <= kPipeMaxB) {
    const FusedFit f = fused_fit<T, VEC, kKindPipe>();
    const int room = f.blocks_per_cu * stream_cus(st, f.cus) - a.G;
    if (f.blocks_per_cu > 0 && room >= 1) {
      a.F = std::min(room, kPipeFin);
      return launch_plan<T, VEC>(a, 1, kKindPipe, st);
    }
  }
  const int kind = fast ? kKindFast : kKindFused;
  const FusedFit f = fast ? fused_fit<T, VEC, kKindFast>() : fused_fit<T, VEC, kKindFused>();
  int plan = 0;
  if (plan_mode == DSPARK_MARKOV_AUTO || plan_mode == DSPARK_MARKOV_REQUEST_GROUPS) {
    if (f.blocks_per_cu > 0 && a.G <= f.blocks_per_cu * stream_cus(st, f.cus)) plan = 1;
  } else if (plan_mode == DSPARK_MARKOV_COOPERATIVE) {
    if (f.coop && f.blocks_per_cu > 0 && a.G <= f.blocks_per_cu * f.cus) plan = 2;
  }
  return launch_plan<T, VEC>(a, plan, kind, st);
}

}  // namespace

void release_markov_chain() {
  std::lock_guard<std::mutex> lk(g_chain.mu);
  for (int dev = 0; dev < 64; ++dev) {
    if (!g_chain.ev[dev]) continue;
    int cur = 0;
    if (hipGetDevice(&cur) == hipSuccess && hipSetDevice(dev) == hipSuccess) {
      (void)hipEventSynchronize(g_chain.ev[dev]);
      (void)hipEventDestroy(g_chain.ev[dev]);
      (void)hipSetDevice(cur);
    }
    g_chain.ev[dev] = nullptr;
    g_chain.last[dev] = nullptr;
  }
}

MarkovPlan plan_markov(int32_t B, int32_t gamma, int32_t V, int32_t r, int32_t d) {
  (void)r;
  (void)d;
  MarkovPlan p{};
  p.C = (V + kChunk - 1) / kChunk;
  p.G = (V + kFusedTokens - 1) / kFusedTokens;
  // one record area, used by whichever plan runs: per-step chunk records
  // (16 B), tagged chunk records (32 B) or tagged workgroup records (56 B)
  const size_t rows = static_cast<size_t>(gamma) * B;
  const size_t rec = std::max({rows * p.C * sizeof(ChunkPart), rows * p.C * 4 * sizeof(uint64_t),
                               rows * p.G * 7 * sizeof(uint64_t)});
  p.off_part = 0;
  size_t off = align_up(rec, 256);
  p.off_xk = off;
  off += align_up(rows * 2 * sizeof(uint64_t), 256);
  p.off_sync = off;
  off += 256;
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
  a.tpart = reinterpret_cast<uint64_t*>(w + plan.off_part);
  a.frec = reinterpret_cast<uint64_t*>(w + plan.off_part);
  a.xk = reinterpret_cast<uint64_t*>(w + plan.off_xk);
  a.sync = reinterpret_cast<uint64_t*>(w + plan.off_sync);
  a.G = plan.G;
  const bool vec = (V % 4 == 0) && (reinterpret_cast<uintptr_t>(backbone) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(q_z) % 16 == 0);
  if (dtype == DSPARK_BF16)
    return vec ? launch_typed<uint16_t, true>(a, plan_mode, st)
               : launch_typed<uint16_t, false>(a, plan_mode, st);
  return vec ? launch_typed<float, true>(a, plan_mode, st) : launch_typed<float, false>(a, plan_mode, st);
}

}  // namespace dspark
