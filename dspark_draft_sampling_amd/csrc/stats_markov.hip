// stats_markov.hip — acceptance statistics of the teacher-forced Markov draft
// on gfx950.
//
// Semantics ("DSpark Speculative Decoding (Draft Training) Design",
// "Semi-autoregressive draft": the Markov head adds a low-rank,
// token-conditioned bias to the parallel logits and is teacher-forced with
// the previous block tokens at training time; "Training objective",
// "Acceptance and confidence"): the draft row of block b at position k is
// backbone[b,k-1,:] + W1[x_{k-1}] . W2^T, x_0 the block's anchor and x_{k-1}
// the teacher token of position k-1; the statistics are those of
// dspark_accept_stats on these rows (definition in include/dspark.h).
//
// The bias is a dense contraction: per look 2 N gamma V r flops (949 GFLOP at
// 2048 x 7 blocks, V = 129280, r = 256), on v_mfma_f32_16x16x32_bf16 with the
// vocabulary as the M side.  As in the one-launch Markov sampler, workgroup g
// owns 512 tokens and keeps their W2 rows in registers (the MFMA A
// fragments) for the whole launch; it walks the rows in tiles of 64 (the N
// side), staging the tile's W1 rows (selected by the forced tokens) in LDS,
// and adds the bias to the backbone values it streams.  Launches, in order:
//  * teacher: per row the forced previous token, the draft value at the
//    teacher token and the row's reference offset (l1norm.hpp) from its
//    first five tokens;
//  * look 1: per (row, workgroup) the normaliser part of the draft and target
//    values of its tokens (l1norm.hpp: the maxima, and the sums under one
//    power-of-two shift shared by both rows where the maxima allow it);
//  * rows: per row the merged part and look 2's constants;
//  * look 2: the bias again, and per (row, workgroup) the share of the row's
//    L1 sum: min(P_v, T_v) for rows whose L1 is at least kFarL1 by look 1's
//    bound, |P_v - T_v| in the form that keeps relative accuracy where the
//    rows nearly agree for the others;
//  * final: per row L1, accept_rate, CE, BCE; then the batch reduction of
//    the plain statistics.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"
#include "l1norm.hpp"

namespace dspark {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSmThreads = 512;  // 8 waves x 64 tokens
constexpr int kSmWaves = kSmThreads / 64;
constexpr int kSmMS = 4;         // 16-token MFMA row blocks per wave
constexpr int kSmTokens = kSmWaves * 16 * kSmMS;
constexpr int kSmTile = 64;      // rows per tile (MFMA N side)
constexpr int kSmMaxR = DSPARK_MAX_RANK;
constexpr int kSmPad = 8;
// The aligned path stages a tile's W1 rows by LDS-DMA buffer loads: each
// wave instruction fills 64 consecutive 16-byte slots, rows of kpad / 8
// slots plus one padding slot (up to 33 x 64 slots), kSmDma instructions
// per wave; slots past the tile land in the buffer's slack (zeros).
constexpr int kSmDma = (kSmTile * (kSmMaxR / 8 + 1) / 64 + kSmWaves - 1) / kSmWaves;
constexpr int kSmABuf = kSmDma * kSmWaves * 64 * 8;  // elements per W1 buffer
static_assert(kSmABuf >= kSmTile * (kSmMaxR + kSmPad), "W1 buffer");

// The looks' per-row constants, 16 bytes (one LDS-DMA slot per row):
//   look 1: x = K (the reference offset)
//   look 2, near rows: x = the common shift, y = K, z = kappa, far = 0
//   look 2, far rows: x = a2d, y = a2t + K log2e, z = lam2, far = 1
// and the final kernel's.
struct SmMeta {
  float x, y, z;
  uint32_t far;
};
struct SmFin {
  float inv_st, isd, lse_d;
  uint32_t flags;  // empty | far << 2
};

struct SmArgs {
  const void* backbone;
  const void* target;
  const int32_t* anchor;
  const uint16_t* w1;
  const uint16_t* w2;
  const int32_t* teacher;
  int32_t rows, gamma, V, r;
  NormPart* rec;    // [rows][G] (look 1)
  float* dteach;    // [rows]: the draft value at the teacher token
  SmFin* norm;      // [rows]: the final kernel's constants (after look 1)
  float* l1part;    // [rows][G][2] (look 2)
  SmMeta* k1;       // [rows]: look 1's per-row constants
  SmMeta* k2;       // [rows]: look 2's per-row constants
  int32_t* xf;      // [rows]: each row's forced previous token, clamped (stats_markov_teacher)
};

// Two of everything: the aligned path stages tile t + 1 and merges tile
// t - 1 while tile t runs (index = tile parity); the unaligned path uses 0.
struct SmLds {
  __attribute__((aligned(16))) uint16_t a[2][kSmABuf];  // staged W1 rows, kSmMaxR + kSmPad apart
  float m[2][kSmWaves][kSmTile], s[2][kSmWaves][kSmTile];  // per (parity, wave, row)
  float u[2][kSmWaves][kSmTile], w[2][kSmWaves][kSmTile], ad[2][kSmWaves][kSmTile];
  SmMeta meta[2][kSmTile];  // per (parity, row): the constants of the look's epilogue
};

__device__ __forceinline__ float rows_max(float v) {
  return __uint_as_float(rows_combine(__float_as_uint(v), [](uint32_t p, uint32_t q) {
    return __float_as_uint(fmaxf(__uint_as_float(p), __uint_as_float(q)));
  }));
}

template <typename T>
struct Quad;
template <>
struct Quad<uint16_t> {
  uint2 u;
  // vec: 4-aligned rows (one 8-byte load for a full quad)
  __device__ void load(const uint16_t* p, int n, bool vec) {
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
struct Quad<float> {
  float4 u;
  __device__ void load(const float* p, int n, bool vec) {
    if (vec && n >= 4) u = *reinterpret_cast<const float4*>(p);
    else u = make_float4(n > 0 ? p[0] : 0.f, n > 1 ? p[1] : 0.f, n > 2 ? p[2] : 0.f, n > 3 ? p[3] : 0.f);
  }
  __device__ float at(int i) const { return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w; }
};

// The forced token before row `row` (flattened b gamma + k - 1).
__device__ __forceinline__ int32_t forced_token(const SmArgs& a, int row) {
  const int k = row % a.gamma;  // k - 1
  const int32_t x = k == 0 ? a.anchor[row / a.gamma] : a.teacher[row - 1];
  return clamp_token(x, a.V);
}

// Token (offset in the wave's 64) of MFMA A row m of 16-token block ms; the
// accumulator element i of lane l holds A row 4 (l >> 4) + i.  Without PERM
// block ms is tokens 16 ms .. 16 ms + 15; with PERM (the aligned path) the
// blocks interleave so that a lane's 16 elements are two runs of 8
// consecutive tokens: 32 (ms / 2) + 8 (m / 4) + 4 (ms % 2) + m % 4.
template <bool PERM>
__device__ __forceinline__ int sm_tok(int ms, int m) {
  return PERM ? 32 * (ms >> 1) + 8 * (m >> 2) + 4 * (ms & 1) + (m & 3) : 16 * ms + m;
}

// One look over the row tile [row0, row0 + 64) for the workgroup's tokens
// (any row alignment): stages the W1 rows, forms the bias tile on MFMA, adds
// the backbone values and calls epi(pass h, d[16], t[16], parity 0) for
// every 16-row pass, element e of the lane's 16 being token
// vb + sm_tok<false>(e / 4, 4 (lane / 16) + e % 4) of row row0 + h 16 +
// lane % 16 (the epilogues reduce over tokens and need no token numbers).
template <typename T, bool VEC, bool LT, class Epi>
__device__ __forceinline__ void sm_tile(const SmArgs& a, const bf16x8 (&af)[kSmMS][kSmMaxR / 32], int tok0,
                                        int row0, SmLds& L, Epi&& epi) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int vb = tok0 + wave * 16 * kSmMS;
  const int V = a.V, r = a.r;
  const int kpad = (r + 31) & ~31, ld = kpad + kSmPad, ksteps = kpad / 32;
  const T* bb = static_cast<const T*>(a.backbone);
  const T* tg = static_cast<const T*>(a.target);

  // stage the tile's W1 rows (MFMA B operand), four 16-byte pieces per
  // thread and round; the pieces are L2-resident after the first tiles
  const int pieces = kpad / 8;
  constexpr int kRound = 4;
  constexpr int kMaxPieces = kSmTile * (kSmMaxR / 8) / kSmThreads;
  static_assert(kMaxPieces % kRound == 0, "staging rounds");
#pragma unroll
  for (int j0 = 0; j0 < kMaxPieces; j0 += kRound) {
    uint4 stage[kRound];
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      const int idx = tid + (j0 + j) * kSmThreads;
      const int rt = idx / pieces, pc = idx - rt * pieces;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (rt < kSmTile && pc * 8 < r && row0 + rt < a.rows) {
        const int32_t x = forced_token(a, row0 + rt);
        val = *reinterpret_cast<const uint4*>(a.w1 + static_cast<size_t>(x) * r + pc * 8);
      }
      stage[j] = val;
    }
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      const int idx = tid + (j0 + j) * kSmThreads;
      const int rt = idx / pieces, pc = idx - rt * pieces;
      if (rt < kSmTile) *reinterpret_cast<uint4*>(L.a[0] + rt * ld + pc * 8) = stage[j];
    }
  }

  // every pass's backbone and target values, in flight during the products
  Quad<T> qd[4][kSmMS], qt[4][kSmMS];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int row = row0 + h * 16 + (lane & 15);
    const size_t off = static_cast<size_t>(row < a.rows ? row : 0) * V;
#pragma unroll
    for (int ms = 0; ms < kSmMS; ++ms) {
      const int v0 = vb + ms * 16 + 4 * (lane >> 4);
      const int n = row < a.rows ? (V - v0 < 4 ? (V - v0 > 0 ? V - v0 : 0) : 4) : 0;
      qd[h][ms].load(bb + off + (n > 0 ? v0 : 0), n, VEC);
      if constexpr (LT) qt[h][ms].load(tg + off + (n > 0 ? v0 : 0), n, VEC);
    }
  }
  __syncthreads();

#pragma unroll
  for (int h = 0; h < 4; ++h) {
    f32x4 acc[kSmMS];
#pragma unroll
    for (int ms = 0; ms < kSmMS; ++ms) acc[ms] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kSmMaxR / 32; ++ks) {
      if (ks < ksteps) {
        const bf16x8 bfr = *reinterpret_cast<const bf16x8*>(L.a[0] + (h * 16 + (lane & 15)) * ld + ks * 32 +
                                                           (lane >> 4) * 8);
#pragma unroll
        for (int ms = 0; ms < kSmMS; ++ms)
          acc[ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ms][ks], bfr, acc[ms], 0, 0, 0);
      }
    }
    // lane: tokens vb + ms 16 + 4 (lane >> 4) + i of row row0 + h 16 + (lane & 15)
    float d[4 * kSmMS], t[4 * kSmMS];
#pragma unroll
    for (int ms = 0; ms < kSmMS; ++ms) {
      const int v0 = vb + ms * 16 + 4 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool in = v0 + i < V;
        d[ms * 4 + i] = in ? qd[h][ms].at(i) + acc[ms][i] : neg_inf();
        t[ms * 4 + i] = LT && in ? qt[h][ms].at(i) : neg_inf();
      }
    }
    epi(h, d, t, 0);
  }
}

// Buffer resources over the backbone and target rows [row0, rows): loads
// past them return zeros, so every load of a tile is unconditional and the
// compiler's wait counts stay exact.
template <typename T>
struct TileRs {
  __amdgpu_buffer_rsrc_t d, t;
};
template <typename T>
__device__ __forceinline__ TileRs<T> tile_rs(const SmArgs& a, int row0) {
  const size_t base = static_cast<size_t>(row0) * a.V;
  const size_t left = (static_cast<size_t>(a.rows) - row0) * a.V * sizeof(T);
  const int bytes = static_cast<int>(left > 0x7fffffffull ? 0x7fffffffull : left);
  return TileRs<T>{__builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(static_cast<const T*>(a.backbone) + base),
                                                     static_cast<short>(0), bytes, kBufferWord3),
                   __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(static_cast<const T*>(a.target) + base),
                                                     static_cast<short>(0), bytes, kBufferWord3)};
}

// The backbone and target quads of passes h0, h0 + 1 (16 rows each) of a tile.
// With the aligned path's token order (sm_tok<true>) a lane's quads ms and
// ms + 1 (ms even) are 8 consecutive tokens: bf16 rows take one 16-byte load
// for both, and a row's 16 lanes read 64 contiguous bytes per load.
template <typename T, bool LT>
__device__ __forceinline__ void load_half(Quad<T> (&qd)[2][kSmMS], Quad<T> (&qt)[2][kSmMS], const TileRs<T>& rs,
                                          int h0, int vb, int lane, int V) {
  auto f4 = [](const u32x4& x) {
    return make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]), __uint_as_float(x[3]));
  };
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const uint32_t n = static_cast<uint32_t>((h0 + hh) * 16 + (lane & 15));
#pragma unroll
    for (int ms = 0; ms < kSmMS; ms += (sizeof(T) == 2 ? 2 : 1)) {
      const uint32_t v0 = static_cast<uint32_t>(vb + sm_tok<true>(ms, 4 * (lane >> 4)));
      const uint32_t off = (n * static_cast<uint32_t>(V) + v0) * sizeof(T);
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs.d, off, 0, 0);
      const u32x4 y = LT ? __builtin_amdgcn_raw_buffer_load_b128(rs.t, off, 0, 0) : u32x4{};
      if constexpr (sizeof(T) == 2) {
        qd[hh][ms].u = make_uint2(x[0], x[1]);
        qd[hh][ms + 1].u = make_uint2(x[2], x[3]);
        if constexpr (LT) {
          qt[hh][ms].u = make_uint2(y[0], y[1]);
          qt[hh][ms + 1].u = make_uint2(y[2], y[3]);
        }
      } else {
        qd[hh][ms].u = f4(x);
        if constexpr (LT) qt[hh][ms].u = f4(y);
      }
    }
  }
}

// All row tiles of one look, for 4-aligned rows, software-pipelined with
// one barrier per tile (LDS buffers indexed by tile parity).  While tile t
// runs: its second half of values is requested before its first half is
// used, and tile t + 1's first half before its second half is used; tile
// t + 1's forced tokens are read during tile t's first half and its W1 rows
// (and, with META, its rows' records from meta[]) go by LDS-DMA loads into
// the other buffers during its second half, holding no registers; tile
// t - 1's partials are merged after tile t's barrier (which waits for the
// DMA).  All global loads are unconditional (past the last row: empty
// resources, zero fills or clamped rows), so the compiler's wait counts stay
// exact.  epi(h, d, t, parity) as for sm_tile (token order sm_tok<true>);
// merge(row0, parity) once
// a tile's partials are complete.
// MASK: tokens past the vocabulary are excluded element by element; without
// it (V a multiple of 64) a wave's tokens are all in or all out, and a wave
// past the vocabulary hands its epilogue -inf values.  RMAX: the rank is
// the maximum (the k loop and the staging indexes are then compile-time).
template <typename T, bool LT, bool MASK, bool RMAX, bool META, class Epi, class Merge>
__device__ __forceinline__ void sm_look_vec(const SmArgs& a, const bf16x8 (&af)[kSmMS][kSmMaxR / 32], int tok0,
                                            SmLds& L, const SmMeta* meta, Epi&& epi, Merge&& merge) {
  typedef __attribute__((address_space(3))) void lds_void;
  if (a.rows <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int vb = tok0 + wave * 16 * kSmMS;
  const int V = a.V, r = RMAX ? kSmMaxR : a.r;
  const bool dead = __builtin_amdgcn_readfirstlane(vb) >= V;  // wave-uniform
  const int kpad = (r + 31) & ~31, ld = kpad + kSmPad, ksteps = kpad / 32;
  const int slots = kpad / 8 + 1;  // 16-byte slots per staged row
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.w1), static_cast<short>(0), V * r * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<SmMeta*>(meta), static_cast<short>(0), META ? a.rows * 16 : 0, kBufferWord3);

  // the forced tokens of the rows of the thread's DMA slots of tile row0
  auto load_xs = [&](int row0, int32_t (&xs)[kSmDma]) {
#pragma unroll
    for (int j = 0; j < kSmDma; ++j) {
      const int n = ((j * kSmWaves + wv) * 64 + lane) / slots;
      xs[j] = a.xf[min(row0 + min(n, kSmTile - 1), a.rows - 1)];
    }
  };
  // tile row0's W1 rows (and records) into buffers buf
  auto stage = [&](int row0, int buf, const int32_t (&xs)[kSmDma]) {
#pragma unroll
    for (int j = 0; j < kSmDma; ++j) {
      const int q = j * kSmWaves + wv;
      const int sl = q * 64 + lane, n = sl / slots, c = sl - n * slots;
      const bool ok = n < kSmTile && c < slots - 1 && c * 8 < r && row0 + n < a.rows;
      const uint32_t off = ok ? static_cast<uint32_t>((xs[j] * r + c * 8) * 2) : 0xfffffff0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(L.a[buf] + q * 64 * 8), 16, off, 0, 0, 0);
    }
    if constexpr (META)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rm, (lds_void*)(L.meta[buf]), 16,
                                               static_cast<uint32_t>(min(row0 + lane, a.rows - 1)) * 16, 0, 0, 0);
  };

  Quad<T> qA[2][kSmMS], tA[2][kSmMS], qB[2][kSmMS], tB[2][kSmMS];
  int32_t xs[kSmDma];
  load_xs(0, xs);
  stage(0, 0, xs);
  load_half<T, LT>(qA, tA, tile_rs<T>(a, 0), 0, vb, lane, V);

  int par = 0;
  for (int row0 = 0; row0 < a.rows; row0 += kSmTile, par ^= 1) {
    __syncthreads();  // tile row0 staged in buffers par; tile row0 - 64's partials complete
    if (row0 > 0) merge(row0 - kSmTile, par ^ 1);
    const int next = min(row0 + kSmTile, a.rows);  // a.rows: nothing left, loads come back empty
    load_half<T, LT>(qB, tB, tile_rs<T>(a, row0), 2, vb, lane, V);
    load_xs(next, xs);

    auto pass = [&](int h, const Quad<T> (&qd)[kSmMS], const Quad<T> (&qt)[kSmMS]) {
      // the accumulator starts from the backbone values: d = backbone + bias
      f32x4 acc[kSmMS];
#pragma unroll
      for (int ms = 0; ms < kSmMS; ++ms) acc[ms] = f32x4{qd[ms].at(0), qd[ms].at(1), qd[ms].at(2), qd[ms].at(3)};
#pragma unroll
      for (int ks = 0; ks < kSmMaxR / 32; ++ks) {
        if (ks < ksteps) {
          const bf16x8 bfr = *reinterpret_cast<const bf16x8*>(L.a[par] + (h * 16 + (lane & 15)) * ld + ks * 32 +
                                                             (lane >> 4) * 8);
#pragma unroll
          for (int ms = 0; ms < kSmMS; ++ms)
            acc[ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ms][ks], bfr, acc[ms], 0, 0, 0);
        }
      }
      float d[4 * kSmMS], t[4 * kSmMS];
#pragma unroll
      for (int ms = 0; ms < kSmMS; ++ms) {
        const int v0 = vb + sm_tok<true>(ms, 4 * (lane >> 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool in = !MASK || v0 + i < V;
          d[ms * 4 + i] = in ? acc[ms][i] : neg_inf();
          t[ms * 4 + i] = LT && in ? qt[ms].at(i) : neg_inf();
        }
      }
      if (!MASK && dead)
#pragma unroll
        for (int e = 0; e < 4 * kSmMS; ++e) d[e] = t[e] = neg_inf();
      epi(h, d, t, par);
    };
    pass(0, qA[0], tA[0]);
    pass(1, qA[1], tA[1]);
    stage(next, par ^ 1, xs);  // buffers par ^ 1 were last read before this tile's barrier
    load_half<T, LT>(qA, tA, tile_rs<T>(a, next), 0, vb, lane, V);
    pass(2, qB[0], tB[0]);
    pass(3, qB[1], tB[1]);
  }
  __syncthreads();
  merge(((a.rows - 1) / kSmTile) * kSmTile, par ^ 1);
}

// W2 fragments of the wave's 16 MS tokens [vb, vb + 16 MS) (A operand), in
// the token order of the path (sm_tok<PERM>).
template <bool PERM>
__device__ __forceinline__ void sm_load_w2(bf16x8 (&af)[kSmMS][kSmMaxR / 32], const uint16_t* w2, int vb, int V,
                                           int r, int lane) {
  const int ksteps = ((r + 31) & ~31) / 32;
#pragma unroll
  for (int ms = 0; ms < kSmMS; ++ms) {
    const int v = vb + sm_tok<PERM>(ms, lane & 15);
#pragma unroll
    for (int ks = 0; ks < kSmMaxR / 32; ++ks) {
      const int k0 = ks * 32 + (lane >> 4) * 8;
      bf16x8 f = {};
      if (ks < ksteps && v < V && k0 < r) f = *reinterpret_cast<const bf16x8*>(w2 + static_cast<size_t>(v) * r + k0);
      af[ms][ks] = f;
    }
  }
}

// Look 1: per (row, workgroup) the normaliser part of the draft and target
// values of its tokens (the teacher's draft value is stats_markov_teacher's).
template <typename T, bool VEC, bool MASK, bool RMAX>
__global__ __launch_bounds__(kSmThreads) void stats_markov_look1_kernel(SmArgs a) {
  __shared__ SmLds L;
  const int g = blockIdx.x, G = gridDim.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok0 = g * kSmTokens;
  bf16x8 af[kSmMS][kSmMaxR / 32];
  sm_load_w2<VEC>(af, a.w2, tok0 + wave * 16 * kSmMS, a.V, a.r, lane);
  // per (wave, row): the part of the lane group's 64 tokens; the shift mode
  // is per row, so per lane here
  auto epi = [&](int h, const float* d, const float* t0, int p) {
    const float K = L.meta[p][h * 16 + (lane & 15)].x;
    float t[4 * kSmMS];
#pragma unroll
    for (int e = 0; e < 4 * kSmMS; ++e) t[e] = t0[e] - K;
    float md = neg_inf(), mt = neg_inf();
#pragma unroll
    for (int e = 0; e < 4 * kSmMS; ++e) {
      md = fmaxf(md, d[e]);
      mt = fmaxf(mt, t[e]);
    }
    md = rows_max(md);
    mt = rows_max(mt);
    const bool common = np_common(md, mt);
    float a2d, a2t;
    np_shifts(md, mt, a2d, a2t);
    float sd = 0.0f, x = 0.0f, ad = 0.0f;
#pragma unroll
    for (int e = 0; e < 4 * kSmMS; ++e) {
      const float D = __builtin_amdgcn_exp2f(fmaf(d[e], kLog2e, -a2d));
      const float Tv = __builtin_amdgcn_exp2f(fmaf(t[e], kLog2e, -a2t));
      const float df = np_diff<true>(d[e], t[e], D, Tv);
      sd += D;
      x += common ? df : Tv;
      ad += fabsf(df);
    }
    sd = rows_sum(sd);
    x = rows_sum(x);
    ad = rows_sum(ad);
    if (lane < 16) {
      const int n = h * 16 + lane;
      L.m[p][wave][n] = md;
      L.s[p][wave][n] = mt;
      L.u[p][wave][n] = sd;
      L.w[p][wave][n] = x;
      L.ad[p][wave][n] = ad;
    }
  };
  auto merge = [&](int row0, int p) {
    if (threadIdx.x < kSmTile && row0 + static_cast<int>(threadIdx.x) < a.rows) {
      const int n = threadIdx.x;
      NormPart q = np_empty();
#pragma unroll
      for (int w = 0; w < kSmWaves; ++w)
        q = np_merge(q, NormPart{L.m[p][w][n], L.s[p][w][n], L.u[p][w][n], L.w[p][w][n], L.ad[p][w][n]});
      a.rec[static_cast<size_t>(row0 + n) * G + g] = q;
    }
  };
  if constexpr (VEC) {
    sm_look_vec<T, true, MASK, RMAX, true>(a, af, tok0, L, a.k1, epi, merge);
  } else {
    for (int row0 = 0; row0 < a.rows; row0 += kSmTile) {
      const int row = row0 + static_cast<int>(threadIdx.x);
      if (threadIdx.x < kSmTile) L.meta[0][threadIdx.x] = a.k1[row < a.rows ? row : 0];
      sm_tile<T, VEC, true>(a, af, tok0, row0, L, epi);  // its staging barrier publishes meta
      __syncthreads();
      merge(row0, 0);
      __syncthreads();  // the LDS tile is reused by the next tile
    }
  }
}

// Per row: the draft value at the teacher token, the backbone's value plus
// W1[x] . W2[teacher] (bf16 products, exact in fp32, summed in fp32), one
// wave per row, and x itself for the looks; x is the row's forced previous
// token (the anchor at the block's first position, else the previous
// position's teacher token).
template <typename T>
__global__ __launch_bounds__(256) void stats_markov_teacher_kernel(SmArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.rows) return;
  const int x = forced_token(a, row);
  const int tch = clamp_token(a.teacher[row], a.V);
  const uint16_t* w1 = a.w1 + static_cast<size_t>(x) * a.r;
  const uint16_t* w2 = a.w2 + static_cast<size_t>(tch) * a.r;
  float s = 0.0f;
  for (int j = lane; j < a.r; j += 64)
    s = fmaf(__uint_as_float(static_cast<uint32_t>(w1[j]) << 16), __uint_as_float(static_cast<uint32_t>(w2[j]) << 16), s);
  s = wave_sum(s);
  // the reference offset: t_v - d_v of tokens 0..4 (bias summed as above)
  const T* bb = static_cast<const T*>(a.backbone) + static_cast<size_t>(row) * a.V;
  const T* tg = static_cast<const T*>(a.target) + static_cast<size_t>(row) * a.V;
  float r[5];
#pragma unroll
  for (int v = 0; v < 5; ++v) {
    const int vv = v < a.V ? v : 0;
    const uint16_t* w2v = a.w2 + static_cast<size_t>(vv) * a.r;
    float b = 0.0f;
    for (int j = lane; j < a.r; j += 64)
      b = fmaf(__uint_as_float(static_cast<uint32_t>(w1[j]) << 16), __uint_as_float(static_cast<uint32_t>(w2v[j]) << 16), b);
    b = wave_sum(b);
    r[v] = v < a.V ? load_logit(tg, vv) - (load_logit(bb, vv) + b) : pos_inf();
  }
  if (lane == 0) {
    a.dteach[row] = load_logit(bb, tch) + s;
    a.xf[row] = x;
    a.k1[row] = SmMeta{ref_offset(r[0], r[1], r[2], r[3], r[4]), 0.0f, 0.0f, 0u};
  }
}

// Per row: the merged part of the row's G look-1 records, look 2's constants
// and the final kernel's (one wave per row, fixed merge order).
__global__ __launch_bounds__(256) void stats_markov_rows_kernel(SmArgs a, int32_t G) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.rows) return;
  const NormPart* rc = a.rec + static_cast<size_t>(row) * G;
  NormPart q = np_empty();
  for (int i = lane; i < G; i += 64) q = np_merge(q, rc[i]);
  const PairK k = pair_k(np_wave_merge(q));
  if (lane == 0) {
    const float K = a.k1[row].x;
    a.k2[row] = k.far ? SmMeta{k.a2d, fmaf(K, kLog2e, k.a2t), k.lam2, 1u} : SmMeta{k.a2d, K, k.kappa, 0u};
    a.norm[row] = SmFin{k.inv_st, k.isd, k.lse_d, k.empty | (k.far << 2)};
  }
}

// Look 2: per (row, workgroup) the share of the row's L1 sum (min(P_v, T_v) Sd
// for far rows, |P_v - T_v| St for near rows; the form is per row, so per
// lane here).
template <typename T, bool VEC, bool MASK, bool RMAX>
__global__ __launch_bounds__(kSmThreads) void stats_markov_look2_kernel(SmArgs a) {
  __shared__ SmLds L;
  const int g = blockIdx.x, G = gridDim.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok0 = g * kSmTokens;
  bf16x8 af[kSmMS][kSmMaxR / 32];
  sm_load_w2<VEC>(af, a.w2, tok0 + wave * 16 * kSmMS, a.V, a.r, lane);
  auto epi = [&](int h, const float* d, const float* t, int p) {
    const SmMeta k = L.meta[p][h * 16 + (lane & 15)];
    float acc = 0.0f;
    if (k.far) {
#pragma unroll
      for (int e = 0; e < 4 * kSmMS; ++e) acc += l1_far(d[e], t[e], k.x, k.y, k.z);
    } else {
#pragma unroll
      for (int e = 0; e < 4 * kSmMS; ++e) acc += l1_near(d[e], t[e] - k.y, k.x, k.z);
    }
    acc = rows_sum(acc);
    if (lane < 16) L.m[p][wave][h * 16 + lane] = acc;
  };
  auto merge = [&](int row0, int p) {
    if (threadIdx.x < kSmTile && row0 + static_cast<int>(threadIdx.x) < a.rows) {
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < kSmWaves; ++w) acc += L.m[p][w][threadIdx.x];
      a.l1part[static_cast<size_t>(row0 + threadIdx.x) * G + g] = acc;
    }
  };
  if constexpr (VEC) {
    sm_look_vec<T, true, MASK, RMAX, true>(a, af, tok0, L, a.k2, epi, merge);
  } else {
    for (int row0 = 0; row0 < a.rows; row0 += kSmTile) {
      const int row = row0 + static_cast<int>(threadIdx.x);
      if (threadIdx.x < kSmTile) L.meta[0][threadIdx.x] = a.k2[row < a.rows ? row : 0];
      sm_tile<T, VEC, true>(a, af, tok0, row0, L, epi);  // its staging barrier publishes meta
      __syncthreads();
      merge(row0, 0);
      __syncthreads();
    }
  }
}

// Per row: L1 from its G shares, then accept_rate, CE and BCE.
__global__ __launch_bounds__(256) void stats_markov_final_kernel(SmArgs a, int32_t G, const float* conf_logits,
                                                                 float* l1, float* accept_rate, float* ce,
                                                                 float* bce) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.rows) return;
  float s = 0.0f;
  for (int i = lane; i < G; i += 64) s += a.l1part[static_cast<size_t>(row) * G + i];
  s = wave_sum(s);
  if (lane == 0) {
    const SmFin f = a.norm[row];
    const float L1 = l1_final(f.flags & 3u, f.flags >> 2, f.inv_st, f.isd, s);
    const float av = fminf(1.0f, fmaxf(0.0f, 1.0f - 0.5f * L1));
    const float c = conf_logits[row];
    l1[row] = L1;
    accept_rate[row] = av;
    ce[row] = f.lse_d - a.dteach[row];
    bce[row] = fmaxf(c, 0.0f) - c * av + log1pf(expf(-fabsf(c)));
  }
}

// One of the looks, in the instance the shapes allow: aligned rows or not,
// V a multiple of 64 or not (the token mask), the maximum rank or not.
template <typename T, int LOOK, bool VEC, bool MASK, bool RMAX>
hipError_t launch_look_inst(const SmArgs& a, int G, hipStream_t st) {
  if constexpr (LOOK == 1)
    DSPARK_LAUNCH("stats_markov_look1", (stats_markov_look1_kernel<T, VEC, MASK, RMAX>), dim3(G), dim3(kSmThreads), 0,
                  st, a);
  else
    DSPARK_LAUNCH("stats_markov_look2", (stats_markov_look2_kernel<T, VEC, MASK, RMAX>), dim3(G), dim3(kSmThreads), 0,
                  st, a);
  return hipGetLastError();
}

template <typename T, int LOOK>
hipError_t launch_look_t(const SmArgs& a, int G, bool vec, bool mask, bool rmax, hipStream_t st) {
  if (!vec) return launch_look_inst<T, LOOK, false, true, false>(a, G, st);
  if (mask) return rmax ? launch_look_inst<T, LOOK, true, true, true>(a, G, st)
                        : launch_look_inst<T, LOOK, true, true, false>(a, G, st);
  return rmax ? launch_look_inst<T, LOOK, true, false, true>(a, G, st)
              : launch_look_inst<T, LOOK, true, false, false>(a, G, st);
}

template <typename T>
hipError_t launch_look(const SmArgs& a, int G, bool vec, bool mask, bool rmax, int look, hipStream_t st) {
  return look == 1 ? launch_look_t<T, 1>(a, G, vec, mask, rmax, st) : launch_look_t<T, 2>(a, G, vec, mask, rmax, st);
}

template <typename T>
hipError_t launch_sm_typed(const SmArgs& a, int G, const float* conf_logits, const uint8_t* block_mask,
                           int32_t N, float w_ce, float w_l1, float w_conf, float* l1, float* accept_rate,
                           float* ce, float* bce, float* tau, float* sums, hipStream_t st) {
  const unsigned rb = static_cast<unsigned>((a.rows + 3) / 4);
  // the aligned path addresses a tile's rows with 32-bit byte offsets
  const bool vec = a.V % 4 == 0 && reinterpret_cast<uintptr_t>(a.backbone) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(a.target) % 16 == 0 &&
                   static_cast<uint64_t>(kSmTile) * a.V * sizeof(T) < 0x7fffffffull &&
                   static_cast<uint64_t>(a.V) * a.r * 2 < 0x7fffffffull &&
                   static_cast<uint64_t>(a.rows) * sizeof(SmMeta) < 0x7fffffffull;
  const bool mask = a.V % 64 != 0, rmax = a.r == kSmMaxR;
  DSPARK_LAUNCH("stats_markov_teacher", stats_markov_teacher_kernel<T>, dim3(rb), dim3(256), 0, st, a);
  hipError_t e = launch_look<T>(a, G, vec, mask, rmax, 1, st);
  if (e != hipSuccess) return e;
  DSPARK_LAUNCH("stats_markov_rows", stats_markov_rows_kernel, dim3(rb), dim3(256), 0, st, a, G);
  e = launch_look<T>(a, G, vec, mask, rmax, 2, st);
  if (e != hipSuccess) return e;
  DSPARK_LAUNCH("stats_markov_final", stats_markov_final_kernel, dim3(rb), dim3(256), 0, st, a, G,
                conf_logits, l1, accept_rate, ce, bce);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_stats_reduce(l1, accept_rate, ce, bce, block_mask, N, a.gamma, w_ce, w_l1, w_conf, tau, sums,
                             st);
}

}  // namespace

StatsMarkovPlan plan_stats_markov(int32_t N, int32_t gamma, int32_t V) {
  StatsMarkovPlan p{};
  const size_t rows = static_cast<size_t>(N) * gamma;
  p.G = (V + kSmTokens - 1) / kSmTokens;
  size_t off = 0;
  p.off_rec = off;
  off = align_up(off + rows * p.G * sizeof(NormPart), 256);
  p.off_norm = off;
  off = align_up(off + rows * sizeof(SmFin), 256);
  p.off_l1 = off;
  off = align_up(off + rows * p.G * sizeof(float), 256);
  p.off_dt = off;
  off = align_up(off + rows * sizeof(float), 256);
  p.off_k1 = off;
  off = align_up(off + rows * sizeof(SmMeta), 256);
  p.off_k2 = off;
  off = align_up(off + rows * sizeof(SmMeta), 256);
  p.off_xf = off;
  off = align_up(off + rows * sizeof(int32_t), 256);
  p.bytes = rows > 0 ? off : 0;
  return p;
}

hipError_t launch_stats_markov(const void* backbone, const void* target, int dtype, const int32_t* anchor,
                               const uint16_t* w1, const uint16_t* w2, int32_t r, const int32_t* teacher,
                               const float* conf_logits, const uint8_t* block_mask, int32_t N, int32_t gamma,
                               int32_t V, float w_ce, float w_l1, float w_conf, float* l1, float* accept_rate,
                               float* ce, float* bce, float* tau, float* sums, void* ws,
                               const StatsMarkovPlan& pl, hipStream_t st) {
  const int32_t rows = N * gamma;
  if (rows == 0)
    return launch_stats_reduce(l1, accept_rate, ce, bce, block_mask, N, gamma, w_ce, w_l1, w_conf, tau, sums, st);
  char* w = static_cast<char*>(ws);
  SmArgs a{backbone, target, anchor, w1, w2, teacher, rows, gamma, V, r,
           reinterpret_cast<NormPart*>(w + pl.off_rec), reinterpret_cast<float*>(w + pl.off_dt),
           reinterpret_cast<SmFin*>(w + pl.off_norm), reinterpret_cast<float*>(w + pl.off_l1),
           reinterpret_cast<SmMeta*>(w + pl.off_k1), reinterpret_cast<SmMeta*>(w + pl.off_k2),
           reinterpret_cast<int32_t*>(w + pl.off_xf)};
  if (dtype == DSPARK_BF16)
    return launch_sm_typed<uint16_t>(a, pl.G, conf_logits, block_mask, N, w_ce, w_l1, w_conf, l1, accept_rate,
                                     ce, bce, tau, sums, st);
  return launch_sm_typed<float>(a, pl.G, conf_logits, block_mask, N, w_ce, w_l1, w_conf, l1, accept_rate, ce,
                                bce, tau, sums, st);
}

}  // namespace dspark
