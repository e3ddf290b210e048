// dspark_oracle.cpp — plain, slow, single-threaded CPU oracle of the DSpark
// per-step sampling and verification engine.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
// CPU-baseline leg may load this library.  It shares no code, header, table or
// constant generator with the GPU library: every constant below is restated
// from the method's definition.
//
// Every real quantity is computed in IEEE binary64 from the exact inputs
// (bf16 and fp32 values convert to binary64 exactly); outputs are binary64.
// Each function restates a definition from these pages:
//   [FT] "[2/3] feat(dsv4): implement exact DSpark speculative decoding"
//        sections "End-to-end speculative cycle", "Checkpoint-faithful DSpark
//        architecture", "Exact decoding semantics" ("Greedy", "Probabilistic").
//   [MB] "DSpark Speculative Decoding (Draft Training) Design"
//        sections "Semi-autoregressive draft", "Training objective",
//        "Acceptance and confidence", "Loss return contract".
//   [PS] "DeepSeek V4 DSpark NPU Serving Dev Notes", section
//        "Speculative decoding (K=7)" ("Acceptance", "Weights").
// Where the pages leave a step open, the reading taken is stated in place.
//
// Decisions that a floating-point margin could flip are reported through the
// `flags` outputs (bit 0) using these rules, with EPS = 1e-6:
//   argmax / Gumbel-max : top-2 score gap <= EPS * max(1, |best score|)
//   accept test         : |u' - p/q| <= EPS
//   top-k boundary      : gap between the k-th and (k+1)-th value
//                         <= EPS * max(1, |k-th value|)   (computed rows only)
//   top-p boundary      : the cumulative mass at the cut within EPS of top_p
// Parity: pinned by the tests under tests/ (fixed points, closed forms, brute
// force, chi-square and a library Philox); see the test module headers.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <numeric>
#include <vector>

namespace {

constexpr double kEps = 1e-6;
constexpr int kChunk = 256;  // tokens per level-1 chunk of the sampler
constexpr int kSub = 16;     // tokens per level-2 sub-chunk of the sampler
constexpr double kNegInf = -std::numeric_limits<double>::infinity();

// flag bits (restated; same meaning as the library's per-row flags)
constexpr uint8_t F_NEAR = 1, F_NONFINITE = 2, F_RESID_ZERO = 4, F_EMPTY = 8,
                  F_BAD_POLICY = 16;

// Philox stream tags (restated)
constexpr uint32_t TAG_DRAFT_TOKEN = 0, TAG_ACCEPT = 1, TAG_TARGET_TOKEN = 2,
                   TAG_DRAFT_CHUNK = 3, TAG_TARGET_CHUNK = 4, TAG_DRAFT_SUB = 5,
                   TAG_TARGET_SUB = 6;

// ---------------------------------------------------------------------------
// Element conversion.  bf16 is the upper half of a binary32.
double bf16_to_double(uint16_t h) {
  uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

// logits element `i` of an array of dtype 1 = bf16, 2 = fp32
// dtype 1: bf16 bits, 2: float32, 3: binary64 (oracle-side rows only)
double logit_at(const void* p, int dtype, size_t i) {
  if (dtype == 1) return bf16_to_double(static_cast<const uint16_t*>(p)[i]);
  if (dtype == 3) return static_cast<const double*>(p)[i];
  return static_cast<double>(static_cast<const float*>(p)[i]);
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// 4x32 Philox S-box on the counter, the 2x32 key bumped by the Weyl
// constants between rounds.
void philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                   uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t p0 = static_cast<uint64_t>(M0) * c0;
    const uint64_t p1 = static_cast<uint64_t>(M1) * c2;
    const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
    const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// The random word for index i: counter (i/4, position, request, tag),
// key = seed split in two 32-bit halves, output word i % 4.
uint32_t philox_word(uint64_t seed, uint32_t i, int32_t position,
                     uint32_t request, uint32_t tag) {
  const uint32_t ctr[4] = {i >> 2, static_cast<uint32_t>(position), request, tag};
  const uint32_t key[2] = {static_cast<uint32_t>(seed & 0xffffffffu),
                           static_cast<uint32_t>(seed >> 32)};
  uint32_t out[4];
  philox4x32_10(ctr, key, out);
  return out[i & 3u];
}

// u = ((w >> 9) + 0.5) * 2^-23, strictly inside (0, 1); returns 1 - u as well
// (both exact in binary64).
void open_uniform(uint32_t w, double* u, double* one_minus_u) {
  const double m = static_cast<double>(w >> 9);  // 0 .. 2^23 - 1
  *u = (m + 0.5) * std::ldexp(1.0, -23);
  *one_minus_u = ((8388608.0 - m) - 0.5) * std::ldexp(1.0, -23);
}

// Gumbel noise g = -ln(-ln u), with -ln u = -log1p(-(1-u)) for accuracy
// near u = 1.
double gumbel(uint64_t seed, uint32_t i, int32_t position, uint32_t request,
              uint32_t tag) {
  double u, omu;
  open_uniform(philox_word(seed, i, position, request, tag), &u, &omu);
  const double e = -std::log1p(-omu);  // = -ln u > 0
  return -std::log(e);
}

// Accept uniform u' = (w >> 8) * 2^-24 in [0, 1).
double accept_uniform(uint64_t seed, int32_t position, uint32_t request) {
  const uint32_t w = philox_word(seed, 0, position, request, TAG_ACCEPT);
  return static_cast<double>(w >> 8) * std::ldexp(1.0, -24);
}

bool near_gap(double best, double second) {
  return (best - second) <= kEps * std::max(1.0, std::fabs(best));
}

// ---------------------------------------------------------------------------
// Three-level Gumbel-max sample from log-weights lw (-inf = excluded).
// The pages fix only that emitted tokens follow the target distribution
// exactly ([FT] "Exact decoding semantics", "Probabilistic"); the draw itself
// is this library's reading: a Gumbel-max descent over a fixed partition of
// the vocabulary.
//   level 1: chunks of kChunk consecutive tokens, chunk c scored by
//            ln(mass of c) + g(c, chunk tag);
//   level 2: inside the chosen chunk, sub-chunks of kSub consecutive tokens,
//            sub-chunk j (global index j = v / kSub) scored by
//            ln(mass of j) + g(j, sub-chunk tag);
//   level 3: inside the chosen sub-chunk, token v scored by lw_v + g(v, token
//            tag).
// Each level's winner is a draw from that level's masses renormalised over
// the chosen parent, with independent noise, so
// P(v) = (W_c / W)(W_j / W_c)(w_v / W_j) = w_v / W exactly.  Ties go to the
// lowest index.  Returns -1 if every weight is zero.  `near` is set if any
// level's top-2 gap is within the margin.
namespace {
struct Best2 {
  int32_t arg = -1;
  double s1 = kNegInf, s2 = kNegInf;
  void offer(double score, int32_t idx) {
    if (score > s1) {
      s2 = s1;
      s1 = score;
      arg = idx;
    } else if (score > s2) {
      s2 = score;
    }
  }
  bool near() const { return arg >= 0 && s2 != kNegInf && near_gap(s1, s2); }
};

// ln(sum of exp(lw_v)) over v in [lo, hi), -inf if every lw_v is -inf
double log_mass(const double* lw, int32_t lo, int32_t hi) {
  double mx = kNegInf;
  for (int32_t v = lo; v < hi; ++v) mx = std::max(mx, lw[v]);
  if (mx == kNegInf) return kNegInf;
  double s = 0.0;
  for (int32_t v = lo; v < hi; ++v)
    if (lw[v] != kNegInf) s += std::exp(lw[v] - mx);
  return mx + std::log(s);
}
}  // namespace

int32_t sample_three_level(const double* lw, int32_t V, uint64_t seed,
                           uint32_t request, int32_t position,
                           uint32_t tag_chunk, uint32_t tag_sub,
                           uint32_t tag_token, bool* near) {
  // level 1: chunks
  Best2 l1;
  const int32_t C = (V + kChunk - 1) / kChunk;
  for (int32_t c = 0; c < C; ++c) {
    const double lm = log_mass(lw, c * kChunk, std::min(V, (c + 1) * kChunk));
    if (lm == kNegInf) continue;
    l1.offer(lm + gumbel(seed, static_cast<uint32_t>(c), position, request, tag_chunk), c);
  }
  if (l1.arg < 0) {
    *near = false;
    return -1;
  }
  // level 2: sub-chunks of the chosen chunk
  Best2 l2;
  const int32_t c_lo = l1.arg * kChunk, c_hi = std::min(V, c_lo + kChunk);
  for (int32_t j = c_lo / kSub; j * kSub < c_hi; ++j) {
    const double lm = log_mass(lw, j * kSub, std::min(c_hi, (j + 1) * kSub));
    if (lm == kNegInf) continue;
    l2.offer(lm + gumbel(seed, static_cast<uint32_t>(j), position, request, tag_sub), j);
  }
  // level 3: tokens of the chosen sub-chunk
  Best2 l3;
  const int32_t j_lo = l2.arg * kSub, j_hi = std::min(c_hi, j_lo + kSub);
  for (int32_t v = j_lo; v < j_hi; ++v) {
    if (lw[v] == kNegInf) continue;
    l3.offer(lw[v] + gumbel(seed, static_cast<uint32_t>(v), position, request, tag_token), v);
  }
  *near = l1.near() || l2.near() || l3.near();
  return l3.arg;
}

// ---------------------------------------------------------------------------
// Row policy ([FT] "Probabilistic": temperature, top-k and top-p are applied to
// both p and q).  Reading taken for the unstated order and ties: temperature,
// then top-k keeping every token tied with the k-th value, then top-p on the
// renormalised top-k set keeping v iff the mass of strictly more probable
// kept tokens is < top_p (top_p <= 0 keeps the argmax set).
struct RowPolicy {
  std::vector<double> z;      // scaled logits (kNegInf where excluded)
  std::vector<uint8_t> kept;  // 1 = in the kept set
  double lse = kNegInf;       // log-sum-exp of z over the kept set
  double thr = kNegInf;       // smallest kept z if truncation active
  int32_t nkept = 0;
  bool near = false;
};

// `exact_order`: the row's ordering is decided on exact input values on the
// device as well (verify rows), so the top-k boundary cannot flip.
void apply_policy(const std::vector<double>& l, double T, int32_t top_k,
                  double top_p, bool exact_order, RowPolicy* out) {
  const int32_t V = static_cast<int32_t>(l.size());
  out->z.assign(V, kNegInf);
  out->kept.assign(V, 0);
  out->near = false;
  for (int32_t v = 0; v < V; ++v)
    if (l[v] != kNegInf) {
      out->z[v] = l[v] / T;
      out->kept[v] = 1;
    }
  bool truncated = false;
  // top-k
  std::vector<int32_t> order;
  order.reserve(V);
  for (int32_t v = 0; v < V; ++v)
    if (out->kept[v]) order.push_back(v);
  const int32_t nfin = static_cast<int32_t>(order.size());
  // descending value, ascending index on ties
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    if (out->z[a] != out->z[b]) return out->z[a] > out->z[b];
    return a < b;
  });
  if (top_k > 0 && top_k < V) {
    truncated = true;
    if (top_k < nfin) {
      const double zk = out->z[order[top_k - 1]];
      const double zk1 = out->z[order[top_k]];
      if (!exact_order && near_gap(zk, zk1)) out->near = true;
      for (int32_t v = 0; v < V; ++v)
        if (out->kept[v] && out->z[v] < zk) out->kept[v] = 0;
    }
  }
  // top-p on the renormalised kept set
  if (top_p < 1.0) {
    truncated = true;
    double mx = kNegInf;
    for (int32_t v = 0; v < V; ++v)
      if (out->kept[v]) mx = std::max(mx, out->z[v]);
    if (mx != kNegInf) {
      double s = 0.0;
      for (int32_t v = 0; v < V; ++v)
        if (out->kept[v]) s += std::exp(out->z[v] - mx);
      const double lse = mx + std::log(s);
      // walk groups of equal value in descending order; the first group is
      // always kept, a later group is kept iff the mass above it is < top_p
      std::vector<int32_t> ko;
      for (int32_t v : order)
        if (out->kept[v]) ko.push_back(v);
      double above = 0.0;  // mass of strictly more probable kept tokens
      double cut_value = out->z[ko[0]], prev_value = cut_value;
      bool first = true;
      size_t i = 0;
      while (i < ko.size()) {
        const double val = out->z[ko[i]];
        size_t j = i;
        double gmass = 0.0;
        while (j < ko.size() && out->z[ko[j]] == val) {
          gmass += std::exp(out->z[ko[j]] - lse);
          ++j;
        }
        if (!first) {
          if (std::fabs(above - top_p) <= kEps) out->near = true;
          if (!(above < top_p)) {
            // a near tie between the last kept and the first dropped value
            // of a computed row could merge or split the groups on device
            if (!exact_order && near_gap(prev_value, val)) out->near = true;
            break;
          }
        }
        cut_value = val;
        prev_value = val;
        above += gmass;
        first = false;
        i = j;
      }
      for (int32_t v = 0; v < V; ++v)
        if (out->kept[v] && out->z[v] < cut_value) out->kept[v] = 0;
    }
  }
  // log-sum-exp over the kept set, threshold
  double mx = kNegInf, mn = std::numeric_limits<double>::infinity();
  int32_t n = 0;
  for (int32_t v = 0; v < V; ++v)
    if (out->kept[v]) {
      mx = std::max(mx, out->z[v]);
      mn = std::min(mn, out->z[v]);
      ++n;
    }
  out->nkept = n;
  if (n == 0) {
    out->lse = kNegInf;
    out->thr = kNegInf;
    return;
  }
  double s = 0.0;
  for (int32_t v = 0; v < V; ++v)
    if (out->kept[v]) s += std::exp(out->z[v] - mx);
  out->lse = mx + std::log(s);
  out->thr = truncated ? mn : kNegInf;
  for (int32_t v = 0; v < V; ++v)
    if (!out->kept[v]) out->z[v] = (l[v] == kNegInf) ? kNegInf : l[v] / T;
}

// Greedy argmax (lowest index on ties) over finite values; -1 if none.
// `near` (if requested) reports a top-2 gap within the margin, ties included.
int32_t argmax_lowest(const std::vector<double>& l, bool* near, bool check_near) {
  const int32_t V = static_cast<int32_t>(l.size());
  int32_t best = -1;
  double b1 = kNegInf;
  for (int32_t v = 0; v < V; ++v)
    if (l[v] != kNegInf && (best < 0 || l[v] > b1)) {
      b1 = l[v];
      best = v;
    }
  if (near) {
    double b2 = kNegInf;
    for (int32_t v = 0; v < V; ++v)
      if (v != best) b2 = std::max(b2, l[v]);
    *near = check_near && best >= 0 && b2 != kNegInf && near_gap(b1, b2);
  }
  return best;
}

// Load a row of logits into binary64, mapping NaN / +inf to -inf.
void load_row(const void* p, int dtype, size_t off, int32_t V,
              std::vector<double>* row, bool* nonfinite) {
  row->resize(V);
  bool nf = false;
  for (int32_t v = 0; v < V; ++v) {
    double x = logit_at(p, dtype, off + v);
    if (std::isnan(x) || x == std::numeric_limits<double>::infinity()) {
      x = kNegInf;
      nf = true;
    }
    (*row)[v] = x;
  }
  *nonfinite = nf;
}

bool bad_temperature(double T) { return !(T > 0.0) || !std::isfinite(T); }

int32_t clamp_token(int32_t x, int32_t V) { return std::min(std::max(x, 0), V - 1); }

}  // namespace

extern "C" {

// ---- primitives exposed for the tests -------------------------------------
void oracle_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out) {
  philox4x32_10(ctr, key, out);
}

uint32_t oracle_philox_word(uint64_t seed, uint32_t i, int32_t position,
                            uint32_t request, uint32_t tag) {
  return philox_word(seed, i, position, request, tag);
}

double oracle_gumbel(uint64_t seed, uint32_t i, int32_t position,
                     uint32_t request, uint32_t tag) {
  return gumbel(seed, i, position, request, tag);
}

double oracle_accept_uniform(uint64_t seed, int32_t position, uint32_t request) {
  return accept_uniform(seed, position, request);
}

// Three-level Gumbel-max over log-weights (for distribution tests).
int32_t oracle_sample_three_level(const double* lw, int32_t V, uint64_t seed,
                                  uint32_t request, int32_t position,
                                  uint32_t tag_chunk, uint32_t tag_sub,
                                  uint32_t tag_token, int32_t* near) {
  bool nr = false;
  const int32_t v = sample_three_level(lw, V, seed, request, position, tag_chunk,
                                       tag_sub, tag_token, &nr);
  if (near) *near = nr ? 1 : 0;
  return v;
}

// Row policy: writes kept[V], z[V] (scaled, -inf where not finite), and
// returns lse / thr / near through pointers.
int32_t oracle_policy_row(const double* l, int32_t V, double T, int32_t top_k,
                          double top_p, int32_t exact_order, uint8_t* kept,
                          double* z, double* lse, double* thr, int32_t* near) {
  std::vector<double> row(l, l + V);
  for (auto& x : row)
    if (std::isnan(x) || x == std::numeric_limits<double>::infinity()) x = kNegInf;
  RowPolicy rp;
  apply_policy(row, T, top_k, top_p, exact_order != 0, &rp);
  for (int32_t v = 0; v < V; ++v) {
    kept[v] = rp.kept[v];
    z[v] = rp.z[v];
  }
  *lse = rp.lse;
  *thr = rp.thr;
  *near = rp.near ? 1 : 0;
  return rp.nkept;
}

// ---------------------------------------------------------------------------
// Markov draft sampling ([FT] "Checkpoint-faithful DSpark architecture";
// [MB] "Semi-autoregressive draft").  For k = 1..gamma in order, with
// x_0 = anchor:
//   y_k = backbone[b,k-1,:] + A[x_{k-1},:] . Bt^T      (A = markov_w1 [V,r],
//                                                       Bt = markov_w2 [V,r])
//   q_k = policy(y_k);  x_k ~ q_k (three-level Gumbel-max, draft tags,
//                       position = anchor position + k)  or argmax if greedy
//   c_k = sigmoid(w[:d] . h[b,k-1,:] + w[d:] . E[x_{k-1},:])   (no bias term,
//         order [h ; embed] as the confidence-head formula writes it)
// forced_tokens (may be NULL; -1 = not forced) replaces x_k after it is drawn,
// so a chain can be replayed along another sampler's tokens.
// q_z may be NULL (not written); otherwise q_z[b,k-1,:] = z for sampled rows.
int32_t oracle_markov_sample(
    const void* backbone, int32_t dtype, const int32_t* anchor,
    const uint16_t* A, const uint16_t* Bt, const uint16_t* h,
    const uint16_t* E, const float* w, const uint8_t* mode,
    const float* temperature, const int32_t* top_k, const float* top_p,
    const uint32_t* request_id, const int32_t* position, uint64_t seed,
    int32_t B, int32_t gamma, int32_t V, int32_t r, int32_t d,
    const int32_t* forced_tokens, int32_t* draft_tokens, double* q_z,
    double* q_lse, double* q_thr, double* q_tok, double* confidence,
    uint8_t* flags) {
  if (B < 0 || gamma < 1 || V < 1 || r < 0 || d < 0) return 1;
  std::vector<double> y(V);
  std::vector<double> a(r);
  for (int32_t b = 0; b < B; ++b) {
    int32_t x_prev = clamp_token(anchor[b], V);
    for (int32_t k = 1; k <= gamma; ++k) {
      const size_t row = static_cast<size_t>(b) * gamma + (k - 1);
      uint8_t fl = 0;
      // confidence head on [h_k ; embed(x_{k-1})]
      double dot = 0.0;
      for (int32_t i = 0; i < d; ++i)
        dot += static_cast<double>(w[i]) * bf16_to_double(h[row * d + i]);
      for (int32_t i = 0; i < d; ++i)
        dot += static_cast<double>(w[d + i]) *
               bf16_to_double(E[static_cast<size_t>(x_prev) * d + i]);
      confidence[row] = 1.0 / (1.0 + std::exp(-dot));
      // y = backbone row + low-rank Markov bias
      for (int32_t i = 0; i < r; ++i)
        a[i] = bf16_to_double(A[static_cast<size_t>(x_prev) * r + i]);
      bool nonfinite = false;
      {
        std::vector<double> bb;
        load_row(backbone, dtype, row * V, V, &bb, &nonfinite);
        for (int32_t v = 0; v < V; ++v) {
          double bias = 0.0;
          for (int32_t i = 0; i < r; ++i)
            bias += a[i] * bf16_to_double(Bt[static_cast<size_t>(v) * r + i]);
          y[v] = (bb[v] == kNegInf) ? kNegInf : bb[v] + bias;
        }
      }
      if (nonfinite) fl |= F_NONFINITE;
      const bool sampled = mode[b] != 0 && !bad_temperature(temperature[b]);
      if (mode[b] != 0 && !sampled) fl |= F_BAD_POLICY;
      int32_t x;
      if (!sampled) {
        bool nr = false;
        x = argmax_lowest(y, &nr, true);
        if (nr) fl |= F_NEAR;
        if (x < 0) {
          x = 0;
          fl |= F_EMPTY;
        }
        q_lse[row] = 0.0;
        q_thr[row] = 0.0;
        q_tok[row] = 1.0;
        if (forced_tokens && forced_tokens[row] >= 0)
          x = clamp_token(forced_tokens[row], V);
      } else {
        RowPolicy rp;
        apply_policy(y, static_cast<double>(temperature[b]), top_k[b],
                     static_cast<double>(top_p[b]), false, &rp);
        if (rp.near) fl |= F_NEAR;
        std::vector<double> lw(V, kNegInf);
        for (int32_t v = 0; v < V; ++v)
          if (rp.kept[v]) lw[v] = rp.z[v];
        bool nr = false;
        x = sample_three_level(lw.data(), V, seed, request_id[b], position[b] + k,
                               TAG_DRAFT_CHUNK, TAG_DRAFT_SUB, TAG_DRAFT_TOKEN, &nr);
        if (nr) fl |= F_NEAR;
        if (x < 0) {
          x = 0;
          fl |= F_EMPTY;
        }
        if (forced_tokens && forced_tokens[row] >= 0)
          x = clamp_token(forced_tokens[row], V);
        q_lse[row] = rp.lse;
        q_thr[row] = rp.thr;
        q_tok[row] = rp.kept[x] ? std::exp(rp.z[x] - rp.lse) : 0.0;
        if (q_z)
          for (int32_t v = 0; v < V; ++v) q_z[row * V + v] = rp.z[v];
      }
      draft_tokens[row] = x;
      flags[row] = fl;
      x_prev = x;
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Exact verify ([FT] "Exact decoding semantics"; [PS] "Acceptance").
// Target row k (k = 0..gamma) is the target distribution after x_k; row k-1
// verifies x_k and row n_draft is the bonus row.
// q_z / q_lse / q_thr / q_tok are the proposal side in the library's stored
// format (fp32): q_v = (q_z[v] >= q_thr) ? exp(q_z[v] - q_lse) : 0.
// p_tok (may be NULL) receives p_{k-1}(x_k) for the tested proposals.
int32_t oracle_verify(const void* target, int32_t dtype,
                      const int32_t* draft_tokens, const float* q_z,
                      const float* q_lse, const float* q_thr,
                      const float* q_tok, const int32_t* n_draft,
                      const uint8_t* mode, const float* temperature,
                      const int32_t* top_k, const float* top_p,
                      const uint32_t* request_id, const int32_t* position,
                      uint64_t seed, int32_t B, int32_t gamma, int32_t V,
                      int32_t* accept_len, int32_t* out_tokens, uint8_t* flags,
                      double* p_tok) {
  if (B < 0 || gamma < 1 || V < 1) return 1;
  const int32_t R = gamma + 1;
  std::vector<double> l;
  for (int32_t b = 0; b < B; ++b) {
    int32_t nd = n_draft ? n_draft[b] : gamma;
    nd = std::min(std::max(nd, 0), gamma);
    uint8_t* fl = flags + static_cast<size_t>(b) * R;
    int32_t* out = out_tokens + static_cast<size_t>(b) * R;
    for (int32_t k = 0; k < R; ++k) {
      fl[k] = 0;
      out[k] = -1;
    }
    std::vector<int32_t> x(gamma + 1, 0);
    for (int32_t k = 1; k <= gamma; ++k)
      x[k] = clamp_token(draft_tokens[static_cast<size_t>(b) * gamma + k - 1], V);
    const bool sampled = mode[b] != 0 && !bad_temperature(temperature[b]);
    if (mode[b] != 0 && !sampled) fl[0] |= F_BAD_POLICY;
    auto row_off = [&](int32_t k) {
      return (static_cast<size_t>(b) * R + k) * static_cast<size_t>(V);
    };
    // data flags of every target row the request owns (rows 0..n_d),
    // whether or not the decision below reaches it
    for (int32_t k = 0; k <= nd; ++k) {
      bool nf = false;
      load_row(target, dtype, row_off(k), V, &l, &nf);
      if (nf) fl[k] |= F_NONFINITE;
      if (argmax_lowest(l, nullptr, false) < 0) fl[k] |= F_EMPTY;
    }
    if (!sampled) {
      // greedy contiguous-prefix match; the target argmax compares exact
      // input values, so no margin applies
      int32_t n = nd;
      std::vector<int32_t> t(nd + 1, 0);
      for (int32_t k = 0; k <= nd; ++k) {
        bool nf = false;
        load_row(target, dtype, row_off(k), V, &l, &nf);
        int32_t tk = argmax_lowest(l, nullptr, false);
        if (tk < 0) tk = 0;
        t[k] = tk;
        if (k >= 1 && x[k] != t[k - 1]) {
          n = k - 1;
          break;
        }
      }
      for (int32_t k = 1; k <= n; ++k) out[k - 1] = x[k];
      out[n] = t[n];
      accept_len[b] = n;
      continue;
    }
    const double T = static_cast<double>(temperature[b]);
    const int32_t pos0 = position[b];
    int32_t j = -1;  // first rejected proposal
    RowPolicy rp;
    for (int32_t k = 1; k <= nd; ++k) {
      bool nf = false;
      load_row(target, dtype, row_off(k - 1), V, &l, &nf);
      apply_policy(l, T, top_k[b], static_cast<double>(top_p[b]), true, &rp);
      if (rp.near) fl[k - 1] |= F_NEAR;
      const double pk = rp.kept[x[k]] ? std::exp(rp.z[x[k]] - rp.lse) : 0.0;
      if (p_tok) p_tok[static_cast<size_t>(b) * gamma + k - 1] = pk;
      const double qk = static_cast<double>(q_tok[static_cast<size_t>(b) * gamma + k - 1]);
      const double u = accept_uniform(seed, pos0 + k, request_id[b]);
      bool accept;
      if (qk > 0.0) {
        const double rho = pk / qk;
        accept = u < rho;
        if (std::fabs(u - rho) <= kEps) fl[k - 1] |= F_NEAR;
      } else {
        accept = pk > 0.0;
      }
      if (!accept) {
        j = k;
        break;
      }
    }
    int32_t emitted;
    if (j > 0) {
      // residual max(p_{j-1} - q_j, 0) over the whole vocabulary; rp holds
      // the policy of target row j-1
      const size_t qrow = (static_cast<size_t>(b) * gamma + (j - 1));
      const double lq = static_cast<double>(q_lse[qrow]);
      const double tq = static_cast<double>(q_thr[qrow]);
      std::vector<double> lw(V, kNegInf);
      bool any = false;
      for (int32_t v = 0; v < V; ++v) {
        const double pv = rp.kept[v] ? std::exp(rp.z[v] - rp.lse) : 0.0;
        const double zq = static_cast<double>(q_z[qrow * V + v]);
        const double qv = (zq >= tq && zq != kNegInf) ? std::exp(zq - lq) : 0.0;
        const double rv = pv - qv;
        if (rv > 0.0) {
          lw[v] = std::log(rv);
          any = true;
        }
      }
      bool nr = false;
      if (!any) {
        fl[j - 1] |= F_RESID_ZERO;
        for (int32_t v = 0; v < V; ++v) lw[v] = rp.kept[v] ? rp.z[v] : kNegInf;
      }
      emitted = sample_three_level(lw.data(), V, seed, request_id[b], pos0 + j,
                                   TAG_TARGET_CHUNK, TAG_TARGET_SUB, TAG_TARGET_TOKEN, &nr);
      if (nr) fl[j - 1] |= F_NEAR;
      if (emitted < 0) emitted = 0;
      for (int32_t k = 1; k < j; ++k) out[k - 1] = x[k];
      out[j - 1] = emitted;
      accept_len[b] = j - 1;
    } else {
      bool nf = false;
      load_row(target, dtype, row_off(nd), V, &l, &nf);
      apply_policy(l, T, top_k[b], static_cast<double>(top_p[b]), true, &rp);
      if (rp.near) fl[nd] |= F_NEAR;
      std::vector<double> lw(V, kNegInf);
      for (int32_t v = 0; v < V; ++v)
        if (rp.kept[v]) lw[v] = rp.z[v];
      bool nr = false;
      emitted = sample_three_level(lw.data(), V, seed, request_id[b],
                                   pos0 + nd + 1, TAG_TARGET_CHUNK,
                                   TAG_TARGET_SUB, TAG_TARGET_TOKEN, &nr);
      if (nr) fl[nd] |= F_NEAR;
      if (emitted < 0) emitted = 0;
      for (int32_t k = 1; k <= nd; ++k) out[k - 1] = x[k];
      out[nd] = emitted;
      accept_len[b] = nd;
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Analytic acceptance statistics ([MB] "Training objective", "Acceptance and
// confidence", "Loss return contract").  Per block b and position k = 1..gamma
// (row k-1), P = softmax(draft row), T = softmax(target row) at temperature 1
// with no truncation (reading: the pages give no training-time policy):
//   l1  = sum_v |P_v - T_v|            (raw; the 1/2 belongs to the label)
//   a   = clamp(1 - l1/2, 0, 1)
//   ce  = logsumexp(draft row) - draft[teacher]
//   bce = max(c,0) - c*a + log1p(exp(-|c|))    (BCE of logit c against a)
//   tau = 1 + sum_k prod_{j<=k} a_j
// Weights w_k = exp(-k/gamma), k 1-based (reading); num_tokens counts the
// supervised positions (reading); the mask is per block (reading).
// sums[12] = {numerator, num_tokens, l1 sum, count, accept sum, count,
//             tau sum, block count, ce sum, count, bce sum, count}.
int32_t oracle_accept_stats2(const void* draft, int32_t ddtype, const void* target,
                             int32_t dtype, const int32_t* teacher,
                             const float* conf_logits, const uint8_t* block_mask,
                             int32_t N, int32_t gamma, int32_t V, double w_ce,
                             double w_l1, double w_conf, double* l1,
                             double* accept_rate, double* ce, double* bce,
                             double* tau, double* sums);

int32_t oracle_accept_stats(const void* draft, const void* target,
                            int32_t dtype, const int32_t* teacher,
                            const float* conf_logits, const uint8_t* block_mask,
                            int32_t N, int32_t gamma, int32_t V, double w_ce,
                            double w_l1, double w_conf, double* l1,
                            double* accept_rate, double* ce, double* bce,
                            double* tau, double* sums) {
  return oracle_accept_stats2(draft, dtype, target, dtype, teacher, conf_logits, block_mask, N,
                              gamma, V, w_ce, w_l1, w_conf, l1, accept_rate, ce, bce, tau, sums);
}

// The same statistics with the draft rows in their own dtype (ddtype).
int32_t oracle_accept_stats2(const void* draft, int32_t ddtype, const void* target,
                             int32_t dtype, const int32_t* teacher,
                             const float* conf_logits, const uint8_t* block_mask,
                             int32_t N, int32_t gamma, int32_t V, double w_ce,
                             double w_l1, double w_conf, double* l1,
                             double* accept_rate, double* ce, double* bce,
                             double* tau, double* sums) {
  if (N < 0 || gamma < 1 || V < 1) return 1;
  for (int i = 0; i < 12; ++i) sums[i] = 0.0;
  std::vector<double> dl, tl;
  for (int32_t b = 0; b < N; ++b) {
    const bool m = block_mask ? block_mask[b] != 0 : true;
    double cum = 1.0, t = 1.0;
    for (int32_t k = 1; k <= gamma; ++k) {
      const size_t row = static_cast<size_t>(b) * gamma + (k - 1);
      bool nf = false;
      load_row(draft, ddtype, row * V, V, &dl, &nf);
      load_row(target, dtype, row * V, V, &tl, &nf);
      double md = kNegInf, mt = kNegInf;
      for (int32_t v = 0; v < V; ++v) {
        md = std::max(md, dl[v]);
        mt = std::max(mt, tl[v]);
      }
      double sd = 0.0, st = 0.0;
      for (int32_t v = 0; v < V; ++v) {
        if (dl[v] != kNegInf) sd += std::exp(dl[v] - md);
        if (tl[v] != kNegInf) st += std::exp(tl[v] - mt);
      }
      const double lse_d = md + std::log(sd), lse_t = mt + std::log(st);
      double dist = 0.0;
      for (int32_t v = 0; v < V; ++v) {
        const double P = (dl[v] == kNegInf) ? 0.0 : std::exp(dl[v] - lse_d);
        const double Q = (tl[v] == kNegInf) ? 0.0 : std::exp(tl[v] - lse_t);
        dist += std::fabs(P - Q);
      }
      const double a = std::min(1.0, std::max(0.0, 1.0 - 0.5 * dist));
      const int32_t tch = clamp_token(teacher[row], V);
      const double c_e = lse_d - dl[tch];
      const double c = static_cast<double>(conf_logits[row]);
      const double b_ce = std::max(c, 0.0) - c * a + std::log1p(std::exp(-std::fabs(c)));
      l1[row] = dist;
      accept_rate[row] = a;
      ce[row] = c_e;
      bce[row] = b_ce;
      cum *= a;
      t += cum;
      if (m) {
        const double wk = std::exp(-static_cast<double>(k) / gamma);
        sums[0] += wk * (w_ce * c_e + w_l1 * dist + w_conf * b_ce);
        sums[1] += 1.0;
        sums[2] += dist;
        sums[3] += 1.0;
        sums[4] += a;
        sums[5] += 1.0;
        sums[8] += c_e;
        sums[9] += 1.0;
        sums[10] += b_ce;
        sums[11] += 1.0;
      }
    }
    tau[b] = t;
    if (m) {
      sums[6] += t;
      sums[7] += 1.0;
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Acceptance statistics of the teacher-forced Markov draft ([MB]
// "Semi-autoregressive draft": the sequential head adds a low-rank,
// token-conditioned bias to the parallel logits and is teacher-forced with
// the previous block tokens at training time; "Training objective").  The
// draft row of block b at position k is
//   backbone[b,k-1,:] + W1[x_{k-1}] . W2^T,
// x_0 = anchor[b] and x_{k-1} = teacher[b,k-2] for k >= 2 (the true token
// before position k; teacher[b,k-1] is the CE target of position k), both
// clamped into [0, V); -inf backbone logits stay -inf.  The statistics are
// then those of oracle_accept_stats on these rows (binary64 throughout).
int32_t oracle_accept_stats_markov(const void* backbone, const void* target, int32_t dtype,
                                   const int32_t* anchor, const uint16_t* A,
                                   const uint16_t* Bt, int32_t r, const int32_t* teacher,
                                   const float* conf_logits, const uint8_t* block_mask,
                                   int32_t N, int32_t gamma, int32_t V, double w_ce,
                                   double w_l1, double w_conf, double* l1,
                                   double* accept_rate, double* ce, double* bce,
                                   double* tau, double* sums) {
  if (N < 0 || gamma < 1 || V < 1 || r < 0) return 1;
  std::vector<double> draft(static_cast<size_t>(N) * gamma * V);
  std::vector<double> a(r), bb;
  for (int32_t b = 0; b < N; ++b)
    for (int32_t k = 1; k <= gamma; ++k) {
      const size_t row = static_cast<size_t>(b) * gamma + (k - 1);
      const int32_t x = clamp_token(k == 1 ? anchor[b] : teacher[row - 1], V);
      for (int32_t i = 0; i < r; ++i) a[i] = bf16_to_double(A[static_cast<size_t>(x) * r + i]);
      bool nf = false;
      load_row(backbone, dtype, row * V, V, &bb, &nf);
      for (int32_t v = 0; v < V; ++v) {
        double bias = 0.0;
        for (int32_t i = 0; i < r; ++i)
          bias += a[i] * bf16_to_double(Bt[static_cast<size_t>(v) * r + i]);
        draft[row * V + v] = (bb[v] == kNegInf) ? kNegInf : bb[v] + bias;
      }
    }
  return oracle_accept_stats2(draft.data(), 3, target, dtype, teacher, conf_logits, block_mask,
                              N, gamma, V, w_ce, w_l1, w_conf, l1, accept_rate, ce, bce, tau,
                              sums);
}

// ---------------------------------------------------------------------------
// Gradient of the acceptance statistics' loss numerator ([MB] "Training
// objective": the draft is trained by 0.1 CE + 0.9 raw L1, and the BCE term
// trains the confidence head against the acceptance label; the target's
// distribution is detached; "Memory contract for the full-vocabulary terms":
// the terms' row chunks are recomputed in the backward).  With the
// numerator of oracle_accept_stats scaled by `scale`, per block b (mask m_b)
// and position k (row k-1), w_k = exp(-k/gamma), P = softmax(draft row),
// T = softmax(target row), a = clamp(1 - L1/2, 0, 1):
//   d/d draft_v = scale m_b w_k [ w_ce (P_v - [v == teacher])
//                                + w_l1 P_v (s_v - sum_u s_u P_u) ]
//   d/d c       = scale m_b w_k w_conf (sigmoid(c) - a)
// with s_u = sign(P_u - T_u) and sign(0) = 0 (the subgradient of |x| that
// vanishes at 0).  Readings: the label a is held fixed in the BCE (it is the
// confidence head's regression target), so the BCE sends no gradient into
// the draft logits; -inf logits have P = 0 and get gradient 0 (teacher
// aside).  sigmoid(c) = 1 / (1 + exp(-c)).
int32_t oracle_accept_stats_backward(const void* draft, const void* target, int32_t dtype,
                                     const int32_t* teacher, const float* conf_logits,
                                     const uint8_t* block_mask, int32_t N, int32_t gamma,
                                     int32_t V, double w_ce, double w_l1, double w_conf,
                                     double scale, double* grad_draft, double* grad_conf) {
  if (N < 0 || gamma < 1 || V < 1) return 1;
  std::vector<double> dl, tl, P, T;
  P.resize(V);
  T.resize(V);
  for (int32_t b = 0; b < N; ++b) {
    const double m = (block_mask ? block_mask[b] != 0 : true) ? 1.0 : 0.0;
    for (int32_t k = 1; k <= gamma; ++k) {
      const size_t row = static_cast<size_t>(b) * gamma + (k - 1);
      bool nf = false;
      load_row(draft, dtype, row * V, V, &dl, &nf);
      load_row(target, dtype, row * V, V, &tl, &nf);
      double md = kNegInf, mt = kNegInf;
      for (int32_t v = 0; v < V; ++v) {
        md = std::max(md, dl[v]);
        mt = std::max(mt, tl[v]);
      }
      double sd = 0.0, st = 0.0;
      for (int32_t v = 0; v < V; ++v) {
        if (dl[v] != kNegInf) sd += std::exp(dl[v] - md);
        if (tl[v] != kNegInf) st += std::exp(tl[v] - mt);
      }
      double l1 = 0.0, S = 0.0;
      for (int32_t v = 0; v < V; ++v) {
        P[v] = (dl[v] == kNegInf) ? 0.0 : std::exp(dl[v] - md) / sd;
        T[v] = (tl[v] == kNegInf) ? 0.0 : std::exp(tl[v] - mt) / st;
        l1 += std::fabs(P[v] - T[v]);
        const double sg = P[v] > T[v] ? 1.0 : (P[v] < T[v] ? -1.0 : 0.0);
        S += sg * P[v];
      }
      const double a = std::min(1.0, std::max(0.0, 1.0 - 0.5 * l1));
      const double alpha = scale * m * std::exp(-static_cast<double>(k) / gamma);
      const int32_t tch = clamp_token(teacher[row], V);
      for (int32_t v = 0; v < V; ++v) {
        const double sg = P[v] > T[v] ? 1.0 : (P[v] < T[v] ? -1.0 : 0.0);
        const double ce_g = P[v] - (v == tch ? 1.0 : 0.0);
        grad_draft[row * V + v] = alpha * (w_ce * ce_g + w_l1 * P[v] * (sg - S));
      }
      const double c = static_cast<double>(conf_logits[row]);
      grad_conf[row] = alpha * w_conf * (1.0 / (1.0 + std::exp(-c)) - a);
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Confidence-scheduled draft width ([FT] "Scope and limitations" and the
// author's reply on hardware-aware width: a measured choice over 0..5
// proposals that declines or shortens speculation when the measured draft
// plus verify cost D + V(k) does not pay; [MB] "Overview": the confidence
// head predicts per-position acceptance so that the server can schedule its
// verify budget).  Reading: c_j is the predicted probability that proposal j
// is accepted given proposals 1..j-1 were, so verifying the first w
// proposals emits E(w) = 1 + sum_{k<=w} prod_{j<=k} c_j tokens in
// expectation (the accepted prefix plus the one token the target always
// emits; E(gamma) is the tau of the acceptance statistics with c for a),
// at cost D + V(w).  Per request, the width w in 0..gamma with the largest
// E(w) / (D + V(w)); ties go to the smaller w; a width whose cost is not a
// finite positive number is not eligible, and with none eligible w = 0.
// c_j is clamped to [0, 1] (NaN -> 0).  cost = {D, V(0), ..., V(gamma)}.
// Evaluated in binary64 in this order: p_k = p_{k-1} c_k, E_k = E_{k-1} + p_k,
// den = D + V(w), ratio = E / den, compared with a strict >.
int32_t oracle_select_width(const float* confidence, const float* cost, int32_t B,
                            int32_t gamma, int32_t* n_draft, double* expected) {
  if (B < 0 || gamma < 1) return 1;
  const double D = static_cast<double>(cost[0]);
  for (int32_t b = 0; b < B; ++b) {
    double p = 1.0, E = 1.0;
    double best = kNegInf, best_E = 1.0;
    int32_t best_w = 0;
    for (int32_t w = 0; w <= gamma; ++w) {
      if (w >= 1) {
        double c = static_cast<double>(confidence[static_cast<size_t>(b) * gamma + (w - 1)]);
        if (!(c > 0.0)) c = 0.0;  // NaN and non-positive
        if (c > 1.0) c = 1.0;
        p = p * c;
        E = E + p;
      }
      const double den = D + static_cast<double>(cost[1 + w]);
      if (!(den > 0.0) || !std::isfinite(den)) continue;
      const double ratio = E / den;
      if (ratio > best) {
        best = ratio;
        best_w = w;
        best_E = E;
      }
    }
    n_draft[b] = best_w;
    expected[b] = best_E;
  }
  return 0;
}

}  // extern "C"
