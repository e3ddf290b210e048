// Host sanitizer driver for the oracle: tests/test_oracle_sanitize.py builds
// this file together with oracle/dspark_oracle.cpp under AddressSanitizer and
// UndefinedBehaviorSanitizer (g++, CPU only) and runs it.  It calls every
// exported oracle function on small inputs: ragged vocabularies, -inf and
// NaN logits, empty rows, truncation on and off, greedy and sampled
// requests, n_draft below gamma, masked blocks, zero ranks.  The values come
// from a fixed linear congruential generator: the run checks memory and
// arithmetic validity, not results (the pinned tests do that).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

extern "C" {
void oracle_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out);
uint32_t oracle_philox_word(uint64_t seed, uint32_t i, int32_t position, uint32_t request, uint32_t tag);
double oracle_gumbel(uint64_t seed, uint32_t i, int32_t position, uint32_t request, uint32_t tag);
double oracle_accept_uniform(uint64_t seed, int32_t position, uint32_t request);
int32_t oracle_sample_three_level(const double* lw, int32_t V, uint64_t seed, uint32_t request, int32_t position,
                                  uint32_t tag_chunk, uint32_t tag_sub, uint32_t tag_token, int32_t* near);
int32_t oracle_policy_row(const double* l, int32_t V, double T, int32_t top_k, double top_p, int32_t exact_order,
                          uint8_t* kept, double* z, double* lse, double* thr, int32_t* near);
int32_t oracle_markov_sample(const void* backbone, int32_t dtype, const int32_t* anchor, const uint16_t* A,
                             const uint16_t* Bt, const uint16_t* h, const uint16_t* E, const float* w,
                             const uint8_t* mode, const float* temperature, const int32_t* top_k,
                             const float* top_p, const uint32_t* request_id, const int32_t* position,
                             uint64_t seed, int32_t B, int32_t gamma, int32_t V, int32_t r, int32_t d,
                             const int32_t* forced_tokens, int32_t* draft_tokens, double* q_z, double* q_lse,
                             double* q_thr, double* q_tok, double* confidence, uint8_t* flags);
int32_t oracle_verify(const void* target, int32_t dtype, const int32_t* draft_tokens, const float* q_z,
                      const float* q_lse, const float* q_thr, const float* q_tok, const int32_t* n_draft,
                      const uint8_t* mode, const float* temperature, const int32_t* top_k, const float* top_p,
                      const uint32_t* request_id, const int32_t* position, uint64_t seed, int32_t B,
                      int32_t gamma, int32_t V, int32_t* accept_len, int32_t* out_tokens, uint8_t* flags,
                      double* p_tok);
int32_t oracle_accept_stats(const void* draft, const void* target, int32_t dtype, const int32_t* teacher,
                            const float* conf_logits, const uint8_t* block_mask, int32_t N, int32_t gamma,
                            int32_t V, double w_ce, double w_l1, double w_conf, double* l1, double* accept_rate,
                            double* ce, double* bce, double* tau, double* sums);
int32_t oracle_accept_stats_markov(const void* backbone, const void* target, int32_t dtype, const int32_t* anchor,
                                   const uint16_t* A, const uint16_t* Bt, int32_t r, const int32_t* teacher,
                                   const float* conf_logits, const uint8_t* block_mask, int32_t N, int32_t gamma,
                                   int32_t V, double w_ce, double w_l1, double w_conf, double* l1,
                                   double* accept_rate, double* ce, double* bce, double* tau, double* sums);
int32_t oracle_accept_stats_backward(const void* draft, const void* target, int32_t dtype, const int32_t* teacher,
                                     const float* conf_logits, const uint8_t* block_mask, int32_t N,
                                     int32_t gamma, int32_t V, double w_ce, double w_l1, double w_conf,
                                     double scale, double* grad_draft, double* grad_conf);
int32_t oracle_select_width(const float* confidence, const float* cost, int32_t B, int32_t gamma,
                            int32_t* n_draft, double* expected);
}

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint32_t next_u32() {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return static_cast<uint32_t>(g_state >> 33);
}
float next_f(float scale) { return scale * (static_cast<float>(next_u32() % 20001) / 10000.0f - 1.0f); }

uint16_t bf16_of(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return static_cast<uint16_t>(u >> 16);
}

// Logits of one dtype (1 = bf16, 2 = fp32): V values per row, some -inf, one
// NaN in row 1, row 2 empty when the batch has it.
std::vector<uint8_t> logits(int dtype, int rows, int V, bool specials) {
  std::vector<float> f(static_cast<size_t>(rows) * V);
  for (auto& x : f) x = next_f(4.0f);
  if (specials) {
    const float ninf = -std::numeric_limits<float>::infinity();
    for (int v = 0; v < V; v += 7) f[v] = ninf;
    if (rows > 1) f[static_cast<size_t>(V) + V / 2] = std::numeric_limits<float>::quiet_NaN();
    if (rows > 2)
      for (int v = 0; v < V; ++v) f[static_cast<size_t>(2) * V + v] = ninf;
  }
  std::vector<uint8_t> out;
  if (dtype == 1) {
    out.resize(f.size() * 2);
    for (size_t i = 0; i < f.size(); ++i) {
      const uint16_t h = bf16_of(f[i]);
      std::memcpy(&out[2 * i], &h, 2);
    }
  } else {
    out.resize(f.size() * 4);
    std::memcpy(out.data(), f.data(), out.size());
  }
  return out;
}

std::vector<uint16_t> weights(size_t n) {
  std::vector<uint16_t> w(n);
  for (auto& x : w) x = bf16_of(next_f(0.05f));
  return w;
}

int run(int dtype, int B, int gamma, int V, int r, int d, bool trunc, bool specials) {
  int bad = 0;
  const auto bb = logits(dtype, B * gamma, V, specials);
  const auto tg = logits(dtype, B * (gamma + 1), V, specials);
  const auto A = weights(static_cast<size_t>(V) * (r > 0 ? r : 1));
  const auto Bt = weights(static_cast<size_t>(V) * (r > 0 ? r : 1));
  const auto h = weights(static_cast<size_t>(B) * gamma * (d > 0 ? d : 1));
  const auto E = weights(static_cast<size_t>(V) * (d > 0 ? d : 1));
  std::vector<float> w(2 * (d > 0 ? d : 1));
  for (auto& x : w) x = next_f(0.1f);
  std::vector<int32_t> anchor(B), top_k(B), pos(B);
  std::vector<uint8_t> mode(B);
  std::vector<float> T(B), top_p(B);
  std::vector<uint32_t> req(B);
  for (int b = 0; b < B; ++b) {
    anchor[b] = static_cast<int32_t>(next_u32() % (V + 3)) - 1;  // some out of range (clamped)
    mode[b] = static_cast<uint8_t>(b % 3 != 0);
    T[b] = b % 5 == 4 ? 0.0f : 0.5f + 0.1f * static_cast<float>(b % 7);  // some invalid
    top_k[b] = trunc ? static_cast<int32_t>(next_u32() % 4) * (V / 4) : 0;
    top_p[b] = trunc ? 0.7f + 0.1f * static_cast<float>(b % 4) : 1.0f;
    req[b] = next_u32();
    pos[b] = static_cast<int32_t>(next_u32() % 1000);
  }
  const size_t BG = static_cast<size_t>(B) * gamma;
  std::vector<int32_t> draft(BG), forced(BG, -1);
  std::vector<double> qz(BG * V), qlse(BG), qthr(BG), qtok(BG), conf(BG);
  std::vector<uint8_t> fl(BG);
  if (BG > 1) forced[1] = static_cast<int32_t>(V - 1);
  bad |= oracle_markov_sample(bb.data(), dtype, anchor.data(), A.data(), Bt.data(), h.data(), E.data(),
                              w.data(), mode.data(), T.data(), top_k.data(), top_p.data(), req.data(),
                              pos.data(), 7, B, gamma, V, r, d, forced.data(), draft.data(), qz.data(),
                              qlse.data(), qthr.data(), qtok.data(), conf.data(), fl.data());
  std::vector<float> qz32(qz.begin(), qz.end()), ql32(qlse.begin(), qlse.end()), qt32(qthr.begin(), qthr.end()),
      qk32(qtok.begin(), qtok.end());
  std::vector<int32_t> nd(B), acc(B), out(static_cast<size_t>(B) * (gamma + 1));
  for (int b = 0; b < B; ++b) nd[b] = static_cast<int32_t>(b % (gamma + 2)) - 1;  // -1 .. gamma (clamped)
  std::vector<uint8_t> vfl(static_cast<size_t>(B) * (gamma + 1));
  std::vector<double> ptok(static_cast<size_t>(B) * (gamma + 1));
  bad |= oracle_verify(tg.data(), dtype, draft.data(), qz32.data(), ql32.data(), qt32.data(), qk32.data(),
                       nd.data(), mode.data(), T.data(), top_k.data(), top_p.data(), req.data(), pos.data(), 7,
                       B, gamma, V, acc.data(), out.data(), vfl.data(), ptok.data());
  // statistics on the same rows (draft = backbone, target = the first gamma target rows)
  std::vector<int32_t> teacher(BG);
  std::vector<float> cl(BG);
  std::vector<uint8_t> bm(B);
  for (size_t i = 0; i < BG; ++i) {
    teacher[i] = static_cast<int32_t>(next_u32() % (V + 2)) - 1;
    cl[i] = next_f(3.0f);
  }
  for (int b = 0; b < B; ++b) bm[b] = static_cast<uint8_t>(b % 2);
  std::vector<double> l1(BG), ar(BG), ce(BG), bce(BG), tau(B), sums(12), gd(BG * V), gc(BG);
  const auto tg_s = logits(dtype, B * gamma, V, specials);
  bad |= oracle_accept_stats(bb.data(), tg_s.data(), dtype, teacher.data(), cl.data(), bm.data(), B, gamma, V,
                             0.1, 0.9, 1.0, l1.data(), ar.data(), ce.data(), bce.data(), tau.data(), sums.data());
  bad |= oracle_accept_stats_markov(bb.data(), tg_s.data(), dtype, anchor.data(), A.data(), Bt.data(), r,
                                    teacher.data(), cl.data(), nullptr, B, gamma, V, 0.1, 0.9, 1.0, l1.data(),
                                    ar.data(), ce.data(), bce.data(), tau.data(), sums.data());
  bad |= oracle_accept_stats_backward(bb.data(), tg_s.data(), dtype, teacher.data(), cl.data(), bm.data(), B,
                                      gamma, V, 0.1, 0.9, 1.0, 0.5, gd.data(), gc.data());
  std::vector<float> cost(gamma + 2);
  for (int i = 0; i < gamma + 2; ++i) cost[i] = 1.0f + static_cast<float>(i);
  if (gamma + 2 > 2) cost[2] = -1.0f;  // a skipped width
  std::vector<int32_t> nw(B);
  std::vector<double> ex(B);
  std::vector<float> cf(BG);
  for (auto& x : cf) x = next_f(1.0f);
  if (!cf.empty()) cf[0] = std::numeric_limits<float>::quiet_NaN();
  bad |= oracle_select_width(cf.data(), cost.data(), B, gamma, nw.data(), ex.data());
  return bad;
}

}  // namespace

int main() {
  int bad = 0;
  uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, o[4];
  oracle_philox4x32_10(ctr, key, o);
  double acc = oracle_gumbel(3, 7, 11, 13, 5) + oracle_accept_uniform(3, 11, 13) +
               static_cast<double>(oracle_philox_word(3, 9, 11, 13, 2));
  for (int V : {1, 5, 16, 17, 300, 1031}) {
    std::vector<double> lw(V);
    for (auto& x : lw) x = next_f(5.0f);
    if (V > 3) lw[2] = -std::numeric_limits<double>::infinity();
    int32_t near = 0;
    acc += oracle_sample_three_level(lw.data(), V, 9, 1, 2, 3, 5, 0, &near);
    std::vector<uint8_t> kept(V);
    std::vector<double> z(V);
    double lse = 0, thr = 0;
    acc += oracle_policy_row(lw.data(), V, 0.7, V / 3, 0.8, 1, kept.data(), z.data(), &lse, &thr, &near);
    acc += oracle_policy_row(lw.data(), V, 1.0, 0, 1.0, 0, kept.data(), z.data(), &lse, &thr, &near);
  }
  bad |= run(2, 3, 4, 1031, 16, 8, true, true);
  bad |= run(1, 4, 5, 600, 32, 16, false, true);
  bad |= run(2, 2, 1, 1, 0, 0, false, false);
  bad |= run(1, 5, 3, 257, 16, 4, true, false);
  std::printf("oracle sanitizer run done (%d, %.3g)\n", bad, acc);
  return bad ? 1 : 0;
}
