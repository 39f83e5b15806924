// DSpark draft-and-verify round: plain fp64 CPU oracle.
//
// TEST INFRASTRUCTURE ONLY. This file is the slow, obviously-correct reference that the
// tests, the smoke check and the CPU-baseline leg of the benchmark compare the GPU library
// against. The GPU library never links, loads or calls it, and it shares no source with the
// GPU library (no headers, helpers, tables or constants).
//
// Sources cited (a reader has these pages):
//   [V41]     blog.javazero.top, "DeepSeek-V4.1 模型结构（6）：解码，DSpark"
//   [ZDS]     zdszero.github.io, spec_dspark (DSpark chapter of a speculative-decoding series)
//   [AIL]     ailearn.mscapital.top, "DSpark：不让大模型更聪明，而让它「吐字更快」"
//   [CSDN]    deepseek.csdn.net, DSpark walk-through (equations numbered (1)-(12))
//
// Every quantity is computed from its plain definition, in double precision, one request at a
// time, with no blocking, fusion or reordering beyond what the definition states. Where the
// pages leave a step open, the reading taken is stated at that step.
//
// Inputs arrive in the same bit patterns the GPU library gets: fp32 logits, bf16 weights
// (uint16 bit patterns, widened exactly to double here), fp32 uniforms.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

extern "C" {

// Plan modes (numbering is part of the shared interface; see the public header of the library).
enum { ORACLE_FULL_VERIFY = 0, ORACLE_EARLY_STOP = 1, ORACLE_FULL_PATH = 2, ORACLE_LAGGED_TOPK = 3 };

// Per-request verify flag bits.
enum { ORACLE_FLAG_NONFINITE = 1u, ORACLE_FLAG_ZERO_RESIDUAL = 2u };

}  // extern "C"

namespace {

double bf16_to_double(uint16_t bits) {
  uint32_t u = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

// Runs f(i) for i in [0, n) on `threads` worker threads (0 = all hardware threads).
template <class F>
void parallel_for(int64_t n, int threads, F f) {
  if (n <= 0) return;
  if (threads <= 0) threads = static_cast<int>(std::thread::hardware_concurrency());
  if (threads <= 0) threads = 1;
  if (threads > n) threads = static_cast<int>(n);
  if (threads == 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::atomic<int64_t> next(0);
  std::vector<std::thread> pool;
  pool.reserve(threads);
  for (int t = 0; t < threads; ++t)
    pool.emplace_back([&]() {
      for (int64_t i = next++; i < n; i = next++) f(i);
    });
  for (auto& th : pool) th.join();
}

// Softmax of fp32 logits in double: p_v = exp(L_v - m) / sum_u exp(L_u - m), m = max L.
// Returns log-sum-exp = m + log(sum). [V41] "Markov head", eq. (4): every position is one
// ordinary softmax, so the exact per-token probability q(x_k) is available.
double softmax_fp64(const float* logits, int V, std::vector<double>& p) {
  p.assign(V, 0.0);
  double m = -std::numeric_limits<double>::infinity();
  for (int v = 0; v < V; ++v) m = std::max(m, static_cast<double>(logits[v]));
  double z = 0.0;
  for (int v = 0; v < V; ++v) {
    p[v] = std::exp(static_cast<double>(logits[v]) - m);
    z += p[v];
  }
  for (int v = 0; v < V; ++v) p[v] /= z;
  return m + std::log(z);
}

// Inverse-CDF draw over token ids in ascending order: the first v with CDF(v) > u.
// Reading: the pages fix only the distribution a draw must follow; the oracle fixes the rule
// "ascending token id, strict >, u in [0,1)" so that results are reproducible bit for bit.
// If rounding leaves no edge above u, the last token with positive probability is taken.
// *margin receives the distance from u to the nearer edge of the chosen token's interval.
int32_t inverse_cdf(const std::vector<double>& p, double u, double* margin) {
  double cdf = 0.0;
  int32_t last_positive = -1;
  for (size_t v = 0; v < p.size(); ++v) {
    const double lo = cdf;
    cdf += p[v];
    if (p[v] > 0.0) last_positive = static_cast<int32_t>(v);
    if (cdf > u) {
      *margin = std::min(u - lo, cdf - u);
      return static_cast<int32_t>(v);
    }
  }
  *margin = 0.0;
  return last_positive >= 0 ? last_positive : 0;
}

// Markov bias of eq. (5): B(prev, v) = W1[prev] . W2[:, v], with W2 stored token-major
// (W2t[v][i] = W2[i][v], the layout of a Linear(r, V) weight). [V41] "Markov head", eq. (5);
// [ZDS] "在 SGLang 里" (markov_w1 = Embedding(V, r), markov_w2 = Linear(r, V)).
void markov_bias_fp64(const uint16_t* W1, const uint16_t* W2t, int V, int r, int32_t prev,
                      std::vector<double>& bias) {
  std::vector<double> e(r);
  for (int i = 0; i < r; ++i) e[i] = bf16_to_double(W1[static_cast<int64_t>(prev) * r + i]);
  bias.assign(V, 0.0);
  for (int v = 0; v < V; ++v) {
    const uint16_t* col = W2t + static_cast<int64_t>(v) * r;
    double s = 0.0;
    for (int i = 0; i < r; ++i) s += e[i] * bf16_to_double(col[i]);
    bias[v] = s;
  }
}

// Draft logits of one position: L_v = fp32(U_v + fp32(B(prev, v))).
// Reading: the official loop adds the bias in place into the fp32 logits tensor before
// sampling ([V41] "Markov head", the serial loop: logits[:, i].add_(bias)), so the draft
// distribution is the softmax of fp32 logits; the bias itself is summed exactly (fp64) and
// rounded once to fp32.
void draft_logits(const float* U_row, const uint16_t* W1, const uint16_t* W2t, int V, int r,
                  int32_t prev, std::vector<float>& L) {
  std::vector<double> bias;
  markov_bias_fp64(W1, W2t, V, r, prev, bias);
  L.assign(V, 0.0f);
  for (int v = 0; v < V; ++v) {
    const float b = static_cast<float>(bias[v]);
    L[v] = U_row[v] + b;  // one fp32 addition, round to nearest
  }
}

// Draft temperature: the official loop samples each position with a temperature ([V41] "Markov
// head", the serial loop: sample(logits, temperature)). Reading: the fp32 logits are multiplied,
// in fp32, by beta = fp32(1 / tau) before the softmax; tau = 1 (beta = 1) leaves them unchanged.
float temperature_beta(float tau) { return static_cast<float>(1.0 / static_cast<double>(tau)); }

void scale_logits(std::vector<float>& L, float beta) {
  if (beta == 1.0f) return;
  for (float& x : L) x = x * beta;  // one fp32 multiplication, round to nearest
}

// Greedy draft (the deployed recipe drafts greedily: [V41] / [AIL] V4 recipe,
// draft_sample_method "greedy"): the token with the largest logit, the smallest id among equal
// maxima; the draft distribution is the point mass on it. *gap receives the distance from the
// largest logit to the largest logit of any other token (0 on a tie).
int32_t greedy_token(const std::vector<float>& L, double* gap) {
  int32_t best = 0;
  for (size_t v = 1; v < L.size(); ++v)
    if (L[v] > L[best]) best = static_cast<int32_t>(v);
  double second = -std::numeric_limits<double>::infinity();
  for (size_t v = 0; v < L.size(); ++v)
    if (static_cast<int32_t>(v) != best) second = std::max(second, static_cast<double>(L[v]));
  *gap = static_cast<double>(L[best]) - second;
  return best;
}

// RNN head, eq. (6) ([CSDN] 4.2 "两种串行头"; [AIL] "RNN 头（可选）"; [V41] "Markov head", the
// smaller-RNN alternative the paper tried): a recurrent state summarises the block's prefix.
// Step k concatenates z_k = [s_{k-1}; W1[x_{k-1}]; h_k] and applies a GRU-like gated update
//   s_k = sigma(W_g z_k) * s_{k-1} + (1 - sigma(W_g z_k)) * tanh(W_c z_k)   (elementwise),
// and the bias of position k is B_k = W2^T tanh(W_o z_k), i.e. B_k(v) = sum_j W2[j][v] e_k[j]
// with e_k = tanh(W_o z_k).
// Readings (the pages fix none of these): the state has r components, the rank of W1 and W2, so
// that e_k feeds W2 directly; s_0 = 0 at the start of every block (the state covers the prefix
// inside the block, whose first conditioning token is the anchor); eq. (6) has no bias terms;
// W_g, W_c and W_o are stacked by rows into one bf16 matrix Wgco [3r][2r + d] (rows 0..r-1 W_g,
// r..2r-1 W_c, 2r..3r-1 W_o) whose columns follow z's order (state, embedding, hidden state);
// h_k is the backbone hidden state of position k, the one the confidence head reads. All of it
// in fp64; the bias is rounded once to fp32 and added to the fp32 U as for the Markov head.
void rnn_update(const uint16_t* Wgco, const uint16_t* W1, const uint16_t* h_row, int r, int d,
                int32_t x_prev, const std::vector<double>& s_prev, std::vector<double>& s_next,
                std::vector<double>& e) {
  const int nz = 2 * r + d;
  std::vector<double> z(nz);
  for (int i = 0; i < r; ++i) z[i] = s_prev[i];
  for (int i = 0; i < r; ++i) z[r + i] = bf16_to_double(W1[static_cast<int64_t>(x_prev) * r + i]);
  for (int i = 0; i < d; ++i) z[2 * r + i] = bf16_to_double(h_row[i]);
  auto row_dot = [&](int row) {
    const uint16_t* w = Wgco + static_cast<int64_t>(row) * nz;
    double a = 0.0;
    for (int i = 0; i < nz; ++i) a += bf16_to_double(w[i]) * z[i];
    return a;
  };
  s_next.assign(r, 0.0);
  e.assign(r, 0.0);
  for (int j = 0; j < r; ++j) {
    const double gate = 1.0 / (1.0 + std::exp(-row_dot(j)));
    const double cand = std::tanh(row_dot(r + j));
    s_next[j] = gate * s_prev[j] + (1.0 - gate) * cand;
    e[j] = std::tanh(row_dot(2 * r + j));
  }
}

// Draft logits of one position under the RNN head: L_v = fp32(U_v + fp32(sum_j W2[j][v] e[j])).
void rnn_draft_logits(const float* U_row, const uint16_t* W2t, int V, int r,
                      const std::vector<double>& e, std::vector<float>& Lr) {
  Lr.assign(V, 0.0f);
  for (int v = 0; v < V; ++v) {
    const uint16_t* col = W2t + static_cast<int64_t>(v) * r;
    double bias = 0.0;
    for (int j = 0; j < r; ++j) bias += bf16_to_double(col[j]) * e[j];
    Lr[v] = U_row[v] + static_cast<float>(bias);
  }
}

double logsumexp_fp32_row(const float* row, int V) {
  double m = -std::numeric_limits<double>::infinity();
  for (int v = 0; v < V; ++v) m = std::max(m, static_cast<double>(row[v]));
  double z = 0.0;
  for (int v = 0; v < V; ++v) z += std::exp(static_cast<double>(row[v]) - m);
  return m + std::log(z);
}

// a_{r,j} = prod_{i<=j} c_{r,i}, sequential product in double of the fp32 confidences.
// [V41] "confidence head": prefix survival a_j; [CSDN] 5.3, a_{r,j} = a_{r,j-1} c_{r,j}.
void survival(const float* conf, int R, int gamma, std::vector<double>& a) {
  a.assign(static_cast<size_t>(R) * gamma, 0.0);
  for (int rq = 0; rq < R; ++rq) {
    double prod = 1.0;
    for (int j = 0; j < gamma; ++j) {
      prod *= static_cast<double>(conf[rq * gamma + j]);
      a[rq * gamma + j] = prod;
    }
  }
}

struct Candidate {
  double a;
  int32_t req, pos;  // pos is 0-based: candidate (req, pos) extends request req to length pos+1
};

// All (request, position) candidates sorted by survival, descending; ties broken by request
// then position, ascending (reading: a deterministic tie-break that keeps every request's
// admitted set a prefix even when c = 1). [V41] "贪心就能解"; [CSDN] 5.3.
std::vector<Candidate> sorted_candidates(const std::vector<double>& a, int R, int gamma) {
  std::vector<Candidate> c;
  c.reserve(static_cast<size_t>(R) * gamma);
  for (int rq = 0; rq < R; ++rq)
    for (int j = 0; j < gamma; ++j) c.push_back({a[rq * gamma + j], rq, j});
  std::sort(c.begin(), c.end(), [](const Candidate& x, const Candidate& y) {
    if (x.a != y.a) return x.a > y.a;
    if (x.req != y.req) return x.req < y.req;
    return x.pos < y.pos;
  });
  return c;
}

// The admission path: theta[i] = tau_i * SPS(R + i), tau_0 = R, tau_i = tau_{i-1} + a_(i).
// [V41] "目标函数": B = sum(1 + l_r), tau = sum(1 + sum_{j<=l_r} a_{r,j}), Theta = tau SPS(B).
// Reading: SPS is indexed by the total number of verified tokens B (not by requests).
void admission_path(const std::vector<Candidate>& cand, int R, const double* sps,
                    std::vector<double>& tau, std::vector<double>& theta) {
  const size_t n = cand.size();
  tau.assign(n + 1, 0.0);
  theta.assign(n + 1, 0.0);
  tau[0] = static_cast<double>(R);
  theta[0] = tau[0] * sps[R];
  for (size_t i = 1; i <= n; ++i) {
    tau[i] = tau[i - 1] + cand[i - 1].a;
    theta[i] = tau[i] * sps[R + i];
  }
}

// Algorithm 1: admit in path order while Theta rises; stop at the first candidate whose
// admission would not raise it (strict >). [V41] "贪心就能解" (once Theta stops rising, stop);
// [CSDN] 5.3.
int64_t early_stop_count(const std::vector<double>& theta, double* margin) {
  const int64_t n = static_cast<int64_t>(theta.size()) - 1;
  int64_t k = 0;
  double mg = std::numeric_limits<double>::infinity();
  while (k < n) {
    const double rel = std::fabs(theta[k + 1] - theta[k]) / std::fabs(theta[k]);
    mg = std::min(mg, rel);
    if (!(theta[k + 1] > theta[k])) break;
    ++k;
  }
  if (margin) *margin = mg;
  return k;
}

// Full-path search: the first maximiser of Theta over the whole path. [AIL] 05 (the
// production variant removes early stop and searches the whole path); [CSDN] 8.
int64_t full_path_count(const std::vector<double>& theta, double* margin) {
  int64_t best = 0;
  for (int64_t i = 1; i < static_cast<int64_t>(theta.size()); ++i)
    if (theta[i] > theta[best]) best = i;
  double mg = std::numeric_limits<double>::infinity();
  for (int64_t i = 0; i < static_cast<int64_t>(theta.size()); ++i)
    if (i != best) mg = std::min(mg, std::fabs(theta[best] - theta[i]) / std::fabs(theta[best]));
  if (margin) *margin = mg;
  return best;
}

}  // namespace

extern "C" {

// Semi-autoregressive Markov-head draft.
// [V41] "Markov head" eqs. (4), (5) and the serial loop: the base logits U_k are given; for
// k = 1..gamma the previous token (x_0 = anchor) selects W1[x_{k-1}], the bias W1[x_{k-1}] W2
// is added to U_k, and x_k is drawn from the softmax; the same W1, W2 serve every position.
// [CSDN] 4.1-4.2, eq. (4): local softmax per position, exact q(x_k).
//
// Layouts: U [B][gamma][V] fp32; W1, W2t [V][r] bf16 bits; anchor [B]; uniforms
// [B][gamma+1][3] fp32 (component 0 of slot k-1 draws position k).
// force_tokens (nullable) [B][gamma]: when given, tokens[] still receives the draw at each
// position, but the token that conditions the next position and whose probability goes to
// q[] is force_tokens[b][k-1] (teacher forcing, used to compare step by step).
// Outputs: tokens [B][gamma], q [B][gamma] = p_k(x_k), lse [B][gamma] = log sum exp L_k,
// logits (nullable) [B][gamma][V] = L_k, margin (nullable) [B][gamma] = distance of u to the
// nearer CDF edge of the drawn token.
// Returns 0, or 2 for a bad shape, 8 for an out-of-range token id.
// With draft options: temperature tau > 0 draws from softmax(beta L), beta = fp32(1 / tau), and
// q / lse refer to that distribution; greedy != 0 drafts the first maximal logit, q = 1 (0 for a
// forced token that is not it), lse = the largest logit, and margin receives the gap between the
// two largest logits instead.
int oracle_markov_draft_opts(int B, int gamma, int V, int r, const float* U, const uint16_t* W1,
                             const uint16_t* W2t, const int32_t* anchor, const float* uniforms,
                             const int32_t* force_tokens, float temperature, int greedy,
                             int32_t* tokens, float* q, double* lse, float* logits, double* margin,
                             int threads) {
  if (B < 0 || gamma < 1 || V < 2 || r < 1) return 2;
  if (!greedy && !(temperature > 0.0f && std::isfinite(temperature))) return 2;
  const float beta = greedy ? 1.0f : temperature_beta(temperature);
  for (int b = 0; b < B; ++b) {
    if (anchor[b] < 0 || anchor[b] >= V) return 8;
    if (force_tokens)
      for (int k = 0; k < gamma; ++k)
        if (force_tokens[b * gamma + k] < 0 || force_tokens[b * gamma + k] >= V) return 8;
  }
  parallel_for(B, threads, [&](int64_t b) {
    std::vector<float> L;
    std::vector<double> p;
    int32_t prev = anchor[b];
    for (int k = 0; k < gamma; ++k) {
      const int64_t bk = b * gamma + k;
      draft_logits(U + bk * V, W1, W2t, V, r, prev, L);
      if (logits) std::memcpy(logits + bk * V, L.data(), sizeof(float) * V);
      double mg = 0.0;
      int32_t x, cond;
      if (greedy) {
        x = greedy_token(L, &mg);
        cond = force_tokens ? force_tokens[bk] : x;
        q[bk] = (cond == x) ? 1.0f : 0.0f;
        lse[bk] = static_cast<double>(L[x]);
      } else {
        scale_logits(L, beta);
        const double l = softmax_fp64(L.data(), V, p);
        const double u = static_cast<double>(uniforms[(b * (gamma + 1) + k) * 3 + 0]);
        x = inverse_cdf(p, u, &mg);
        cond = force_tokens ? force_tokens[bk] : x;
        q[bk] = static_cast<float>(p[cond]);
        lse[bk] = l;
      }
      tokens[bk] = x;
      if (margin) margin[bk] = mg;
      prev = cond;
    }
  });
  return 0;
}

int oracle_markov_draft(int B, int gamma, int V, int r, const float* U, const uint16_t* W1,
                        const uint16_t* W2t, const int32_t* anchor, const float* uniforms,
                        const int32_t* force_tokens, int32_t* tokens, float* q, double* lse,
                        float* logits, double* margin, int threads) {
  return oracle_markov_draft_opts(B, gamma, V, r, U, W1, W2t, anchor, uniforms, force_tokens, 1.0f,
                                  0, tokens, q, lse, logits, margin, threads);
}

// Confidence head, eq. (7), with the STS temperature applied at inference:
// z = w . [h_k ; W1[x_{k-1}]] (no bias term: eq. (7) has none), c_k = sigmoid(z / T_k).
// [V41] "confidence head" eq. (7) (the input holds x_{k-1}, not x_k; x_0 = anchor);
// [ZDS] "在 SGLang 里" (Linear(h + r, 1), sigmoid(raw / T) with the STS temperature).
// Layouts: h [B][gamma][d] bf16; w [d + r] bf16 (first d entries multiply h_k); T [gamma];
// tokens [B][gamma] (the drafted tokens; x_{k-1} = tokens[b][k-2] for k >= 2).
// Outputs: conf [B][gamma] fp32; z_out (nullable) [B][gamma] = the pre-sigmoid value.
int oracle_confidence(int B, int gamma, int V, int r, int d, const uint16_t* h, const uint16_t* W1,
                      const uint16_t* w, const float* T, const int32_t* anchor,
                      const int32_t* tokens, float* conf, double* z_out, int threads) {
  if (B < 0 || gamma < 1 || V < 2 || r < 1 || d < 1) return 2;
  for (int b = 0; b < B; ++b) {
    if (anchor[b] < 0 || anchor[b] >= V) return 8;
    for (int k = 0; k < gamma; ++k)
      if (tokens[b * gamma + k] < 0 || tokens[b * gamma + k] >= V) return 8;
  }
  parallel_for(static_cast<int64_t>(B) * gamma, threads, [&](int64_t bk) {
    const int64_t b = bk / gamma, k = bk % gamma;
    const int32_t prev = (k == 0) ? anchor[b] : tokens[b * gamma + k - 1];
    double z = 0.0;
    for (int i = 0; i < d; ++i) z += bf16_to_double(w[i]) * bf16_to_double(h[bk * d + i]);
    for (int i = 0; i < r; ++i)
      z += bf16_to_double(w[d + i]) * bf16_to_double(W1[static_cast<int64_t>(prev) * r + i]);
    const double c = 1.0 / (1.0 + std::exp(-z / static_cast<double>(T[k])));
    conf[bk] = static_cast<float>(c);
    if (z_out) z_out[bk] = z;
  });
  return 0;
}

// Hardware-aware verify planner. [V41] "调度器" ("目标函数", "贪心就能解", "按置信度截断在什么
// 条件下不改变分布"); [ZDS] "调度" and "在 SGLang 里" (lengths 1 + l_r in [1, gamma+1], a flat
// SPS table degrades to full verify, confidence relayed through a ring with lag 2, no lag
// without overlap); [CSDN] 5.3, 5.4, 8.
//
// Modes: FULL_VERIFY admits everything (l_r = gamma); EARLY_STOP is Algorithm 1;
// FULL_PATH takes the first maximiser of Theta over the whole path (the retrospective search
// that is biased when applied to the current round, Appendix A); LAGGED_TOPK takes the
// capacity K from the confidences of two rounds back (full-path search on those), then admits
// the top K - R candidates of the current round's own order.
// Ring (LAGGED_TOPK only) [2][B][gamma]: slot (round % 2) holds round-2's confidences; it is
// read first, then overwritten with this round's. Reading for the warm-up: rounds 0 and 1
// have no lagged confidences and use EARLY_STOP (no lag without overlap).
// Outputs: draft_len [B] (l_r in [0, gamma]); row_offsets [B+1], the exclusive scan of
// (1 + l_r); stats[4] = {B_tot, tau, Theta, K} at the admitted point (K = capacity for
// LAGGED_TOPK after warm-up, else B_tot); margin (nullable) = smallest relative Theta gap
// among the comparisons that decided the admission count; theta_path (nullable) [B*gamma+1]
// = Theta_i along this round's admission path.
// sps [sps_len] fp64: sps[n] = steps per second with n verified tokens; sps_len must exceed
// B * (gamma + 1). Returns 0, 2 (shape), 5 (SPS table too short), 7 (bad mode / missing ring).
int oracle_plan(int B, int gamma, const float* conf, const double* sps, int sps_len, int mode,
                float* ring, int round_index, int32_t* draft_len, int32_t* row_offsets,
                double* stats, double* margin, double* theta_path) {
  if (B < 1 || gamma < 1) return 2;
  if (sps_len < B * (gamma + 1) + 1) return 5;
  if (mode < ORACLE_FULL_VERIFY || mode > ORACLE_LAGGED_TOPK) return 7;
  if (mode == ORACLE_LAGGED_TOPK && ring == nullptr) return 7;
  if (mode != ORACLE_FULL_VERIFY && conf == nullptr) return 7;

  const int64_t n = static_cast<int64_t>(B) * gamma;
  std::vector<double> a, tau, theta;
  std::vector<Candidate> cand;
  int64_t admit = 0;
  double mg = std::numeric_limits<double>::infinity();
  double capacity = 0.0;
  bool lagged = false;

  if (mode == ORACLE_FULL_VERIFY) {
    // Static mode: no planner, every drafted token is verified. Without confidences the
    // survivals (and so tau and Theta) are unknown and reported as NaN.
    admit = n;
    if (conf) {
      survival(conf, B, gamma, a);
      cand = sorted_candidates(a, B, gamma);
    } else {
      for (int rq = 0; rq < B; ++rq)
        for (int j = 0; j < gamma; ++j)
          cand.push_back({std::numeric_limits<double>::quiet_NaN(), rq, j});
    }
    admission_path(cand, B, sps, tau, theta);
  } else {
    survival(conf, B, gamma, a);
    cand = sorted_candidates(a, B, gamma);
    admission_path(cand, B, sps, tau, theta);
    if (mode == ORACLE_EARLY_STOP || (mode == ORACLE_LAGGED_TOPK && round_index < 2)) {
      admit = early_stop_count(theta, &mg);
    } else if (mode == ORACLE_FULL_PATH) {
      admit = full_path_count(theta, &mg);
    } else {
      // Capacity from the confidences of two rounds back: [V41] last paragraph before
      // "训练"; [CSDN] 8: K from two steps back, order from the current survivals.
      const float* lag = ring + static_cast<int64_t>(round_index % 2) * n;
      std::vector<double> a_lag, tau_lag, theta_lag;
      survival(lag, B, gamma, a_lag);
      std::vector<Candidate> cand_lag = sorted_candidates(a_lag, B, gamma);
      admission_path(cand_lag, B, sps, tau_lag, theta_lag);
      const int64_t k_lag = full_path_count(theta_lag, &mg);
      admit = std::min<int64_t>(k_lag, n);
      capacity = static_cast<double>(B) + static_cast<double>(k_lag);
      lagged = true;
    }
  }
  if (mode == ORACLE_LAGGED_TOPK)
    std::memcpy(ring + static_cast<int64_t>(round_index % 2) * n, conf, sizeof(float) * n);

  for (int rq = 0; rq < B; ++rq) draft_len[rq] = 0;
  for (int64_t i = 0; i < admit; ++i) draft_len[cand[i].req] += 1;
  row_offsets[0] = 0;
  for (int rq = 0; rq < B; ++rq) row_offsets[rq + 1] = row_offsets[rq] + 1 + draft_len[rq];

  const double b_tot = static_cast<double>(B) + static_cast<double>(admit);
  if (stats) {
    stats[0] = b_tot;
    stats[1] = tau[admit];
    stats[2] = theta[admit];
    stats[3] = lagged ? capacity : b_tot;
  }
  if (margin) *margin = mg;
  if (theta_path)
    for (size_t i = 0; i < theta.size(); ++i) theta_path[i] = theta[i];
  return 0;
}

// Lossless verify with the standard rejection rule.
// [V41] "投机解码：让小的先猜，大的一次验一串" (accept x ~ q with probability min(1, p(x)/q(x));
// on reject resample from norm(max(0, p - q)); check left to right, the first reject voids the
// rest; at least one token per round: the bonus from the target when all are accepted, the
// resample otherwise; that token is the next anchor); [AIL] 02 (worked A/B example, the
// correction distribution); [CSDN] 2.1.
//
// Row layout: the rows of request b are target[row_offsets[b] .. row_offsets[b] + l_b], row j
// holding the target logits of position j + 1 (row l_b is the bonus position).
// Accept test at position k (reading, equivalent to u < min(1, p_t/q) with u in [0,1)):
//   u[b][k-1][1] * q[b][k-1] < p_t(x_k), all in double, q as given (fp32).
// On the first reject at position k the draft distribution p_d of position k is recomputed
// from U, W1, W2 and the previous token (same definition as the draft), and the next token is
// drawn from max(0, p_t - p_d) / sum with u[b][k-1][2]; if that mass is not positive
// (impossible in exact arithmetic after a reject) the draw falls back to p_t and flag bit 2 is
// set. When every verified token is accepted, the bonus is drawn from p_t of row l_b with
// u[b][l_b][2]. A row whose log-sum-exp is not finite sets flag bit 1.
// Outputs: accept_len [B]; next_token [B]; beta_emit (nullable) [B] = sum_v min(p_t, p_d) at a
// residual emission row, -1 at a bonus row; flags (nullable) [B]; accept_margin (nullable)
// [B][gamma] = |u - p_t/q| for each tested position with p_t/q < 1 (+inf otherwise);
// emit_margin (nullable) [B]; resid_mass (nullable) [B] = sum_v max(0, p_t - p_d) (-1 at bonus).
// With draft options (as for the draft): the draft distribution p_d whose residual is drawn from
// is softmax(beta L) at temperature tau, or, for a greedy draft, the point mass on the drafted
// token (q = 1 in the accept test).
}  // extern "C"

namespace {

// The verify of one batch, given the draft distribution of a rejected position: draft_pd(b, k,
// pd) fills p_d of request b at its 1-based position k (the draft head's own definition). The
// accept test, the residual, the bonus and the flags are those stated above.
template <class DraftPd>
void verify_core(int B, int gamma, int V, const float* target, const int32_t* row_offsets,
                 const int32_t* draft_len, const int32_t* tokens, const float* q,
                 const float* uniforms, int greedy, DraftPd draft_pd, int32_t* accept_len,
                 int32_t* next_token, float* beta_emit, uint32_t* flags, double* accept_margin,
                 double* emit_margin, double* resid_mass, int threads) {
  const double inf = std::numeric_limits<double>::infinity();
  parallel_for(B, threads, [&](int64_t b) {
    const int ell = draft_len[b];
    const int64_t off = row_offsets[b];
    uint32_t fl = 0;
    int accepted = 0;
    int reject_pos = -1;  // 1-based position of the first reject
    if (accept_margin)
      for (int k = 0; k < gamma; ++k) accept_margin[b * gamma + k] = inf;
    for (int k = 1; k <= ell; ++k) {
      const float* row = target + (off + k - 1) * static_cast<int64_t>(V);
      const double l = logsumexp_fp32_row(row, V);
      if (!std::isfinite(l)) fl |= ORACLE_FLAG_NONFINITE;
      const int32_t x = tokens[b * gamma + k - 1];
      const double pt = std::exp(static_cast<double>(row[x]) - l);
      const double u = static_cast<double>(uniforms[(b * (gamma + 1) + (k - 1)) * 3 + 1]);
      const double qk = static_cast<double>(q[b * gamma + k - 1]);
      if (accept_margin && pt < qk) accept_margin[b * gamma + k - 1] = std::fabs(u - pt / qk);
      if (u * qk < pt) {
        ++accepted;
      } else {
        reject_pos = k;
        break;
      }
    }
    std::vector<double> pt, pd, w;
    double mg = 0.0;
    int32_t tok = 0;
    if (reject_pos < 0) {
      // Bonus token from the target at position ell + 1.
      const float* row = target + (off + ell) * static_cast<int64_t>(V);
      const double l = softmax_fp64(row, V, pt);
      if (!std::isfinite(l)) fl |= ORACLE_FLAG_NONFINITE;
      const double u = static_cast<double>(uniforms[(b * (gamma + 1) + ell) * 3 + 2]);
      tok = inverse_cdf(pt, u, &mg);
      if (beta_emit) beta_emit[b] = -1.0f;
      if (resid_mass) resid_mass[b] = -1.0;
    } else {
      const int k = reject_pos;
      const float* row = target + (off + k - 1) * static_cast<int64_t>(V);
      const double lt = softmax_fp64(row, V, pt);
      if (!std::isfinite(lt)) fl |= ORACLE_FLAG_NONFINITE;
      if (greedy) {
        pd.assign(V, 0.0);
        pd[tokens[b * gamma + k - 1]] = 1.0;
      } else {
        draft_pd(b, k, pd);
      }
      w.assign(V, 0.0);
      double mass = 0.0, beta = 0.0;
      for (int v = 0; v < V; ++v) {
        w[v] = std::max(0.0, pt[v] - pd[v]);
        mass += w[v];
        beta += std::min(pt[v], pd[v]);
      }
      const double u = static_cast<double>(uniforms[(b * (gamma + 1) + (k - 1)) * 3 + 2]);
      if (mass > 0.0 && std::isfinite(mass)) {
        for (int v = 0; v < V; ++v) w[v] /= mass;
        tok = inverse_cdf(w, u, &mg);
      } else {
        fl |= ORACLE_FLAG_ZERO_RESIDUAL;
        tok = inverse_cdf(pt, u, &mg);
      }
      if (beta_emit) beta_emit[b] = static_cast<float>(beta);
      if (resid_mass) resid_mass[b] = mass;
    }
    accept_len[b] = accepted;
    next_token[b] = tok;
    if (flags) flags[b] = fl;
    if (emit_margin) emit_margin[b] = mg;
  });
}

}  // namespace

extern "C" {

int oracle_verify_opts(int B, int gamma, int V, int r, const float* target,
                       const int32_t* row_offsets, const int32_t* draft_len, const float* U,
                       const uint16_t* W1, const uint16_t* W2t, const int32_t* anchor,
                       const int32_t* tokens, const float* q, const float* uniforms,
                       float temperature, int greedy, int32_t* accept_len, int32_t* next_token,
                       float* beta_emit, uint32_t* flags, double* accept_margin,
                       double* emit_margin, double* resid_mass, int threads) {
  if (B < 0 || gamma < 1 || V < 2 || r < 1) return 2;
  if (!greedy && !(temperature > 0.0f && std::isfinite(temperature))) return 2;
  const float beta = greedy ? 1.0f : temperature_beta(temperature);
  for (int b = 0; b < B; ++b) {
    if (draft_len[b] < 0 || draft_len[b] > gamma) return 2;
    if (row_offsets[b + 1] - row_offsets[b] != draft_len[b] + 1) return 2;
    if (anchor[b] < 0 || anchor[b] >= V) return 8;
    for (int k = 0; k < gamma; ++k)
      if (tokens[b * gamma + k] < 0 || tokens[b * gamma + k] >= V) return 8;
  }
  // Markov head: p_d of position k from U, W1, W2 and the previous token.
  auto markov_pd = [&](int64_t b, int k, std::vector<double>& pd) {
    const int32_t prev = (k == 1) ? anchor[b] : tokens[b * gamma + k - 2];
    std::vector<float> L;
    draft_logits(U + (b * gamma + k - 1) * static_cast<int64_t>(V), W1, W2t, V, r, prev, L);
    scale_logits(L, beta);
    softmax_fp64(L.data(), V, pd);
  };
  verify_core(B, gamma, V, target, row_offsets, draft_len, tokens, q, uniforms, greedy, markov_pd,
              accept_len, next_token, beta_emit, flags, accept_margin, emit_margin, resid_mass,
              threads);
  return 0;
}

int oracle_verify(int B, int gamma, int V, int r, const float* target, const int32_t* row_offsets,
                  const int32_t* draft_len, const float* U, const uint16_t* W1,
                  const uint16_t* W2t, const int32_t* anchor, const int32_t* tokens,
                  const float* q, const float* uniforms, int32_t* accept_len,
                  int32_t* next_token, float* beta_emit, uint32_t* flags, double* accept_margin,
                  double* emit_margin, double* resid_mass, int threads) {
  return oracle_verify_opts(B, gamma, V, r, target, row_offsets, draft_len, U, W1, W2t, anchor,
                            tokens, q, uniforms, 1.0f, 0, accept_len, next_token, beta_emit, flags,
                            accept_margin, emit_margin, resid_mass, threads);
}

// RNN-head draft, eqs. (4) and (6): per request, s_0 = 0 and x_0 = the anchor; at position k
// the state update of eq. (6) on z_k = [s_{k-1}; W1[x_{k-1}]; h_k] gives s_k and e_k =
// tanh(W_o z_k); L_k = fp32(U_k + fp32(W2^T e_k)); x_k is drawn as in the Markov draft (same
// uniforms, temperature, greedy rule and forcing); the conditioning token x_k (drawn or forced)
// feeds position k + 1. h [B][gamma][d] bf16 bits; Wgco [3r][2r + d] bf16 bits (see
// rnn_update). Outputs as oracle_markov_draft_opts, plus e_out (nullable) [B][gamma][r] =
// e_k in fp64.
int oracle_rnn_draft(int B, int gamma, int V, int r, int d, const float* U, const uint16_t* W1,
                     const uint16_t* W2t, const uint16_t* Wgco, const uint16_t* h,
                     const int32_t* anchor, const float* uniforms, const int32_t* force_tokens,
                     float temperature, int greedy, int32_t* tokens, float* q, double* lse,
                     float* logits, double* margin, double* e_out, int threads) {
  if (B < 0 || gamma < 1 || V < 2 || r < 1 || d < 0) return 2;
  if (!greedy && !(temperature > 0.0f && std::isfinite(temperature))) return 2;
  const float beta = greedy ? 1.0f : temperature_beta(temperature);
  for (int b = 0; b < B; ++b) {
    if (anchor[b] < 0 || anchor[b] >= V) return 8;
    if (force_tokens)
      for (int k = 0; k < gamma; ++k)
        if (force_tokens[b * gamma + k] < 0 || force_tokens[b * gamma + k] >= V) return 8;
  }
  parallel_for(B, threads, [&](int64_t b) {
    std::vector<double> state(r, 0.0), next_state, e, p;
    std::vector<float> Lr;
    int32_t x_prev = anchor[b];
    for (int k = 0; k < gamma; ++k) {
      const int64_t bk = b * gamma + k;
      rnn_update(Wgco, W1, h + bk * static_cast<int64_t>(d), r, d, x_prev, state, next_state, e);
      state.swap(next_state);
      if (e_out)
        for (int j = 0; j < r; ++j) e_out[bk * r + j] = e[j];
      rnn_draft_logits(U + bk * V, W2t, V, r, e, Lr);
      if (logits) std::memcpy(logits + bk * V, Lr.data(), sizeof(float) * V);
      double mg = 0.0;
      int32_t x, x_cond;
      if (greedy) {
        x = greedy_token(Lr, &mg);
        x_cond = force_tokens ? force_tokens[bk] : x;
        q[bk] = (x_cond == x) ? 1.0f : 0.0f;
        lse[bk] = static_cast<double>(Lr[x]);
      } else {
        scale_logits(Lr, beta);
        const double l = softmax_fp64(Lr.data(), V, p);
        const double u = static_cast<double>(uniforms[(b * (gamma + 1) + k) * 3 + 0]);
        x = inverse_cdf(p, u, &mg);
        x_cond = force_tokens ? force_tokens[bk] : x;
        q[bk] = static_cast<float>(p[x_cond]);
        lse[bk] = l;
      }
      tokens[bk] = x;
      if (margin) margin[bk] = mg;
      x_prev = x_cond;
    }
  });
  return 0;
}

// Verify of an RNN-head draft: as oracle_verify_opts, with p_d of the rejected position k
// recomputed from eq. (6) by running the state from s_0 = 0 along the anchor and the drafted
// tokens x_1 .. x_{k-1}.
int oracle_rnn_verify(int B, int gamma, int V, int r, int d, const float* target,
                      const int32_t* row_offsets, const int32_t* draft_len, const float* U,
                      const uint16_t* W1, const uint16_t* W2t, const uint16_t* Wgco,
                      const uint16_t* h, const int32_t* anchor, const int32_t* tokens,
                      const float* q, const float* uniforms, float temperature, int greedy,
                      int32_t* accept_len, int32_t* next_token, float* beta_emit, uint32_t* flags,
                      double* accept_margin, double* emit_margin, double* resid_mass,
                      int threads) {
  if (B < 0 || gamma < 1 || V < 2 || r < 1 || d < 0) return 2;
  if (!greedy && !(temperature > 0.0f && std::isfinite(temperature))) return 2;
  const float beta = greedy ? 1.0f : temperature_beta(temperature);
  for (int b = 0; b < B; ++b) {
    if (draft_len[b] < 0 || draft_len[b] > gamma) return 2;
    if (row_offsets[b + 1] - row_offsets[b] != draft_len[b] + 1) return 2;
    if (anchor[b] < 0 || anchor[b] >= V) return 8;
    for (int k = 0; k < gamma; ++k)
      if (tokens[b * gamma + k] < 0 || tokens[b * gamma + k] >= V) return 8;
  }
  auto rnn_pd = [&](int64_t b, int k, std::vector<double>& pd) {
    std::vector<double> state(r, 0.0), next_state, e;
    int32_t x_prev = anchor[b];
    for (int i = 1; i <= k; ++i) {
      const int64_t bi = b * gamma + i - 1;
      rnn_update(Wgco, W1, h + bi * static_cast<int64_t>(d), r, d, x_prev, state, next_state, e);
      state.swap(next_state);
      x_prev = tokens[bi];
    }
    std::vector<float> Lr;
    rnn_draft_logits(U + (b * gamma + k - 1) * static_cast<int64_t>(V), W2t, V, r, e, Lr);
    scale_logits(Lr, beta);
    softmax_fp64(Lr.data(), V, pd);
  };
  verify_core(B, gamma, V, target, row_offsets, draft_len, tokens, q, uniforms, greedy, rnn_pd,
              accept_len, next_token, beta_emit, flags, accept_margin, emit_margin, resid_mass,
              threads);
  return 0;
}

}  // extern "C"

// ---- PCTree: tree drafting scored by the Markov head, and its lossless verify ----------------
//
// [ZDS] "后续工作" (PCTree): the single draft chain becomes a tree. The Markov head already
// scores every child token under a given parent token, so it picks the candidate children of
// each parent node directly, and the most likely paths are kept within a fixed verify budget;
// no retraining and no extra backbone pass. Readings taken where the page is silent:
//   - The backbone's base logits U_k of a position are shared by every node at that depth (the
//     backbone runs once); a node's token x scores the next depth's children by
//     softmax(fp32(U_k + fp32(W1[x] W2))) (eqs. (4), (5)), the root being the anchor.
//   - A node expands its c best children: the c largest fp32 logits, the smaller id first on a
//     tie.
//   - A node's path probability P is the product of the Markov probabilities along its path
//     (fp64). Depth 1 expands the root; depth k >= 2 expands the M nodes of depth k - 1 with the
//     largest P (key (-P, index), the index counting a depth's candidates parent by parent in
//     the expanded order and child by child in rank order).
//   - The verify budget N keeps the N candidates of all depths with the largest P (key (-P,
//     depth, index)). A child's P is at most its parent's and the key puts the parent first on a
//     tie, so the kept set is a tree.
namespace {

struct TreeCand {
  double P;        // path probability
  double q;        // the Markov probability of the token under its parent
  int depth;       // 1..gamma
  int idx;         // index within its depth's candidates
  int parent;      // position of the parent in `all` (-1: the root)
  int32_t token;
};

// The c largest logits of L (the smaller id first on a tie), and the smallest gap between two
// consecutive logits of the c + 1 largest (the decisions that fix the children and their order).
void top_children(const std::vector<float>& L, int c, std::vector<int32_t>& out, double* gap) {
  const int V = static_cast<int>(L.size());
  const int n = std::min(V, c + 1);
  std::vector<int32_t> ids(V);
  for (int v = 0; v < V; ++v) ids[v] = v;
  std::partial_sort(ids.begin(), ids.begin() + n, ids.end(), [&](int32_t a, int32_t b) {
    if (L[a] != L[b]) return L[a] > L[b];
    return a < b;
  });
  out.assign(ids.begin(), ids.begin() + c);
  for (int i = 0; i + 1 < n; ++i)
    *gap = std::min(*gap, static_cast<double>(L[ids[i]]) - static_cast<double>(L[ids[i + 1]]));
}

// Smallest relative gap between consecutive path probabilities of a ranked list among ranks
// 0 .. upto (so with upto = the number kept, the boundary with the first one left out counts).
void rank_gaps(const std::vector<double>& P, int upto, double* gap) {
  const int n = std::min<int>(static_cast<int>(P.size()), upto + 1);
  for (int i = 0; i + 1 < n; ++i)
    if (P[i] > 0.0) *gap = std::min(*gap, (P[i] - P[i + 1]) / P[i]);
}

}  // namespace

extern "C" {

// Tree draft. U [B][gamma][V] f32, W1/W2t bf16 [V][r], anchor [B]; c children a node, M nodes
// expanded a depth (depth >= 2), N nodes kept. Outputs per request, nodes in rank order (key
// (-P, depth, index)): node_token, node_depth (1..gamma), node_parent (rank of the parent node,
// -1 for the root) [B][N] int32; node_q (the token's Markov probability under its parent) and
// node_path (P) [B][N] f64. logit_margin / path_margin (nullable, [B]): the smallest logit gap
// among any expanded node's c + 1 largest logits, and the smallest relative gap between
// consecutive path probabilities in the depth rankings (up to the M-th) and the final ranking
// (up to the N-th). Returns 1 on bad sizes (1 <= M <= c <= V, 1 <= N <= the candidate count).
int oracle_tree_draft(int B, int gamma, int V, int r, int c, int M, int N, const float* U,
                      const uint16_t* W1, const uint16_t* W2t, const int32_t* anchor,
                      int32_t* node_token, int32_t* node_depth, int32_t* node_parent,
                      double* node_q, double* node_path, double* logit_margin,
                      double* path_margin, int threads) {
  if (B < 1 || gamma < 1 || V < 2 || r < 1 || c < 1 || M < 1 || M > c || c > V) return 1;
  int64_t total = c, width = c;
  for (int k = 2; k <= gamma; ++k) {
    width = std::min<int64_t>(M, width) * c;
    total += width;
  }
  if (N < 1 || N > total) return 1;
  parallel_for(B, threads, [&](int64_t b) {
    double lgap = std::numeric_limits<double>::infinity();
    double pgap = std::numeric_limits<double>::infinity();
    std::vector<TreeCand> all;
    std::vector<int> frontier = {-1};            // positions in `all`; -1 = the root
    std::vector<float> L;
    std::vector<double> p;
    std::vector<int32_t> kids;
    for (int k = 1; k <= gamma; ++k) {
      const float* U_row = U + (b * gamma + (k - 1)) * static_cast<int64_t>(V);
      const size_t first = all.size();
      for (size_t m = 0; m < frontier.size(); ++m) {
        const int par = frontier[m];
        const int32_t x = (par < 0) ? anchor[b] : all[par].token;
        const double Ppar = (par < 0) ? 1.0 : all[par].P;
        draft_logits(U_row, W1, W2t, V, r, x, L);
        softmax_fp64(L.data(), V, p);
        top_children(L, c, kids, &lgap);
        for (int i = 0; i < c; ++i) {
          TreeCand t;
          t.q = p[kids[i]];
          t.P = Ppar * t.q;
          t.depth = k;
          t.idx = static_cast<int>(m) * c + i;
          t.parent = par;
          t.token = kids[i];
          all.push_back(t);
        }
      }
      if (k == gamma) break;
      // The M best nodes of this depth are the parents of the next.
      std::vector<int> order;
      for (size_t i = first; i < all.size(); ++i) order.push_back(static_cast<int>(i));
      std::stable_sort(order.begin(), order.end(), [&](int a, int bb) {
        if (all[a].P != all[bb].P) return all[a].P > all[bb].P;
        return all[a].idx < all[bb].idx;
      });
      std::vector<double> Ps;
      for (int i : order) Ps.push_back(all[i].P);
      const int keep = std::min<int>(M, static_cast<int>(order.size()));
      rank_gaps(Ps, std::min<int>(keep, static_cast<int>(order.size()) - 1), &pgap);
      frontier.assign(order.begin(), order.begin() + keep);
    }
    // The verify budget: the N best candidates of every depth.
    std::vector<int> rank(all.size());
    for (size_t i = 0; i < all.size(); ++i) rank[i] = static_cast<int>(i);
    std::stable_sort(rank.begin(), rank.end(), [&](int a, int bb) {
      if (all[a].P != all[bb].P) return all[a].P > all[bb].P;
      if (all[a].depth != all[bb].depth) return all[a].depth < all[bb].depth;
      return all[a].idx < all[bb].idx;
    });
    std::vector<double> Ps;
    for (int i : rank) Ps.push_back(all[i].P);
    rank_gaps(Ps, std::min<int>(N, static_cast<int>(rank.size()) - 1), &pgap);
    std::vector<int> pos_of(all.size(), -1);
    for (int n = 0; n < N; ++n) pos_of[rank[n]] = n;
    for (int n = 0; n < N; ++n) {
      const TreeCand& t = all[rank[n]];
      const int64_t o = b * static_cast<int64_t>(N) + n;
      node_token[o] = t.token;
      node_depth[o] = t.depth;
      node_parent[o] = (t.parent < 0) ? -1 : pos_of[t.parent];
      node_q[o] = t.q;
      node_path[o] = t.P;
    }
    if (logit_margin) logit_margin[b] = lgap;
    if (path_margin) path_margin[b] = pgap;
  });
  return 0;
}

// Lossless verify of a tree. target [B][N + 1][V] f32: row 0 of a request holds the target
// logits of position 1 (after the anchor), row 1 + n those of the position after node n (its
// depth + 1), given the node's path. Tree as written by oracle_tree_draft (nodes in rank order;
// a node's children are the nodes whose parent it is, in rank order).
// The walk ([V41] "投机解码…": a draft is kept only as far as the target's own draws agree with
// it; [ZDS] "后续工作"; reading): at the current node (the root first), y is drawn from p_t of
// its row with u = uniforms[b][depth][2] by the inverse CDF whose order puts the node's
// children first (in rank order) and then every other token in ascending id. If y is a child,
// it is accepted and the walk moves to it; otherwise y is the emitted token (a correction, or,
// at a node without children, the bonus) and the walk stops. Every emitted token is thus a draw
// from the target's distribution given the accepted path: the tree changes how far the round
// gets, never the distribution. For one child this is the point-mass rule of a greedy draft
// (accept with probability p_t(x), else draw from p_t without x), taken with one uniform.
// Outputs: accept_len [B] (accepted tree tokens), path [B][gamma] (the accepted tokens, -1 past
// accept_len), next_token [B], flags [B] (NONFINITE when a row the walk read has a non-finite
// log-sum-exp), margin [B] (nullable: the smallest distance from u to a boundary the walk
// compared it with).
int oracle_tree_verify(int B, int gamma, int V, int N, const float* target,
                       const int32_t* node_token, const int32_t* node_depth,
                       const int32_t* node_parent, const float* uniforms, int32_t* accept_len,
                       int32_t* path, int32_t* next_token, uint32_t* flags, double* margin,
                       int threads) {
  if (B < 1 || gamma < 1 || V < 2 || N < 1) return 1;
  parallel_for(B, threads, [&](int64_t b) {
    const int32_t* tok = node_token + b * static_cast<int64_t>(N);
    const int32_t* dep = node_depth + b * static_cast<int64_t>(N);
    const int32_t* par = node_parent + b * static_cast<int64_t>(N);
    std::vector<double> pt;
    std::vector<char> excluded(V, 0);
    double mg = std::numeric_limits<double>::infinity();
    uint32_t fl = 0;
    int cur = -1, depth = 0, accepted = 0;
    int32_t y = 0;
    for (int k = 0; k < gamma; ++k) path[b * gamma + k] = -1;
    for (;;) {
      const float* row = target + (b * static_cast<int64_t>(N + 1) + (cur + 1)) * V;
      const double lt = softmax_fp64(row, V, pt);
      if (!std::isfinite(lt)) fl |= ORACLE_FLAG_NONFINITE;
      const double u = static_cast<double>(uniforms[(b * (gamma + 1) + depth) * 3 + 2]);
      double S = 0.0;
      int chosen = -1;
      std::vector<int32_t> kids;
      for (int n = 0; n < N; ++n) {
        if (par[n] != cur) continue;
        kids.push_back(tok[n]);
        const double lo = S;
        S += pt[tok[n]];
        if (S > u) {
          mg = std::min(mg, std::min(u - lo, S - u));
          chosen = n;
          break;
        }
        mg = std::min(mg, u - S);
      }
      if (chosen >= 0) {
        path[b * gamma + accepted] = tok[chosen];
        ++accepted;
        cur = chosen;
        depth = dep[chosen];
        continue;
      }
      // Emission: the first token outside the children whose cumulative mass passes u.
      for (int32_t x : kids) excluded[x] = 1;
      double cdf = S;
      int32_t last_positive = -1;
      y = -1;
      for (int v = 0; v < V; ++v) {
        if (excluded[v]) continue;
        const double lo = cdf;
        cdf += pt[v];
        if (pt[v] > 0.0) last_positive = v;
        if (u < cdf) {
          mg = std::min(mg, std::min(u - lo, cdf - u));
          y = v;
          break;
        }
      }
      if (y < 0) {
        mg = 0.0;
        y = last_positive >= 0 ? last_positive : 0;
      }
      for (int32_t x : kids) excluded[x] = 0;
      break;
    }
    accept_len[b] = accepted;
    next_token[b] = y;
    if (flags) flags[b] = fl;
    if (margin) margin[b] = mg;
  });
  return 0;
}

}  // extern "C"
