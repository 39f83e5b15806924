/*
 * dspark.h — C ABI of the MI355X (gfx950) DSpark draft-and-verify library (libdspark.so).
 *
 * One speculative-decoding round of DSpark for a batch of B requests:
 *   dspark_markov_draft  semi-autoregressive Markov-head draft of gamma tokens per request
 *   dspark_confidence    confidence head c_k = sigmoid(w . [h_k ; W1[x_{k-1}]] / T_k)
 *   dspark_plan          survival-ordered greedy planner that maximises Theta = tau * SPS(B)
 *   dspark_verify        lossless rejection-sampling verify, residual resample, bonus token
 *   dspark_markov_draft_opts, dspark_verify_opts   the same with a draft temperature or greedy
 *   dspark_rnn_draft, dspark_rnn_verify   the draft and verify with the RNN head of eq. (6)
 *   dspark_markov_draft_plan, dspark_rnn_draft_plan   draft, confidence and plan of a round
 *                        in one call, the plan computed beside the last position's draft step
 *   dspark_tree_draft, dspark_tree_verify   PCTree: a draft tree scored by the Markov head
 *                        within a verify budget, and its lossless verify
 *
 * Sources (cited below by tag; each gives the page title and the section or equation):
 *   [V41]  blog.javazero.top, "DeepSeek-V4.1 模型结构（6）：解码，DSpark"
 *   [ZDS]  zdszero.github.io, spec_dspark (the DSpark chapter of a speculative-decoding series)
 *   [AIL]  ailearn.mscapital.top, "DSpark：不让大模型更聪明，而让它「吐字更快」"
 *   [CSDN] deepseek.csdn.net, DSpark walk-through with equations (1)-(12)
 *
 * Conventions shared by every entry point
 *   - Every array argument is a DEVICE pointer (HIP device memory or memory the device can
 *     read), row-major and contiguous, allocated and owned by the caller. The library keeps no
 *     state between calls and allocates no device memory: scratch space comes in through the
 *     `ws`/`ws_bytes` workspace argument, sized by dspark_workspace_bytes().
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the null stream) and
 *     returns without waiting for it. Results are valid once the stream reaches that point.
 *   - Argument checks run on the host, synchronously, before anything is enqueued; a failed
 *     check returns its status and enqueues nothing. A launch failure returns DSPARK_ERR_HIP.
 *     No C++ exception crosses this interface.
 *   - Alignment (DSPARK_ERR_ALIGN otherwise): the bulk tensors that kernels read in 16-byte
 *     vectors (U, target, W1, W2t, h, w) must be 16-byte aligned, the workspace 256-byte
 *     aligned, and every other array aligned to its element size. bf16 tensors are passed as
 *     uint16_t bit patterns.
 *   - Random draws are never generated inside the library: the caller passes
 *     uniforms [B][gamma+1][3] fp32 in [0,1), so a round is reproducible bit for bit.
 *     Component 0 of slot k-1 draws the draft token of position k; component 1 of slot k-1 is
 *     the accept test of position k; component 2 of slot k-1 draws the token emitted at
 *     position k (the residual resample after a reject at k, or the bonus at k = l_b + 1).
 *   - Sampling rule: a draw from a distribution p over token ids with uniform u returns the
 *     smallest id v whose cumulative probability (ids in ascending order) exceeds u. The pages
 *     fix only the distribution a draw must follow; this rule makes it reproducible.
 *   - Results are deterministic: two identical calls give bitwise identical outputs.
 *   - Token ids the caller passes (anchors, forced or drafted tokens, tree node tokens) are
 *     clamped into [0, V) on the device, and verify lengths into [0, gamma], before any address
 *     is formed from them: a call with such values reads nothing outside its tensors and gives
 *     the results of the clamped values (which are then not meaningful).
 */
#ifndef DSPARK_H_
#define DSPARK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define DSPARK_API __attribute__((visibility("default")))
#else
#define DSPARK_API
#endif

/* Problem sizes. B requests, gamma draft positions, V vocabulary, r Markov rank, d hidden size
 * (d is read only by dspark_confidence). Supported: B >= 1, 1 <= gamma <= 255, 2 <= V <= 2^19,
 * r in {16, 32, 64, 128, 256, 512}, d % 8 == 0, B * (gamma + 1) <= 65535, and for
 * dspark_plan and the draft-and-plan calls B * gamma <= 8192. */
typedef struct dspark_dims {
  int32_t B;
  int32_t gamma;
  int32_t V;
  int32_t r;
  int32_t d;
} dspark_dims;

typedef int32_t dspark_status;
#define DSPARK_OK 0
#define DSPARK_ERR_NULL 1        /* a required pointer is NULL */
#define DSPARK_ERR_SHAPE 2       /* a size is out of the supported range */
#define DSPARK_ERR_ALIGN 3       /* a pointer is not 16-byte aligned */
#define DSPARK_ERR_WORKSPACE 4   /* ws_bytes < dspark_workspace_bytes(...) */
#define DSPARK_ERR_SPS 5         /* sps_len <= B * (gamma + 1) */
#define DSPARK_ERR_HIP 6         /* a HIP launch failed */
#define DSPARK_ERR_MODE 7        /* unknown plan mode, or LAGGED_TOPK without a ring */
#define DSPARK_ERR_OPTS 8        /* draft options out of range (temperature not positive, finite) */

/* Plan modes. [ZDS] "在 SGLang 里": the static mode verifies every drafted token (no planner);
 * the compact mode plans with the SPS table. */
#define DSPARK_PLAN_FULL_VERIFY 0 /* l_b = gamma for every request */
#define DSPARK_PLAN_EARLY_STOP 1  /* Algorithm 1: admit by survival while Theta rises */
#define DSPARK_PLAN_FULL_PATH 2   /* first maximiser of Theta over the whole admission path */
#define DSPARK_PLAN_LAGGED_TOPK 3 /* capacity from confidences two rounds back, order now */

/* Operation ids for dspark_workspace_bytes. */
#define DSPARK_OP_DRAFT 0
#define DSPARK_OP_CONFIDENCE 1
#define DSPARK_OP_PLAN 2
#define DSPARK_OP_VERIFY 3
#define DSPARK_OP_RNN_DRAFT 4
#define DSPARK_OP_RNN_VERIFY 5
#define DSPARK_OP_TREE_DRAFT 6   /* sized by dspark_tree_workspace_bytes */
#define DSPARK_OP_TREE_VERIFY 7

/* Per-request verify flag bits. */
#define DSPARK_FLAG_NONFINITE 1u     /* a verified target row has a non-finite log-sum-exp */
#define DSPARK_FLAG_ZERO_RESIDUAL 2u /* residual mass not positive: token drawn from p_t */

/* Human-readable name of a status code (static storage; never NULL). */
DSPARK_API const char* dspark_status_string(dspark_status status);

/* Library version string (static storage). */
DSPARK_API const char* dspark_version(void);

/* Bytes of workspace the operation `op` (DSPARK_OP_*) needs for `dims`; 0 if it needs none,
 * (size_t)-1 for unsupported dims or op. */
DSPARK_API size_t dspark_workspace_bytes(dspark_dims dims, int32_t op);

/*
 * Semi-autoregressive Markov-head draft.
 * [V41] "Markov head", eqs. (4) and (5) and the serial loop; [CSDN] 4.1-4.2, eq. (4);
 * [ZDS] "insight 一" (p_k = softmax(U_k + W1[x_{k-1}] W2), then bias position k+1).
 * For k = 1..gamma: with x_0 = anchor,
 *   L_k = U_k + W1[x_{k-1}] . W2   (bf16 operands, fp32 accumulation, fp32 logits)
 *   x_k ~ softmax(L_k)             (inverse-CDF draw with uniforms[b][k-1][0])
 * The same W1, W2 serve every position; the draft always produces all gamma tokens.
 *   U         [B][gamma][V] fp32   base logits of the parallel drafter
 *   W1        [V][r] bf16          Markov embedding table (Embedding(V, r) layout)
 *   W2t       [V][r] bf16          Markov projection stored token-major: W2t[v][i] = W2[i][v]
 *                                  (the weight layout of Linear(r, V))
 *   anchor    [B] int32            x_0, the last token the target emitted
 *   uniforms  [B][gamma+1][3] fp32
 *   tokens    [B][gamma] int32     out: drafted tokens x_1..x_gamma
 *   q_tok     [B][gamma] fp32      out: q_k = p_k(x_k), the draft probability of the token
 *   lse       [B][gamma] fp64      out: log sum_v exp L_k(v)
 *   logits_dbg  nullable [B][gamma][V] fp32: out, L_k (costs an extra write of the logits)
 *   force_tokens nullable [B][gamma] int32: teacher forcing for step-by-step comparison; when
 *              given, tokens[] still receives each draw, but force_tokens[b][k-1] conditions
 *              position k+1 and q_tok[b][k-1] is the probability of force_tokens[b][k-1].
 * Token ids in anchor / force_tokens must lie in [0, V) (not checked on the device).
 * A row whose logits are not finite yields token 0 and q = lse = NaN.
 */
DSPARK_API dspark_status dspark_markov_draft(dspark_dims dims, const float* U, const uint16_t* W1,
                                             const uint16_t* W2t, const int32_t* anchor,
                                             const float* uniforms, int32_t* tokens, float* q_tok,
                                             double* lse, float* logits_dbg,
                                             const int32_t* force_tokens, void* ws, size_t ws_bytes,
                                             void* stream);

/*
 * Draft sampling options. [V41] "Markov head", the serial loop (each position is sampled with a
 * temperature); [V41] / [AIL] the deployed recipe drafts greedily (draft_sample_method "greedy").
 *   temperature  > 0 and finite: the fp32 logits L_k are multiplied, in fp32, by
 *                beta = fp32(1 / temperature) and x_k ~ softmax(beta L_k); q_tok and lse refer to
 *                that distribution (temperature 1 is the plain draft, bit for bit).
 *   greedy       nonzero: x_k is the first token with the largest logit L_k (the temperature is
 *                ignored); q_tok = 1 (the point mass; 0 for a forced token other than x_k) and
 *                lse = max_v L_k(v). With non-finite logits the greedy token is unspecified.
 */
typedef struct dspark_draft_opts {
  float temperature;
  int32_t greedy;
} dspark_draft_opts;

/*
 * dspark_markov_draft with draft options (opts NULL: temperature 1, sampling). logits_dbg
 * receives L_k before the temperature. Returns DSPARK_ERR_OPTS for a temperature that is not
 * positive and finite (when greedy is 0); the other arguments and checks are those of
 * dspark_markov_draft.
 */
DSPARK_API dspark_status dspark_markov_draft_opts(dspark_dims dims, const float* U,
                                                  const uint16_t* W1, const uint16_t* W2t,
                                                  const int32_t* anchor, const float* uniforms,
                                                  int32_t* tokens, float* q_tok, double* lse,
                                                  float* logits_dbg, const int32_t* force_tokens,
                                                  void* ws, size_t ws_bytes,
                                                  const dspark_draft_opts* opts, void* stream);

/*
 * Confidence head, eq. (7), with the STS temperature applied at inference:
 *   c_k = sigmoid( (w . [h_k ; W1[x_{k-1}]]) / T_k ),  x_0 = anchor.
 * [V41] "confidence head", eq. (7) (input holds x_{k-1}, not x_k; no bias term);
 * [ZDS] "在 SGLang 里" (Linear(h + r, 1), sigmoid(raw / T) with per-position STS temperatures).
 *   h       [B][gamma][d] bf16   drafter hidden states
 *   W1      [V][r] bf16          the Markov embedding table
 *   w       [d + r] bf16         head weights; w[0..d) multiply h_k, w[d..d+r) multiply W1 row
 *   T       [gamma] fp32         per-position temperature (> 0)
 *   anchor  [B] int32, tokens [B][gamma] int32 (the drafted tokens)
 *   conf    [B][gamma] fp32      out
 * The dot product is accumulated in fp64.
 */
DSPARK_API dspark_status dspark_confidence(dspark_dims dims, const uint16_t* h, const uint16_t* W1,
                                           const uint16_t* w, const float* T,
                                           const int32_t* anchor, const int32_t* tokens,
                                           float* conf, void* stream);

/*
 * Hardware-aware verify planner.
 * [V41] "调度器" ("目标函数", "贪心就能解", "按置信度截断在什么条件下不改变分布", Appendix A);
 * [ZDS] "调度" and "在 SGLang 里"; [CSDN] 5.3, 5.4, 8.
 *   a_{b,j} = prod_{i<=j} c_{b,i} (fp64, sequential),  B_tot = sum_b (1 + l_b),
 *   tau = sum_b (1 + sum_{j<=l_b} a_{b,j}),            Theta = tau * SPS(B_tot).
 * Candidates (b, j) are ordered by a descending, ties by b then j ascending; admitting them
 * one by one along that order traces Theta_i = (B + sum of the first i survivals) * sps[B + i].
 *   FULL_VERIFY  admit all (conf may be NULL; tau and Theta are then NaN in stats)
 *   EARLY_STOP   admit while Theta_{i+1} > Theta_i (stop at the first non-increase)
 *   FULL_PATH    admit the first maximiser of Theta_i over i = 0..B*gamma
 *   LAGGED_TOPK  K = B + (FULL_PATH count computed on the confidences of round round_index-2,
 *                read from ring[round_index % 2]); admit the first K - B candidates of this
 *                round's own order. Rounds 0 and 1 plan with EARLY_STOP. In every round the
 *                ring slot round_index % 2 is then overwritten with this round's conf.
 *   conf        [B][gamma] fp32
 *   sps         [sps_len] fp64, sps[n] = engine steps per second with n verified tokens;
 *               sps_len must exceed B * (gamma + 1)
 *   ring        [2][B][gamma] fp32, required for LAGGED_TOPK (NULL otherwise)
 *   draft_len   [B] int32        out: l_b in [0, gamma]; request b verifies 1 + l_b rows
 *   row_offsets [B+1] int32      out: exclusive scan of (1 + l_b), the packed row layout
 *   stats       [4] fp64         out (nullable): {B_tot, tau, Theta, K} at the admitted point
 *                                (K = B_tot except for LAGGED_TOPK after warm-up)
 * Runs as a single workgroup; nothing returns to the host.
 */
DSPARK_API dspark_status dspark_plan(dspark_dims dims, const float* conf, const double* sps,
                                     int32_t sps_len, int32_t mode, float* ring,
                                     int32_t round_index, int32_t* draft_len,
                                     int32_t* row_offsets, double* stats, void* stream);

/*
 * The draft side of one round in a single call: the Markov-head draft (as
 * dspark_markov_draft_opts without logits_dbg or force_tokens), the confidence head (as
 * dspark_confidence) and the planner (as dspark_plan), with the same arguments, checks and
 * outputs as those three calls made one after the other. Passages: those of the three calls;
 * the planner depends only on the confidences, which depend only on x_0 .. x_{gamma-1}
 * ([V41] "confidence head", eq. (7)), so it is computed while the last position is drafted.
 * Order on the stream: draft positions 1 .. gamma-1, the confidence head, then the last
 * position's step with the planner on one extra workgroup of the same launch (for r in
 * {64, 128, 256}, V % 4 == 0 and B * gamma <= 4096; other shapes launch the planner and the
 * step one after the other), then the last position's sampler. The results are bit-identical to
 * the three separate calls.
 *   ws, ws_bytes   the draft workspace (dspark_workspace_bytes(dims, DSPARK_OP_DRAFT))
 *   opts           nullable; temperature / greedy as in dspark_markov_draft_opts
 * A failing check of any of the three calls returns its status, and nothing is launched.
 */
DSPARK_API dspark_status dspark_markov_draft_plan(
    dspark_dims dims, const float* U, const uint16_t* W1, const uint16_t* W2t,
    const int32_t* anchor, const float* uniforms, const uint16_t* h, const uint16_t* w,
    const float* T, const double* sps, int32_t sps_len, int32_t mode, float* ring,
    int32_t round_index, int32_t* tokens, float* q_tok, double* lse, float* conf,
    int32_t* draft_len, int32_t* row_offsets, double* stats, void* ws, size_t ws_bytes,
    const dspark_draft_opts* opts, void* stream);

/*
 * Lossless verify.
 * [V41] "投机解码：让小的先猜，大的一次验一串" and the derivation after it (accept with
 * min(1, p/q), on reject resample from norm(max(0, p - q)), left to right, the first reject
 * voids the rest, the bonus from the target when all are accepted, the emitted token is the
 * next anchor); [AIL] 02 (A/B worked example); [CSDN] 2.1.
 * Rows of request b: target[row_offsets[b] + j] (j = 0..draft_len[b]) holds the target logits
 * of position j+1; row draft_len[b] is the bonus position. FULL_VERIFY is the dense layout
 * row_offsets[b] = b * (gamma + 1).
 *   Accept test at position k:  uniforms[b][k-1][1] * q_tok[b][k-1] < p_t(x_k)   (fp64)
 *   First reject at k: next_token ~ max(0, p_t - p_d) / sum, p_d the draft distribution of
 *   position k recomputed from U, W1, W2t and x_{k-1} (uniforms[b][k-1][2]); all accepted:
 *   next_token ~ p_t of row draft_len[b] (uniforms[b][draft_len[b]][2]).
 *   target      [row_offsets[B]][V] fp32 (device-resident; sized for the plan's rows, of which
 *               there are at least B: each request verifies 1 + draft_len[b] >= 1 rows, and
 *               rows 0..B-1 may be read before row_offsets[B] is)
 *   row_offsets [B+1], draft_len [B] int32 (as written by dspark_plan)
 *   U, W1, W2t, anchor, tokens, q_tok, lse, uniforms: as given to / written by the draft
 *   accept_len  [B] int32   out: number of drafted tokens accepted (0..draft_len[b]); the
 *                           round emits tokens[b][0..accept_len) followed by next_token[b]
 *   next_token  [B] int32   out: the residual or bonus token (the next anchor)
 *   beta_emit   nullable [B] fp32: out, sum_v min(p_t, p_d) at a residual emission row (the
 *               acceptance rate of that position, eq. (8)); -1 at a bonus row
 *   flags       nullable [B] uint32: out, DSPARK_FLAG_* bits
 */
DSPARK_API dspark_status dspark_verify(dspark_dims dims, const float* target,
                                       const int32_t* row_offsets, const int32_t* draft_len,
                                       const float* U, const uint16_t* W1, const uint16_t* W2t,
                                       const int32_t* anchor, const int32_t* tokens,
                                       const float* q_tok, const double* lse,
                                       const float* uniforms, int32_t* accept_len,
                                       int32_t* next_token, float* beta_emit, uint32_t* flags,
                                       void* ws, size_t ws_bytes, void* stream);

/*
 * dspark_verify for a draft made with options (opts NULL: temperature 1, sampling). The accept
 * test is unchanged (q_tok is the draft probability the options produced: 1 for a greedy
 * draft, which is accepted iff u < p_t(x)); after a reject at position j the residual is
 * max(0, p_t - p_d) with p_d = softmax(beta L_j) at the draft temperature, or the point mass
 * on x_j for a greedy draft (so the correction draws from p_t without x_j). lse must be the
 * draft's output under the same options. [V41] "投机解码…" (the accept / resample rule holds for
 * any draft distribution, a point mass included). Returns DSPARK_ERR_OPTS as the draft does.
 */
DSPARK_API dspark_status dspark_verify_opts(dspark_dims dims, const float* target,
                                            const int32_t* row_offsets, const int32_t* draft_len,
                                            const float* U, const uint16_t* W1, const uint16_t* W2t,
                                            const int32_t* anchor, const int32_t* tokens,
                                            const float* q_tok, const double* lse,
                                            const float* uniforms, int32_t* accept_len,
                                            int32_t* next_token, float* beta_emit, uint32_t* flags,
                                            void* ws, size_t ws_bytes,
                                            const dspark_draft_opts* opts, void* stream);

/*
 * PCTree tree drafting. [ZDS] "后续工作" (PCTree): the draft chain becomes a tree; the Markov
 * head scores every child token under a parent token, so it picks each parent's candidate
 * children, and the most likely paths are kept within a fixed verify budget, with no retraining
 * and no extra backbone pass; [V41] "Markov head" eqs. (4), (5) (the scores).
 * Per request, with x the token of a node (the anchor at the root) and U_k the base logits of
 * depth k (shared by every node of the depth):
 *   - a node of depth k - 1 scores the tokens of depth k by softmax(fp32(U_k + fp32(W1[x] W2)))
 *     and expands its c best children: the c largest fp32 logits, the smaller id on a tie;
 *   - a node's path probability P is the product of those probabilities along its path (fp64);
 *   - depth 1 expands the root; depth k >= 2 expands the M nodes of depth k - 1 with the
 *     largest P (ties: the earlier candidate, numbering candidates parent by parent and child
 *     by child in rank order);
 *   - the N candidates of all depths with the largest P (ties: the smaller depth, then the
 *     earlier candidate) are kept; they form a tree (a child's P never exceeds its parent's).
 * Outputs, nodes in that rank order, [B][N] each:
 *   node_token   int32   the node's token
 *   node_depth   int32   1..gamma (the token's position)
 *   node_parent  int32   rank of the parent node, -1 for a child of the root
 *   node_q       f64     the token's Markov probability under its parent (exp(L - lse))
 *   node_path    f64     P
 * U, W1, W2t, anchor as for dspark_markov_draft (no temperature; anchors are clamped into
 * [0, V)). Shape limits (else DSPARK_ERR_SHAPE): r <= 256, 1 <= M <= c <= 8, M a power of
 * two, c <= V, c + (gamma - 1) M c <= 1024 candidates, 1 <= N <= min(that, 256), and
 * ceil(V / 32) <= 32 * (1024 / M). Workspace: dspark_tree_workspace_bytes(dims, shape,
 * DSPARK_OP_TREE_DRAFT). Precision: the logits are bit-identical to the chain draft's; lse from
 * the tile partials (fp32 tile sums, fp64 across tiles), probabilities in fp64.
 */
typedef struct dspark_tree_shape {
  int32_t c;   /* children expanded per node */
  int32_t M;   /* nodes expanded per depth (depth >= 2) */
  int32_t N;   /* nodes kept: the verify budget */
} dspark_tree_shape;
DSPARK_API size_t dspark_tree_workspace_bytes(dspark_dims dims, dspark_tree_shape shape,
                                              int32_t op);
DSPARK_API dspark_status dspark_tree_draft(dspark_dims dims, dspark_tree_shape shape,
                                           const float* U, const uint16_t* W1,
                                           const uint16_t* W2t, const int32_t* anchor,
                                           int32_t* node_token, int32_t* node_depth,
                                           int32_t* node_parent, double* node_q,
                                           double* node_path, void* ws, size_t ws_bytes,
                                           void* stream);

/*
 * Lossless verify of a draft tree. [V41] "投机解码：让小的先猜，大的一次验一串" (a drafted
 * token is kept only as far as the target's own draw agrees with it; every round emits at least
 * one token from the target); [ZDS] "后续工作" (PCTree). Rows: target[b][0] holds the target
 * logits of position 1 (after the anchor), target[b][1 + n] those of the position after kept
 * node n, given the node's path. The walk: at the current node (the root first, depth 0), y is
 * drawn from p_t of its row with u = uniforms[b][depth][2], by the inverse CDF whose order puts
 * the node's children (in rank order) first and then every other token by ascending id. A child
 * is accepted and the walk moves to it; any other y is emitted (the correction, or at a node
 * without children the bonus) and the walk stops. Every emitted token is a draw from the
 * target given the accepted path, so the round is lossless whatever the tree.
 *   target      [B][N + 1][V] fp32
 *   node_token, node_parent   [B][N] as written by dspark_tree_draft (clamped into range)
 *   uniforms    [B][gamma + 1][3] fp32; component 2 of slot depth is used
 *   accept_len  [B] int32 out: tree tokens accepted (0..gamma)
 *   path        [B][gamma] int32 out: the accepted tokens, -1 past accept_len
 *   next_token  [B] int32 out: the emitted token (the next anchor)
 *   flags       nullable [B] uint32 out: DSPARK_FLAG_NONFINITE when a row the walk read has a
 *               non-finite log-sum-exp
 * Shape limits and errors as for dspark_tree_draft; workspace: dspark_tree_workspace_bytes(
 * dims, shape, DSPARK_OP_TREE_VERIFY).
 */
DSPARK_API dspark_status dspark_tree_verify(dspark_dims dims, dspark_tree_shape shape,
                                            const float* target, const int32_t* node_token,
                                            const int32_t* node_parent, const float* uniforms,
                                            int32_t* accept_len, int32_t* path,
                                            int32_t* next_token, uint32_t* flags, void* ws,
                                            size_t ws_bytes, void* stream);

/*
 * The verify of dspark_verify_opts for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, and harnesses that forbid hipMalloc. Arguments,
 * results, checks and kernels are those of dspark_verify_opts, without `ws` / `ws_bytes`: the
 * scratch space is a fixed array in the library's device memory, DSPARK_NOALLOC_SCRATCH_BYTES
 * (48 MiB) per GPU, held from the library's first use on that GPU until the process ends.
 * Sizes whose workspace (dspark_workspace_bytes(dims, DSPARK_OP_VERIFY)) exceeds it return
 * DSPARK_ERR_WORKSPACE before anything is enqueued; every workload from 4 to 512 requests at
 * V <= 151936 and gamma <= 15 fits. The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine). Every call on one GPU shares that GPU's array and leaves its
 * contents behind; each call clears what it needs cleared itself. Calls that overlap on one
 * GPU (concurrent streams or host threads) race on the array and must be serialised by the
 * caller. DSPARK_ERR_HIP if the array's device address cannot be obtained.
 */
#define DSPARK_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
DSPARK_API dspark_status dspark_verify_noalloc(dspark_dims dims, const float* target,
                                               const int32_t* row_offsets,
                                               const int32_t* draft_len, const float* U,
                                               const uint16_t* W1, const uint16_t* W2t,
                                               const int32_t* anchor, const int32_t* tokens,
                                               const float* q_tok, const double* lse,
                                               const float* uniforms, int32_t* accept_len,
                                               int32_t* next_token, float* beta_emit,
                                               uint32_t* flags, const dspark_draft_opts* opts,
                                               void* stream);

/*
 * Draft with the RNN head instead of the Markov head. [CSDN] 4.2, eq. (6); [AIL] "RNN 头（可选）";
 * [V41] "Markov head" (the paper's small-RNN alternative): a recurrent state s summarises the
 * block's prefix. Per request s_0 = 0 and x_0 = anchor[b]; at position k (1-based)
 *   z_k = [s_{k-1}; W1[x_{k-1}]; h_k],
 *   s_k = sigmoid(W_g z_k) * s_{k-1} + (1 - sigmoid(W_g z_k)) * tanh(W_c z_k)   (elementwise),
 *   e_k = tanh(W_o z_k),   B_k = W2^T e_k,   p_k = softmax(U_k + B_k),
 * and x_k is drawn, forced and reported as in dspark_markov_draft_opts (same uniforms, options,
 * q_tok, lse, logits_dbg). The state has r components and eq. (6) has no bias terms.
 *   Wgco      bf16 [3r][2r + d]: rows 0..r-1 W_g, r..2r-1 W_c, 2r..3r-1 W_o; columns in z's
 *             order: state (r), embedding (r), hidden state (d).
 *   h         bf16 [B][gamma][d]: the backbone hidden states h_k (those of the confidence head).
 *   e_rows    out, fp32 [B][gamma][r]: e_k = tanh(W_o z_k), the bias vectors; the verify of the
 *             round takes them (dspark_rnn_verify).
 * Precision: pre-activations in fp64 (the hidden block as bf16 MFMA products summed in fp32
 * over 128 products, then in fp64); e_k rounded to fp32, and the bias contraction takes it as
 * three bf16 terms whose sum is that fp32 value, with fp32 accumulation.
 * Requires r <= 256 and d a positive multiple of 8 (else DSPARK_ERR_SHAPE); workspace:
 * dspark_workspace_bytes(dims, DSPARK_OP_RNN_DRAFT). Other checks and errors as in
 * dspark_markov_draft_opts.
 */
DSPARK_API dspark_status dspark_rnn_draft(dspark_dims dims, const float* U, const uint16_t* W1,
                                          const uint16_t* W2t, const uint16_t* Wgco,
                                          const uint16_t* h, const int32_t* anchor,
                                          const float* uniforms, int32_t* tokens, float* q_tok,
                                          double* lse, float* e_rows, float* logits_dbg,
                                          const int32_t* force_tokens, void* ws, size_t ws_bytes,
                                          const dspark_draft_opts* opts, void* stream);

/*
 * Verify of an RNN-head draft: as dspark_verify_opts, with the draft distribution of a rejected
 * position j recomputed from the draft's bias vector e_j (e_rows, fp32 [B][gamma][r], as
 * dspark_rnn_draft wrote it, taken as the same three bf16 terms): p_d = softmax(beta (U_j + W2^T
 * e_j)). No embedding table or anchor is needed. Requires r <= 256 and d as for the draft;
 * workspace: dspark_workspace_bytes(dims, DSPARK_OP_RNN_VERIFY).
 */
DSPARK_API dspark_status dspark_rnn_verify(dspark_dims dims, const float* target,
                                           const int32_t* row_offsets, const int32_t* draft_len,
                                           const float* U, const uint16_t* W2t,
                                           const float* e_rows, const int32_t* tokens,
                                           const float* q_tok, const double* lse,
                                           const float* uniforms, int32_t* accept_len,
                                           int32_t* next_token, float* beta_emit, uint32_t* flags,
                                           void* ws, size_t ws_bytes,
                                           const dspark_draft_opts* opts, void* stream);

/*
 * The draft side of one round with the RNN head in a single call: dspark_rnn_draft (without
 * logits_dbg or force_tokens), dspark_confidence and dspark_plan, with their arguments, checks
 * and outputs, in the order and with the planner placement of dspark_markov_draft_plan (the
 * planner beside the last position's step for r in {64, 128, 256} and V % 4 == 0,
 * B * gamma <= 4096). Passages: those of the three calls. The results are bit-identical to the
 * three separate calls.
 *   ws, ws_bytes   the RNN draft workspace (dspark_workspace_bytes(dims, DSPARK_OP_RNN_DRAFT))
 */
DSPARK_API dspark_status dspark_rnn_draft_plan(
    dspark_dims dims, const float* U, const uint16_t* W1, const uint16_t* W2t,
    const uint16_t* Wgco, const uint16_t* h, const int32_t* anchor, const float* uniforms,
    const uint16_t* w, const float* T, const double* sps, int32_t sps_len, int32_t mode,
    float* ring, int32_t round_index, int32_t* tokens, float* q_tok, double* lse, float* e_rows,
    float* conf, int32_t* draft_len, int32_t* row_offsets, double* stats, void* ws,
    size_t ws_bytes, const dspark_draft_opts* opts, void* stream);

/*
 * Kernel timing with HIP events (measurement support; not part of the method).
 * dspark_profile_begin(capacity) arms up to `capacity` event pairs; while armed, every kernel
 * launch of the library records a pair with its dispatch on the launch stream (the start and
 * stop events of hipExtLaunchKernel, taken around the kernel by the command processor).
 * dspark_profile_end() waits for the recorded events and returns, per kernel name, the number
 * of launches and their summed duration in milliseconds (names[i] has static storage), then
 * disarms. Returns the number of kernel names written (at most max_names), or -1 on error.
 * Not thread-safe; only for single-threaded benchmarking.
 */
DSPARK_API int32_t dspark_profile_begin(int32_t capacity);
DSPARK_API int32_t dspark_profile_end(const char** names, int32_t* counts, double* total_ms,
                                      int32_t max_names);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif /* DSPARK_H_ */
