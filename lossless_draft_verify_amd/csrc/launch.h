// Kernel argument blocks and launchers (internal to libdspark.so).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

// One draft step k: L = U[:, k] + W1[prev] . W2 -> per-tile partials.
struct StepArgs {
  int B, V, gamma, k, ntiles;
  const float* U;
  const uint16_t* W1;
  const uint16_t* W2t;
  const int32_t* prev;  // conditioning token of request b at prev[b * prev_stride]
  int prev_stride;
  float2* part;         // [B][ntiles] (tile max, sum exp(L - tile max))
  float* dbg;           // nullable [B][gamma][V] (the logits L, before the temperature)
  int persistent_wgs;   // workgroups of the persistent step kernel (one per compute unit)
  float beta;           // logits are scaled by beta = fp32(1 / temperature) (1: unscaled)
  // Bias rows: 1 = the Markov embedding row W1[prev]; 3 = the RNN head's bias vector of
  // (b, k) as three bf16 terms, E [B][gamma][3r] (prev unused).
  int e_terms = 1;
  const uint16_t* E = nullptr;
  // The same bias rows by MFMA operand (e_terms = 3; nullable): for each block of 32 requests and
  // position, k-step s of the 3r / 16, half h and column c hold 8 bf16 at
  // (((blk * gamma + k) * (3r / 16) + s) * 2 + h) * 256 + 8 c, so a wave's k-step is 1 KB.
  const uint16_t* E2 = nullptr;
  // Rows that share a request's base logits: row b reads U row (b >> u_shift) (tree drafting:
  // the 2^u_shift expanded nodes of one request score their children from the same U_k).
  int u_shift = 0;
};

struct SampleArgs {
  int B, V, gamma, k, ntiles;
  const float* U;
  const uint16_t* W1;
  const uint16_t* W2t;
  const int32_t* prev;
  int prev_stride;
  const float2* part;
  const float* uniforms;
  const int32_t* force;  // nullable [B][gamma]
  int32_t* tokens;
  float* q;
  double* lse;
  float beta;   // as in StepArgs
  int greedy;   // draft the first maximal logit (point-mass q)
  int e_terms = 1;               // as in StepArgs
  const uint16_t* E = nullptr;
};

struct ConfArgs {
  int B, gamma, r, d;
  const uint16_t* h;
  const uint16_t* W1;
  const uint16_t* w;
  const float* T;
  const int32_t* anchor;
  const int32_t* tokens;
  float* conf;
  int V;                  // token ids are clamped into [0, V)
};

struct PlanArgs {
  int B, gamma, sps_len, mode, round_index;
  const float* conf;   // nullable for FULL_VERIFY
  const double* sps;
  float* ring;         // nullable unless LAGGED_TOPK
  int32_t* draft_len;
  int32_t* row_offsets;
  double* stats;       // nullable
};

// Emission kinds written by the accept scan.
enum : int32_t { kEmitBonus = 0, kEmitResidual = 1 };

// One residual emission, appended by the accept scan (in no particular order: the kernels that
// read the list give every request the same result whatever its slot).
struct ResRec {
  int32_t b;       // request
  int32_t j;       // 1-based emission position (the first rejected draft position)
  int32_t erow;    // packed target row of position j
  int32_t prev;    // token before position j (the anchor for j = 1)
  int32_t tok;     // the drafted token of position j (the point mass of a greedy draft)
  double lse_d;    // log-sum-exp of the draft logits of position j
  double lse_t;    // log-sum-exp of the target row
};

struct VerifyWs {
  float* seg_max;    // [B*(gamma+1)][nseg]
  double* seg_sum;   // [B*(gamma+1)][nseg]
  int32_t* ekind;    // [B]
  int32_t* epos;     // [B] 1-based position of the emission
  int32_t* erow;     // [B] packed target row of the emission
  double* erow_lse;  // [B] log-sum-exp of that target row
  uint32_t* eflags;  // [B]
  int32_t* eprev;    // [B] conditioning token of a residual emission's position (its bias row)
  double* rsum;      // [B][ntiles] residual mass per 32-token tile
  double* rmin;      // [B][ntiles] sum of min(p_t, p_d) per tile
  int32_t* rcount;   // [1] residual emissions (zeroed by the target pass, counted by accept)
  ResRec* rrec;      // [B] their records
};

struct VerifyArgs {
  int B, V, gamma, r, ntiles, nseg;
  const float* target;
  const int32_t* row_offsets;
  const int32_t* draft_len;
  const float* U;
  const uint16_t* W1;
  const uint16_t* W2t;
  const int32_t* anchor;
  const int32_t* tokens;
  const float* q;
  const double* lse;
  const float* uniforms;
  int32_t* accept_len;
  int32_t* next_token;
  float* beta_emit;   // nullable
  uint32_t* flags;    // nullable
  int persistent_wgs; // workgroups of the pipelined residual kernel (one per compute unit)
  float beta;         // the draft distribution: softmax(beta L), beta = fp32(1 / temperature)
  int greedy;         // or the point mass on the drafted token (greedy drafts)
  VerifyWs ws;
  int e_terms = 1;               // bias rows as in StepArgs (3: E [B][gamma][3r], in ws)
  const uint16_t* E = nullptr;
  int dense_rows = 0;            // > 0: the target pass takes this many rows (no row_offsets)
  // Nullable: fp32 bias vectors e [B gamma][r] whose bf16 terms the target pass writes to
  // E_split [B gamma][3r] (the E above) before the passes that read them.
  const float* e_split = nullptr;
  uint16_t* E_split = nullptr;
};

// PCTree ([ZDS] "后续工作"). Candidates of a request are numbered depth by depth, and within a
// depth parent by parent (in the order the depth's expanded nodes were ranked) and child by
// child in rank order; T = c + (gamma - 1) M c of them.
constexpr int kTreeMaxRows = 8;        // nodes expanded per request and depth (M)
constexpr int kTreeMaxChildren = 8;    // children per expanded node (c)
constexpr int kTreeMaxCand = 1024;     // candidates per request over all depths (T)
constexpr int kTreeMaxNodes = 256;     // kept nodes per request (N)
struct TreeCandWs {
  int32_t* tok;      // [B][T]
  int32_t* parent;   // [B][T] candidate number of the parent (-1: the root)
  double* P;         // [B][T] path probability
  double* q;         // [B][T] Markov probability of the token under its parent
};
struct TreeSelectArgs {
  int B, V, gamma, k, ntiles;   // k: 0-based depth (the children sit at position k + 1)
  int c, M, rows;               // rows: expanded nodes per request at this depth (1 or M)
  int T, cand_base;             // candidates per request; number of this depth's first one
  const float* U;
  const uint16_t* W1;
  const uint16_t* W2t;
  const int32_t* prev;          // [B rows] token of each expanded node (the anchor at depth 1)
  const double* prevP;          // [B rows] its path probability (nullptr: 1)
  const int32_t* prevCand;      // [B rows] its candidate number (nullptr: the root)
  const float2* part;           // [B rows][ntiles] the step kernel's partials
  TreeCandWs cand;
  int32_t* front_tok;           // [B][M] out: the next depth's expanded nodes (k < gamma - 1)
  double* front_P;
  int32_t* front_cand;
  int last;                     // k == gamma - 1: write the kept nodes instead
  int N;
  int32_t* node_token;          // [B][N] out, rank order
  int32_t* node_depth;
  int32_t* node_parent;
  double* node_q;
  double* node_path;
};
struct TreeWalkArgs {
  int B, V, gamma, N, nseg;
  const float* target;          // [B][N + 1][V]
  const int32_t* node_token;    // [B][N]
  const int32_t* node_parent;   // [B][N]
  const float* uniforms;        // [B][gamma + 1][3]
  const float* seg_max;         // [B (N + 1)][nseg]
  const double* seg_sum;
  int32_t* accept_len;          // [B]
  int32_t* path;                // [B][gamma]
  int32_t* next_token;          // [B]
  uint32_t* flags;              // nullable [B]
};

// RNN head, eq. (6). P [kRnnPreSplits][M][3r] = the hidden-state block of Wgco applied to every
// h_k (M = B gamma rows (b, k)), one part per slice of the hidden dimension (summed in fp64,
// stored as fp32); computed once per round, off the serial chain.
constexpr int kRnnPreSplits = 4;
struct RnnPreArgs {
  int M, r, d;
  const uint16_t* h;      // [M][d] bf16
  const uint16_t* Wgco;   // [3r][2r + d] bf16: rows W_g, W_c, W_o; columns state | embedding | hidden
  float* P;               // [kRnnPreSplits][M][3r]
};

// One step of the RNN state: pre-activations a = P[b][k] + Wgco[:, state] s_{k-1} +
// Wgco[:, embedding] W1[x_{k-1}] (fp64), s_k, e_k = tanh(a_o); e_k as fp32 and as three bf16
// terms (the bias rows of the step kernel).
struct RnnStateArgs {
  int B, gamma, k, r, d;
  const float* P;         // [kRnnPreSplits][M][3r] (rnn_pre)
  const uint16_t* Wgco;
  const uint16_t* W1;
  const int32_t* prev;    // conditioning token of request b at prev[b * prev_stride]
  int prev_stride;
  const double* s_in;     // [B][r] s_{k-1} (ignored at k = 0: s_0 = 0)
  double* s_out;          // [B][r] s_k
  float* e_out;           // [B][gamma][r] e_k (fp32)
  uint16_t* E;            // [B][gamma][3r] bf16 terms of e_k
  uint16_t* E2;           // the same terms by MFMA operand (StepArgs::E2)
  int V;                  // token ids are clamped into [0, V)
};


// Kernel timing: the event pair the next launch records with its dispatch (hipExtLaunchKernel
// start and stop events, taken by the command processor around the kernel itself), or none.
struct LaunchTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
LaunchTiming& launch_timing();   // per host thread

// Every kernel of the library is launched through here.
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                          hipStream_t s, Args... args) {
  LaunchTiming& t = launch_timing();
  if (t.start) {
    hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(shmem), s, t.start, t.stop, 0,
                          args...);
    t = LaunchTiming{};
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
  }
}

hipError_t launch_markov_step(const StepArgs& a, int r, hipStream_t s);
hipError_t launch_draft_sample(const SampleArgs& a, int r, hipStream_t s);
hipError_t launch_confidence(const ConfArgs& a, hipStream_t s);
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
// The last position's draft step with the planner beside it (one launch); fits() says
// whether this shape can take it (else the step and the plan are launched one after the other).
bool markov_step_plan_fits(const StepArgs& a, int r, int B, int gamma);
hipError_t launch_markov_step_plan(const StepArgs& a, const PlanArgs& pa, int r, hipStream_t s);
hipError_t launch_target_stats(const VerifyArgs& a, hipStream_t s);
hipError_t launch_accept(const VerifyArgs& a, hipStream_t s);
hipError_t launch_residual_partials(const VerifyArgs& a, hipStream_t s);
hipError_t launch_emit_sample(const VerifyArgs& a, hipStream_t s);
hipError_t launch_rnn_pre(const RnnPreArgs& a, hipStream_t s);
hipError_t launch_rnn_state(const RnnStateArgs& a, hipStream_t s);
hipError_t launch_tree_select(const TreeSelectArgs& a, int r, hipStream_t s);
hipError_t launch_tree_walk(const TreeWalkArgs& a, hipStream_t s);

}  // namespace dspark
