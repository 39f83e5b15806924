// C ABI of libdspark.so: host-side argument checks, workspace layout and launch order.
// The operations and their sources are documented in include/dspark.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "dspark.h"
#include "device.h"
#include "launch.h"
#include "tiles.h"

namespace dspark {
LaunchTiming& launch_timing() {
  thread_local LaunchTiming t;
  return t;
}
}  // namespace dspark

namespace {

using namespace dspark;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int ntiles_of(int V) { return (V + kTileTokens - 1) / kTileTokens; }
int nseg_of(int V) { return (V + kSegTokens - 1) / kSegTokens; }

bool rank_ok(int r) {
  return r == 16 || r == 32 || r == 64 || r == 128 || r == 256 || r == 512;
}

// B * (gamma + 1) verified rows index grid dimension y of the target pass (<= 65535); the
// planner sorts all B * gamma candidates in one workgroup's LDS (<= 8192).
bool dims_ok(const dspark_dims& d) {
  if (d.B < 1 || d.gamma < 1 || d.gamma > kMaxGamma || d.V < 2 || d.V > kMaxVocab || !rank_ok(d.r))
    return false;
  if (static_cast<int64_t>(d.B) * (d.gamma + 1) > 65535) return false;
  return true;
}
bool plan_dims_ok(const dspark_dims& d) {
  return dims_ok(d) && static_cast<int64_t>(d.B) * d.gamma <= 8192;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Draft options: beta = fp32(1 / temperature) (1 for greedy or no options). False when the
// temperature is not positive and finite.
bool draft_options(const dspark_draft_opts* opts, float* beta, int* greedy) {
  *beta = 1.0f;
  *greedy = 0;
  if (!opts) return true;
  if (opts->greedy) {
    *greedy = 1;
    return true;
  }
  const float t = opts->temperature;
  if (!(t > 0.0f) || !std::isfinite(t)) return false;
  *beta = static_cast<float>(1.0 / static_cast<double>(t));
  return true;
}

// Compute units of the current device (cached per device id).
int compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// ---- workspace layouts ----------------------------------------------------------------------
struct DraftWs {
  float2* part;
};
size_t draft_ws(const dspark_dims& d, void* base, DraftWs* out) {
  const size_t n = static_cast<size_t>(d.B) * ntiles_of(d.V);
  if (out) out->part = static_cast<float2*>(base);
  return align_up(n * sizeof(float2));
}

// RNN-head draft: the step partials, then P [kRnnPreSplits][B gamma][3r] fp32 (slices of the
// hidden block), the state ping-pong [2][B][r] fp64 and the bias rows E [B gamma][3r] bf16.
struct RnnDraftWs {
  DraftWs draft;
  float* P;
  double* s[2];
  uint16_t* E;
  uint16_t* E2;   // the bias terms by MFMA operand, [ceil(B / 32)][gamma][3r / 16][2][32][8]
};
size_t rnn_draft_ws(const dspark_dims& d, void* base, RnnDraftWs* out) {
  const size_t M = static_cast<size_t>(d.B) * d.gamma;
  char* b = static_cast<char*>(base);
  size_t off = draft_ws(d, base, out ? &out->draft : nullptr);
  auto take = [&](size_t bytes) {
    char* p = b ? b + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  char* P = take(static_cast<size_t>(kRnnPreSplits) * M * 3 * d.r * sizeof(float));
  char* s0 = take(static_cast<size_t>(d.B) * d.r * sizeof(double));
  char* s1 = take(static_cast<size_t>(d.B) * d.r * sizeof(double));
  char* E = take(M * kRnnTerms * d.r * sizeof(uint16_t));
  const size_t nblk = (static_cast<size_t>(d.B) + 31) / 32;
  char* E2 = take(nblk * 32 * d.gamma * kRnnTerms * d.r * sizeof(uint16_t));
  if (out) {
    out->P = reinterpret_cast<float*>(P);
    out->s[0] = reinterpret_cast<double*>(s0);
    out->s[1] = reinterpret_cast<double*>(s1);
    out->E = reinterpret_cast<uint16_t*>(E);
    out->E2 = reinterpret_cast<uint16_t*>(E2);
  }
  return off;
}

size_t verify_ws(const dspark_dims& d, void* base, VerifyWs* out) {
  const size_t rows = static_cast<size_t>(d.B) * (d.gamma + 1);
  const size_t nseg = nseg_of(d.V), nt = ntiles_of(d.V), B = d.B;
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t bytes) {   // a null base only sizes the layout
    char* p = b ? b + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  VerifyWs w;
  w.seg_max = reinterpret_cast<float*>(take(rows * nseg * sizeof(float)));
  w.seg_sum = reinterpret_cast<double*>(take(rows * nseg * sizeof(double)));
  w.ekind = reinterpret_cast<int32_t*>(take(B * sizeof(int32_t)));
  w.epos = reinterpret_cast<int32_t*>(take(B * sizeof(int32_t)));
  w.erow = reinterpret_cast<int32_t*>(take(B * sizeof(int32_t)));
  w.erow_lse = reinterpret_cast<double*>(take(B * sizeof(double)));
  w.eflags = reinterpret_cast<uint32_t*>(take(B * sizeof(uint32_t)));
  w.eprev = reinterpret_cast<int32_t*>(take(B * sizeof(int32_t)));
  w.rsum = reinterpret_cast<double*>(take(B * nt * sizeof(double)));
  w.rmin = reinterpret_cast<double*>(take(B * nt * sizeof(double)));
  w.rcount = reinterpret_cast<int32_t*>(take(sizeof(int32_t)));
  w.rrec = reinterpret_cast<ResRec*>(take(B * sizeof(ResRec)));
  if (out) *out = w;
  return off;
}

// Verify of an RNN-head draft: the verify workspace, then the bias rows E [B gamma][3r] bf16.
size_t rnn_verify_ws(const dspark_dims& d, void* base, VerifyWs* out, uint16_t** E) {
  const size_t off = verify_ws(d, base, out);
  if (E) *E = base ? reinterpret_cast<uint16_t*>(static_cast<char*>(base) + off) : nullptr;
  return off + align_up(static_cast<size_t>(d.B) * d.gamma * kRnnTerms * d.r * sizeof(uint16_t));
}

// ---- PCTree ------------------------------------------------------------------------------
// Candidates of a request: c at depth 1, M c at every later depth (M <= c).
int64_t tree_candidates(const dspark_dims& d, const dspark_tree_shape& t) {
  return static_cast<int64_t>(t.c) + static_cast<int64_t>(d.gamma - 1) * t.M * t.c;
}
bool tree_shape_ok(const dspark_dims& d, const dspark_tree_shape& t) {
  if (!dims_ok(d) || d.r > 256) return false;
  if (t.c < 1 || t.c > kTreeMaxChildren || t.c > d.V) return false;
  if (t.M < 1 || t.M > t.c || (t.M & (t.M - 1)) != 0) return false;
  const int64_t T = tree_candidates(d, t);
  if (T > kTreeMaxCand || t.N < 1 || t.N > T || t.N > kTreeMaxNodes) return false;
  // a select workgroup gives each expanded node 1024 / M threads of at most 32 tile partials
  if (static_cast<int64_t>(ntiles_of(d.V)) > 32LL * (1024 / t.M)) return false;
  return static_cast<int64_t>(d.B) * (t.N + 1) <= (1LL << 24);
}
struct TreeDraftWs {
  float2* part;
  int32_t* ftok[2];
  double* fP[2];
  int32_t* fcand[2];
  TreeCandWs cand;
};
size_t tree_draft_ws(const dspark_dims& d, const dspark_tree_shape& t, void* base, TreeDraftWs* out) {
  const size_t B = d.B, M = t.M, T = static_cast<size_t>(tree_candidates(d, t));
  char* b = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = b ? b + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  TreeDraftWs w;
  w.part = reinterpret_cast<float2*>(take(B * M * ntiles_of(d.V) * sizeof(float2)));
  for (int i = 0; i < 2; ++i) {
    w.ftok[i] = reinterpret_cast<int32_t*>(take(B * M * sizeof(int32_t)));
    w.fP[i] = reinterpret_cast<double*>(take(B * M * sizeof(double)));
    w.fcand[i] = reinterpret_cast<int32_t*>(take(B * M * sizeof(int32_t)));
  }
  w.cand.tok = reinterpret_cast<int32_t*>(take(B * T * sizeof(int32_t)));
  w.cand.parent = reinterpret_cast<int32_t*>(take(B * T * sizeof(int32_t)));
  w.cand.P = reinterpret_cast<double*>(take(B * T * sizeof(double)));
  w.cand.q = reinterpret_cast<double*>(take(B * T * sizeof(double)));
  if (out) *out = w;
  return off;
}
// Tree verify: the segment statistics of the B (N + 1) rows (and the target pass's counter).
size_t tree_verify_ws(const dspark_dims& d, const dspark_tree_shape& t, void* base, VerifyWs* out) {
  const size_t rows = static_cast<size_t>(d.B) * (t.N + 1), nseg = nseg_of(d.V);
  char* b = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = b ? b + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  VerifyWs w{};
  w.seg_max = reinterpret_cast<float*>(take(rows * nseg * sizeof(float)));
  w.seg_sum = reinterpret_cast<double*>(take(rows * nseg * sizeof(double)));
  w.rcount = reinterpret_cast<int32_t*>(take(sizeof(int32_t)));
  if (out) *out = w;
  return off;
}

// The RNN head needs the hidden states (d a positive multiple of 8) and r <= 256 (the three
// bf16 terms of a bias row fill at most two 1 KB copies of one wave).
bool rnn_dims_ok(const dspark_dims& d) { return dims_ok(d) && d.r <= 256 && d.d >= 8 && d.d % 8 == 0; }

// ---- kernel timing ----------------------------------------------------------------------------
enum KernelId {
  kMarkovStep = 0,
  kDraftSample,
  kConfidence,
  kPlan,
  kTargetStats,
  kAccept,
  kResidualPartials,
  kEmitSample,
  kRnnPre,
  kRnnState,
  kTreeSelect,
  kTreeWalk,
  kNumKernels
};
const char* const kKernelNames[kNumKernels] = {"markov_step",  "draft_sample", "confidence",
                                               "plan",         "target_stats", "accept",
                                               "residual_partials", "emit_sample",
                                               "rnn_pre",      "rnn_state",
                                               "tree_select",  "tree_walk"};

struct Profiler {
  bool armed = false;
  int capacity = 0;
  int used = 0;
  std::vector<hipEvent_t> events;
  std::vector<int> ids;
};
Profiler g_prof;

// While the profiler is armed, the launch made by `launch` records the next event pair with
// its dispatch (launch_kernel); if it launched nothing, the pair is recorded back to back.
template <class F>
hipError_t timed(KernelId id, hipStream_t s, F launch) {
  const bool rec = g_prof.armed && g_prof.used < g_prof.capacity;
  LaunchTiming& t = launch_timing();
  if (rec) t = LaunchTiming{g_prof.events[2 * g_prof.used], g_prof.events[2 * g_prof.used + 1]};
  const hipError_t e = launch();
  if (rec) {
    if (t.start) {
      (void)hipEventRecord(t.start, s);
      (void)hipEventRecord(t.stop, s);
      t = LaunchTiming{};
    }
    g_prof.ids[g_prof.used] = id;
    ++g_prof.used;
  }
  return e;
}

// The serial draft loop shared by the two heads: per position the bias step (bias rows from
// W1[prev], or from E after the RNN state step) and the sampler.
struct RnnDraftInputs {
  const uint16_t* Wgco;
  const uint16_t* h;
  float* e_rows;
  RnnDraftWs w;
};

// The confidence head and the plan of a round, when the draft call also makes them: they need
// only the tokens before the last position, so they are launched before the last step, and the
// plan runs on one workgroup of that step's launch where the shape allows.
struct RoundPlan {
  ConfArgs conf;
  PlanArgs plan;
};

dspark_status draft_loop(const dspark_dims& dims, const float* U, const uint16_t* W1,
                         const uint16_t* W2t, const int32_t* anchor, const float* uniforms,
                         int32_t* tokens, float* q_tok, double* lse, float* logits_dbg,
                         const int32_t* force_tokens, float2* part, float beta, int greedy,
                         const RnnDraftInputs* rnn, hipStream_t s,
                         const RoundPlan* round_plan = nullptr) {
  const int nt = ntiles_of(dims.V);
  const int cus = compute_units();
  if (rnn) {
    RnnPreArgs pa{dims.B * dims.gamma, dims.r, dims.d, rnn->h, rnn->Wgco, rnn->w.P};
    if (timed(kRnnPre, s, [&] { return launch_rnn_pre(pa, s); }) != hipSuccess)
      return DSPARK_ERR_HIP;
  }
  for (int k = 0; k < dims.gamma; ++k) {
    const int32_t* prev = anchor;
    int stride = 1;
    if (k > 0) {
      prev = (force_tokens ? force_tokens : tokens) + (k - 1);
      stride = dims.gamma;
    }
    if (rnn) {
      RnnStateArgs ra{dims.B,        dims.gamma,       k,          dims.r,
                      dims.d,        rnn->w.P,         rnn->Wgco,  W1,
                      prev,          stride,           k > 0 ? rnn->w.s[(k + 1) & 1] : nullptr,
                      rnn->w.s[k & 1], rnn->e_rows,    rnn->w.E,   rnn->w.E2,
                      dims.V};
      if (timed(kRnnState, s, [&] { return launch_rnn_state(ra, s); }) != hipSuccess)
        return DSPARK_ERR_HIP;
    }
    StepArgs sa{dims.B, dims.V, dims.gamma, k, nt, U, W1, W2t, prev, stride, part, logits_dbg,
                cus, beta};
    SampleArgs pa{dims.B, dims.V, dims.gamma, k, nt, U, W1, W2t, prev, stride, part,
                  uniforms, force_tokens, tokens, q_tok, lse, beta, greedy};
    if (rnn) {
      sa.e_terms = pa.e_terms = kRnnTerms;
      sa.E = pa.E = rnn->w.E;
      sa.E2 = rnn->w.E2;
    }
    if (round_plan && k == dims.gamma - 1) {
      if (timed(kConfidence, s, [&] { return launch_confidence(round_plan->conf, s); }) !=
          hipSuccess)
        return DSPARK_ERR_HIP;
      if (markov_step_plan_fits(sa, dims.r, dims.B, dims.gamma)) {
        if (timed(kMarkovStep, s, [&] {
              return launch_markov_step_plan(sa, round_plan->plan, dims.r, s);
            }) != hipSuccess)
          return DSPARK_ERR_HIP;
      } else {
        if (timed(kPlan, s, [&] { return launch_plan(round_plan->plan, s); }) != hipSuccess)
          return DSPARK_ERR_HIP;
        if (timed(kMarkovStep, s, [&] { return launch_markov_step(sa, dims.r, s); }) !=
            hipSuccess)
          return DSPARK_ERR_HIP;
      }
    } else if (timed(kMarkovStep, s, [&] { return launch_markov_step(sa, dims.r, s); }) !=
               hipSuccess) {
      return DSPARK_ERR_HIP;
    }
    if (timed(kDraftSample, s, [&] { return launch_draft_sample(pa, dims.r, s); }) != hipSuccess)
      return DSPARK_ERR_HIP;
  }
  return DSPARK_OK;
}

// The four verify passes, shared by the two heads (bias rows from W1[prev], or E).
dspark_status verify_passes(const dspark_dims& dims, VerifyArgs& a, hipStream_t s) {
  if (timed(kTargetStats, s, [&] { return launch_target_stats(a, s); }) != hipSuccess)
    return DSPARK_ERR_HIP;
  if (timed(kAccept, s, [&] { return launch_accept(a, s); }) != hipSuccess) return DSPARK_ERR_HIP;
  if (timed(kResidualPartials, s, [&] { return launch_residual_partials(a, s); }) != hipSuccess)
    return DSPARK_ERR_HIP;
  if (timed(kEmitSample, s, [&] { return launch_emit_sample(a, s); }) != hipSuccess)
    return DSPARK_ERR_HIP;
  (void)dims;
  return DSPARK_OK;
}

// Argument checks of the confidence head and of the planner (shared by their own entry points
// and the draft call that also makes them).
dspark_status check_confidence(const dspark_dims& dims, const uint16_t* h, const uint16_t* W1,
                               const uint16_t* w, const float* T, const int32_t* anchor,
                               const int32_t* tokens, const float* conf) {
  if (!h || !W1 || !w || !T || !anchor || !tokens || !conf) return DSPARK_ERR_NULL;
  if (!dims_ok(dims) || dims.d < 8 || dims.d % 8 != 0) return DSPARK_ERR_SHAPE;
  if (!aligned(h, 16) || !aligned(W1, 16) || !aligned(w, 16) || !aligned(T, 4) ||
      !aligned(anchor, 4) || !aligned(tokens, 4) || !aligned(conf, 4))
    return DSPARK_ERR_ALIGN;
  return DSPARK_OK;
}

dspark_status check_plan(const dspark_dims& dims, const float* conf, const double* sps,
                         int32_t sps_len, int32_t mode, const float* ring, int32_t round_index,
                         const int32_t* draft_len, const int32_t* row_offsets,
                         const double* stats) {
  if (!sps || !draft_len || !row_offsets) return DSPARK_ERR_NULL;
  if (mode < DSPARK_PLAN_FULL_VERIFY || mode > DSPARK_PLAN_LAGGED_TOPK) return DSPARK_ERR_MODE;
  if (mode != DSPARK_PLAN_FULL_VERIFY && !conf) return DSPARK_ERR_NULL;
  if (mode == DSPARK_PLAN_LAGGED_TOPK && !ring) return DSPARK_ERR_MODE;
  if (!plan_dims_ok(dims) || round_index < 0) return DSPARK_ERR_SHAPE;
  if (static_cast<int64_t>(sps_len) < static_cast<int64_t>(dims.B) * (dims.gamma + 1) + 1)
    return DSPARK_ERR_SPS;
  if ((conf && !aligned(conf, 4)) || !aligned(sps, 8) || (ring && !aligned(ring, 4)) ||
      !aligned(draft_len, 4) || !aligned(row_offsets, 4) || (stats && !aligned(stats, 8)))
    return DSPARK_ERR_ALIGN;
  return DSPARK_OK;
}

// Scratch space of dspark_verify_noalloc: a fixed array in device memory, one copy per GPU
// (each device that loads the library holds its own, until the process ends). Host code never
// passes the array's name to a kernel: that is a host-side stand-in, not a device address. The
// device address of the current device's copy comes from hipGetSymbolAddress, once per device,
// and is kept here.
constexpr size_t kScratchBytes = DSPARK_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, or nullptr if HIP cannot give it.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* dspark_status_string(dspark_status s) {
  switch (s) {
    case DSPARK_OK: return "ok";
    case DSPARK_ERR_NULL: return "a required pointer is NULL";
    case DSPARK_ERR_SHAPE: return "a size is out of the supported range";
    case DSPARK_ERR_ALIGN: return "a pointer is not aligned";
    case DSPARK_ERR_WORKSPACE: return "workspace too small";
    case DSPARK_ERR_SPS: return "SPS table shorter than B * (gamma + 1) + 1";
    case DSPARK_ERR_HIP: return "HIP launch failed";
    case DSPARK_ERR_MODE: return "unknown plan mode or missing ring";
    case DSPARK_ERR_OPTS: return "draft temperature not positive and finite";
    default: return "unknown status";
  }
}

const char* dspark_version(void) { return "dspark-gfx950 0.1"; }

size_t dspark_workspace_bytes(dspark_dims dims, int32_t op) {
  if (!dims_ok(dims)) return static_cast<size_t>(-1);
  switch (op) {
    case DSPARK_OP_DRAFT: return draft_ws(dims, nullptr, nullptr);
    case DSPARK_OP_CONFIDENCE: return 0;
    case DSPARK_OP_PLAN: return 0;
    case DSPARK_OP_VERIFY: return verify_ws(dims, nullptr, nullptr);
    case DSPARK_OP_RNN_DRAFT:
      return rnn_dims_ok(dims) ? rnn_draft_ws(dims, nullptr, nullptr) : static_cast<size_t>(-1);
    case DSPARK_OP_RNN_VERIFY:
      return rnn_dims_ok(dims) ? rnn_verify_ws(dims, nullptr, nullptr, nullptr)
                               : static_cast<size_t>(-1);
    default: return static_cast<size_t>(-1);
  }
}

dspark_status dspark_markov_draft_opts(dspark_dims dims, const float* U, const uint16_t* W1,
                                       const uint16_t* W2t, const int32_t* anchor,
                                       const float* uniforms, int32_t* tokens, float* q_tok,
                                       double* lse, float* logits_dbg,
                                       const int32_t* force_tokens, void* ws, size_t ws_bytes,
                                       const dspark_draft_opts* opts, void* stream) {
  if (!U || !W1 || !W2t || !anchor || !uniforms || !tokens || !q_tok || !lse || !ws)
    return DSPARK_ERR_NULL;
  float beta = 1.0f;
  int greedy = 0;
  if (!draft_options(opts, &beta, &greedy)) return DSPARK_ERR_OPTS;
  if (!dims_ok(dims)) return DSPARK_ERR_SHAPE;
  if (!aligned(U, 16) || !aligned(W1, 16) || !aligned(W2t, 16) || !aligned(anchor, 4) ||
      !aligned(uniforms, 4) || !aligned(tokens, 4) || !aligned(q_tok, 4) || !aligned(lse, 8) ||
      (logits_dbg && !aligned(logits_dbg, 4)) || (force_tokens && !aligned(force_tokens, 4)) ||
      !aligned(ws, kAlign))
    return DSPARK_ERR_ALIGN;
  if (ws_bytes < draft_ws(dims, nullptr, nullptr)) return DSPARK_ERR_WORKSPACE;
  DraftWs w;
  draft_ws(dims, ws, &w);
  return draft_loop(dims, U, W1, W2t, anchor, uniforms, tokens, q_tok, lse, logits_dbg,
                    force_tokens, w.part, beta, greedy, nullptr, static_cast<hipStream_t>(stream));
}

dspark_status dspark_rnn_draft(dspark_dims dims, const float* U, const uint16_t* W1,
                               const uint16_t* W2t, const uint16_t* Wgco, const uint16_t* h,
                               const int32_t* anchor, const float* uniforms, int32_t* tokens,
                               float* q_tok, double* lse, float* e_rows, float* logits_dbg,
                               const int32_t* force_tokens, void* ws, size_t ws_bytes,
                               const dspark_draft_opts* opts, void* stream) {
  if (!U || !W1 || !W2t || !Wgco || !h || !anchor || !uniforms || !tokens || !q_tok || !lse ||
      !e_rows || !ws)
    return DSPARK_ERR_NULL;
  float beta = 1.0f;
  int greedy = 0;
  if (!draft_options(opts, &beta, &greedy)) return DSPARK_ERR_OPTS;
  if (!rnn_dims_ok(dims)) return DSPARK_ERR_SHAPE;
  if (!aligned(U, 16) || !aligned(W1, 16) || !aligned(W2t, 16) || !aligned(Wgco, 16) ||
      !aligned(h, 16) || !aligned(anchor, 4) || !aligned(uniforms, 4) || !aligned(tokens, 4) ||
      !aligned(q_tok, 4) || !aligned(lse, 8) || !aligned(e_rows, 4) ||
      (logits_dbg && !aligned(logits_dbg, 4)) || (force_tokens && !aligned(force_tokens, 4)) ||
      !aligned(ws, kAlign))
    return DSPARK_ERR_ALIGN;
  if (ws_bytes < rnn_draft_ws(dims, nullptr, nullptr)) return DSPARK_ERR_WORKSPACE;
  RnnDraftInputs rnn{Wgco, h, e_rows, {}};
  rnn_draft_ws(dims, ws, &rnn.w);
  return draft_loop(dims, U, W1, W2t, anchor, uniforms, tokens, q_tok, lse, logits_dbg,
                    force_tokens, rnn.w.draft.part, beta, greedy, &rnn,
                    static_cast<hipStream_t>(stream));
}

dspark_status dspark_rnn_draft_plan(dspark_dims dims, const float* U, const uint16_t* W1,
                                    const uint16_t* W2t, const uint16_t* Wgco, const uint16_t* h,
                                    const int32_t* anchor, const float* uniforms,
                                    const uint16_t* w, const float* T, const double* sps,
                                    int32_t sps_len, int32_t mode, float* ring,
                                    int32_t round_index, int32_t* tokens, float* q_tok,
                                    double* lse, float* e_rows, float* conf, int32_t* draft_len,
                                    int32_t* row_offsets, double* stats, void* ws,
                                    size_t ws_bytes, const dspark_draft_opts* opts, void* stream) {
  if (!U || !W2t || !Wgco || !uniforms || !q_tok || !lse || !e_rows || !ws) return DSPARK_ERR_NULL;
  dspark_status st = check_confidence(dims, h, W1, w, T, anchor, tokens, conf);
  if (st != DSPARK_OK) return st;
  st = check_plan(dims, conf, sps, sps_len, mode, ring, round_index, draft_len, row_offsets, stats);
  if (st != DSPARK_OK) return st;
  float beta = 1.0f;
  int greedy = 0;
  if (!draft_options(opts, &beta, &greedy)) return DSPARK_ERR_OPTS;
  if (!rnn_dims_ok(dims)) return DSPARK_ERR_SHAPE;
  if (!aligned(U, 16) || !aligned(W2t, 16) || !aligned(Wgco, 16) || !aligned(uniforms, 4) ||
      !aligned(q_tok, 4) || !aligned(lse, 8) || !aligned(e_rows, 4) || !aligned(ws, kAlign))
    return DSPARK_ERR_ALIGN;
  if (ws_bytes < rnn_draft_ws(dims, nullptr, nullptr)) return DSPARK_ERR_WORKSPACE;
  RnnDraftInputs rnn{Wgco, h, e_rows, {}};
  rnn_draft_ws(dims, ws, &rnn.w);
  const RoundPlan rp{{dims.B, dims.gamma, dims.r, dims.d, h, W1, w, T, anchor, tokens, conf, dims.V},
                     {dims.B, dims.gamma, sps_len, mode, round_index, conf, sps, ring, draft_len,
                      row_offsets, stats}};
  return draft_loop(dims, U, W1, W2t, anchor, uniforms, tokens, q_tok, lse, nullptr, nullptr,
                    rnn.w.draft.part, beta, greedy, &rnn, static_cast<hipStream_t>(stream), &rp);
}

dspark_status dspark_markov_draft(dspark_dims dims, const float* U, const uint16_t* W1,
                                  const uint16_t* W2t, const int32_t* anchor,
                                  const float* uniforms, int32_t* tokens, float* q_tok,
                                  double* lse, float* logits_dbg, const int32_t* force_tokens,
                                  void* ws, size_t ws_bytes, void* stream) {
  return dspark_markov_draft_opts(dims, U, W1, W2t, anchor, uniforms, tokens, q_tok, lse,
                                  logits_dbg, force_tokens, ws, ws_bytes, nullptr, stream);
}

dspark_status dspark_confidence(dspark_dims dims, const uint16_t* h, const uint16_t* W1,
                                const uint16_t* w, const float* T, const int32_t* anchor,
                                const int32_t* tokens, float* conf, void* stream) {
  const dspark_status st = check_confidence(dims, h, W1, w, T, anchor, tokens, conf);
  if (st != DSPARK_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ConfArgs a{dims.B, dims.gamma, dims.r, dims.d, h, W1, w, T, anchor, tokens, conf, dims.V};
  if (timed(kConfidence, s, [&] { return launch_confidence(a, s); }) != hipSuccess)
    return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

dspark_status dspark_plan(dspark_dims dims, const float* conf, const double* sps, int32_t sps_len,
                          int32_t mode, float* ring, int32_t round_index, int32_t* draft_len,
                          int32_t* row_offsets, double* stats, void* stream) {
  const dspark_status st =
      check_plan(dims, conf, sps, sps_len, mode, ring, round_index, draft_len, row_offsets, stats);
  if (st != DSPARK_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  PlanArgs a{dims.B, dims.gamma, sps_len, mode, round_index, conf, sps, ring, draft_len,
             row_offsets, stats};
  if (timed(kPlan, s, [&] { return launch_plan(a, s); }) != hipSuccess) return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

dspark_status dspark_markov_draft_plan(dspark_dims dims, const float* U, const uint16_t* W1,
                                       const uint16_t* W2t, const int32_t* anchor,
                                       const float* uniforms, const uint16_t* h,
                                       const uint16_t* w, const float* T, const double* sps,
                                       int32_t sps_len, int32_t mode, float* ring,
                                       int32_t round_index, int32_t* tokens, float* q_tok,
                                       double* lse, float* conf, int32_t* draft_len,
                                       int32_t* row_offsets, double* stats, void* ws,
                                       size_t ws_bytes, const dspark_draft_opts* opts,
                                       void* stream) {
  if (!U || !W2t || !uniforms || !q_tok || !lse || !ws) return DSPARK_ERR_NULL;
  dspark_status st = check_confidence(dims, h, W1, w, T, anchor, tokens, conf);
  if (st != DSPARK_OK) return st;
  st = check_plan(dims, conf, sps, sps_len, mode, ring, round_index, draft_len, row_offsets, stats);
  if (st != DSPARK_OK) return st;
  float beta = 1.0f;
  int greedy = 0;
  if (!draft_options(opts, &beta, &greedy)) return DSPARK_ERR_OPTS;
  if (!aligned(U, 16) || !aligned(W2t, 16) || !aligned(uniforms, 4) || !aligned(q_tok, 4) ||
      !aligned(lse, 8) || !aligned(ws, kAlign))
    return DSPARK_ERR_ALIGN;
  if (ws_bytes < draft_ws(dims, nullptr, nullptr)) return DSPARK_ERR_WORKSPACE;
  DraftWs dw;
  draft_ws(dims, ws, &dw);
  const RoundPlan rp{{dims.B, dims.gamma, dims.r, dims.d, h, W1, w, T, anchor, tokens, conf, dims.V},
                     {dims.B, dims.gamma, sps_len, mode, round_index, conf, sps, ring, draft_len,
                      row_offsets, stats}};
  return draft_loop(dims, U, W1, W2t, anchor, uniforms, tokens, q_tok, lse, nullptr, nullptr,
                    dw.part, beta, greedy, nullptr, static_cast<hipStream_t>(stream), &rp);
}

dspark_status dspark_verify_opts(dspark_dims dims, const float* target,
                                 const int32_t* row_offsets, const int32_t* draft_len,
                                 const float* U, const uint16_t* W1, const uint16_t* W2t,
                                 const int32_t* anchor, const int32_t* tokens, const float* q_tok,
                                 const double* lse, const float* uniforms, int32_t* accept_len,
                                 int32_t* next_token, float* beta_emit, uint32_t* flags, void* ws,
                                 size_t ws_bytes, const dspark_draft_opts* opts, void* stream) {
  if (!target || !row_offsets || !draft_len || !U || !W1 || !W2t || !anchor || !tokens ||
      !q_tok || !lse || !uniforms || !accept_len || !next_token || !ws)
    return DSPARK_ERR_NULL;
  float beta = 1.0f;
  int greedy = 0;
  if (!draft_options(opts, &beta, &greedy)) return DSPARK_ERR_OPTS;
  if (!dims_ok(dims)) return DSPARK_ERR_SHAPE;
  if (!aligned(target, 16) || !aligned(U, 16) || !aligned(W1, 16) || !aligned(W2t, 16) ||
      !aligned(row_offsets, 4) || !aligned(draft_len, 4) || !aligned(anchor, 4) ||
      !aligned(tokens, 4) || !aligned(q_tok, 4) || !aligned(lse, 8) || !aligned(uniforms, 4) ||
      !aligned(accept_len, 4) || !aligned(next_token, 4) || (beta_emit && !aligned(beta_emit, 4)) ||
      (flags && !aligned(flags, 4)) || !aligned(ws, kAlign))
    return DSPARK_ERR_ALIGN;
  if (ws_bytes < verify_ws(dims, nullptr, nullptr)) return DSPARK_ERR_WORKSPACE;
  VerifyArgs a;
  a.B = dims.B;
  a.V = dims.V;
  a.gamma = dims.gamma;
  a.r = dims.r;
  a.ntiles = ntiles_of(dims.V);
  a.nseg = nseg_of(dims.V);
  a.target = target;
  a.row_offsets = row_offsets;
  a.draft_len = draft_len;
  a.U = U;
  a.W1 = W1;
  a.W2t = W2t;
  a.anchor = anchor;
  a.tokens = tokens;
  a.q = q_tok;
  a.lse = lse;
  a.uniforms = uniforms;
  a.accept_len = accept_len;
  a.next_token = next_token;
  a.beta_emit = beta_emit;
  a.flags = flags;
  a.persistent_wgs = compute_units();
  a.beta = beta;
  a.greedy = greedy;
  verify_ws(dims, ws, &a.ws);
  return verify_passes(dims, a, static_cast<hipStream_t>(stream));
}

size_t dspark_tree_workspace_bytes(dspark_dims dims, dspark_tree_shape shape, int32_t op) {
  if (!tree_shape_ok(dims, shape)) return static_cast<size_t>(-1);
  if (op == DSPARK_OP_TREE_DRAFT) return tree_draft_ws(dims, shape, nullptr, nullptr);
  if (op == DSPARK_OP_TREE_VERIFY) return tree_verify_ws(dims, shape, nullptr, nullptr);
  return static_cast<size_t>(-1);
}

dspark_status dspark_tree_draft(dspark_dims dims, dspark_tree_shape shape, const float* U,
                                const uint16_t* W1, const uint16_t* W2t, const int32_t* anchor,
                                int32_t* node_token, int32_t* node_depth, int32_t* node_parent,
                                double* node_q, double* node_path, void* ws, size_t ws_bytes,
                                void* stream) {
  if (!U || !W1 || !W2t || !anchor || !node_token || !node_depth || !node_parent || !node_q ||
      !node_path || !ws)
    return DSPARK_ERR_NULL;
  if (!tree_shape_ok(dims, shape)) return DSPARK_ERR_SHAPE;
  if (!aligned(U, 16) || !aligned(W1, 16) || !aligned(W2t, 16) || !aligned(anchor, 4) ||
      !aligned(node_token, 4) || !aligned(node_depth, 4) || !aligned(node_parent, 4) ||
      !aligned(node_q, 8) || !aligned(node_path, 8) || !aligned(ws, kAlign))
    return DSPARK_ERR_ALIGN;
  if (ws_bytes < tree_draft_ws(dims, shape, nullptr, nullptr)) return DSPARK_ERR_WORKSPACE;
  TreeDraftWs w;
  tree_draft_ws(dims, shape, ws, &w);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nt = ntiles_of(dims.V);
  const int cus = compute_units();
  const int T = static_cast<int>(tree_candidates(dims, shape));
  int shift = 0;
  while ((1 << shift) < shape.M) ++shift;
  for (int k = 0; k < dims.gamma; ++k) {
    const int rows = (k == 0) ? 1 : shape.M;
    const int pb = (k + 1) & 1;   // buffer the previous depth's select wrote (k - 1) & 1
    const int32_t* prev = (k == 0) ? anchor : w.ftok[pb];
    StepArgs sa{dims.B * rows, dims.V, dims.gamma, k, nt, U, W1, W2t, prev, 1, w.part, nullptr,
                cus, 1.0f};
    sa.u_shift = (k == 0) ? 0 : shift;
    if (timed(kMarkovStep, s, [&] { return launch_markov_step(sa, dims.r, s); }) != hipSuccess)
      return DSPARK_ERR_HIP;
    TreeSelectArgs ta{};
    ta.B = dims.B;
    ta.V = dims.V;
    ta.gamma = dims.gamma;
    ta.k = k;
    ta.ntiles = nt;
    ta.c = shape.c;
    ta.M = shape.M;
    ta.rows = rows;
    ta.T = T;
    ta.cand_base = (k == 0) ? 0 : shape.c + (k - 1) * shape.M * shape.c;
    ta.U = U;
    ta.W1 = W1;
    ta.W2t = W2t;
    ta.prev = prev;
    ta.prevP = (k == 0) ? nullptr : w.fP[pb];
    ta.prevCand = (k == 0) ? nullptr : w.fcand[pb];
    ta.part = w.part;
    ta.cand = w.cand;
    ta.front_tok = w.ftok[k & 1];
    ta.front_P = w.fP[k & 1];
    ta.front_cand = w.fcand[k & 1];
    ta.last = (k == dims.gamma - 1) ? 1 : 0;
    ta.N = shape.N;
    ta.node_token = node_token;
    ta.node_depth = node_depth;
    ta.node_parent = node_parent;
    ta.node_q = node_q;
    ta.node_path = node_path;
    if (timed(kTreeSelect, s, [&] { return launch_tree_select(ta, dims.r, s); }) != hipSuccess)
      return DSPARK_ERR_HIP;
  }
  return DSPARK_OK;
}

dspark_status dspark_tree_verify(dspark_dims dims, dspark_tree_shape shape, const float* target,
                                 const int32_t* node_token, const int32_t* node_parent,
                                 const float* uniforms, int32_t* accept_len, int32_t* path,
                                 int32_t* next_token, uint32_t* flags, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (!target || !node_token || !node_parent || !uniforms || !accept_len || !path ||
      !next_token || !ws)
    return DSPARK_ERR_NULL;
  if (!tree_shape_ok(dims, shape)) return DSPARK_ERR_SHAPE;
  if (!aligned(target, 16) || !aligned(node_token, 4) || !aligned(node_parent, 4) ||
      !aligned(uniforms, 4) || !aligned(accept_len, 4) || !aligned(path, 4) ||
      !aligned(next_token, 4) || (flags && !aligned(flags, 4)) || !aligned(ws, kAlign))
    return DSPARK_ERR_ALIGN;
  if (ws_bytes < tree_verify_ws(dims, shape, nullptr, nullptr)) return DSPARK_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  VerifyArgs a;
  a.B = dims.B;
  a.V = dims.V;
  a.gamma = dims.gamma;
  a.r = dims.r;
  a.ntiles = ntiles_of(dims.V);
  a.nseg = nseg_of(dims.V);
  a.target = target;
  a.row_offsets = nullptr;
  a.dense_rows = dims.B * (shape.N + 1);
  a.persistent_wgs = compute_units();
  tree_verify_ws(dims, shape, ws, &a.ws);
  if (timed(kTargetStats, s, [&] { return launch_target_stats(a, s); }) != hipSuccess)
    return DSPARK_ERR_HIP;
  TreeWalkArgs wa{dims.B, dims.V, dims.gamma, shape.N, a.nseg, target, node_token, node_parent,
                  uniforms, a.ws.seg_max, a.ws.seg_sum, accept_len, path, next_token, flags};
  if (timed(kTreeWalk, s, [&] { return launch_tree_walk(wa, s); }) != hipSuccess)
    return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

dspark_status dspark_verify_noalloc(dspark_dims dims, const float* target,
                                    const int32_t* row_offsets, const int32_t* draft_len,
                                    const float* U, const uint16_t* W1, const uint16_t* W2t,
                                    const int32_t* anchor, const int32_t* tokens,
                                    const float* q_tok, const double* lse, const float* uniforms,
                                    int32_t* accept_len, int32_t* next_token, float* beta_emit,
                                    uint32_t* flags, const dspark_draft_opts* opts, void* stream) {
  // Sizes beyond the scratch array are refused before its address is looked up; the other
  // checks are those of dspark_verify_opts, which runs the call on the array.
  if (!dims_ok(dims)) return DSPARK_ERR_SHAPE;
  if (verify_ws(dims, nullptr, nullptr) > kScratchBytes) return DSPARK_ERR_WORKSPACE;
  if (!target || !row_offsets || !draft_len || !U || !W1 || !W2t || !anchor || !tokens ||
      !q_tok || !lse || !uniforms || !accept_len || !next_token)
    return DSPARK_ERR_NULL;
  void* ws = scratch_address();
  if (!ws) return DSPARK_ERR_HIP;
  return dspark_verify_opts(dims, target, row_offsets, draft_len, U, W1, W2t, anchor, tokens,
                            q_tok, lse, uniforms, accept_len, next_token, beta_emit, flags, ws,
                            kScratchBytes, opts, stream);
}

dspark_status dspark_rnn_verify(dspark_dims dims, const float* target, const int32_t* row_offsets,
                                const int32_t* draft_len, const float* U, const uint16_t* W2t,
                                const float* e_rows, const int32_t* tokens, const float* q_tok,
                                const double* lse, const float* uniforms, int32_t* accept_len,
                                int32_t* next_token, float* beta_emit, uint32_t* flags, void* ws,
                                size_t ws_bytes, const dspark_draft_opts* opts, void* stream) {
  if (!target || !row_offsets || !draft_len || !U || !W2t || !e_rows || !tokens || !q_tok ||
      !lse || !uniforms || !accept_len || !next_token || !ws)
    return DSPARK_ERR_NULL;
  float beta = 1.0f;
  int greedy = 0;
  if (!draft_options(opts, &beta, &greedy)) return DSPARK_ERR_OPTS;
  if (!rnn_dims_ok(dims)) return DSPARK_ERR_SHAPE;
  if (!aligned(target, 16) || !aligned(U, 16) || !aligned(W2t, 16) || !aligned(e_rows, 4) ||
      !aligned(row_offsets, 4) || !aligned(draft_len, 4) || !aligned(tokens, 4) ||
      !aligned(q_tok, 4) || !aligned(lse, 8) || !aligned(uniforms, 4) ||
      !aligned(accept_len, 4) || !aligned(next_token, 4) || (beta_emit && !aligned(beta_emit, 4)) ||
      (flags && !aligned(flags, 4)) || !aligned(ws, kAlign))
    return DSPARK_ERR_ALIGN;
  if (ws_bytes < rnn_verify_ws(dims, nullptr, nullptr, nullptr)) return DSPARK_ERR_WORKSPACE;
  VerifyArgs a;
  a.B = dims.B;
  a.V = dims.V;
  a.gamma = dims.gamma;
  a.r = dims.r;
  a.ntiles = ntiles_of(dims.V);
  a.nseg = nseg_of(dims.V);
  a.target = target;
  a.row_offsets = row_offsets;
  a.draft_len = draft_len;
  a.U = U;
  a.W1 = nullptr;
  a.W2t = W2t;
  a.anchor = nullptr;
  a.tokens = tokens;
  a.q = q_tok;
  a.lse = lse;
  a.uniforms = uniforms;
  a.accept_len = accept_len;
  a.next_token = next_token;
  a.beta_emit = beta_emit;
  a.flags = flags;
  a.persistent_wgs = compute_units();
  a.beta = beta;
  a.greedy = greedy;
  uint16_t* E = nullptr;
  rnn_verify_ws(dims, ws, &a.ws, &E);
  a.e_terms = kRnnTerms;
  a.E = E;
  a.e_split = e_rows;   // the target pass splits the bias vectors into E
  a.E_split = E;
  return verify_passes(dims, a, static_cast<hipStream_t>(stream));
}

dspark_status dspark_verify(dspark_dims dims, const float* target, const int32_t* row_offsets,
                            const int32_t* draft_len, const float* U, const uint16_t* W1,
                            const uint16_t* W2t, const int32_t* anchor, const int32_t* tokens,
                            const float* q_tok, const double* lse, const float* uniforms,
                            int32_t* accept_len, int32_t* next_token, float* beta_emit,
                            uint32_t* flags, void* ws, size_t ws_bytes, void* stream) {
  return dspark_verify_opts(dims, target, row_offsets, draft_len, U, W1, W2t, anchor, tokens,
                            q_tok, lse, uniforms, accept_len, next_token, beta_emit, flags, ws,
                            ws_bytes, nullptr, stream);
}

int32_t dspark_profile_begin(int32_t capacity) {
  if (capacity < 1 || g_prof.armed) return -1;
  g_prof.events.assign(2 * static_cast<size_t>(capacity), nullptr);
  for (auto& e : g_prof.events)
    if (hipEventCreate(&e) != hipSuccess) return -1;
  g_prof.ids.assign(capacity, 0);
  g_prof.capacity = capacity;
  g_prof.used = 0;
  g_prof.armed = true;
  return 0;
}

int32_t dspark_profile_end(const char** names, int32_t* counts, double* total_ms,
                           int32_t max_names) {
  if (!g_prof.armed) return -1;
  int32_t rc = 0;
  std::vector<double> ms(kNumKernels, 0.0);
  std::vector<int> cnt(kNumKernels, 0);
  if (g_prof.used > 0 && hipEventSynchronize(g_prof.events[2 * g_prof.used - 1]) != hipSuccess)
    rc = -1;
  for (int i = 0; rc == 0 && i < g_prof.used; ++i) {
    float t = 0.0f;
    if (hipEventElapsedTime(&t, g_prof.events[2 * i], g_prof.events[2 * i + 1]) != hipSuccess) {
      rc = -1;
      break;
    }
    ms[g_prof.ids[i]] += t;
    cnt[g_prof.ids[i]] += 1;
  }
  for (auto& e : g_prof.events) (void)hipEventDestroy(e);
  g_prof.events.clear();
  g_prof.armed = false;
  g_prof.used = 0;
  if (rc != 0) return rc;
  int32_t n = 0;
  for (int k = 0; k < kNumKernels && n < max_names; ++k) {
    if (names) names[n] = kKernelNames[k];
    if (counts) counts[n] = cnt[k];
    if (total_ms) total_ms[n] = ms[k];
    ++n;
  }
  return n;
}

}  // extern "C"
