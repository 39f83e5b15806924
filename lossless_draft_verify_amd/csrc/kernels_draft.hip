// Markov-head draft for gfx950.
//
// Sources: [V41] blog.javazero.top "DeepSeek-V4.1 模型结构（6）：解码，DSpark", "Markov head"
// (eqs. (4), (5), the serial loop); [ZDS] zdszero.github.io spec_dspark, "insight 一";
// [CSDN] deepseek.csdn.net DSpark walk-through, 4.1-4.2. The last position's step can carry the
// verify planner (plan.h) on one extra workgroup.
//
// One draft step k (the serial dependency: step k+1 needs every request's x_k):
//   markov_step  streams W2t and the U slice of position k once, forms
//                L = U_k + W1[x_{k-1}] . W2 tile by tile with bf16 MFMA (fp32 accumulate) and
//                writes, per request and 32-token tile, the tile max and the fp32 sum of
//                exp(L - tile max). The [B][V] logits are never written (unless asked for).
//   draft_sample one workgroup per request: combines the tile partials in fp64, finds the tile
//                that holds u * Z, recomputes that tile's 32 logits with the same MFMA sequence
//                (bit-identical), and walks them in fp64 to the drawn token.
#include <type_traits>

#include "device.h"
#include "launch.h"
#include "dma.h"
#include "tiles.h"
#include "plan.h"

namespace dspark {

namespace {

// Persistent draft step: one 512-thread workgroup per compute unit walks work items (a
// 128-token tile of the vocabulary x a group of up to kBG requests). The group's embedding
// rows sit in LDS; each item's U block is loaded row-contiguously (512 B per request row) and
// staged through LDS into the MFMA output layout. Wave w computes tokens 32 (w % 4) .. +32 for
// requests 64 (w / 4) .. +64 of the group (two 32-request MFMA tiles), so each SIMD runs two
// waves. The next item's U block is loaded right after the current one is staged, and the
// next W2 tile right after the current MFMAs; LDS hand-offs use lds_barrier(), which leaves
// those loads in flight.
constexpr int kStepThreads = 512;

template <int KS, bool VEC4, int NT>
struct StepKernel {
  using C = StepCfg<KS * NT>;                         // LDS rows hold NT r bf16 (the bias row)
  static constexpr int r = 16 * KS;                   // rank: W2 columns
  static constexpr int BG = C::kBG;                   // requests per group (128, or 64 for r=512)
  static constexpr int kNTW = BG / 64;                // 32-request MFMA tiles per wave
  static constexpr int kTok = 4 * kTileTokens;        // tokens per item
  static constexpr int kUrow = kTok + 4;              // padded LDS row of the staged U block
  static constexpr int kURows = BG / 16;              // U rows per thread (32 threads per row)
  static constexpr int kPR = NT * r / 8;              // 16-byte pieces per bias row
  static constexpr int kEPieces = (BG * kPR + kStepThreads - 1) / kStepThreads;

  const StepArgs& p;
  uint16_t* E;
  float* Us;
  int tid, lane, half, col, ts, bh, ngroups;

  __device__ StepKernel(const StepArgs& p_, uint16_t* E_, float* Us_) : p(p_), E(E_), Us(Us_) {
    tid = threadIdx.x;
    lane = tid & 63;
    half = lane >> 5;
    col = lane & 31;
    ts = (tid >> 6) & 3;   // token sub-tile of the wave
    bh = tid >> 8;         // request half of the wave
    ngroups = (p.B + BG - 1) / BG;
  }

  // Request rows past B read row B-1 (never used): no branch in the load sequence.
  __device__ __forceinline__ void load_u(float4 (&u)[kURows], int it) const {
    const int tile = it / ngroups, group = it % ngroups;
    const int v = tile * kTok + 4 * (tid & 31);
#pragma unroll
    for (int i = 0; i < kURows; ++i) {
      const int b = min(group * BG + i * 16 + (tid >> 5), p.B - 1);
      const float* row = p.U + (static_cast<size_t>(b >> p.u_shift) * p.gamma + p.k) * p.V;
      if (VEC4) {
        u[i] = (v + 3 < p.V) ? *reinterpret_cast<const float4*>(row + v) : make_float4(0.f, 0.f, 0.f, 0.f);
      } else {
        float o[4];
        load4(row, v, p.V, false, o);
        u[i] = make_float4(o[0], o[1], o[2], o[3]);
      }
    }
  }

  __device__ __forceinline__ void load_a(u16x8_t (&a)[KS], int it) const {
    load_w2_tile<KS>(a, p.W2t, (it / ngroups) * kTok + ts * kTileTokens + col, p.V, half);
  }

  // Bias rows of one request group into LDS (Markov: token ids first, then rows).
  __device__ void load_embeddings(int group) const {
    // piece c = i * kStepThreads + tid covers row c / kPR, bytes 16 (c % kPR); pieces past the
    // group (c >= BG * kPR) are clamped to the last one and not stored.
    int32_t ids[kEPieces];
#pragma unroll
    for (int i = 0; i < kEPieces; ++i) {
      const int c = min(i * kStepThreads + tid, BG * kPR - 1);
      const int b = min(group * BG + c / kPR, p.B - 1);
      ids[i] = (NT == 1) ? clamp_token(p.prev[static_cast<size_t>(b) * p.prev_stride], p.V) : b;
    }
    u16x8_t e[kEPieces];
#pragma unroll
    for (int i = 0; i < kEPieces; ++i) {
      const int c = min(i * kStepThreads + tid, BG * kPR - 1);
      const int64_t pos = static_cast<int64_t>(ids[i]) * p.gamma + p.k;
      e[i] = load_u16x8(bias_row<NT>(p.W1, p.E, r, ids[i], pos) + (c % kPR) * 8);
    }
#pragma unroll
    for (int i = 0; i < kEPieces; ++i) {
      const int c = i * kStepThreads + tid;
      if (c >= BG * kPR) break;
      const bool valid = group * BG + c / kPR < p.B;
      *reinterpret_cast<u16x8_t*>(&E[(c / kPR) * C::kLdsRow + (c % kPR) * 8]) = valid ? e[i] : zero_u16x8();
    }
  }

  __device__ __forceinline__ void stage_u(const float4 (&u)[kURows]) const {
#pragma unroll
    for (int i = 0; i < kURows; ++i)
      *reinterpret_cast<float4*>(&Us[(i * 16 + (tid >> 5)) * kUrow + 4 * (tid & 31)]) = u[i];
  }

  // MFMA (independent chains over the wave's request tiles, embedding reads one k-step ahead).
  __device__ __forceinline__ void mfma(const u16x8_t (&a)[KS], f32x16_t (&acc)[kNTW]) const {
    u16x8_t e0[kNTW], e1[kNTW];
#pragma unroll
    for (int nt = 0; nt < kNTW; ++nt) {
      acc[nt] = f32x16_t{};
      e0[nt] = load_u16x8(&E[((bh * kNTW + nt) * 32 + col) * C::kLdsRow + 8 * half]);
    }
#pragma unroll
    for (int s2 = 0; s2 < NT * KS; ++s2) {
      u16x8_t (&cur)[kNTW] = (s2 & 1) ? e1 : e0;
      u16x8_t (&nxt)[kNTW] = (s2 & 1) ? e0 : e1;
      if (s2 + 1 < NT * KS) {
#pragma unroll
        for (int nt = 0; nt < kNTW; ++nt)
          nxt[nt] = load_u16x8(&E[((bh * kNTW + nt) * 32 + col) * C::kLdsRow + 8 * half + 16 * (s2 + 1)]);
      }
#pragma unroll
      for (int nt = 0; nt < kNTW; ++nt) acc[nt] = mfma_32x32x16(a[s2 % KS], cur[nt], acc[nt]);
    }
  }

  // Epilogue: L = U + bias (written out as the debug logits when asked), scaled by the draft
  // temperature, tile max, fp32 sum of exp(x - max), one float2 per (request, tile).
  __device__ __forceinline__ void epilogue(f32x16_t (&acc)[kNTW], int it) const {
    const int tile = it / ngroups, group = it % ngroups;
    const int tok0 = tile * kTok + ts * kTileTokens;
    const bool full = tok0 + kTileTokens <= p.V;
    float m[kNTW], sm[kNTW];
#pragma unroll
    for (int nt = 0; nt < kNTW; ++nt) {
      const int rt = bh * kNTW + nt;
      const float* urow = &Us[(rt * 32 + col) * kUrow + ts * kTileTokens + 4 * half];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 uu = *reinterpret_cast<const float4*>(urow + 8 * g);
        acc[nt][4 * g + 0] += uu.x;
        acc[nt][4 * g + 1] += uu.y;
        acc[nt][4 * g + 2] += uu.z;
        acc[nt][4 * g + 3] += uu.w;
      }
      if (!full) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (tok0 + tile_token(j, half) >= p.V) acc[nt][j] = kNegInf;
      }
      const int b = group * BG + rt * 32 + col;
      if (p.dbg && b < p.B) {   // the logits L themselves, before the temperature
        const size_t drow = (static_cast<size_t>(b) * p.gamma + p.k) * p.V;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int v = tok0 + tile_token(j, half);
          if (v < p.V) p.dbg[drow + v] = acc[nt][j];
        }
      }
      if (p.beta != 1.0f) {   // beta = 1: unchanged, no multiply
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[nt][j] *= p.beta;
      }
      float L[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) L[j] = acc[nt][j];
      m[nt] = max16(L);
    }
#pragma unroll
    for (int nt = 0; nt < kNTW; ++nt) m[nt] = fmaxf(m[nt], __uint_as_float(lane_xor<32>(__float_as_uint(m[nt]))));
#pragma unroll
    for (int nt = 0; nt < kNTW; ++nt) {
      float t[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) t[j] = exp_term(acc[nt][j] - m[nt]);
      sm[nt] = (m[nt] == kNegInf) ? 0.0f : sum16(t);
    }
#pragma unroll
    for (int nt = 0; nt < kNTW; ++nt) sm[nt] = sm[nt] + __uint_as_float(lane_xor<32>(__float_as_uint(sm[nt])));
#pragma unroll
    for (int nt = 0; nt < kNTW; ++nt) {
      const int b = group * BG + (bh * kNTW + nt) * 32 + col;
      if (b >= p.B) continue;
      if (half == 0) p.part[static_cast<size_t>(b) * p.ntiles + tok0 / kTileTokens] = make_float2(m[nt], sm[nt]);
    }
  }
};

template <int KS, bool VEC4, int NT>
__global__ __launch_bounds__(kStepThreads, 1) void markov_step_kernel(StepArgs p) {
  using K = StepKernel<KS, VEC4, NT>;
  __shared__ __attribute__((aligned(16))) uint16_t E[K::BG * K::C::kLdsRow];
  __shared__ __attribute__((aligned(16))) float Us[K::BG * K::kUrow];
  const K k(p, E, Us);
  const int nitems = ((p.V + K::kTok - 1) / K::kTok) * k.ngroups;
  int it = blockIdx.x;
  if (it >= nitems) return;
  u16x8_t a[KS];
  float4 u[K::kURows];
  f32x16_t acc[K::kNTW];
  int cur_group = -1;
  k.load_a(a, it);
  k.load_u(u, it);
  for (; it < nitems; it += gridDim.x) {
    const int group = it % k.ngroups;
    if (group != cur_group) k.load_embeddings(group);
    cur_group = group;
    k.stage_u(u);
    const int nxt = it + gridDim.x;
    const bool has_next = nxt < nitems;
    if (has_next) k.load_u(u, nxt);
    lds_barrier();
    const bool active = (it / k.ngroups) * K::kTok + k.ts * kTileTokens < p.V &&
                        group * K::BG + k.bh * K::kNTW * 32 < p.B;
    if (active) k.mfma(a, acc);
    if (has_next) k.load_a(a, nxt);
    if (active) k.epilogue(acc, it);
    lds_barrier();
  }
}

// ---- Pipelined draft step: tiles copied into LDS by LDS-DMA loads ----------------------------
//
// One 512-thread workgroup per compute unit, on a persistent grid whose size is a multiple of
// the number of 128-request groups, so every workgroup keeps one group for the whole launch.
// A work item is 64 tokens (two 32-token tiles): its 64 W2t rows and the group's U block
// (128 request rows x 64 tokens, fp32) are copied from HBM into one of two LDS stages by
// global_load_lds_dwordx4, which writes LDS directly and holds no registers, so the next item
// is in flight while one is computed. Wave w computes tile w / 4 of the item for requests
// 32 (w % 4) .. +32, whose embedding rows (the MFMA B operand) it holds in registers for the
// whole launch; each SIMD runs two waves. Both LDS blocks are XOR-swizzled in 16-byte chunks
// (chunk c of row t is stored at c ^ (t & 15)), so the rows one ds_read_b128 touches fall on
// distinct banks.
//
// The copies are awaited explicitly: s_waitcnt vmcnt(n) with n the number of copies this wave
// issued after the awaited item, then s_barrier for the other waves' copies. No global store is
// issued inside the pipelined loop (the partials collect in LDS and are written when the buffer
// is full, followed by a full drain, and after the loop), so the vector-memory counter only
// ever holds copies, in issue order.
constexpr int kDmaThreads = 512;
constexpr int kDmaGroup = 128;   // requests per group: 4 waves x 32 per tile
constexpr int kDmaTiles = 2;     // 32-token tiles per item
constexpr int kXcds = 8;         // accelerator complex dies of an MI355X, each with its own L2

// Bias rows of a wave's 32 requests in MFMA operand form (lane (h, c): k-step s is bf16
// 16 s + 8 h .. + 8 of request c's row): from the operand layout E2 when the RNN state step wrote
// it (one contiguous 1 KB a k-step), else from the rows. blk is the wave's 32-request block, row
// its request within the 128-request group.
template <int KS, int NT>
__device__ __forceinline__ void load_bias_operands(const StepArgs& p, int blk, int row, int half,
                                                   int col, u16x8_t (&e)[NT * KS]) {
  if (NT > 1 && p.E2) {
    const int nblk = (p.B + 31) / 32;
    const uint16_t* src = p.E2 +
        ((static_cast<size_t>(min(blk, nblk - 1)) * p.gamma + p.k) * (NT * KS) * 2 + half) * 256 +
        8 * col;
#pragma unroll
    for (int s = 0; s < NT * KS; ++s) e[s] = load_u16x8(src + 512 * s);
    return;
  }
  const int b = min((blk / 4) * kDmaGroup + row, p.B - 1);
  const int32_t prev =
      (NT == 1) ? clamp_token(p.prev[static_cast<size_t>(b) * p.prev_stride], p.V) : 0;
  const uint16_t* erow =
      bias_row<NT>(p.W1, p.E, 16 * KS, prev, static_cast<int64_t>(b) * p.gamma + p.k) + 8 * half;
#pragma unroll
  for (int s = 0; s < NT * KS; ++s) e[s] = load_u16x8(erow + 16 * s);
}

template <int KS>
struct DmaStep {
  static constexpr int r = 16 * KS;
  static constexpr int kThreads = kDmaThreads;
  static constexpr int kTok = kDmaTiles * kTileTokens;              // 64 tokens per item
  static constexpr int kW2Chunks = 2 * KS;                          // 16-byte chunks per row
  static constexpr int kW2Bytes = kTok * kW2Chunks * 16;            // 64 W2t rows
  static constexpr int kUChunks = kTok / 4;                         // 16 per U row segment
  static constexpr int kUBytes = kDmaGroup * kUChunks * 16;         // 32 KB
  static constexpr int kStageBytes = kW2Bytes + kUBytes;
  static constexpr int kStages = 2;
  static constexpr int kPartItems = 8;                              // items of partials in LDS
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kW2Copies = kW2Bytes / 1024 / kWaves;        // copies per wave per item
  static constexpr int kUCopies = kUBytes / 1024 / kWaves;
  static constexpr int kCopies = kW2Copies + kUCopies;
  static constexpr int kECopies = kDmaGroup * kW2Chunks * 16 / 1024 / kWaves;   // embedding rows
  static_assert(kDmaGroup * kW2Chunks * 16 <= kStageBytes, "embedding rows fit in one stage");
  static constexpr int kW2Swz = (kW2Chunks >= 16) ? 15 : kW2Chunks - 1;   // W2 swizzle mask
  static constexpr int kAOffs = (KS < 8) ? KS : 8;                   // distinct lane offsets
  static_assert(KS >= 4 && KS <= 16, "one to four 1 KB W2 copies per wave per item");
  static_assert((kStages - 1) * kCopies <= 63, "vmcnt range");
};

// LDS of the pipelined step: the copy stages, the partials of kPartItems items, and the
// group's previous tokens.
template <int KS>
struct DmaLds {
  using D = DmaStep<KS>;
  __attribute__((aligned(1024))) unsigned char stage[D::kStages * D::kStageBytes];
  float2 pbuf[D::kPartItems * kDmaTiles * kDmaGroup];
  __attribute__((aligned(256))) int32_t pid[kDmaGroup];
};

// Workgroup -> (request group, vocabulary range) of the pipelined step. Workgroup w of a group
// takes a contiguous range of items, so that the partials of one request that it produces are
// contiguous in memory (full-line writes). Blocks are dispatched round-robin over the XCDs
// (hardware blocks h and h + kXcds share one): with several request groups, the groups of one
// range go to blocks that share an XCD, so that the range's W2t rows come from HBM once and then
// from that XCD's L2. `first` hardware blocks come before the step's (the planner's block of
// the fused last step); each XCD's step blocks form whole sets of ngroups, and blocks left over
// take no item (group = -1).
struct StepMap {
  int group, wg, nwg;
};
__device__ __forceinline__ StepMap step_map(int B, int h, int nblk_hw, int first) {
  const int ngroups = (B + kDmaGroup - 1) / kDmaGroup;
  const int nstep = nblk_hw - first;
  if (ngroups == 1) return StepMap{0, h - first, nstep};
  if (nstep < kXcds * ngroups) {   // too few blocks for whole sets on every XCD: consecutive
    const int s = h - first, nwg = nstep / ngroups;
    return (s < nwg * ngroups) ? StepMap{s % ngroups, s / ngroups, nwg} : StepMap{-1, 0, nwg};
  }
  // step blocks on XCD x: hardware blocks first .. nblk_hw - 1 with h % kXcds == x
  auto on_xcd = [&](int x) {
    const int lo = (first + kXcds - 1 - x) / kXcds;        // first slot with h >= first
    const int hi = (nblk_hw - 1 - x + kXcds) / kXcds;      // slots with h < nblk_hw
    return max(0, hi - lo);
  };
  const int x = h % kXcds;
  const int slot = h / kXcds - (first + kXcds - 1 - x) / kXcds;   // index among x's step blocks
  int before = 0, total = 0;
  for (int y = 0; y < kXcds; ++y) {
    const int ranges = on_xcd(y) / ngroups;
    if (y < x) before += ranges;
    total += ranges;
  }
  const int ranges_x = on_xcd(x) / ngroups;
  if (slot >= ranges_x * ngroups) return StepMap{-1, 0, total};
  return StepMap{slot % ngroups, before + slot / ngroups, total};
}

// The pipelined step as run by the workgroup that step_map placed at (group, wg of nwg).
template <int KS, int NT, bool kUShared = false>
__device__ __forceinline__ void markov_step_dma(const StepArgs& p, StepMap mp, DmaLds<KS>& lds) {
  using D = DmaStep<KS>;
  unsigned char* stage = lds.stage;
  float2* pbuf = lds.pbuf;
  int32_t* pid = lds.pid;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int sub = wave >> 2, rq = wave & 3;   // tile within the item, request quarter
  if (mp.group < 0) return;
  const int group = mp.group, wg = mp.wg, nwg = mp.nwg;
  const int nitems = (p.V + D::kTok - 1) / D::kTok;
  const int item_lo = static_cast<int>(static_cast<int64_t>(nitems) * wg / nwg);
  const int n = static_cast<int>(static_cast<int64_t>(nitems) * (wg + 1) / nwg) - item_lo;
  if (n <= 0) return;
  const int row_own = 32 * rq + col;                    // request row within the group
  const bool wave_active = group * kDmaGroup + 32 * rq < p.B;
  // kUShared (u_shift > 0: the expanded nodes of one request read one U row): the rows that
  // share a U row share one copy of it; the stage holds the group's nd = kDmaGroup >> u_shift
  // distinct U rows, four to a 1 KB copy, and the copies are spread over the waves (ucopies_w of
  // them per item on this wave). Otherwise every row has its own U row, kUCopies per wave.
  const int ush = kUShared ? p.u_shift : 0;
  const int u0 = (group * kDmaGroup) >> ush;            // the group's first U row
  const int nd = max(1, kDmaGroup >> ush);
  const int ucopies = max(1, nd * D::kUChunks * 16 / 1024);
  const int uper =
      kUShared ? __builtin_amdgcn_readfirstlane(max(1, ucopies / D::kWaves)) : D::kUCopies;
  const int ucopies_w =
      kUShared ? __builtin_amdgcn_readfirstlane(max(0, min(uper, ucopies - wave * uper)))
               : D::kUCopies;
  const int urow_own = ((group * kDmaGroup + row_own) >> ush) - u0;   // lane's U row in the stage

  // Per-lane LDS offsets: k-step s of the A operand (W2t row 32 sub + col, chunk 2s + half) is
  // at a_off[s % 8] + 256 (s / 8) (the swizzle depends only on col); U chunk 8 sub + 2g + half of
  // the lane's U row at u_off[g].
  const uint32_t stage_addr = lds_addr(stage);
  uint32_t a_off[D::kAOffs], u_off[4];
  {
    const int wrow = 32 * sub + col;
#pragma unroll
    for (int t = 0; t < D::kAOffs; ++t)
      a_off[t] = 16 * (wrow * D::kW2Chunks + ((2 * t + half) ^ (wrow & D::kW2Swz)));
#pragma unroll
    for (int g = 0; g < 4; ++g)
      u_off[g] = D::kW2Bytes + 16 * (urow_own * D::kUChunks +
                                     ((8 * sub + 2 * g + half) ^ (urow_own & 15)));
  }
  // Item j is complete once at most the next item's copies (this wave's count) are in flight.
  auto wait_item = [&]() {
    if constexpr (kUShared)
      wait_copies_upto<D::kW2Copies, 1, D::kUCopies>(ucopies_w);
    else
      wait_copies<D::kCopies>();
  };

  // This wave's share of item j's copies into stage j % kStages. Rows past V or B are clamped
  // to the last valid one (all addresses stay inside the tensors); the epilogue masks them.
  auto issue = [&](int j) {
    const int tok0 = (item_lo + j) * D::kTok;
    const uint32_t base = stage_addr + (j % D::kStages) * D::kStageBytes;
#pragma unroll
    for (int i = 0; i < D::kW2Copies; ++i) {
      const int q = wave * D::kW2Copies + i;
      const int slot = 64 * q + lane;
      const int row = slot / D::kW2Chunks;
      const int c = (slot % D::kW2Chunks) ^ (row & D::kW2Swz);
      const int tok = min(tok0 + row, p.V - 1);
      copy16_to_lds(p.W2t + static_cast<size_t>(tok) * D::r + 8 * c, base + 1024 * q);
    }
#pragma unroll
    for (int i = 0; i < D::kUCopies; ++i) {
      if constexpr (kUShared) {
        if (i < ucopies_w) {   // wave-uniform
          const int q = wave * uper + i;
          const int slot = 64 * q + lane;
          const int d = slot / D::kUChunks;             // U row within the stage
          const int c = (slot % D::kUChunks) ^ (d & 15);
          const int ub = min(u0 + d, (p.B - 1) >> ush);
          const int v = min(tok0 + 4 * c, p.V - 4);
          copy16_to_lds_nt(p.U + (static_cast<size_t>(ub) * p.gamma + p.k) * p.V + v,
                           __builtin_amdgcn_readfirstlane(base + D::kW2Bytes + 1024 * q));
        }
      } else {
        const int q = wave * D::kUCopies + i;
        const int slot = 64 * q + lane;
        const int row = slot / D::kUChunks;
        const int c = (slot % D::kUChunks) ^ (row & 15);
        const int b = min(group * kDmaGroup + row, p.B - 1);
        const int v = min(tok0 + 4 * c, p.V - 4);
        copy16_to_lds_nt(p.U + (static_cast<size_t>(b) * p.gamma + p.k) * p.V + v,
                         base + D::kW2Bytes + 1024 * q);
      }
    }
  };

  // Partials of items j0 .. j1-1 (after a barrier), to global memory by the whole workgroup.
  // With kSlots the power of two at or above their tile count, thread t takes tile slot
  // t % kSlots (item j0 + slot / kDmaTiles) of the rows t / kSlots + kRowStep i: consecutive
  // threads write consecutive tiles of one request (whole lines), and all of a thread's LDS reads
  // go out before its stores.
  auto flush_slots = [&](int j0, int j1, auto slots_c) {
    constexpr int kSlots = decltype(slots_c)::value;
    constexpr int kRowStep = D::kThreads / kSlots;
    constexpr int kPasses = (kDmaGroup + kRowStep - 1) / kRowStep;
    static_assert(D::kThreads % kSlots == 0 && kSlots <= D::kPartItems * kDmaTiles, "flush mapping");
    const int tt = tid % kSlots, r0 = tid / kSlots;
    const int j = j0 + tt / kDmaTiles;
    const int tile = (item_lo + j0) * kDmaTiles + tt;
    const bool ok = tt < (j1 - j0) * kDmaTiles && tile < p.ntiles;
    const float2* src = pbuf + ((j % D::kPartItems) * kDmaTiles + tt % kDmaTiles) * kDmaGroup;
    float2 v[kPasses];
#pragma unroll
    for (int i = 0; i < kPasses; ++i) v[i] = src[min(r0 + kRowStep * i, kDmaGroup - 1)];
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
      const int row = r0 + kRowStep * i;
      const int b = group * kDmaGroup + row;
      if (ok && row < kDmaGroup && b < p.B) p.part[static_cast<size_t>(b) * p.ntiles + tile] = v[i];
    }
  };
  auto flush = [&](int j0, int j1) {
    const int per = (j1 - j0) * kDmaTiles;   // uniform
    if (per <= 2) {
      flush_slots(j0, j1, std::integral_constant<int, 2>{});
    } else if (per <= 4) {
      flush_slots(j0, j1, std::integral_constant<int, 4>{});
    } else if (per <= 8) {
      flush_slots(j0, j1, std::integral_constant<int, 8>{});
    } else {
      flush_slots(j0, j1, std::integral_constant<int, D::kPartItems * kDmaTiles>{});
    }
  };

  // Prologue. Markov head, all copies: the group's previous tokens into LDS; then the
  // embedding rows W1[prev] (each row once per workgroup, swizzled like W2t) into stage 1, with
  // item 0 behind them into stage 0; each wave reads its rows into registers and releases
  // stage 1. RNN head: each lane loads its request's bias row (both terms) straight into
  // registers, and those loads are drained before the copy pipeline starts.
  u16x8_t e[NT * KS];
  if constexpr (NT == 1) {
    if (wave < kDmaGroup / 64) {
      const int b = min(group * kDmaGroup + 64 * wave + lane, p.B - 1);
      copy4_to_lds(p.prev + static_cast<size_t>(b) * p.prev_stride, lds_addr(pid) + 256 * wave);
    }
    wait_copies<0>();
    asm volatile("s_barrier" ::: "memory");
    {
      const uint32_t ebase = stage_addr + D::kStageBytes;
#pragma unroll
      for (int i = 0; i < D::kECopies; ++i) {
        const int q = wave * D::kECopies + i;
        const int slot = 64 * q + lane;
        const int row = slot / D::kW2Chunks;
        const int c = (slot % D::kW2Chunks) ^ (row & D::kW2Swz);
        copy16_to_lds(p.W1 + static_cast<size_t>(clamp_token(pid[row], p.V)) * D::r + 8 * c,
                      ebase + 1024 * q);
      }
    }
    issue(0);
    wait_item();                                // the embedding rows (item 0 may be in flight)
    asm volatile("s_barrier" ::: "memory");
    {
      const unsigned char* eb = stage + D::kStageBytes;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        e[s] = *reinterpret_cast<const u16x8_t*>(
            eb + 16 * (row_own * D::kW2Chunks + ((2 * s + half) ^ (row_own & D::kW2Swz))));
    }
    lds_barrier();                              // stage 1 is free for item 1
  } else {
    load_bias_operands<KS, NT>(p, group * kDmaGroup / 32 + rq, row_own, half, col, e);
    __builtin_amdgcn_s_waitcnt(0);
    issue(0);
  }
  int flushed = 0;
  for (int j = 0; j < n; ++j) {
    if (j + 1 < n) {
      issue(j + 1);
      wait_item();
    } else {
      wait_copies<0>();
    }
    asm volatile("s_barrier" ::: "memory");

    const int tok0 = (item_lo + j) * D::kTok + sub * kTileTokens;
    if (wave_active && tok0 < p.V) {
      const unsigned char* base = stage + (j % D::kStages) * D::kStageBytes;
      u16x8_t a[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s)
        a[s] = *reinterpret_cast<const u16x8_t*>(base + 256 * (s >> 3) + a_off[s % D::kAOffs]);
      float4 uu[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) uu[g] = *reinterpret_cast<const float4*>(base + u_off[g]);
      f32x16_t acc = {};
#pragma unroll
      for (int s = 0; s < NT * KS; ++s) acc = mfma_32x32x16(a[s % KS], e[s], acc);
      // Epilogue: L = U + bias, tile max, fp32 sum of exp(L - max) (the order of the
      // register-prefetch step kernel, so both give the same partials bit for bit).
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        acc[4 * g + 0] += uu[g].x;
        acc[4 * g + 1] += uu[g].y;
        acc[4 * g + 2] += uu[g].z;
        acc[4 * g + 3] += uu[g].w;
      }
      if (tok0 + kTileTokens > p.V) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
          if (tok0 + tile_token(jj, half) >= p.V) acc[jj] = kNegInf;
      }
      float L[16];   // the draft temperature scales the logits (beta = 1: unchanged, no multiply)
      if (p.beta != 1.0f) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) L[jj] = acc[jj] * p.beta;
      } else {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) L[jj] = acc[jj];
      }
      float m = max16(L);
      m = fmaxf(m, other_half(m, half));
      float t[16];
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) t[jj] = exp_term(L[jj] - m);
      float sm = (m == kNegInf) ? 0.0f : sum16(t);
      sm = sm + other_half(sm, half);
      if (half == 0)
        pbuf[((j % D::kPartItems) * kDmaTiles + sub) * kDmaGroup + row_own] = make_float2(m, sm);
    }
    lds_barrier();   // stage j % kStages is free for item j + kStages
    if ((j + 1) % D::kPartItems == 0 && j + 1 < n) {
      flush(flushed, j + 1);
      flushed = j + 1;
      wait_copies<0>();   // the stores join the counter: drain it so later counts hold copies only
    }
  }
  flush(flushed, n);
}

template <int KS, int NT, bool kUShared>
__global__ __launch_bounds__(kDmaThreads, 1) void markov_step_dma_kernel(StepArgs p) {
  __shared__ DmaLds<KS> lds;
  markov_step_dma<KS, NT, kUShared>(p, step_map(p.B, blockIdx.x, gridDim.x, 0), lds);
}


// The pipelined step for bias rows held in registers with one wave per SIMD (the RNN head's
// three-term rows at r = 256): 32-token items in four 32 KB stages, so that three items stream
// while a wave runs the 48 MFMA k-steps of its tile (with 64-token items in two stages only one
// item was in flight behind them). Wave w computes the item's tile for request quarter w with
// the MFMA sequence and epilogue of the other step kernels, so the partials are bit-identical.
// The bias rows come from the operand layout where the state step wrote it.
template <int KS>
struct Deep4Step {
  static constexpr int r = 16 * KS;
  static constexpr int kThreads = 256;
  static constexpr int kWaves = 4;
  static constexpr int kTok = kTileTokens;                          // one tile per item
  static constexpr int kW2Chunks = 2 * KS;
  static constexpr int kW2Bytes = kTok * kW2Chunks * 16;            // 16 KB at r = 256
  static constexpr int kUChunks = kTok / 4;                         // 8 per U row segment
  static constexpr int kUBytes = kDmaGroup * kUChunks * 16;         // 16 KB
  static constexpr int kStageBytes = kW2Bytes + kUBytes;
  static constexpr int kStages = 4;
  static constexpr int kPartItems = 16;
  static constexpr int kW2Copies = kW2Bytes / 1024 / kWaves;
  static constexpr int kUCopies = kUBytes / 1024 / kWaves;
  static constexpr int kCopies = kW2Copies + kUCopies;
  static constexpr int kW2Swz = 15;
  static_assert(KS == 16, "r = 256");
  static_assert((kStages - 1) * kCopies <= 63, "vmcnt range");
};

template <int KS>
struct Deep4Lds {
  using D = Deep4Step<KS>;
  __attribute__((aligned(1024))) unsigned char stage[D::kStages * D::kStageBytes];
  float2 pbuf[D::kPartItems * kDmaGroup];
};

template <int KS, int NT>
__device__ __forceinline__ void markov_step_deep4(const StepArgs& p, StepMap mp,
                                                  Deep4Lds<KS>& lds) {
  using D = Deep4Step<KS>;
  unsigned char* stage = lds.stage;
  float2* pbuf = lds.pbuf;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  if (mp.group < 0) return;
  const int group = mp.group;
  const int nitems = p.ntiles;
  const int item_lo = static_cast<int>(static_cast<int64_t>(nitems) * mp.wg / mp.nwg);
  const int n = static_cast<int>(static_cast<int64_t>(nitems) * (mp.wg + 1) / mp.nwg) - item_lo;
  if (n <= 0) return;
  const int row_own = 32 * wave + col;
  const bool wave_active = group * kDmaGroup + 32 * wave < p.B;
  const uint32_t stage_addr = lds_addr(stage);
  // A operand (W2t row col, chunk 2s + half) of k-step s at a_off[s % 8] + 256 (s / 8); U chunk
  // 2g + half of row row_own at u_off[g].
  uint32_t a_off[8], u_off[4];
#pragma unroll
  for (int t = 0; t < 8; ++t) a_off[t] = 16 * (col * D::kW2Chunks + ((2 * t + half) ^ (col & D::kW2Swz)));
#pragma unroll
  for (int g = 0; g < 4; ++g)
    u_off[g] = D::kW2Bytes + 16 * (row_own * D::kUChunks + ((2 * g + half) ^ (row_own & 7)));

  // This wave's share of item j's copies into stage j % kStages; rows past V or B are clamped
  // to the last valid one and masked in the epilogue.
  auto issue = [&](int j) {
    const int tok0 = (item_lo + j) * D::kTok;
    const uint32_t base = stage_addr + (j % D::kStages) * D::kStageBytes;
#pragma unroll
    for (int i = 0; i < D::kW2Copies; ++i) {
      const int q = wave * D::kW2Copies + i;
      const int slot = 64 * q + lane;
      const int row = slot / D::kW2Chunks;
      const int c = (slot % D::kW2Chunks) ^ (row & D::kW2Swz);
      const int tok = min(tok0 + row, p.V - 1);
      copy16_to_lds(p.W2t + static_cast<size_t>(tok) * D::r + 8 * c, base + 1024 * q);
    }
#pragma unroll
    for (int i = 0; i < D::kUCopies; ++i) {
      const int q = wave * D::kUCopies + i;
      const int slot = 64 * q + lane;
      const int row = slot / D::kUChunks;
      const int c = (slot % D::kUChunks) ^ (row & 7);
      const int b = min(group * kDmaGroup + row, p.B - 1);
      const int v = min(tok0 + 4 * c, p.V - 4);
      copy16_to_lds_nt(p.U + (static_cast<size_t>(b >> p.u_shift) * p.gamma + p.k) * p.V + v,
                       base + D::kW2Bytes + 1024 * q);
    }
  };
  // Partials of items j0 .. j1-1 (one tile each), mapped as in the two-stage kernel's flush.
  auto flush_slots = [&](int j0, int j1, auto slots_c) {
    constexpr int kSlots = decltype(slots_c)::value;
    constexpr int kRowStep = D::kThreads / kSlots;
    constexpr int kPasses = (kDmaGroup + kRowStep - 1) / kRowStep;
    static_assert(D::kThreads % kSlots == 0 && kSlots <= D::kPartItems, "flush mapping");
    const int tt = tid % kSlots, r0 = tid / kSlots;
    const bool ok = tt < j1 - j0;
    const float2* src = pbuf + ((j0 + tt) % D::kPartItems) * kDmaGroup;
    float2 v[kPasses];
#pragma unroll
    for (int i = 0; i < kPasses; ++i) v[i] = src[min(r0 + kRowStep * i, kDmaGroup - 1)];
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
      const int row = r0 + kRowStep * i;
      const int b = group * kDmaGroup + row;
      if (ok && row < kDmaGroup && b < p.B)
        p.part[static_cast<size_t>(b) * p.ntiles + item_lo + j0 + tt] = v[i];
    }
  };
  auto flush = [&](int j0, int j1) {
    const int per = j1 - j0;   // uniform
    if (per <= 2) {
      flush_slots(j0, j1, std::integral_constant<int, 2>{});
    } else if (per <= 4) {
      flush_slots(j0, j1, std::integral_constant<int, 4>{});
    } else if (per <= 8) {
      flush_slots(j0, j1, std::integral_constant<int, 8>{});
    } else {
      flush_slots(j0, j1, std::integral_constant<int, D::kPartItems>{});
    }
  };

  // Prologue: the first kStages - 1 items' copies, then each lane's bias rows (all NT terms)
  // into registers behind them; all of it is drained before the loop, whose waits then count
  // copies only.
#pragma unroll
  for (int j = 0; j < D::kStages - 1; ++j)
    if (j < n) issue(j);
  u16x8_t e[NT * KS];
  load_bias_operands<KS, NT>(p, group * kDmaGroup / 32 + wave, row_own, half, col, e);
  __builtin_amdgcn_s_waitcnt(0);
  int flushed = 0;
  for (int j = 0; j < n; ++j) {
    if (j + D::kStages - 1 < n) issue(j + D::kStages - 1);
    // item j is complete once at most the copies of the items issued after it are in flight
    wait_copies_upto<0, D::kCopies, D::kStages - 1>(min(D::kStages - 1, n - 1 - j));
    asm volatile("s_barrier" ::: "memory");
    const int tok0 = (item_lo + j) * D::kTok;
    if (wave_active) {
      const unsigned char* base = stage + (j % D::kStages) * D::kStageBytes;
      u16x8_t a[KS];
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2)
        a[s2] = *reinterpret_cast<const u16x8_t*>(base + 256 * (s2 >> 3) + a_off[s2 & 7]);
      float4 uu[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) uu[g] = *reinterpret_cast<const float4*>(base + u_off[g]);
      f32x16_t acc = {};
#pragma unroll
      for (int s2 = 0; s2 < NT * KS; ++s2) acc = mfma_32x32x16(a[s2 % KS], e[s2], acc);
      // Epilogue as in the other step kernels (the same partials bit for bit).
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        acc[4 * g + 0] += uu[g].x;
        acc[4 * g + 1] += uu[g].y;
        acc[4 * g + 2] += uu[g].z;
        acc[4 * g + 3] += uu[g].w;
      }
      if (tok0 + kTileTokens > p.V) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
          if (tok0 + tile_token(jj, half) >= p.V) acc[jj] = kNegInf;
      }
      float L[16];   // beta = 1: unchanged, no multiply
      if (p.beta != 1.0f) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) L[jj] = acc[jj] * p.beta;
      } else {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) L[jj] = acc[jj];
      }
      float m = max16(L);
      m = fmaxf(m, other_half(m, half));
      float t[16];
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) t[jj] = exp_term(L[jj] - m);
      float sm = (m == kNegInf) ? 0.0f : sum16(t);
      sm = sm + other_half(sm, half);
      if (half == 0) pbuf[(j % D::kPartItems) * kDmaGroup + row_own] = make_float2(m, sm);
    }
    lds_barrier();   // stage j % kStages is free for item j + kStages
    if ((j + 1) % D::kPartItems == 0 && j + 1 < n) {
      flush(flushed, j + 1);
      flushed = j + 1;
      wait_copies<0>();   // the stores join the counter: drain it so later counts hold copies only
    }
  }
  flush(flushed, n);
}

template <int KS, int NT>
__global__ __launch_bounds__(256, 1) void markov_step_deep4_kernel(StepArgs p) {
  __shared__ Deep4Lds<KS> lds;
  markov_step_deep4<KS, NT>(p, step_map(p.B, blockIdx.x, gridDim.x, 0), lds);
}


// The last draft position's step with the verify planner beside it: workgroup 0 plans (its LDS
// holds the planner's arrays in place of the copy stages), the others run the step. The plan
// needs only the confidences, which need only the tokens before the last position, so it costs
// the round no time of its own; no workgroup waits for another.
constexpr int kFusedPlanMax = 4096;   // B * gamma limit of the fused planner

template <int KS, int NT>
__global__ __launch_bounds__(kDmaThreads, 1) void markov_step_plan_kernel(StepArgs p,
                                                                               PlanArgs pa) {
  __shared__ DmaLds<KS> lds;
  static_assert(sizeof(plan::Smem<kFusedPlanMax>) <= sizeof(lds.stage), "planner fits the stages");
  if (blockIdx.x == 0) {
    plan::run<kDmaThreads>(pa, *reinterpret_cast<plan::Smem<kFusedPlanMax>*>(lds.stage));
    return;
  }
  markov_step_dma<KS, NT>(p, step_map(p.B, blockIdx.x, gridDim.x, 1), lds);
}

// The same with the verify planner on workgroup 0 (its arrays in place of the copy stages), for
// the last position of an RNN-head draft at r = 256.
template <int KS, int NT>
__global__ __launch_bounds__(256, 1) void markov_step_deep4_plan_kernel(StepArgs p, PlanArgs pa) {
  __shared__ Deep4Lds<KS> lds;
  static_assert(sizeof(plan::Smem<kFusedPlanMax>) <= sizeof(lds.stage), "planner fits the stages");
  if (blockIdx.x == 0) {
    plan::run<256>(pa, *reinterpret_cast<plan::Smem<kFusedPlanMax>*>(lds.stage));
    return;
  }
  markov_step_deep4<KS, NT>(p, step_map(p.B, blockIdx.x, gridDim.x, 1), lds);
}

// One 1024-thread workgroup per request. Thread t holds a contiguous range of at most 16 tile
// partials (V <= 2^19) in registers: the row max comes from a block reduction, and each thread
// writes its tile masses exp(m - M) * s (fp32 exponential, fp64 product) to LDS with their sum.
// Wave 0 then locates the draw u * Z in three levels, each a wave scan and a ballot: the group
// of threads, the thread, and the tile (the last candidate with positive mass whose exclusive
// prefix is <= u * Z at the first two levels, the first tile whose inclusive prefix passes it at
// the last). Wave 0 recomputes that tile's logits and walks them to the token. The logits are
// scaled by the draft temperature as in the step kernel; a greedy draft instead takes the first
// maximal logit (the first tile whose max is the row max, then its first lane holding it).
// r = 512 takes 512 threads: its 32-step tile recompute needs more than 128 registers a lane.
// kHalf: 512 threads at r <= 256 for batches past 256 requests, up to 16 tiles a thread
// (V <= 262144). The kernel holds more than 64 registers a lane, so a CU takes 16 of its waves:
// one 1024-thread workgroup, or two of 512, and B = 512 then runs in one round of workgroups
// instead of two.
template <int KS, bool kHalf = false>
struct SampleCfg {
  static constexpr int kThreads = (KS >= 32 || kHalf) ? 512 : 1024;
  static constexpr int kPer = kHalf ? 16 : kMaxVocab / kTileTokens / kThreads;   // tiles a thread
};
constexpr int kHalfSampleMinB = 257;

__device__ __forceinline__ double tile_mass(float m, float s, float M) {
  return (m == kNegInf) ? 0.0 : static_cast<double>(exp_term(m - M)) * static_cast<double>(s);
}

template <int KS, int NT, bool kHalf = false>
__global__ __launch_bounds__((SampleCfg<KS, kHalf>::kThreads)) void draft_sample_kernel(SampleArgs p) {
  constexpr int kSampleThreads = SampleCfg<KS, kHalf>::kThreads;
  constexpr int kSamplePer = SampleCfg<KS, kHalf>::kPer;
  __shared__ float red_f[kSampleThreads / 64];
  __shared__ int red_i[kSampleThreads / 64];
  __shared__ double ssum[kSampleThreads];
  extern __shared__ double mass[];   // [ntiles], dynamic
  __shared__ float Ls[kTileTokens];
  __shared__ float Lc[kTileTokens];

  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int nt = p.ntiles;
  const float2* part = p.part + static_cast<size_t>(b) * nt;
  const size_t urow = (static_cast<size_t>(b) * p.gamma + p.k) * p.V;
  const size_t out = static_cast<size_t>(b) * p.gamma + p.k;

  // The partials' loads go out first, unconditionally (index clamped into the row), the count
  // picked by a uniform branch. The embedding row W1[prev] then goes to LDS by an LDS-DMA copy,
  // so it costs no registers while the partials are processed (the tile recompute reads it
  // back); the previous token is loaded before the partials, so both latencies overlap. The
  // validity of each partial is applied only after the copy is issued.
  const int per = (nt + kSampleThreads - 1) / kSampleThreads;   // uniform, <= kSamplePer
  const int c0 = min(nt, tid * per), c1 = min(nt, c0 + per);
  const int32_t prevtok = clamp_token(p.prev[static_cast<size_t>(b) * p.prev_stride], p.V);
  const int32_t forced = p.force ? clamp_token(p.force[out], p.V) : 0;   // conditioning token
  // The draw's uniform, loaded with the rest at entry (wave 0 reads it after the reductions).
  const float u_draw = (tid < 64) ? p.uniforms[(static_cast<size_t>(b) * (p.gamma + 1) + p.k) * 3]
                                  : 0.0f;
  __shared__ __attribute__((aligned(16))) uint16_t Es[16 * KS * NT];
  float2 v[kSamplePer];
  auto load_parts = [&](auto n_c) {
    constexpr int n = decltype(n_c)::value;
    float2 t[n];
#pragma unroll
    for (int i = 0; i < n; ++i) t[i] = part[min(c0 + i, nt - 1)];
    if (tid < 64)
      copy_row_to_lds<2 * KS * NT>(
          bias_row<NT>(p.W1, p.E, 16 * KS, prevtok, static_cast<int64_t>(out)), lds_addr(Es), tid);
#pragma unroll
    for (int i = 0; i < kSamplePer; ++i)
      v[i] = (i < n && i < per && c0 + i < c1) ? t[min(i, n - 1)] : make_float2(kNegInf, 0.0f);
  };
  if (per <= 4) {
    load_parts(std::integral_constant<int, 4>{});
  } else if (per <= 8) {
    load_parts(std::integral_constant<int, 8>{});
  } else {
    load_parts(std::integral_constant<int, kSamplePer>{});
  }
  float m = kNegInf;
#pragma unroll
  for (int i = 0; i < kSamplePer; ++i) m = fmaxf(m, v[i].x);
  const float M = block_max_lds<kSampleThreads>(m, red_f);
  int gtile = 0x7fffffff;
  if (p.greedy) {
    // Greedy draft (the partials hold unscaled logits): the first tile whose max is the row max.
    int first = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kSamplePer; ++i)
      if (i < per && c0 + i < c1 && v[i].x == M) first = min(first, c0 + i);
    gtile = block_min_int_lds<kSampleThreads>(first, red_i);
  } else {
    double S = 0.0;
#pragma unroll
    for (int i = 0; i < kSamplePer; ++i) {
      if (i < per && c0 + i < c1) {
        const double mi = tile_mass(v[i].x, v[i].y, M);
        mass[c0 + i] = mi;
        S += mi;
      }
    }
    ssum[tid] = S;
    lds_barrier();   // the embedding-row copy stays in flight (waited for before the recompute)
  }
  if (tid >= 64) return;
  Located L;
  double lse;
  if (p.greedy) {
    L.chunk = (gtile == 0x7fffffff) ? -1 : gtile;
    L.before = 0.0;
    L.target = 0.0;
    L.take_last = 0;
    lse = static_cast<double>(M);
  } else {
    const double u = static_cast<double>(u_draw);
    L = wave_locate<kSampleThreads>(
        ssum, nt, per, [u](double Z) { return u * Z; }, [&](int c) { return mass[c]; });
    lse = static_cast<double>(M) + log(L.total);
  }
  if (L.chunk < 0) {  // logits not finite: documented fallback
    if (tid == 0) {
      p.tokens[out] = 0;
      p.q[out] = __builtin_nanf("");
      p.lse[out] = __builtin_nan("");
    }
    return;
  }
  const float tm = part[L.chunk].x;   // goes out with the tile's loads
  wait_copies<0>();   // the embedding row copy (issued with the partials' loads)
  const int tok0 = L.chunk * kTileTokens;
  recompute_tile_lds<KS, NT>(Es, p.W2t, p.U + urow, tok0, p.V, Ls);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  int x;
  double qc;
  if (p.greedy) {
    // The first token of the tile holding the row max in the bit-identical recompute; the draft
    // distribution is the point mass on it.
    const unsigned long long hit =
        __ballot(lane < kTileTokens && tok0 + lane < p.V && Ls[lane] == M);
    x = tok0 + (hit ? __ffsll(static_cast<long long>(hit)) - 1 : 0);
    qc = ((p.force ? forced : x) == x) ? 1.0 : 0.0;
  } else {
    const double f = static_cast<double>(exp_term(tm - M));
    // Lane j's token mass for the walk and its probability exp(x_j - lse) (independent of the
    // walk, so the two overlap; the reported one is read from its lane afterwards).
    double w = 0.0, qj = 0.0;
    if (lane < kTileTokens && tok0 + lane < p.V) {
      const float xl = Ls[lane] * p.beta;   // as the step kernel scaled it
      w = f * static_cast<double>(exp_term(xl - tm));
      qj = exp(static_cast<double>(xl) - lse);
    }
    x = tok0 + walk_tile(w, L.before, L.target, L.take_last != 0);
    // The token whose probability is reported (and that conditions the next position).
    const int32_t cond = p.force ? forced : x;
    if (cond / kTileTokens != L.chunk) {
      recompute_tile_lds<KS, NT>(Es, p.W2t, p.U + urow, (cond / kTileTokens) * kTileTokens, p.V,
                                 Lc);
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
      qc = exp(static_cast<double>(Lc[cond % kTileTokens] * p.beta) - lse);
    } else {
      qc = read_lane(qj, cond % kTileTokens);
    }
  }
  if (tid == 0) {
    p.tokens[out] = x;
    p.q[out] = static_cast<float>(qc);
    p.lse[out] = lse;
  }
}

}  // namespace

// One step workgroup per compute unit (step_map places them), at least one per request group.
static int step_grid(const StepArgs& a, int first) {
  const int ngroups = (a.B + kDmaGroup - 1) / kDmaGroup;
  const int nstep = a.persistent_wgs - first;
  return first + (nstep > ngroups ? nstep : ngroups);
}

template <int KS, int NT>
static hipError_t launch_step_dma(const StepArgs& a, hipStream_t s) {
  // Tree depths past the first read one U row per request for several rows (u_shift > 0).
  if (a.u_shift > 0)
    launch_kernel(markov_step_dma_kernel<KS, NT, true>, dim3(step_grid(a, 0)), dim3(kDmaThreads), 0,
                  s, a);
  else
    launch_kernel(markov_step_dma_kernel<KS, NT, false>, dim3(step_grid(a, 0)), dim3(kDmaThreads),
                  0, s, a);
  return hipGetLastError();
}

template <int KS, int NT>
static hipError_t launch_step_deep4(const StepArgs& a, hipStream_t s) {
  launch_kernel(markov_step_deep4_kernel<KS, NT>, dim3(step_grid(a, 0)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int KS, int NT>
static hipError_t launch_step_plan(const StepArgs& a, const PlanArgs& pa, hipStream_t s) {
  const int grid = step_grid(a, 1);
  launch_kernel(markov_step_plan_kernel<KS, NT>, dim3(grid), dim3(kDmaThreads), 0, s,
                a, pa);
  return hipGetLastError();
}

template <int KS, int NT>
static hipError_t launch_step_prefetch(const StepArgs& a, hipStream_t s) {
  const int items = ((a.V + 4 * kTileTokens - 1) / (4 * kTileTokens)) *
                    ((a.B + StepCfg<KS * NT>::kBG - 1) / StepCfg<KS * NT>::kBG);
  const int grid = items < a.persistent_wgs ? items : a.persistent_wgs;
  if ((a.V & 3) == 0)
    launch_kernel(markov_step_kernel<KS, true, NT>, dim3(grid), dim3(kStepThreads), 0, s, a);
  else
    launch_kernel(markov_step_kernel<KS, false, NT>, dim3(grid), dim3(kStepThreads), 0, s,
                       a);
  return hipGetLastError();
}

template <int KS, int NT>
static hipError_t launch_step_kind(const StepArgs& a, hipStream_t s) {
  // The pipelined kernel copies 16-byte U chunks (rows 16-byte aligned: V % 4 == 0), one to four
  // 1 KB W2 copies per wave (64 <= r <= 256; two r = 512 stages would not fit in LDS), and the
  // debug-logits output would put global stores inside its copy pipeline: other requests take
  // the register-prefetch kernel.
  if constexpr (KS >= 4 && KS <= 16) {
    if (a.dbg == nullptr && (a.V & 3) == 0) return launch_step_dma<KS, NT>(a, s);
  }
  return launch_step_prefetch<KS, NT>(a, s);
}
// Bias rows of three bf16 terms (the RNN head) are built for r <= 256; the pipelined steps hold
// them in registers, with eight waves up to r = 128 and, at r = 256, with four (one per SIMD)
// over 32-token items in four stages.
template <int KS>
static hipError_t launch_step_ks(const StepArgs& a, hipStream_t s) {
  if (a.e_terms == 1) return launch_step_kind<KS, 1>(a, s);
  if constexpr (KS <= 8) {
    if (a.e_terms == kRnnTerms) return launch_step_kind<KS, kRnnTerms>(a, s);
  } else if constexpr (KS == 16) {
    if (a.e_terms == kRnnTerms) {
      if (a.dbg == nullptr && (a.V & 3) == 0) return launch_step_deep4<KS, kRnnTerms>(a, s);
      return launch_step_prefetch<KS, kRnnTerms>(a, s);
    }
  }
  return hipErrorInvalidValue;
}
template <int KS>
static hipError_t launch_sample_ks(const SampleArgs& a, hipStream_t s) {
  const size_t lds = static_cast<size_t>(a.ntiles) * sizeof(double);
  if constexpr (KS <= 16) {
    constexpr int kHalfThreads = SampleCfg<KS, true>::kThreads;
    if (a.B >= kHalfSampleMinB && a.ntiles <= kHalfThreads * SampleCfg<KS, true>::kPer) {
      if (a.e_terms == 1) {
        launch_kernel(draft_sample_kernel<KS, 1, true>, dim3(a.B), dim3(kHalfThreads), lds, s, a);
        return hipGetLastError();
      }
      if (a.e_terms == kRnnTerms) {
        launch_kernel(draft_sample_kernel<KS, kRnnTerms, true>, dim3(a.B), dim3(kHalfThreads), lds,
                      s, a);
        return hipGetLastError();
      }
      return hipErrorInvalidValue;
    }
  }
  if (a.e_terms == 1) {
    launch_kernel(draft_sample_kernel<KS, 1>, dim3(a.B), dim3(SampleCfg<KS>::kThreads), lds,
                       s, a);
    return hipGetLastError();
  }
  if constexpr (KS <= 16) {
    if (a.e_terms == kRnnTerms) {
      launch_kernel(draft_sample_kernel<KS, kRnnTerms>, dim3(a.B),
                         dim3(SampleCfg<KS>::kThreads), lds, s, a);
      return hipGetLastError();
    }
  }
  return hipErrorInvalidValue;
}

#define DSPARK_DISPATCH_KS(r, fn, ...)             \
  switch (r) {                                     \
    case 16: return fn<1>(__VA_ARGS__);            \
    case 32: return fn<2>(__VA_ARGS__);            \
    case 64: return fn<4>(__VA_ARGS__);            \
    case 128: return fn<8>(__VA_ARGS__);           \
    case 256: return fn<16>(__VA_ARGS__);          \
    case 512: return fn<32>(__VA_ARGS__);          \
    default: return hipErrorInvalidValue;          \
  }

hipError_t launch_markov_step(const StepArgs& a, int r, hipStream_t s) {
  DSPARK_DISPATCH_KS(r, launch_step_ks, a, s)
}
// The shapes the pipelined step with the planner beside it takes (eight waves; the four-stage
// kernel for the RNN head's three-term bias rows at r = 256).
bool markov_step_plan_fits(const StepArgs& a, int r, int B, int gamma) {
  return (r == 64 || r == 128 || r == 256) && (a.e_terms == 1 || a.e_terms == kRnnTerms) &&
         a.dbg == nullptr && (a.V & 3) == 0 &&
         static_cast<int64_t>(B) * gamma <= kFusedPlanMax &&
         a.persistent_wgs > (B + kDmaGroup - 1) / kDmaGroup;
}
hipError_t launch_markov_step_plan(const StepArgs& a, const PlanArgs& pa, int r, hipStream_t s) {
  if (a.e_terms == kRnnTerms) {
    switch (r) {
      case 64: return launch_step_plan<4, kRnnTerms>(a, pa, s);
      case 128: return launch_step_plan<8, kRnnTerms>(a, pa, s);
      case 256: {
        launch_kernel(markov_step_deep4_plan_kernel<16, kRnnTerms>, dim3(step_grid(a, 1)), dim3(256),
                      0, s, a, pa);
        return hipGetLastError();
      }
      default: return hipErrorInvalidValue;
    }
  }
  switch (r) {
    case 64: return launch_step_plan<4, 1>(a, pa, s);
    case 128: return launch_step_plan<8, 1>(a, pa, s);
    case 256: return launch_step_plan<16, 1>(a, pa, s);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_draft_sample(const SampleArgs& a, int r, hipStream_t s) {
  DSPARK_DISPATCH_KS(r, launch_sample_ks, a, s)
}

}  // namespace dspark
