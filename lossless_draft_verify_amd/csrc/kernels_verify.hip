// Lossless verify for gfx950.
//
// Sources: [V41] blog.javazero.top "DeepSeek-V4.1 模型结构（6）：解码，DSpark",
// "投机解码：让小的先猜，大的一次验一串" and the derivation that follows (accept with
// min(1, p/q); on reject resample from norm(max(0, p - q)); left to right, the first reject
// voids the rest; at least one token per round, the bonus from the target when all are
// accepted; that token is the next anchor); [AIL] ailearn.mscapital.top "DSpark：...", 02;
// [CSDN] deepseek.csdn.net DSpark walk-through, 2.1.
//
// Kernels, in stream order (no host synchronisation; grids are sized for the largest plan and
// read the actual row count from row_offsets[B] on the device):
//   target_stats       every verified target row, 4096-token segments: segment max and fp64 sum
//                      of exp(t - segment max); for an RNN-head draft it also splits the given
//                      fp32 bias vectors into their three bf16 terms for the later passes
//   accept             one wave per request: row log-sum-exp from the segments, left-to-right
//                      accept test u * q < p_t(x), emission kind / position / row
//   residual_partials  requests that rejected: the draft logits of the rejected position are
//                      recomputed with the draft's MFMA sequence (bit-identical), fused with the
//                      target row into w = max(0, p_t - p_d) and min(p_t, p_d), summed per tile
//   emit_sample        one workgroup per request: inverse-CDF draw from the residual tiles, or
//                      from the target row's segments for a bonus (or a zero-mass residual)
#include <type_traits>

#include "device.h"
#include "launch.h"
#include "dma.h"
#include "tiles.h"

namespace dspark {

namespace {

// Target row statistics, one 256-thread block per (row, 4096-token segment) work item on a
// grid-stride loop over the rows the plan produced (read on the device). Each thread holds 16
// values of an item in one of two register buffers; the next item's loads go into the other
// buffer before the current one is reduced, and the block reductions use LDS-only barriers, so
// those loads stay in flight through them. The vector-memory counter is in-order, so the loop
// is written for the compiler's wait placement: the loop is unrolled over the two buffers (no
// copy between them waits for a load), the next item's loads are issued on every pass (past the
// last item they read one line at the row start), and each item's statistics are kept in LDS
// and written when the block is done (a store between two loads would be waited for with them).
constexpr int kStatsBlocksPerCU = 8;        // up to 1023 rows
constexpr int kStatsBlocksPerCULarge = 4;   // 1024 rows and more
// Statistics held in LDS between writes: 64 items, so that the in-loop write runs for long row
// sets (b128-v151936-g15 and the PCTree rows give a block 68-76 items) as well as at the end.
constexpr int kStatsKept = 64;

// The row is read once per round: non-temporal loads, so that it displaces less of the W2
// columns the residual pass reads next. With V % 4 == 0 the four 16-byte loads are unguarded
// (addresses past the row are clamped to its last four values, and the reduction masks them),
// so they go out back to back; a guarded fallback writing the same registers would make the
// compiler wait for each load before issuing the next.
template <bool kVec4>
__device__ __forceinline__ void issue_segment(const VerifyArgs& p, int it, bool live,
                                              float (&x)[16]) {
  typedef float nt_f4 __attribute__((ext_vector_type(4)));
  const float* __restrict__ trow = p.target + static_cast<size_t>(it / p.nseg) * p.V;
  const int t0 = (it % p.nseg) * kSegTokens;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = t0 + 1024 * i + 4 * threadIdx.x;
    if constexpr (kVec4) {
      const float* src = live ? trow + min(v, p.V - 4) : p.target;
      const nt_f4 t = __builtin_nontemporal_load(reinterpret_cast<const nt_f4*>(src));
      x[4 * i + 0] = t.x;
      x[4 * i + 1] = t.y;
      x[4 * i + 2] = t.z;
      x[4 * i + 3] = t.w;
    } else {
      float o[4];
      load4(live ? trow : p.target, live ? v : 0, p.V, false, o);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * i + e] = o[e];
    }
  }
}

// Segment max and fp64 sum of exp(t - max) of item `it` (values past the row end are -inf), to
// LDS slot `slot`.
__device__ __forceinline__ void reduce_segment(const VerifyArgs& p, int it, float (&x)[16],
                                               float* red_f, double* red_d, float* kept_m,
                                               double* kept_s, int slot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t0 = (it % p.nseg) * kSegTokens;
  if (t0 + kSegTokens > p.V) {   // a row's last, partial segment (uniform over the block)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (t0 + 1024 * i + 4 * static_cast<int>(threadIdx.x) + e >= p.V) x[4 * i + e] = kNegInf;
  }
  float m = max16(x);
  m = wave_max(m);
  lds_barrier();
  if (lane == 0) red_f[w] = m;
  lds_barrier();
  m = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
  double s = 0.0;
  if (m != kNegInf) {
#pragma unroll
    for (int j = 0; j < 16; ++j) s += static_cast<double>(exp_term(x[j] - m));
  }
  s = wave_sum(s);
  if (lane == 0) red_d[w] = s;
  lds_barrier();
  if (threadIdx.x == 0) {
    kept_m[slot] = m;
    kept_s[slot] = (red_d[0] + red_d[1]) + (red_d[2] + red_d[3]);
  }
}

template <bool kSplit, bool kVec4>
__global__ __launch_bounds__(kBlock) void target_stats_kernel(VerifyArgs p) {
  __shared__ float red_f[kBlock / 64];
  __shared__ double red_d[kBlock / 64];
  __shared__ float kept_m[kStatsKept];
  __shared__ double kept_s[kStatsKept];
  const int G = gridDim.x;
  // Every request verifies at least one row, so rows 0 .. B-1 exist whatever the plan (the
  // row count is at least B): a first item among them goes out before the row count is read,
  // and that load's round trip no longer precedes the stream. Only a block whose first item
  // lies past them (a grid larger than B * nseg items) reads the count first.
  auto row_count = [&]() { return p.dense_rows > 0 ? p.dense_rows : p.row_offsets[p.B]; };
  int it = blockIdx.x;
  if (it >= p.B * p.nseg) {
    if (it >= row_count() * p.nseg) return;
  }
  float xa[16], xb[16];
  if constexpr (kSplit) {
    // The RNN head's bias terms for the later passes (a grid-strided share per thread): the
    // first value goes out with the first segment, and the split runs while it is loading.
    const int nsplit = p.B * p.gamma * p.r;
    const int i0 = blockIdx.x * kBlock + threadIdx.x;
    const float e0 = (i0 < nsplit) ? p.e_split[i0] : 0.0f;
    issue_segment<kVec4>(p, it, true, xa);
    for (int i = i0; i < nsplit; i += gridDim.x * kBlock)
      split_terms(i == i0 ? e0 : p.e_split[i],
                  p.E_split + static_cast<size_t>(i / p.r) * (kRnnTerms * p.r) + i % p.r, p.r);
  } else {
    issue_segment<kVec4>(p, it, true, xa);
  }
  const int nitems = row_count() * p.nseg;
  // Item k of this block is it0 + k G; its statistics go to output item it0 + k G too (the
  // item number is the (row, segment) offset of the output arrays).
  const int it0 = it;
  int k = 0;
  auto write_kept = [&](int k0, int cnt) {
    lds_barrier();
    if (static_cast<int>(threadIdx.x) < cnt) {
      const size_t o = static_cast<size_t>(it0) + static_cast<size_t>(k0 + threadIdx.x) * G;
      p.ws.seg_max[o] = kept_m[threadIdx.x];
      p.ws.seg_sum[o] = kept_s[threadIdx.x];
    }
    lds_barrier();
    // Drained here (once per kStatsKept items), so that the loop's own waits need not count
    // these stores: the compiler would otherwise wait for them, and for every load, at the top
    // of each pass.
    __builtin_amdgcn_s_waitcnt(0);
  };
  auto step = [&](float (&cur)[16], float (&nxt)[16]) {
    issue_segment<kVec4>(p, it + G, it + G < nitems, nxt);
    __builtin_amdgcn_sched_barrier(0);   // the loads stay ahead of the reduction's first wait
    reduce_segment(p, it, cur, red_f, red_d, kept_m, kept_s, k % kStatsKept);
    if (++k % kStatsKept == 0) write_kept(k - kStatsKept, kStatsKept);
    it += G;
  };
  while (true) {
    step(xa, xb);
    if (it >= nitems) break;
    step(xb, xa);
    if (it >= nitems) break;
  }
  if (k % kStatsKept) write_kept(k - k % kStatsKept, k % kStatsKept);
  // The residual list starts empty (accept appends to it). Written last: with no store ahead of
  // them, the row-count reads are known unclobbered and go through the scalar cache, so waiting
  // for the count does not wait for the segment loads issued before it.
  if (blockIdx.x == 0 && threadIdx.x == 0) *p.ws.rcount = 0;
}

// One wave per request. The log-sum-exp of all its verified rows and the accept-test inputs of
// all its positions are loaded together (no dependent chain per position); lane k then tests
// position k + 1 and the first failing lane, found with a ballot, is the first reject.
constexpr int kAcceptRows = 16;    // rows reduced per batch (one batch when gamma < 16)

__global__ __launch_bounds__(kBlock) void accept_kernel(VerifyArgs p) {
  __shared__ double lse_s[kBlock / 64][kMaxGamma + 1];   // each row's sum z, then its lse
  __shared__ float lse_m[kBlock / 64][kMaxGamma + 1];    // each row's max M
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.x * (kBlock / 64) + w;
  if (b >= p.B) return;
  const int ell = min(max(p.draft_len[b], 0), p.gamma);   // a length past gamma is clamped
  const int off = p.row_offsets[b];
  uint32_t fl = 0;
  // 0. The accept-test inputs of the first 64 positions go out with (ell, off), for every
  //    drafted position (lanes past ell are masked where they are used); then, needing only those,
  //    the segment statistics of every verified row (for nseg <= 32) and the target values of
  //    the drafted tokens.
  float tx0 = 0.0f, u0 = 0.0f, q0 = 0.0f;
  int32_t x0 = 0;
  double lsed0 = 0.0;
  const int32_t anc = p.anchor ? clamp_token(p.anchor[b], p.V) : 0;   // none for the RNN head
  if (lane < p.gamma) {
    x0 = clamp_token(p.tokens[static_cast<size_t>(b) * p.gamma + lane], p.V);
    lsed0 = p.lse[static_cast<size_t>(b) * p.gamma + lane];
    u0 = p.uniforms[(static_cast<size_t>(b) * (p.gamma + 1) + lane) * 3 + 1];
    q0 = p.q[static_cast<size_t>(b) * p.gamma + lane];
  }
  if (p.nseg <= 32) {
    // Rows in pairs: lanes 0..31 take row 2 pr, lanes 32..63 row 2 pr + 1, lane & 31 a segment.
    // A 32-lane butterfly reduces both rows at once, adding the same values in the same order
    // as a 64-lane one over one row (whose other lanes would add exact zeros).
    const int half = lane >> 5, sgi = lane & 31;
    for (int r0 = 0; r0 <= ell; r0 += kAcceptRows) {
      float mx[kAcceptRows / 2];
      double sg[kAcceptRows / 2];
#pragma unroll
      for (int pr = 0; pr < kAcceptRows / 2; ++pr) {
        const int row = r0 + 2 * pr + half;
        const bool valid = row <= ell && sgi < p.nseg;
        const size_t o =
            static_cast<size_t>(off + min(row, ell)) * p.nseg + min(sgi, p.nseg - 1);
        const float m0 = p.ws.seg_max[o];
        const double s0 = p.ws.seg_sum[o];
        mx[pr] = valid ? m0 : kNegInf;
        sg[pr] = valid ? s0 : 0.0;
      }
      if (r0 == 0 && lane < ell) tx0 = p.target[static_cast<size_t>(off + lane) * p.V + x0];
#pragma unroll
      for (int pr = 0; pr < kAcceptRows / 2; ++pr) {
        if (r0 + 2 * pr > ell) break;
        float M = mx[pr];
        M = fmaxf(M, __uint_as_float(lane_xor<16>(__float_as_uint(M))));
        M = fmaxf(M, __uint_as_float(lane_xor<8>(__float_as_uint(M))));
        M = fmaxf(M, __uint_as_float(lane_xor<4>(__float_as_uint(M))));
        M = fmaxf(M, __uint_as_float(lane_xor<2>(__float_as_uint(M))));
        M = fmaxf(M, __uint_as_float(lane_xor<1>(__float_as_uint(M))));
        double z = partial_mass(mx[pr], sg[pr], M);
        z += lane_xor<16>(z);
        z += lane_xor<8>(z);
        z += lane_xor<4>(z);
        z += lane_xor<2>(z);
        z += lane_xor<1>(z);
        const int row = r0 + 2 * pr + half;
        if (sgi == 0 && row <= ell) {
          lse_s[w][row] = z;
          lse_m[w][row] = M;
        }
      }
    }
  } else {
    if (lane < ell) tx0 = p.target[static_cast<size_t>(off + lane) * p.V + x0];
    // 1. log-sum-exp of rows off .. off + ell (segments: lane + 64 i, i < 2, nseg <= 128).
    for (int r0 = 0; r0 <= ell; r0 += kAcceptRows) {
      float mx[kAcceptRows][2];
      double sg[kAcceptRows][2];
#pragma unroll
      for (int r = 0; r < kAcceptRows; ++r)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int sgi = lane + 64 * i;
          const bool valid = (r0 + r <= ell) && sgi < p.nseg;
          const size_t o = static_cast<size_t>(off + min(r0 + r, ell)) * p.nseg + min(sgi, p.nseg - 1);
          const float m0 = p.ws.seg_max[o];
          const double s0 = p.ws.seg_sum[o];
          mx[r][i] = valid ? m0 : kNegInf;
          sg[r][i] = valid ? s0 : 0.0;
        }
#pragma unroll
      for (int r = 0; r < kAcceptRows; ++r) {
        if (r0 + r > ell) break;
        const float M = wave_max(fmaxf(mx[r][0], mx[r][1]));
        const double z = wave_sum(partial_mass(mx[r][0], sg[r][0], M) + partial_mass(mx[r][1], sg[r][1], M));
        if (lane == 0) {
          lse_s[w][r0 + r] = z;
          lse_m[w][r0 + r] = M;
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  // The rows' log-sum-exps M + log z, one row a lane (the fp64 log once for up to 64 rows).
  for (int r = lane; r <= ell; r += 64) lse_s[w][r] = static_cast<double>(lse_m[w][r]) + log(lse_s[w][r]);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  // 2. accept tests, 64 positions per batch: lane k tests position k0 + k + 1.
  int accepted = ell;
  for (int k0 = 0; k0 < ell; k0 += 64) {
    const int k = k0 + lane;
    bool ok = true;
    if (k < ell) {
      float tx = tx0, uk = u0, qk = q0;
      if (k0 > 0) {
        const int row = off + k;
        const int32_t x = clamp_token(p.tokens[static_cast<size_t>(b) * p.gamma + k], p.V);
        tx = p.target[static_cast<size_t>(row) * p.V + x];
        uk = p.uniforms[(static_cast<size_t>(b) * (p.gamma + 1) + k) * 3 + 1];
        qk = p.q[static_cast<size_t>(b) * p.gamma + k];
      }
      const double pt = exp(static_cast<double>(tx) - lse_s[w][k]);
      ok = static_cast<double>(uk) * static_cast<double>(qk) < pt;
    }
    const unsigned long long fail = __ballot(!ok);
    if (fail) {
      accepted = k0 + __ffsll(static_cast<long long>(fail)) - 1;
      break;
    }
  }
  // Rows tested before the first reject, and the emission row, feed the non-finite flag.
  const bool rejected = accepted < ell;
  const int last = rejected ? accepted : ell;    // 0-based row of the emission
  for (int k = lane; k <= last; k += 64)
    if (!isfinite(lse_s[w][k])) fl |= 1u;
  fl = (__ballot(fl != 0u) != 0ull) ? 1u : 0u;
  // Inputs of the residual record: positions 0..63 come from the registers loaded in step 0,
  // later ones from memory.
  int32_t prev_x = anc, xtok = 0;
  double lse_d = 0.0;
  if (rejected) {
    const int32_t xs = read_lane(static_cast<int>(x0), (last + 63) & 63);   // last: wave-uniform
    const int32_t xr = read_lane(static_cast<int>(x0), last & 63);
    const double ls = read_lane(lsed0, last & 63);
    prev_x = (last == 0) ? anc
             : (last - 1 < 64 ? xs
                              : clamp_token(p.tokens[static_cast<size_t>(b) * p.gamma + last - 1], p.V));
    xtok = (last < 64) ? xr : p.tokens[static_cast<size_t>(b) * p.gamma + last];
    lse_d = (last < 64) ? ls : p.lse[static_cast<size_t>(b) * p.gamma + last];
  }
  if (lane == 0) {
    if (rejected) {
      ResRec r;
      r.b = b;
      r.j = last + 1;
      r.erow = off + last;
      r.prev = prev_x;
      r.tok = xtok;
      r.lse_d = lse_d;
      r.lse_t = lse_s[w][last];
      p.ws.rrec[atomicAdd(p.ws.rcount, 1)] = r;
    }
    p.accept_len[b] = accepted;
    p.ws.ekind[b] = rejected ? kEmitResidual : kEmitBonus;
    p.ws.epos[b] = last + 1;
    p.ws.erow[b] = off + last;
    p.ws.erow_lse[b] = lse_s[w][last];
    p.ws.eflags[b] = fl;
    p.ws.eprev[b] = prev_x;
  }
}

// Previous token of emission position j (1-based): the anchor for j = 1.
__device__ __forceinline__ int32_t emit_prev(const VerifyArgs& p, int b, int j) {
  return clamp_token((j == 1) ? p.anchor[b] : p.tokens[static_cast<size_t>(b) * p.gamma + j - 2], p.V);
}

// Draft probability of one token in fp32 (prob_f32): softmax(beta L) of the position (cd its
// log-sum-exp times log2(e), beta the draft temperature's multiplier, applied in fp32 as in the
// draft), or, for a greedy draft, the point mass on the drafted token.
__device__ __forceinline__ float draft_prob(float L, float beta, double cd, bool greedy,
                                            bool drafted) {
  return greedy ? (drafted ? 1.0f : 0.0f) : prob_f32(L * beta, cd);
}
// The same with the kind of draft fixed at compile time (the residual passes, where a run-time
// select per token is measurable; a greedy pass never reads the draft logits).
template <bool Greedy>
__device__ __forceinline__ float draft_prob_t(float L, float beta, double cd, bool drafted) {
  if constexpr (Greedy) {
    return drafted ? 1.0f : 0.0f;
  } else {
    return prob_f32(L * beta, cd);
  }
}

// a or b by a wave-uniform byte selector: v_perm_b32 takes bytes 0-3 of (b, a) from a for
// 0x03020100 and from b for 0x07060504. A byte permute, so that the choice between two elements
// of a register array stays one instruction: a select there would be folded into a run-time
// register index.
constexpr uint32_t kPickA = 0x03020100u, kPickB = 0x07060504u;
__device__ __forceinline__ float pick(float a, float b, uint32_t sel) {
  return __uint_as_float(__builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), sel));
}

// Residual weight and overlap of one token in fp32: w = max(0, p_t - p_d), o = min(p_t, p_d),
// with p_t = exp(t - lse_t) from prob_f32 (ct = lse_t log2(e)). Every site that forms these
// terms (the residual pass, its fallback and the emission's tile walk) calls this, so the walk
// sees the bits the tile sums were made of.
__device__ __forceinline__ void residual_pair(float pd, float t, double ct, float& w, float& o) {
  const float pt = prob_f32(t, ct);
  const float d = pt - pd;
  w = (0.0f < d) ? d : 0.0f;
  o = (pd < pt) ? pd : pt;
}

// Sum of eight fp32 terms as a balanced tree (three rounding levels), widened to fp64.
__device__ __forceinline__ double sum8(const float (&x)[8]) {
  return static_cast<double>(((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7])));
}

template <int KS, bool Greedy, int NT>
__global__ __launch_bounds__(kBlock, 2) void residual_partials_kernel(VerifyArgs p) {
  using C = StepCfg<KS * NT>;   // LDS rows hold the NT r bf16 of a bias row
  constexpr int r = 16 * KS;
  __shared__ __attribute__((aligned(16))) uint16_t E[C::kBG * C::kLdsRow];
  __shared__ int list[C::kBG];
  __shared__ int red_i[kBlock / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int tok0 = blockIdx.x * (4 * kTileTokens) + wave * kTileTokens;
  const bool active = tok0 < p.V;
  const bool vec4 = (p.V & 3) == 0;

  // Residual requests in request order: contiguous request ranges per thread + block scan.
  const int per = (p.B + kBlock - 1) / kBlock;
  const int b0 = min(p.B, tid * per), b1 = min(p.B, b0 + per);
  int cnt = 0;
  for (int b = b0; b < b1; ++b) cnt += (p.ws.ekind[b] == kEmitResidual) ? 1 : 0;
  int nres;
  const int first = block_exclusive_scan_int<kBlock>(cnt, red_i, &nres);
  if (nres == 0) return;

  u16x8_t a[KS];
  load_w2_tile<KS>(a, p.W2t, tok0 + col, p.V, half);

  for (int g0 = 0; g0 < nres; g0 += C::kBG) {
    const int nb = min(C::kBG, nres - g0);
    int rank = first;
    for (int b = b0; b < b1; ++b) {
      if (p.ws.ekind[b] == kEmitResidual) {
        if (rank >= g0 && rank < g0 + C::kBG) list[rank - g0] = b;
        ++rank;
      }
    }
    __syncthreads();
    constexpr int kChunks = NT * r / 8;
    for (int c = tid; c < C::kBG * kChunks; c += kBlock) {
      const int i = c / kChunks, q = c % kChunks;
      u16x8_t v = zero_u16x8();
      if (i < nb) {
        const int b = list[i];
        const int j = p.ws.epos[b];
        const int32_t prevtok = (NT == 1) ? emit_prev(p, b, j) : 0;
        const int64_t pos = static_cast<int64_t>(b) * p.gamma + j - 1;
        v = load_u16x8(bias_row<NT>(p.W1, p.E, r, prevtok, pos) + q * 8);
      }
      *reinterpret_cast<u16x8_t*>(&E[i * C::kLdsRow + q * 8]) = v;
    }
    __syncthreads();
    if (active) {
      for (int nt = 0; nt * 32 < nb; ++nt) {
        const uint16_t* erow = &E[(nt * 32 + col) * C::kLdsRow + 8 * half];
        f32x16_t acc = {};
#pragma unroll
        for (int s = 0; s < NT * KS; ++s)
          acc = mfma_32x32x16(a[s % KS], load_u16x8(erow + 16 * s), acc);
        const int i = nt * 32 + col;
        if (i < nb) {
          const int b = list[i];
          const int j = p.ws.epos[b];
          const float* Urow = p.U + (static_cast<size_t>(b) * p.gamma + j - 1) * p.V;
          const float* trow = p.target + static_cast<size_t>(p.ws.erow[b]) * p.V;
          const double cd = p.lse[static_cast<size_t>(b) * p.gamma + j - 1] * kLog2e64;
          const double ct = p.ws.erow_lse[b] * kLog2e64;
          const int32_t xtok = p.tokens[static_cast<size_t>(b) * p.gamma + j - 1];
          float L[16];
          tile_logits(acc, Urow, tok0, p.V, half, vec4, L);
          float w8[2][8], o8[2][8];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int v = tok0 + 8 * g + 4 * half;
            float t[4];
            load4(trow, v, p.V, vec4, t);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float w = 0.0f, o = 0.0f;
              if (v + e < p.V)
                residual_pair(draft_prob_t<Greedy>(L[4 * g + e], p.beta, cd, v + e == xtok),
                              t[e], ct, w, o);
              w8[g >> 1][4 * (g & 1) + e] = w;
              o8[g >> 1][4 * (g & 1) + e] = o;
            }
          }
          double W = sum8(w8[0]) + sum8(w8[1]);
          double O = sum8(o8[0]) + sum8(o8[1]);
          W = W + lane_xor<32>(W);
          O = O + lane_xor<32>(O);
          if (half == 0) {
            const size_t o = static_cast<size_t>(b) * p.ntiles + tok0 / kTileTokens;
            p.ws.rsum[o] = W;
            p.ws.rmin[o] = O;
          }
        }
      }
    }
    __syncthreads();
  }
}

// ---- Pipelined residual pass --------------------------------------------------------------
//
// The structure of the pipelined draft step, for the requests that rejected: a persistent grid
// whose workgroups split the residual list into groups of 64 (records written by the accept
// scan) and the vocabulary into contiguous ranges of 64-token items. Per item, the 64 W2t rows,
// the group's U row segments (draft position j) and target row segments are copied into one of
// two LDS stages; waves (sub, rq, part) recompute the logits of tile `sub` for requests
// 32 rq .. +32 with the draft's MFMA sequence (bit-identical logits; the two waves of a pair
// compute the same tile) and reduce w = max(0, p_t - p_d) and min(p_t, p_d) in fp64 over half of
// the tile each (the fp64 exponentials dominate, so eight waves share them).
constexpr int kResThreads = 512;
constexpr int kResGroup = 64;
constexpr int kXcds = 8;          // accelerator complex dies of an MI355X, each with its own L2
constexpr int kResTiles = 2;

// PW: halves of a tile's epilogue each wave takes (1: eight waves, two per tile; 2: four waves,
// one per tile and SIMD, with room for the RNN head's three-term bias rows at r = 256).
template <int KS, int PW = 1>
struct ResStep {
  static constexpr int r = 16 * KS;
  static constexpr int kThreads = kResThreads / PW;
  static constexpr int kTok = kResTiles * kTileTokens;              // 64 tokens per item
  static constexpr int kW2Chunks = 2 * KS;
  static constexpr int kW2Bytes = kTok * kW2Chunks * 16;
  static constexpr int kRowChunks = kTok / 4;                       // 16 per row segment
  static constexpr int kRowBytes = kResGroup * kRowChunks * 16;     // 16 KB
  static constexpr int kStageBytes = kW2Bytes + 2 * kRowBytes;      // W2t | U rows | target rows
  static constexpr int kStages = 2;
  static constexpr int kPartItems = 4;
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kW2Copies = kW2Bytes / 1024 / kWaves;
  static constexpr int kRowCopies = kRowBytes / 1024 / kWaves;
  static constexpr int kCopies = kW2Copies + 2 * kRowCopies;
  static constexpr int kECopies = kResGroup * kW2Chunks * 16 / 1024 / kWaves;
  static constexpr int kW2Swz = (kW2Chunks >= 16) ? 15 : kW2Chunks - 1;
  static constexpr int kAOffs = (KS < 8) ? KS : 8;
  static_assert(KS >= 8 && KS <= 16, "one or two 1 KB W2 copies per wave per item");
  static_assert(kRowCopies >= 1 && kCopies <= 63, "copy counts");
  static_assert(kResGroup * kW2Chunks * 16 <= kStageBytes, "embedding rows fit in one stage");
};

template <int KS, bool Greedy, int NT, int PW>
__device__ __forceinline__ void residual_dma(const VerifyArgs& p) {
  using D = ResStep<KS, PW>;
  __shared__ __attribute__((aligned(1024))) unsigned char stage[D::kStages * D::kStageBytes];
  __shared__ double2 pbuf[D::kPartItems * kResTiles * 2 * kResGroup];   // (sum w, sum min)
  __shared__ ResRec rec[kResGroup];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int sub = (wave >> 1) & 1, rq = wave & 1;
  const int part = (PW == 1) ? (wave >> 2) : 0;   // the wave's (first) half of the tile
  const uint32_t part_sel = part ? kPickB : kPickA;
  const int nres = *p.ws.rcount;
  if (nres <= 0) return;
  const int ngroups = (nres + kResGroup - 1) / kResGroup;   // <= gridDim.x (launch sizing)
  const int nwg = gridDim.x / ngroups;
  const int bid = blockIdx.x;
  if (bid >= nwg * ngroups) return;
  // Block -> (group, vocabulary range). Blocks are dispatched round-robin over the XCDs, so
  // blocks b and b + kXcds share one; with several groups, the groups of one range go to blocks
  // that share an XCD, and the range's W2t rows come from HBM once and then from that XCD's L2
  // (a bijection when nwg is a multiple of kXcds; otherwise consecutive blocks).
  int group, wg;
  if (ngroups > 1 && nwg % kXcds == 0) {
    const int xcd = bid % kXcds, slot = bid / kXcds;
    group = slot % ngroups;
    wg = (slot / ngroups) * kXcds + xcd;
  } else {
    group = bid % ngroups;
    wg = bid / ngroups;
  }
  const int gcount = min(kResGroup, nres - group * kResGroup);
  const int nitems = (p.V + D::kTok - 1) / D::kTok;
  const int item_lo = static_cast<int>(static_cast<int64_t>(nitems) * wg / nwg);
  const int n = static_cast<int>(static_cast<int64_t>(nitems) * (wg + 1) / nwg) - item_lo;
  if (n <= 0) return;
  if (tid < kResGroup) rec[tid] = p.ws.rrec[group * kResGroup + min(tid, gcount - 1)];
  __syncthreads();
  const int row_own = 32 * rq + col;
  const bool wave_active = 32 * rq < gcount;
  // Copies of request rows are issued only for rows below gcount (a 1 KB copy covers
  // 1024 / (16 kRowChunks) rows; a wave's copies cover consecutive rows, so its valid ones are a
  // prefix): nrow_w row copies per kind and ne_w embedding-row copies for this wave. The waits
  // use this wave's exact count of copies per item.
  constexpr int kRowsPerCopy = 1024 / (16 * D::kRowChunks);
  constexpr int kERowsPerCopy = 1024 / (16 * D::kW2Chunks);
  const int nrow_w = min(D::kRowCopies, max(0, (gcount - kRowsPerCopy * D::kRowCopies * wave +
                                                kRowsPerCopy - 1) / kRowsPerCopy));
  const int ne_w = (NT == 1) ? min(D::kECopies, max(0, (gcount - kERowsPerCopy * D::kECopies * wave +
                                                        kERowsPerCopy - 1) / kERowsPerCopy))
                             : 0;
  auto wait_item = [&]() { wait_copies_upto<D::kW2Copies, 2, D::kRowCopies>(nrow_w); };

  const uint32_t stage_addr = lds_addr(stage);
  uint32_t a_off[D::kAOffs], u_off[PW][2];
  {
    const int wrow = 32 * sub + col;
#pragma unroll
    for (int t = 0; t < D::kAOffs; ++t)
      a_off[t] = 16 * (wrow * D::kW2Chunks + ((2 * t + half) ^ (wrow & D::kW2Swz)));
#pragma unroll
    for (int pp = 0; pp < PW; ++pp)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int g = 2 * (part + pp) + h;
        u_off[pp][h] = D::kW2Bytes + 16 * (row_own * D::kRowChunks +
                                           ((8 * sub + 2 * g + half) ^ (row_own & 15)));
      }
  }

  // This wave's share of item j's copies. Positions past V are clamped (masked later).
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
    for (int i = 0; i < D::kRowCopies; ++i) {
      if (i >= nrow_w) break;   // wave-uniform: copies past the group's rows are not issued
      const int q = wave * D::kRowCopies + i;
      const int slot = 64 * q + lane;
      const int row = slot / D::kRowChunks;
      const int c = (slot % D::kRowChunks) ^ (row & 15);
      const int v = min(tok0 + 4 * c, p.V - 4);
      const ResRec& R = rec[row];
      copy16_to_lds_nt(p.U + (static_cast<size_t>(R.b) * p.gamma + R.j - 1) * p.V + v,
                       base + D::kW2Bytes + 1024 * q);
      copy16_to_lds_nt(p.target + static_cast<size_t>(R.erow) * p.V + v,
                       base + D::kW2Bytes + D::kRowBytes + 1024 * q);
    }
  };

  // Tile sums of items j0 .. j1-1 (after a barrier) to rsum / rmin: with kSlots the power of two
  // at or above their tile count, thread t takes tile slot t % kSlots of the rows t / kSlots +
  // kRowStep i, so consecutive threads write consecutive tiles of one request, and its LDS reads
  // all go out before its stores.
  auto flush_slots = [&](int j0, int j1, auto slots_c) {
    constexpr int kSlots = decltype(slots_c)::value;
    constexpr int kRowStep = D::kThreads / kSlots;
    constexpr int kPasses = (kResGroup + kRowStep - 1) / kRowStep;
    static_assert(D::kThreads % kSlots == 0 && kSlots <= D::kPartItems * kResTiles, "flush mapping");
    const int tt = tid % kSlots, r0 = tid / kSlots;   // tile slot, first row
    const int j = j0 + tt / kResTiles;
    const int tile = (item_lo + j0) * kResTiles + tt;
    const bool ok = tt < (j1 - j0) * kResTiles && tile < p.ntiles;
    const int slot = ((j % D::kPartItems) * kResTiles + tt % kResTiles) * 2;
    double2 v0[kPasses], v1[kPasses];
    int rb[kPasses];
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
      const int row = min(r0 + kRowStep * i, kResGroup - 1);
      v0[i] = pbuf[slot * kResGroup + row];
      v1[i] = pbuf[(slot + 1) * kResGroup + row];
      rb[i] = rec[row].b;
    }
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
      if (ok && r0 + kRowStep * i < gcount) {
        const size_t o = static_cast<size_t>(rb[i]) * p.ntiles + tile;
        p.ws.rsum[o] = v0[i].x + v1[i].x;
        p.ws.rmin[o] = v0[i].y + v1[i].y;
      }
    }
  };
  auto flush = [&](int j0, int j1) {
    const int per = (j1 - j0) * kResTiles;   // uniform
    if (per <= 2) {
      flush_slots(j0, j1, std::integral_constant<int, 2>{});
    } else if (per <= 4) {
      flush_slots(j0, j1, std::integral_constant<int, 4>{});
    } else {
      flush_slots(j0, j1, std::integral_constant<int, D::kPartItems * kResTiles>{});
    }
  };

  // Prologue. Markov head: embedding rows W1[prev] of the group into stage 1, item 0 into
  // stage 0. RNN head: each lane loads its request's bias row (both terms) into registers,
  // drained before the copies start.
  u16x8_t e[NT * KS];
  if constexpr (NT > 1) {
    const ResRec& R = rec[row_own];
    const uint16_t* erow =
        bias_row<NT>(p.W1, p.E, D::r, 0, static_cast<int64_t>(R.b) * p.gamma + R.j - 1) + 8 * half;
#pragma unroll
    for (int s = 0; s < NT * KS; ++s) e[s] = load_u16x8(erow + 16 * s);
    __builtin_amdgcn_s_waitcnt(0);
  }
  {
    const uint32_t ebase = stage_addr + D::kStageBytes;
#pragma unroll
    for (int i = 0; i < D::kECopies; ++i) {
      if (i >= ne_w) break;   // wave-uniform
      const int q = wave * D::kECopies + i;
      const int slot = 64 * q + lane;
      const int row = slot / D::kW2Chunks;
      const int c = (slot % D::kW2Chunks) ^ (row & D::kW2Swz);
      copy16_to_lds(p.W1 + static_cast<size_t>(rec[row].prev) * D::r + 8 * c, ebase + 1024 * q);
    }
  }
  issue(0);
  wait_item();   // the embedding rows (issued first) have landed
  asm volatile("s_barrier" ::: "memory");
  if constexpr (NT == 1) {
    const unsigned char* eb = stage + D::kStageBytes;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      e[s] = *reinterpret_cast<const u16x8_t*>(
          eb + 16 * (row_own * D::kW2Chunks + ((2 * s + half) ^ (row_own & D::kW2Swz))));
  }
  const double cd = rec[row_own].lse_d * kLog2e64, ct = rec[row_own].lse_t * kLog2e64;
  const int32_t xtok = rec[row_own].tok;
  lds_barrier();
  int flushed = 0;
  for (int j = 0; j < n; ++j) {
    if (j + 1 < n) {
      issue(j + 1);
      wait_item();   // outstanding: at most item j + 1's copies
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
      float4 uu[PW][2], tt[PW][2];
#pragma unroll
      for (int pp = 0; pp < PW; ++pp)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uu[pp][h] = *reinterpret_cast<const float4*>(base + u_off[pp][h]);
          tt[pp][h] = *reinterpret_cast<const float4*>(base + u_off[pp][h] + D::kRowBytes);
        }
      f32x16_t acc = {};
#pragma unroll
      for (int s = 0; s < NT * KS; ++s) acc = mfma_32x32x16(a[s % KS], e[s], acc);
#pragma unroll
      for (int pp = 0; pp < PW; ++pp) {
        const int pt = part + pp;
        // This half of the tile (accumulator slot groups 2 pt, 2 pt + 1), in token order. With
        // eight waves the half is a run-time choice and its slots are taken by byte permutes (a
        // select here becomes a register-indexing sequence per term); only a tile that reaches
        // past V checks its tokens.
        float Lh[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          Lh[q] = (PW == 1) ? pick(acc[q], acc[8 + q], part_sel) : acc[8 * pp + q];
        float w8[8], o8[8];
        auto half_tile = [&](auto checked) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int v = tok0 + 8 * (2 * pt + h) + 4 * half;
            const float u4[4] = {uu[pp][h].x, uu[pp][h].y, uu[pp][h].z, uu[pp][h].w};
            const float t4[4] = {tt[pp][h].x, tt[pp][h].y, tt[pp][h].z, tt[pp][h].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float w = 0.0f, o = 0.0f;
              if (!decltype(checked)::value || v + i < p.V)
                residual_pair(draft_prob_t<Greedy>(u4[i] + Lh[4 * h + i], p.beta, cd,
                                                   v + i == xtok),
                              t4[i], ct, w, o);
              w8[4 * h + i] = w;
              o8[4 * h + i] = o;
            }
          }
        };
        if (tok0 + kTileTokens <= p.V)
          half_tile(std::false_type{});
        else
          half_tile(std::true_type{});
        double W = sum8(w8), O = sum8(o8);
        W = W + other_half(W, half);
        O = O + other_half(O, half);
        if (half == 0 && row_own < gcount)
          pbuf[(((j % D::kPartItems) * kResTiles + sub) * 2 + pt) * kResGroup + row_own] =
              make_double2(W, O);
      }
    }
    lds_barrier();
    if ((j + 1) % D::kPartItems == 0 && j + 1 < n) {
      flush(flushed, j + 1);
      flushed = j + 1;
      wait_copies<0>();   // the stores join the counter: drain it so later counts hold copies only
    }
  }
  flush(flushed, n);
}

template <int KS, bool Greedy, int NT>
__global__ __launch_bounds__(kResThreads, 1) void residual_dma_kernel(VerifyArgs p) {
  residual_dma<KS, Greedy, NT, 1>(p);
}

// Four waves, one per tile and SIMD, each taking both halves of its tile's epilogue in turn (the
// same half sums as the eight-wave kernel): 512 registers a lane hold the RNN head's three-term
// bias rows at r = 256.
template <int KS, bool Greedy, int NT>
__global__ __launch_bounds__(kResThreads / 2, 1) void residual_dma_wave4_kernel(VerifyArgs p) {
  residual_dma<KS, Greedy, NT, 2>(p);
}

template <int KS, int NT>
__global__ __launch_bounds__(kBlock) void emit_sample_kernel(VerifyArgs p) {
  extern __shared__ double stage[];   // padded: residual tile masses, or one segment's terms
  __shared__ double ssum[kBlock];     // per-thread sums over contiguous ranges (wave-0 search)
  __shared__ double osum[kBlock];     // per-thread overlap sums (beta)
  __shared__ Located loc;
  __shared__ float seg_m, row_m;     // the chosen segment's max, the row's largest segment max
  __shared__ float Ls[kTileTokens];
  __shared__ __attribute__((aligned(16))) uint16_t Es[16 * KS * NT];

  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int kind = p.ws.ekind[b];
  const int j = p.ws.epos[b];
  const int erow = p.ws.erow[b];
  uint32_t fl = p.ws.eflags[b];
  const int32_t eprev = p.ws.eprev[b];
  const float* trow = p.target + static_cast<size_t>(erow) * p.V;
  bool from_target = (kind == kEmitBonus);
  int token = 0;
  // The residual tile masses and overlap partials of this request's first batch are loaded
  // with the records, before the kind is known (a bonus emission does not use them), so that
  // they do not wait for it; so are the uniform and the inputs of the residual terms of the tile
  // walk (they need only the position).
  constexpr int kBatch = 16;
  const int nt = p.ntiles;
  const size_t rbase = static_cast<size_t>(b) * nt;
  double w0[kBatch], ov0[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    const int c = min(i * kBlock + tid, nt - 1);
    w0[i] = p.ws.rsum[rbase + c];
    ov0[i] = p.ws.rmin[rbase + c];
  }
  const size_t pos = static_cast<size_t>(b) * p.gamma + j - 1;
  const double u = static_cast<double>(p.uniforms[(static_cast<size_t>(b) * (p.gamma + 1) + j - 1) * 3 + 2]);
  const int32_t xtok = p.tokens[pos];
  const double lse_d = p.lse[pos], lse_t = p.ws.erow_lse[b];

  if (kind == kEmitResidual) {
    // Residual tile masses into LDS (16 loads in flight per thread) with the overlap partials;
    // the embedding row of the position's previous token (accept's record) is copied into LDS
    // behind them and waited for only before the recompute.
    const int32_t prevtok = (NT == 1) ? clamp_token(eprev, p.V) : 0;
    if (tid < 64)
      copy_row_to_lds<2 * KS * NT>(
          bias_row<NT>(p.W1, p.E, 16 * KS, prevtok, static_cast<int64_t>(pos)), lds_addr(Es),
          tid);
    double o = 0.0;
    for (int c0 = 0; c0 < nt; c0 += kBlock * kBatch) {
      double w[kBatch], ov[kBatch];
      if (c0 == 0) {
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          w[i] = w0[i];
          ov[i] = ov0[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const int c = min(c0 + i * kBlock + tid, nt - 1);
          w[i] = p.ws.rsum[rbase + c];
          ov[i] = p.ws.rmin[rbase + c];
        }
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int c = c0 + i * kBlock + tid;
        if (c < nt) {
          stage[padded(c)] = w[i];
          o += ov[i];
        }
      }
    }
    lds_barrier();
    const int per = (nt + kBlock - 1) / kBlock;   // <= 64 (V <= 2^19)
    const int c0 = min(nt, tid * per), c1 = min(nt, c0 + per);
    double S = 0.0;
    for (int c = c0; c < c1; ++c) S += stage[padded(c)];
    ssum[tid] = S;
    osum[tid] = o;
    lds_barrier();
    if (tid < 64) {
      double og = 0.0;
#pragma unroll
      for (int i = 0; i < kBlock / 64; ++i) og += osum[(kBlock / 64) * lane + i];
      og = wave_sum(og);
      if (tid == 0 && p.beta_emit) p.beta_emit[b] = static_cast<float>(og);
      const Located L = wave_locate<kBlock>(
          ssum, nt, per, [u](double Z) { return u * Z; }, [&](int c) { return stage[padded(c)]; });
      if (tid == 0) loc = L;
    }
    lds_barrier();
    const Located L = loc;
    if (L.chunk < 0) {
      fl |= 2u;
      from_target = true;
    } else {
      if (tid >= 64) return;
      const int tok0 = L.chunk * kTileTokens;
      const float* Urow = p.U + pos * p.V;
      const float tv = (lane < kTileTokens && tok0 + lane < p.V) ? trow[tok0 + lane] : 0.0f;
      wait_copies<0>();   // the embedding row
      recompute_tile_lds<KS, NT>(Es, p.W2t, Urow, tok0, p.V, Ls);
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
      float w = 0.0f;
      if (lane < kTileTokens && tok0 + lane < p.V) {
        float ov;
        residual_pair(draft_prob(Ls[lane], p.beta, lse_d * kLog2e64, p.greedy, tok0 + lane == xtok),
                      tv, lse_t * kLog2e64, w, ov);
      }
      token = tok0 + walk_tile(static_cast<double>(w), L.before, L.target, L.take_last != 0);
    }
  } else if (tid == 0 && p.beta_emit) {
    p.beta_emit[b] = -1.0f;
  }

  if (from_target) {
    // Draw from p_t of the emission row. Wave 0 picks the segment: lane l owns segments 2l,
    // 2l + 1 (nseg <= 128), masses relative to the row's largest segment max.
    const size_t base = static_cast<size_t>(erow) * p.nseg;
    if (tid < 64) {
      float m[2];
      double sg[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int s = 2 * lane + i;
        m[i] = (s < p.nseg) ? p.ws.seg_max[base + s] : kNegInf;
        sg[i] = (s < p.nseg) ? p.ws.seg_sum[base + s] : 0.0;
      }
      const float M = wave_max(fmaxf(m[0], m[1]));
      double S = 0.0;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const double ms = partial_mass(m[i], sg[i], M);
        stage[2 * lane + i] = ms;
        S += ms;
      }
      ssum[lane] = S;
      __builtin_amdgcn_s_waitcnt(0);   // this wave's LDS writes, read back by other lanes
      __builtin_amdgcn_wave_barrier();
      const Located Sg = wave_locate<64>(
          ssum, p.nseg, 2, [u](double Z) { return u * Z; }, [&](int c) { return stage[c]; });
      if (tid == 0) {
        loc = Sg;
        row_m = M;
      }
      if (Sg.chunk >= 0 && lane == (Sg.chunk >> 1)) seg_m = m[Sg.chunk & 1];
    }
    __syncthreads();
    const Located S = loc;
    if (S.chunk < 0) {
      token = 0;
    } else {
      // The segment's 4096 terms exp(t - segment max): thread t takes tokens 16 t .. 16 t + 15.
      const int t0 = S.chunk * kSegTokens;
      const int n = min(kSegTokens, p.V - t0);
      const float sm = seg_m;
      const bool vec4 = (p.V & 3) == 0;
      double Sum = 0.0;
      float x16[16];
      load16(trow, t0 + 16 * tid, p.V, vec4, x16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 16 * tid + 4 * i + e;
          const double ms = (c < n) ? static_cast<double>(exp_term(x16[4 * i + e] - sm)) : 0.0;
          stage[padded(c)] = ms;
          Sum += ms;
        }
      }
      ssum[tid] = Sum;
      __syncthreads();
      if (tid >= 64) return;
      const double f = exp(static_cast<double>(sm) - static_cast<double>(row_m));
      const double tgt = S.take_last ? __builtin_inf() : (S.target - S.before) / f;
      const Located T = wave_locate<kBlock>(
          ssum, n, kSegTokens / kBlock, [tgt](double) { return tgt; },
          [&](int c) { return stage[padded(c)]; });
      token = t0 + (T.chunk >= 0 ? T.chunk : 0);
    }
  }
  if (tid == 0) {
    p.next_token[b] = token;
    if (p.flags) p.flags[b] = fl;
  }
}

}  // namespace

hipError_t launch_target_stats(const VerifyArgs& a, hipStream_t s) {
  // Blocks per CU by the largest row count the call can have (the plan's actual count is read on
  // the device): 8 for up to 1023 rows, where the launch's fixed cost dominates, and 4 from 1024
  // rows on, where the steady stream is faster with fewer segment loads in flight (b128-v151936-g15
  // target_stats over 2048 rows: 193.7 us at 4, 195.2 at 6, 206.1 at 8; over 334 rows at
  // b128-v129280-g5: 29.1, 28.6 and 28.2 us).
  const long max_rows = a.dense_rows > 0 ? a.dense_rows : static_cast<long>(a.B) * (a.gamma + 1);
  const int per_cu = (max_rows >= 1024) ? kStatsBlocksPerCULarge : kStatsBlocksPerCU;
  const dim3 grid(a.persistent_wgs * per_cu);
  const bool vec4 = (a.V & 3) == 0;
  if (a.e_split) {
    if (vec4)
      launch_kernel(target_stats_kernel<true, true>, grid, dim3(kBlock), 0, s, a);
    else
      launch_kernel(target_stats_kernel<true, false>, grid, dim3(kBlock), 0, s, a);
  } else {
    if (vec4)
      launch_kernel(target_stats_kernel<false, true>, grid, dim3(kBlock), 0, s, a);
    else
      launch_kernel(target_stats_kernel<false, false>, grid, dim3(kBlock), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_accept(const VerifyArgs& a, hipStream_t s) {
  const int grid = (a.B + (kBlock / 64) - 1) / (kBlock / 64);
  launch_kernel(accept_kernel, dim3(grid), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <int KS, bool Greedy, int NT>
static hipError_t launch_resid_kind(const VerifyArgs& a, hipStream_t s) {
  // The pipelined pass copies 16-byte row chunks (V % 4 == 0) and 1-2 KB of W2t per wave
  // (128 <= r <= 256) and holds a wave's bias rows in registers: eight waves, or four for the
  // three terms of the RNN head at r = 256; other shapes take the register-load kernel.
  if constexpr (KS >= 8 && KS <= 16) {
    if ((a.V & 3) == 0) {
      const int groups = (a.B + kResGroup - 1) / kResGroup;
      const int grid = a.persistent_wgs > groups ? a.persistent_wgs : groups;
      if constexpr (NT == 1 || KS <= 8) {
        launch_kernel(residual_dma_kernel<KS, Greedy, NT>, dim3(grid), dim3(kResThreads), 0, s, a);
      } else {
        launch_kernel(residual_dma_wave4_kernel<KS, Greedy, NT>, dim3(grid), dim3(kResThreads / 2),
                      0, s, a);
      }
      return hipGetLastError();
    }
  }
  const int grid = (a.V + 4 * kTileTokens - 1) / (4 * kTileTokens);
  launch_kernel(residual_partials_kernel<KS, Greedy, NT>, dim3(grid), dim3(kBlock), 0, s,
                     a);
  return hipGetLastError();
}
template <int KS, int NT>
static hipError_t launch_resid_terms(const VerifyArgs& a, hipStream_t s) {
  return a.greedy ? launch_resid_kind<KS, true, NT>(a, s) : launch_resid_kind<KS, false, NT>(a, s);
}
// Bias rows of three bf16 terms (the RNN head) are built for r <= 256.
template <int KS>
static hipError_t launch_resid_ks(const VerifyArgs& a, hipStream_t s) {
  if (a.e_terms == 1) return launch_resid_terms<KS, 1>(a, s);
  if constexpr (KS <= 16) {
    if (a.e_terms == kRnnTerms) return launch_resid_terms<KS, kRnnTerms>(a, s);
  }
  return hipErrorInvalidValue;
}
template <int KS>
static hipError_t launch_emit_ks(const VerifyArgs& a, hipStream_t s) {
  const int slots = padded(a.ntiles > kSegTokens ? a.ntiles : kSegTokens);
  const size_t lds = static_cast<size_t>(slots) * sizeof(double);
  if (a.e_terms == 1) {
    launch_kernel(emit_sample_kernel<KS, 1>, dim3(a.B), dim3(kBlock), lds, s, a);
    return hipGetLastError();
  }
  if constexpr (KS <= 16) {
    if (a.e_terms == kRnnTerms) {
      launch_kernel(emit_sample_kernel<KS, kRnnTerms>, dim3(a.B), dim3(kBlock), lds, s, a);
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

hipError_t launch_residual_partials(const VerifyArgs& a, hipStream_t s) {
  DSPARK_DISPATCH_KS(a.r, launch_resid_ks, a, s)
}
hipError_t launch_emit_sample(const VerifyArgs& a, hipStream_t s) {
  DSPARK_DISPATCH_KS(a.r, launch_emit_ks, a, s)
}

}  // namespace dspark
