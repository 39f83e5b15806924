// Survival-ordered verify planner, as a device routine for one workgroup: the standalone planner
// kernel runs it on 1024 threads, and the pipelined draft step can run it on one of its 512-thread
// workgroups (LDS borrowed from the step's copy stages) beside the last position's step.
//
// Sources: [V41] blog.javazero.top "DeepSeek-V4.1 模型结构（6）：解码，DSpark", "调度器"
// ("目标函数": B, tau, Theta; "贪心就能解": sort the survivals, admit one by one, stop once
// Theta stops rising; the asynchronous production variant in the last paragraph before "训练");
// [ZDS] zdszero.github.io spec_dspark, "调度" and "在 SGLang 里" (lengths in [1, gamma+1], a
// flat SPS table degrades to full verify, confidences relayed through a ring, lag 2);
// [CSDN] deepseek.csdn.net DSpark walk-through, 5.3 and 8.
//
// Steps: a_{b,j} = prod c (sequential fp64 per request) -> merge sort of (a desc, b, j) ->
// prefix sums tau_i -> Theta_i = tau_i * sps[B + i] -> admission count by mode -> l_b from
// the rank of each candidate -> row_offsets. LAGGED_TOPK first runs the full-path search on
// the ring slot holding the confidences of two rounds back, then overwrites that slot.
//
// Every result is independent of the block size: the sort places each element by exact
// comparisons, the admission searches and offsets are exact, and the prefix sums always use
// the partition of a 1024-thread block (below).
#pragma once

#include <limits.h>

#include "device.h"
#include "launch.h"

namespace dspark {

namespace plan {

enum { kFullVerify = 0, kEarlyStop = 1, kFullPath = 2, kLaggedTopK = 3 };

// The prefix sums split the N survivals into this many contiguous ranges whatever the block
// size (a thread of a smaller block takes several), so tau is the same sum in every launch.
constexpr int kScanRanges = 1024;

template <int MaxN>
struct Smem {
  double a[MaxN];   // survivals, then prefix sums tau
  int idx[MaxN];    // candidate index b * gamma + j, sorted alongside a
  double red_d[kScanRanges / 64];
  int red_i[kScanRanges / 64];
  int n_admit;
};

// "Before" order of candidates: survival descending, then candidate index ascending.
__device__ __forceinline__ bool before(double ai, int ii, double aj, int ij) {
  return (ai > aj) || (ai == aj && ii < ij);
}

// One compare-exchange of a bitonic stage with partner lane l ^ S (within the wave); `up`
// selects the direction of the bitonic sequence the lane belongs to.
template <int S>
__device__ __forceinline__ void exchange(double& a, int& ix, int l, bool up) {
  const double pa = lane_xor<S>(a);
  const int pi = static_cast<int>(lane_xor<S>(static_cast<uint32_t>(ix)));
  const bool lower = (l & S) == 0;
  const bool other_first = before(pa, pi, a, ix);
  if ((lower == up) ? other_first : !other_first) {
    a = pa;
    ix = pi;
  }
}

// The global inputs of candidate i = tid, issued together at entry so that their latencies
// overlap each other and the sort (other candidates are read where they are used): its
// confidence, its lag-slot value, and sps[B + i], sps[B + i + 1] for the admission tests.
struct Inputs {
  float c, lag;
  double s0, s1;
};

__device__ __forceinline__ void load_inputs(Inputs& in, const PlanArgs& p, bool lagged) {
  const int i = threadIdx.x, N = p.B * p.gamma;
  const float* lag = p.ring + static_cast<size_t>(p.round_index % 2) * N;
  in.c = (p.conf != nullptr && i < N) ? p.conf[i] : 0.0f;
  in.lag = (lagged && i < N) ? lag[i] : 0.0f;
  in.s0 = (i <= N) ? p.sps[p.B + i] : 0.0;
  in.s1 = (i < N) ? p.sps[p.B + i + 1] : 0.0;
}

// Fill survivals from the confidences src (c0 = src[tid], already loaded), sort, and turn a[]
// into tau_i (a[i] = tau_{i+1}). Results in sm.
//
// The sort runs over Np = N rounded up to a power of two (at least 64): entries N .. Np-1 hold
// -inf with the highest candidate indices, so they sort last and every run below is full. Every
// 64-element chunk is sorted inside one wave (bitonic, no LDS traffic), then merge levels double
// the runs. A merge level places every element directly: its position is its rank in its own run
// plus the number of elements of the partner run that come before it. The left run holds the
// lower candidate indices, so for x in the left run a right element comes first iff it is > x,
// and for x in the right run a left element comes first iff it is >= x, that is > the next
// double below x: one threshold per element, one comparison per probe of a fixed-step base-4
// search. A padding element comes after every real one and after the padding of lower index.
template <int NT, int MaxN>
__device__ void sorted_path(Smem<MaxN>& sm, const float* __restrict__ src, float c0, int B,
                            int gamma) {
  constexpr int kPer = MaxN / NT;   // candidates per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = B * gamma;
  const int Np = (N <= kWave) ? kWave : (1 << (32 - __clz(N - 1)));
  for (int i = tid; i < Np; i += NT) {
    sm.a[i] = (i < N) ? static_cast<double>(i == tid ? c0 : src[i]) : -__builtin_inf();
    sm.idx[i] = i;
  }
  __syncthreads();
  // a_{b,j}: running product along each request's path, in place (one thread per request).
  for (int b = tid; b < B; b += NT) {
    double prod = 1.0;
    for (int j = 0; j < gamma; ++j) {
      prod *= sm.a[b * gamma + j];
      sm.a[b * gamma + j] = prod;
    }
  }
  __syncthreads();
  // Runs of 64: each wave sorts 64-element chunks in registers with a bitonic network whose
  // exchanges go through DPP / lane swaps.
  for (int c = wave; c * kWave < Np; c += NT / kWave) {
    const int i = c * kWave + lane;
    double a = sm.a[i];
    int ix = sm.idx[i];
#pragma unroll
    for (int size = 2; size <= kWave; size <<= 1) {
      const bool up = (lane & size) == 0 || size == kWave;
      if (size >= 64) exchange<32>(a, ix, lane, up);
      if (size >= 32) exchange<16>(a, ix, lane, up);
      if (size >= 16) exchange<8>(a, ix, lane, up);
      if (size >= 8) exchange<4>(a, ix, lane, up);
      if (size >= 4) exchange<2>(a, ix, lane, up);
      exchange<1>(a, ix, lane, up);
    }
    sm.a[i] = a;
    sm.idx[i] = ix;
  }
  __syncthreads();
  for (int run = kWave; run < Np; run *= 2) {
    double ka[kPer];
    int ki[kPer], pos[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int p = tid + q * NT;
      pos[q] = -1;
      if (p < Np) {
        ka[q] = sm.a[p];
        ki[q] = sm.idx[p];
        const int base = p & ~(2 * run - 1);
        const bool left = p - base < run;
        const int own = left ? p - base : p - base - run;
        const int o0 = left ? base + run : base;
        int cnt;
        if (ki[q] >= N) {
          const int real = min(max(N - o0, 0), run);
          cnt = left ? real : run;
        } else {
          const double thr = left ? ka[q] : nextafter(ka[q], -__builtin_inf());
          const double* r = sm.a + o0;
          // Base-4 lifting: three independent probes a step (one binary step first when the run
          // length is an odd power of two), then the last position.
          int lo = 0, len = run;
          if (__builtin_ctz(run) & 1) {
            lo += (r[len / 2 - 1] > thr) ? len / 2 : 0;
            len /= 2;
          }
          for (; len >= 4; len >>= 2) {
            const int qq = len >> 2;
            const int n1 = (r[lo + qq - 1] > thr) ? 1 : 0;
            const int n2 = (r[lo + 2 * qq - 1] > thr) ? 1 : 0;
            const int n3 = (r[lo + 3 * qq - 1] > thr) ? 1 : 0;
            lo += qq * (n1 + n2 + n3);
          }
          lo += (r[lo] > thr) ? 1 : 0;
          cnt = lo;
        }
        pos[q] = base + own + cnt;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      if (pos[q] >= 0) {
        sm.a[pos[q]] = ka[q];
        sm.idx[pos[q]] = ki[q];
      }
    }
    __syncthreads();
  }
  // Inclusive prefix sums of the sorted survivals, plus B: a[i] <- tau_{i+1}. Range g of the
  // kScanRanges ranges (ceil(N / kScanRanges) survivals each) is summed in order by thread
  // g % NT; the range sums are scanned 64 at a time by a wave and the 16 wave totals are added
  // in order, as one range per thread of a 1024-thread block would do.
  constexpr int kRangesPerThread = kScanRanges / NT;
  static_assert(kRangesPerThread * NT == kScanRanges, "block size divides the scan ranges");
  const int per = (N + kScanRanges - 1) / kScanRanges;
  double exc[kRangesPerThread];
#pragma unroll
  for (int v = 0; v < kRangesPerThread; ++v) {
    const int g = tid + v * NT;
    const int i0 = min(N, g * per), i1 = min(N, i0 + per);
    double s = 0.0;
    for (int i = i0; i < i1; ++i) s += sm.a[i];
    const double inc = wave_inclusive_scan(s, lane);
    exc[v] = wave_exclusive_of(inc, lane);
    if (lane == 63) sm.red_d[(g >> 6)] = inc;
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < kRangesPerThread; ++v) {
    const int g = tid + v * NT, gw = g >> 6;
    double before_sum = 0.0;
#pragma unroll
    for (int i = 0; i < kScanRanges / 64; ++i)
      if (i < gw) before_sum += sm.red_d[i];
    const int i0 = min(N, g * per), i1 = min(N, i0 + per);
    double run = static_cast<double>(B) + (before_sum + exc[v]);
    for (int i = i0; i < i1; ++i) {
      run += sm.a[i];
      sm.a[i] = run;
    }
  }
  __syncthreads();
}

template <int MaxN>
__device__ __forceinline__ double tau_at(const Smem<MaxN>& sm, int i, int B) {
  return i == 0 ? static_cast<double>(B) : sm.a[i - 1];
}

// Admission count along the current path for EARLY_STOP or FULL_PATH.
template <int NT, int MaxN>
__device__ int admit_count(Smem<MaxN>& sm, const Inputs& in, const double* __restrict__ sps,
                           int B, int N, int mode) {
  const int tid = threadIdx.x;
  if (mode == kEarlyStop) {
    int first = N;
    for (int i = tid; i < N; i += NT) {
      const double t0 = tau_at(sm, i, B) * (i == tid ? in.s0 : sps[B + i]);
      const double t1 = tau_at(sm, i + 1, B) * (i == tid ? in.s1 : sps[B + i + 1]);
      if (!(t1 > t0)) first = min(first, i);
    }
    return block_min_int<NT>(first, sm.red_i);
  }
  // FULL_PATH: first maximiser of Theta_i, i = 0..N.
  double best = -__builtin_inf();
  int best_i = INT_MAX;
  for (int i = tid; i <= N; i += NT) {
    const double th = tau_at(sm, i, B) * (i == tid ? in.s0 : sps[B + i]);
    if (th > best) {
      best = th;
      best_i = i;
    }
  }
  // block max of Theta, then the smallest index attaining it
  double w = wave_max(best);
  __syncthreads();
  if ((tid & 63) == 0) sm.red_d[tid >> 6] = w;
  __syncthreads();
  double gmax = sm.red_d[0];
  for (int k = 1; k < NT / 64; ++k) gmax = fmax(gmax, sm.red_d[k]);
  return block_min_int<NT>(best == gmax ? best_i : INT_MAX, sm.red_i);
}

// The whole planner on one workgroup of NT threads (B * gamma <= MaxN).
template <int NT, int MaxN>
__device__ void run(const PlanArgs& p, Smem<MaxN>& sm) {
  const int tid = threadIdx.x;
  const int B = p.B, gamma = p.gamma, N = B * gamma;

  int n_admit = N;
  double capacity = -1.0;
  const bool lagged = (p.mode == kLaggedTopK) && (p.round_index >= 2);
  Inputs in;
  load_inputs(in, p, lagged);
  if (lagged) {
    sorted_path<NT>(sm, p.ring + static_cast<size_t>(p.round_index % 2) * N, in.lag, B, gamma);
    const int k_lag = admit_count<NT>(sm, in, p.sps, B, N, kFullPath);
    capacity = static_cast<double>(B) + static_cast<double>(k_lag);
    n_admit = min(k_lag, N);
    __syncthreads();
  }
  const bool have_conf = p.conf != nullptr;
  if (have_conf) {
    sorted_path<NT>(sm, p.conf, in.c, B, gamma);
    if (p.mode == kEarlyStop || (p.mode == kLaggedTopK && !lagged)) {
      n_admit = admit_count<NT>(sm, in, p.sps, B, N, kEarlyStop);
    } else if (p.mode == kFullPath) {
      n_admit = admit_count<NT>(sm, in, p.sps, B, N, kFullPath);
    } else if (p.mode == kFullVerify) {
      n_admit = N;
    }
  }
  if (tid == 0) {
    const double tau = have_conf ? tau_at(sm, n_admit, B) : __builtin_nan("");
    if (p.stats) {
      p.stats[0] = static_cast<double>(B + n_admit);
      p.stats[1] = tau;
      p.stats[2] = tau * p.sps[B + n_admit];
      p.stats[3] = lagged ? capacity : static_cast<double>(B + n_admit);
    }
    sm.n_admit = n_admit;
  }
  __syncthreads();
  if (p.mode == kLaggedTopK) {
    float* slot = p.ring + static_cast<size_t>(p.round_index % 2) * N;
    for (int i = tid; i < N; i += NT) slot[i] = (i == tid) ? in.c : p.conf[i];
  }
  // Ranks: candidate (b, j) is admitted iff its sorted position is < n_admit. Reuse a[] as an
  // int array of positions per candidate.
  int* rank = reinterpret_cast<int*>(sm.a);
  if (have_conf) {
    for (int i = tid; i < N; i += NT) rank[sm.idx[i]] = i;
  } else {
    for (int i = tid; i < N; i += NT) rank[i] = 0;
  }
  __syncthreads();
  // l_b and row offsets (exclusive scan of 1 + l_b over contiguous request ranges).
  const int per = (B + NT - 1) / NT;
  const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
  int cnt = 0;
  for (int b = b0; b < b1; ++b) {
    int l = 0;
    for (int j = 0; j < gamma; ++j) l += (rank[b * gamma + j] < n_admit) ? 1 : 0;
    p.draft_len[b] = l;
    cnt += 1 + l;
  }
  int total;
  int off = block_exclusive_scan_int<NT>(cnt, sm.red_i, &total);
  for (int b = b0; b < b1; ++b) {
    p.row_offsets[b] = off;
    int l = 0;
    for (int j = 0; j < gamma; ++j) l += (rank[b * gamma + j] < n_admit) ? 1 : 0;
    off += 1 + l;
  }
  if (tid == 0) p.row_offsets[B] = total;
}

}  // namespace plan

}  // namespace dspark
