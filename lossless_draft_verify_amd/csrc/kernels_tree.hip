// PCTree tree drafting and its lossless verify for gfx950.
//
// Sources: [ZDS] zdszero.github.io spec_dspark, "后续工作" (PCTree: the single draft chain
// becomes a tree; the Markov head scores the child tokens under each parent token, picks each
// parent's candidate children with it, and the most likely paths are kept within a fixed verify
// budget, with no retraining and no extra backbone pass); [V41] blog.javazero.top
// "DeepSeek-V4.1 模型结构（6）：解码，DSpark", "Markov head" eqs. (4) and (5) (the scores),
// "投机解码：让小的先猜，大的一次验一串" (only draws of the target decide what is kept).
//
// A depth of the tree is one launch of the draft step kernel over the depth's expanded nodes
// (rows b M + m share request b's base logits U_k) followed by one tree_select launch:
//   tree_select  one 1024-thread workgroup per request. Each expanded node's row is taken by
//                1024 / rows threads: the row's log-sum-exp from the tile partials; its c best
//                children, which lie in the c tiles with the largest maxima (a token among the
//                c best can have at most c - 1 tiles ranked above its own), so only those tiles
//                are recomputed (the step's MFMA sequence, bit-identical logits) and ranked;
//                their probabilities and path probabilities. Then the depth's M most likely
//                nodes become the next depth's expanded nodes, or, after the last depth, the N
//                most likely candidates of every depth are written in rank order.
//   tree_walk    one workgroup per request (after the target pass's segment statistics): every
//                tree row's log-sum-exp, p_t of every kept node under its parent, the walk from
//                the root (children first in the draw's order), and the emitted token drawn from
//                p_t without the stop node's children.
#include "device.h"
#include "dma.h"
#include "launch.h"
#include "tiles.h"

namespace dspark {

namespace {

constexpr int kTreeThreads = 1024;
constexpr int kTreePer = 32;          // tile partials per thread, at most (checked by the host)
constexpr int kWalkThreads = 256;

// Order-preserving unsigned image of an fp32 value (larger value, larger key).
__device__ __forceinline__ uint32_t float_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
// Key of (value, index): larger value first, then the smaller index; 0 = none.
__device__ __forceinline__ uint64_t rank_key(float x, int index) {
  return (static_cast<uint64_t>(float_key(x)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(index));
}
__device__ __forceinline__ int key_index(uint64_t k) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(k));
}

template <int S>
__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t v) {
  const uint32_t lo = lane_xor<S>(static_cast<uint32_t>(v));
  const uint32_t hi = lane_xor<S>(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o;
  o = lane_xor_u64<32>(v); v = o > v ? o : v;
  o = lane_xor_u64<16>(v); v = o > v ? o : v;
  o = lane_xor_u64<8>(v);  v = o > v ? o : v;
  o = lane_xor_u64<4>(v);  v = o > v ? o : v;
  o = lane_xor_u64<2>(v);  v = o > v ? o : v;
  o = lane_xor_u64<1>(v);  v = o > v ? o : v;
  return v;
}

// Mass of a tile partial relative to the row max M, as the chain's sampler forms it.
__device__ __forceinline__ double tree_tile_mass(float m, float s, float M) {
  return (m == kNegInf) ? 0.0 : static_cast<double>(exp_term(m - M)) * static_cast<double>(s);
}

// CM: a power of two >= c, the length of each thread's sorted list of best tiles.
template <int KS, int CM>
__global__ __launch_bounds__(kTreeThreads) void tree_select_kernel(TreeSelectArgs p) {
  constexpr int r = 16 * KS;
  __shared__ __attribute__((aligned(16))) uint16_t Es[kTreeMaxRows][r];
  __shared__ unsigned long long redk[kTreeThreads / 64][kTreeMaxChildren];
  __shared__ float redf[kTreeThreads / 64];
  __shared__ double redd[kTreeThreads / 64];
  __shared__ float Lt[kTreeMaxRows][kTreeMaxChildren][kTileTokens];
  __shared__ int tile_of[kTreeMaxRows][kTreeMaxChildren];
  __shared__ double cP[kTreeMaxCand];
  __shared__ int cTok[kTreeMaxRows * kTreeMaxChildren];
  __shared__ int rank_of[kTreeMaxCand];

  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = p.rows;                       // 1, 2, 4 or 8 expanded nodes
  const int G = kTreeThreads / R;             // threads per node row
  const int WS = G / 64;                      // waves per node row
  const int sub = tid / G, stid = tid - sub * G, wsub = wave - sub * WS;
  const int row = b * R + sub;
  const int nt = p.ntiles, c = p.c;
  const size_t cb = static_cast<size_t>(b) * p.T;

  // The node's token (clamped into the vocabulary) and its embedding row, copied into LDS by
  // the row's first wave while the partials load.
  const int32_t ptok = min(max(p.prev[row], 0), p.V - 1);
  if (wsub == 0)
    copy_row_to_lds<2 * KS>(p.W1 + static_cast<size_t>(ptok) * r,
                            __builtin_amdgcn_readfirstlane(lds_addr(&Es[sub][0])), lane);
  // The row's partials, thread stid taking tiles stid + G i in batches of 8. First pass: the
  // thread's maximum and its c best tiles by key (tile max, then the smaller tile), kept sorted
  // in registers. Second pass (the partials again, now from the cache): the masses relative to
  // the row maximum, as the chain's sampler forms them.
  const float2* part = p.part + static_cast<size_t>(row) * nt;
  float m_thr = kNegInf;
  uint64_t best[CM];
#pragma unroll
  for (int j = 0; j < CM; ++j) best[j] = 0;
  constexpr int kBatch = 8;
  for (int i0 = 0; i0 < kTreePer && G * i0 < nt; i0 += kBatch) {
    // Loads at clamped indices, unconditionally, and the range applied afterwards: a guarded
    // load per element would make each one wait for the one before it.
    float tm[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) tm[i] = part[min(stid + G * (i0 + i), nt - 1)].x;
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (stid + G * (i0 + i) >= nt) tm[i] = kNegInf;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int t = stid + G * (i0 + i);
      m_thr = fmaxf(m_thr, tm[i]);
      uint64_t key = (t < nt) ? rank_key(tm[i], t) : 0ull;
#pragma unroll
      for (int j = 0; j < CM; ++j) {
        const uint64_t x = best[j];
        const bool swap = key > x;
        best[j] = swap ? key : x;
        key = swap ? x : key;
      }
    }
  }

  // Row maximum and log-sum-exp (wave sums, then the row's waves in order).
  const float mw = wave_max(m_thr);
  if (lane == 0) redf[wave] = mw;
  __syncthreads();
  float M = kNegInf;
  for (int w = 0; w < WS; ++w) M = fmaxf(M, redf[sub * WS + w]);
  double z = 0.0;
  for (int i0 = 0; i0 < kTreePer && G * i0 < nt; i0 += kBatch) {
    float2 pv[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) pv[i] = part[min(stid + G * (i0 + i), nt - 1)];
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (stid + G * (i0 + i) >= nt) pv[i] = make_float2(kNegInf, 0.0f);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) z += tree_tile_mass(pv[i].x, pv[i].y, M);
  }
  z = wave_sum(z);
  if (lane == 0) redd[wave] = z;
  __syncthreads();
  double Z = 0.0;
  for (int w = 0; w < WS; ++w) Z += redd[sub * WS + w];
  const double lse = static_cast<double>(M) + log(Z);

  // The row's c best tiles. Each wave first takes its own c best, one per round: every lane
  // offers the head of its sorted list, and the one lane whose head was taken (keys are unique)
  // shifts its list. The row's first wave then takes the c best of its waves' WS c (<= 128,
  // two a lane), the same set in the same order as c rounds over the whole row.
  for (int j = 0; j < c; ++j) {
    const uint64_t kb = wave_max_u64(best[0]);
    const bool taken = kb != 0 && best[0] == kb;
#pragma unroll
    for (int i = 0; i + 1 < CM; ++i) best[i] = taken ? best[i + 1] : best[i];
    best[CM - 1] = taken ? 0ull : best[CM - 1];
    if (lane == 0) redk[wave][j] = kb;
  }
  __syncthreads();
  if (wsub == 0) {
    const int nc = WS * c;
    const int f0 = lane, f1 = lane + 64;
    uint64_t k0 = (f0 < nc) ? redk[sub * WS + f0 / c][f0 % c] : 0ull;
    uint64_t k1 = (f1 < nc) ? redk[sub * WS + f1 / c][f1 % c] : 0ull;
    if (k1 > k0) {
      const uint64_t t = k0;
      k0 = k1;
      k1 = t;
    }
    for (int j = 0; j < c; ++j) {
      const uint64_t kb = wave_max_u64(k0);
      const bool taken = kb != 0 && k0 == kb;
      k0 = taken ? k1 : k0;
      k1 = taken ? 0ull : k1;
      if (lane == 0) tile_of[sub][j] = kb ? key_index(kb) : -1;
    }
  }

  // Recompute those tiles with the step's instruction sequence.
  if (wsub == 0) wait_copies<0>();   // the embedding row
  __syncthreads();
  const float* Urow = p.U + (static_cast<size_t>(b) * p.gamma + p.k) * p.V;
  for (int j = wsub; j < c; j += WS) {
    const int t = tile_of[sub][j];
    if (t >= 0) recompute_tile_lds<KS, 1>(&Es[sub][0], p.W2t, Urow, t * kTileTokens, p.V, &Lt[sub][j][0]);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // The row's c best tokens among those tiles' c * 32 (by logit, the smaller id on a tie).
  if (wsub == 0) {
    uint64_t keys[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = lane + 64 * i;
      const int j = f >> 5, off = f & 31;
      uint64_t key = 0;
      if (j < c) {
        const int t = tile_of[sub][j];
        const int tok = t * kTileTokens + off;
        if (t >= 0 && tok < p.V) key = rank_key(Lt[sub][j][off], tok);
      }
      keys[i] = key;
    }
    // sort the lane's four keys (descending), then take heads as above
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int q = 0; q < 3 - i; ++q) {
        const uint64_t hi = keys[q] > keys[q + 1] ? keys[q] : keys[q + 1];
        const uint64_t lo = keys[q] > keys[q + 1] ? keys[q + 1] : keys[q];
        keys[q] = hi;
        keys[q + 1] = lo;
      }
    uint64_t mine = 0;
    for (int i = 0; i < c; ++i) {
      const uint64_t kb = wave_max_u64(keys[0]);
      const bool taken = kb != 0 && keys[0] == kb;
      keys[0] = taken ? keys[1] : keys[0];
      keys[1] = taken ? keys[2] : keys[1];
      keys[2] = taken ? keys[3] : keys[2];
      keys[3] = taken ? 0ull : keys[3];
      if (lane == i) mine = kb;
    }
    if (lane < c) {
      const int tok = mine ? key_index(mine) : 0;
      const double q = mine ? exp(static_cast<double>(key_float(static_cast<uint32_t>(mine >> 32))) - lse)
                            : 0.0;
      const double Pp = p.prevP ? p.prevP[row] : 1.0;
      const int gi = p.cand_base + sub * c + lane;
      p.cand.tok[cb + gi] = tok;
      p.cand.parent[cb + gi] = p.prevCand ? p.prevCand[row] : -1;
      p.cand.P[cb + gi] = Pp * q;
      p.cand.q[cb + gi] = q;
      cP[sub * c + lane] = Pp * q;
      cTok[sub * c + lane] = tok;
    }
  }
  __syncthreads();

  if (!p.last) {
    // The depth's M most likely nodes, key (-P, candidate number): the next expanded nodes.
    const int n = R * c;   // <= 64
    if (wave == 0) {
      const double Pl = (lane < n) ? cP[lane] : -1.0;
      int rank = 0;
      for (int j = 0; j < n; ++j) {
        const double Pj = cP[j];
        rank += (Pj > Pl || (Pj == Pl && j < lane)) ? 1 : 0;
      }
      if (lane < n && rank < p.M) {
        const size_t o = static_cast<size_t>(b) * p.M + rank;
        p.front_tok[o] = cTok[lane];
        p.front_P[o] = Pl;
        p.front_cand[o] = p.cand_base + lane;
      }
    }
    return;
  }
  // Last depth: the N most likely candidates of every depth, key (-P, candidate number), in
  // rank order. This workgroup wrote the last depth's candidates above (visible after the
  // barrier); earlier launches wrote the others.
  const int T = p.T;
  for (int i = tid; i < T; i += kTreeThreads) cP[i] = p.cand.P[cb + i];
  __syncthreads();
  for (int i = tid; i < T; i += kTreeThreads) {
    const double Pi = cP[i];
    int rank = 0;
    for (int j = 0; j < T; ++j) {
      const double Pj = cP[j];
      rank += (Pj > Pi || (Pj == Pi && j < i)) ? 1 : 0;
    }
    rank_of[i] = rank;
  }
  __syncthreads();
  for (int i = tid; i < T; i += kTreeThreads) {
    const int n = rank_of[i];
    if (n >= p.N) continue;
    const size_t o = static_cast<size_t>(b) * p.N + n;
    const int par = p.cand.parent[cb + i];
    p.node_token[o] = p.cand.tok[cb + i];
    p.node_depth[o] = (i < c) ? 1 : 2 + (i - c) / (p.M * c);
    p.node_parent[o] = (par < 0) ? -1 : rank_of[par];
    p.node_q[o] = p.cand.q[cb + i];
    p.node_path[o] = cP[i];
  }
}

// The tree walk and the emitted token of one request. Phase 1 gathers the tree and every kept
// node's target logit under its parent's row; phase 2 forms every row's log-sum-exp from its
// segment statistics (a wave a row); phase 3 walks from the root on one thread (ALU only);
// phase 4 draws the emitted token from the stop row without the stop node's children, by
// segment (wave 0) and then by token within the segment (the segment's terms staged in LDS).
__global__ __launch_bounds__(kWalkThreads) void tree_walk_kernel(TreeWalkArgs p) {
  extern __shared__ double stage[];   // padded: segment masses, then one segment's terms
  __shared__ int tok[kTreeMaxNodes], par[kTreeMaxNodes];
  __shared__ float tval[kTreeMaxNodes];
  __shared__ double lse[kTreeMaxNodes + 1];     // each row's sum z, then its lse
  __shared__ float lse_m[kTreeMaxNodes + 1];    // each row's max M
  __shared__ double ptn[kTreeMaxNodes];
  __shared__ float us[kMaxGamma + 1];
  __shared__ double ssum[kWalkThreads];
  __shared__ int stop_s, acc_s, nexc_s;
  __shared__ uint32_t fl_s;
  __shared__ int exc[kTreeMaxChildren];
  __shared__ float exc_t[kTreeMaxChildren];
  __shared__ Located loc;
  __shared__ float seg_m, row_m;

  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = p.N, V = p.V, nseg = p.nseg;
  const size_t base = static_cast<size_t>(b) * (N + 1);

  // 1. The tree (out-of-range tokens and parents clamped) and each node's target logit.
  for (int n = tid; n < N; n += kWalkThreads) {
    const int t = min(max(p.node_token[static_cast<size_t>(b) * N + n], 0), V - 1);
    const int q = min(max(p.node_parent[static_cast<size_t>(b) * N + n], -1), N - 1);
    tok[n] = t;
    par[n] = q;
    tval[n] = p.target[(base + q + 1) * V + t];
  }
  for (int k = tid; k <= p.gamma; k += kWalkThreads)
    us[k] = p.uniforms[(static_cast<size_t>(b) * (p.gamma + 1) + k) * 3 + 2];
  // 2. Log-sum-exp of rows 0 .. N (lane l holds segments 2l, 2l + 1; nseg <= 128): a wave
  //    takes rows wave, wave + 4, ..., the loads of up to 8 of its rows going out together.
  constexpr int kRowsBatch = 8;
  for (int r0 = wave; r0 <= N; r0 += kRowsBatch * (kWalkThreads / 64)) {
    float ms[kRowsBatch][2];
    double sg[kRowsBatch][2];
#pragma unroll
    for (int j = 0; j < kRowsBatch; ++j) {
      const int rr = min(r0 + j * (kWalkThreads / 64), N);
      const size_t o = (base + rr) * nseg;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int sgi = min(2 * lane + i, nseg - 1);
        ms[j][i] = p.seg_max[o + sgi];
        sg[j][i] = p.seg_sum[o + sgi];
      }
    }
#pragma unroll
    for (int j = 0; j < kRowsBatch; ++j) {
      const int rr = r0 + j * (kWalkThreads / 64);
      if (rr > N) break;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (2 * lane + i >= nseg) {
          ms[j][i] = kNegInf;
          sg[j][i] = 0.0;
        }
      const float Mr = wave_max(fmaxf(ms[j][0], ms[j][1]));
      const double zr =
          wave_sum(partial_mass(ms[j][0], sg[j][0], Mr) + partial_mass(ms[j][1], sg[j][1], Mr));
      if (lane == 0) {
        lse[rr] = zr;
        lse_m[rr] = Mr;
      }
    }
  }
  __syncthreads();
  // The rows' log-sum-exps M + log z, one row a thread (the fp64 log in one pass).
  for (int rr = tid; rr <= N; rr += kWalkThreads) lse[rr] = static_cast<double>(lse_m[rr]) + log(lse[rr]);
  __syncthreads();
  for (int n = tid; n < N; n += kWalkThreads)
    ptn[n] = exp(static_cast<double>(tval[n]) - lse[par[n] + 1]);
  __syncthreads();
  // 3. The walk on wave 0: at a node, its children in rank order take the first part of the
  //    draw's order; the first child whose cumulative mass passes u is accepted. A depth is a
  //    ballot and a scan over the nodes (64 a batch), the cumulative mass carried across batches.
  if (wave == 0) {
    int cur = -1, acc = 0;
    uint32_t fl = 0;
    for (;;) {
      if (!isfinite(lse[cur + 1])) fl |= 1u;
      const double u = static_cast<double>(us[acc]);
      double before = 0.0;
      int chosen = -1;
      for (int i0 = 0; i0 < N; i0 += 64) {
        const int n = i0 + lane;
        const bool child = n < N && par[n] == cur;
        const double inc = before + wave_inclusive_scan(child ? ptn[n] : 0.0, lane);
        const unsigned long long hit = __ballot(child && inc > u);
        if (hit) {
          chosen = i0 + __ffsll(static_cast<long long>(hit)) - 1;
          break;
        }
        before = read_lane(inc, 63);
      }
      if (chosen < 0 || acc >= p.gamma) break;
      if (lane == 0) p.path[static_cast<size_t>(b) * p.gamma + acc] = tok[chosen];
      ++acc;
      cur = chosen;
    }
    if (lane == 0)
      for (int k = acc; k < p.gamma; ++k) p.path[static_cast<size_t>(b) * p.gamma + k] = -1;
    // the stop node's children (at most c), in rank order: excluded from the emission
    int ne = 0;
    for (int i0 = 0; i0 < N; i0 += 64) {
      const int n = i0 + lane;
      const bool child = n < N && par[n] == cur;
      const unsigned long long m = __ballot(child);
      const int pos = ne + __popcll(m & ((1ull << lane) - 1ull));
      if (child && pos < kTreeMaxChildren) {
        exc[pos] = tok[n];
        exc_t[pos] = tval[n];
      }
      ne += __popcll(m);
    }
    if (lane == 0) {
      stop_s = cur;
      acc_s = acc;
      fl_s = fl;
      nexc_s = min(ne, kTreeMaxChildren);
    }
  }
  __syncthreads();
  const int stop = stop_s, acc = acc_s, ne = nexc_s;
  const double u = static_cast<double>(us[acc]);
  const float* trow = p.target + (base + stop + 1) * V;
  // 4a. Wave 0 picks the segment of the draw over the complement of the children: the
  //     children's mass (in the units of the segment masses) comes first, so the complement's
  //     target is u Z minus it.
  const size_t so = (base + stop + 1) * nseg;
  if (tid < 64) {
    float ms[2];
    double sg[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int sgi = 2 * lane + i;
      ms[i] = (sgi < nseg) ? p.seg_max[so + sgi] : kNegInf;
      sg[i] = (sgi < nseg) ? p.seg_sum[so + sgi] : 0.0;
    }
    const float Mr = wave_max(fmaxf(ms[0], ms[1]));
    double full = 0.0, kids = 0.0, S2 = 0.0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int sgi = 2 * lane + i;
      const double f = (ms[i] == kNegInf) ? 0.0 : exp(static_cast<double>(ms[i]) - static_cast<double>(Mr));
      double kin = 0.0;
      for (int e = 0; e < ne; ++e)
        if (exc[e] / kSegTokens == sgi) kin += f * static_cast<double>(exp_term(exc_t[e] - ms[i]));
      const double mfull = partial_mass(ms[i], sg[i], Mr);
      const double mc = fmax(mfull - kin, 0.0);
      full += mfull;
      kids += kin;
      if (sgi < nseg) stage[sgi] = mc;
      S2 += (sgi < nseg) ? mc : 0.0;
    }
    ssum[lane] = S2;
    const double Zr = wave_sum(full), Kr = wave_sum(kids);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's LDS writes, read back by other lanes
    __builtin_amdgcn_wave_barrier();
    const double tgt = fmax(u * Zr - Kr, 0.0);
    const Located Sg = wave_locate<64>(
        ssum, nseg, 2, [tgt](double) { return tgt; }, [&](int ch) { return stage[ch]; });
    if (tid == 0) {
      loc = Sg;
      row_m = Mr;
    }
    if (Sg.chunk >= 0 && lane == (Sg.chunk >> 1)) seg_m = ms[Sg.chunk & 1];
  }
  __syncthreads();
  const Located S = loc;
  int token = 0;
  if (S.chunk >= 0) {
    // 4b. The segment's terms exp(t - segment max), the children's set to 0: thread t takes
    //     tokens 16 t .. 16 t + 15.
    const int t0 = S.chunk * kSegTokens;
    const int n = min(kSegTokens, V - t0);
    const float sm = seg_m;
    const bool vec4 = (V & 3) == 0;
    double Sum = 0.0;
    float x16[16];
    load16(trow, t0 + 16 * tid, V, vec4, x16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = 16 * tid + 4 * i + e;
        bool skip = ch >= n;
        for (int x = 0; x < ne; ++x) skip = skip || (exc[x] == t0 + ch);
        const double ms = skip ? 0.0 : static_cast<double>(exp_term(x16[4 * i + e] - sm));
        stage[padded(ch)] = ms;
        Sum += ms;
      }
    }
    ssum[tid] = Sum;
    __syncthreads();
    if (tid < 64) {
      const double f = exp(static_cast<double>(sm) - static_cast<double>(row_m));
      const double tgt = S.take_last ? __builtin_inf() : (S.target - S.before) / f;
      const Located T = wave_locate<kWalkThreads>(
          ssum, n, kSegTokens / kWalkThreads, [tgt](double) { return tgt; },
          [&](int ch) { return stage[padded(ch)]; });
      token = t0 + (T.chunk >= 0 ? T.chunk : 0);
    }
  }
  if (tid == 0) {
    p.accept_len[b] = acc;
    p.next_token[b] = token;
    if (p.flags) p.flags[b] = fl_s;
  }
}

}  // namespace

template <int KS>
static hipError_t launch_tree_select_ks(const TreeSelectArgs& a, hipStream_t s) {
  if (a.c <= 1) {
    launch_kernel(tree_select_kernel<KS, 1>, dim3(a.B), dim3(kTreeThreads), 0, s, a);
  } else if (a.c <= 2) {
    launch_kernel(tree_select_kernel<KS, 2>, dim3(a.B), dim3(kTreeThreads), 0, s, a);
  } else if (a.c <= 4) {
    launch_kernel(tree_select_kernel<KS, 4>, dim3(a.B), dim3(kTreeThreads), 0, s, a);
  } else {
    launch_kernel(tree_select_kernel<KS, 8>, dim3(a.B), dim3(kTreeThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_tree_select(const TreeSelectArgs& a, int r, hipStream_t s) {
  switch (r) {
    case 16: return launch_tree_select_ks<1>(a, s);
    case 32: return launch_tree_select_ks<2>(a, s);
    case 64: return launch_tree_select_ks<4>(a, s);
    case 128: return launch_tree_select_ks<8>(a, s);
    case 256: return launch_tree_select_ks<16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_tree_walk(const TreeWalkArgs& a, hipStream_t s) {
  const size_t lds = static_cast<size_t>(padded(kSegTokens)) * sizeof(double);
  launch_kernel(tree_walk_kernel, dim3(a.B), dim3(kWalkThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace dspark
