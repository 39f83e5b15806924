// Device building blocks for the gfx950 DSpark kernels: MFMA tiles, exact-order reductions and
// the fp32 exponential used for every softmax term.
//
// Determinism: every reduction below combines values in a fixed order, and the HIP sources are
// compiled with -ffp-contract=off, so the same inputs give the same bits in every kernel that
// calls these helpers (a sampler can recompute a term exactly as the streaming pass made it).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(uint16_t)))) uint16_t u16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kWave = 64;
constexpr int kBlock = 256;          // threads per workgroup for the streaming kernels
constexpr int kTileTokens = 32;      // tokens per MFMA tile = tokens per draft partial
constexpr int kSegTokens = 4096;     // tokens per target-row segment
constexpr int kMaxGamma = 255;       // draft positions per request (accept scan LDS)
constexpr int kMaxVocab = 1 << 19;   // a sampler stages one row's tile partials in LDS (8 B each)
constexpr float kNegInf = -__builtin_inff();

// A token id read from an input, clamped into [0, V): every address formed from a token id stays
// inside its table whatever the caller passed (the results of a round with such an id are not
// meaningful, but no access leaves the tensors).
__device__ __forceinline__ int32_t clamp_token(int32_t x, int V) { return min(max(x, 0), V - 1); }

// One 32x32x16 bf16 MFMA step (fp32 accumulate). Lane l holds A[m = l % 32][k = 8 (l / 32) + i]
// and B[k = 8 (l / 32) + i][n = l % 32], i = 0..7; the result lane l, slot j holds
// C[m = 8 (j / 4) + 4 (l / 32) + j % 4][n = l % 32]. In the kernels m indexes tokens and n
// indexes requests: out[token][request] = sum_i W2t[token][i] * E[request][i].
__device__ __forceinline__ f32x16_t mfma_32x32x16(u16x8_t a, u16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Token offset (within a 32-token tile) of accumulator slot j in a lane of half `half`.
__device__ __forceinline__ int tile_token(int j, int half) {
  return 8 * (j >> 2) + 4 * half + (j & 3);
}

__device__ __forceinline__ u16x8_t load_u16x8(const uint16_t* p) {
  return *reinterpret_cast<const u16x8_t*>(p);
}

__device__ __forceinline__ u16x8_t zero_u16x8() {
  u16x8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
  return z;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// exp(x) for x <= 0 in fp32, as exp2(x * log2 e) on the hardware exp2 (about 1 ulp). x is a
// logit minus its tile maximum, so the terms that carry the probability mass have small |x| and
// a small rounding error in the product. exp2(-inf) = 0; NaN propagates.
__device__ __forceinline__ float exp_term(float x) {
  return __builtin_amdgcn_exp2f(x * 1.44269504088896340736f);
}

// A probability exp(x - lse) in fp32 from an fp32 logit x and c = lse * log2(e) (fp64, formed
// once per row). The exponent a = x log2(e) - c is taken in fp64 and split into its nearest
// integer n and a remainder f in [-1/2, 1/2] (exact in fp64); 2^f comes from the hardware exp2
// on fp32(f) and 2^n is applied exactly. Rounding f to fp32 moves the result by at most
// 2^-25 ln 2 relative, so the error is that of the hardware exp2 on [-1/2, 1/2] plus 2e-8,
// whatever the size of a (no fp32 rounding of a itself). Below 2^-1000 (and for x = -inf or a
// NaN exponent) the result is 0; it underflows to 0 below 2^-149.
constexpr double kLog2e64 = 1.4426950408889634073599;
__device__ __forceinline__ float prob_f32(float x, double c) {
  double a = __builtin_fma(static_cast<double>(x), kLog2e64, -c);
  a = (a > -1000.0) ? a : -1000.0;
  const double n = __builtin_rint(a);
  const float f = static_cast<float>(a - n);
  return __builtin_amdgcn_ldexpf(__builtin_amdgcn_exp2f(f), static_cast<int>(n));
}

// Workgroup barrier for an LDS hand-off that leaves global loads in flight: __syncthreads()
// carries a workgroup fence, which waits for every outstanding global load before s_barrier
// and would serialise a software prefetch issued just before it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Value held by lane l ^ S (S = 1, 2, 4, 8, 16, 32) without going through LDS: DPP quad
// permutes for 1 and 2, DPP row shifts for 4 and 8, and the gfx950 row-pair / half-wave swaps
// for 16 and 32.
template <int S>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
  const int lane = threadIdx.x & 63;
  if constexpr (S == 1) {
    return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  } else if constexpr (S == 2) {
    return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  } else if constexpr (S == 4 || S == 8) {
    const uint32_t up = __builtin_amdgcn_mov_dpp(x, 0x100 + S, 0xF, 0xF, false);   // row_shl:S
    const uint32_t dn = __builtin_amdgcn_mov_dpp(x, 0x110 + S, 0xF, 0xF, false);   // row_shr:S
    return (lane & S) ? dn : up;
  } else if constexpr (S == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    static_assert(S == 32, "lane_xor: S in 1..32");
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}
template <int S>
__device__ __forceinline__ double lane_xor(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t lo = lane_xor<S>(static_cast<uint32_t>(u));
  const uint32_t hi = lane_xor<S>(static_cast<uint32_t>(u >> 32));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Lane l - S of the same 16-lane row, 0 for the first S lanes of each row (DPP row_shr with
// zero fill).
template <int S>
__device__ __forceinline__ uint32_t row_shr_zero(uint32_t x) {
  return __builtin_amdgcn_update_dpp(0u, x, 0x110 + S, 0xF, 0xF, true);
}
template <int S>
__device__ __forceinline__ double row_shr_zero(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t lo = row_shr_zero<S>(static_cast<uint32_t>(u));
  const uint32_t hi = row_shr_zero<S>(static_cast<uint32_t>(u >> 32));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}
// Value of lane l (uniform l) in every lane.
__device__ __forceinline__ double read_lane(double x, int l) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(u), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(u >> 32), l);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}
__device__ __forceinline__ int read_lane(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

// ---- wave (64-lane) reductions: butterfly 32, 16, ..., 1 through lane_xor (no LDS traffic);
// every lane ends with the same value (the pairwise sums only swap operands between partners).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __uint_as_float(lane_xor<32>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(lane_xor<16>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(lane_xor<8>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(lane_xor<4>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(lane_xor<2>(__float_as_uint(v))));
  return fmaxf(v, __uint_as_float(lane_xor<1>(__float_as_uint(v))));
}
__device__ __forceinline__ double wave_max(double v) {
  v = fmax(v, lane_xor<32>(v));
  v = fmax(v, lane_xor<16>(v));
  v = fmax(v, lane_xor<8>(v));
  v = fmax(v, lane_xor<4>(v));
  v = fmax(v, lane_xor<2>(v));
  return fmax(v, lane_xor<1>(v));
}
__device__ __forceinline__ double wave_sum(double v) {
  v += lane_xor<32>(v);
  v += lane_xor<16>(v);
  v += lane_xor<8>(v);
  v += lane_xor<4>(v);
  v += lane_xor<2>(v);
  return v + lane_xor<1>(v);
}
__device__ __forceinline__ int wave_max_int(int v) {
  v = max(v, static_cast<int>(lane_xor<32>(static_cast<uint32_t>(v))));
  v = max(v, static_cast<int>(lane_xor<16>(static_cast<uint32_t>(v))));
  v = max(v, static_cast<int>(lane_xor<8>(static_cast<uint32_t>(v))));
  v = max(v, static_cast<int>(lane_xor<4>(static_cast<uint32_t>(v))));
  v = max(v, static_cast<int>(lane_xor<2>(static_cast<uint32_t>(v))));
  return max(v, static_cast<int>(lane_xor<1>(static_cast<uint32_t>(v))));
}
__device__ __forceinline__ int wave_min_int(int v) {
  v = min(v, static_cast<int>(lane_xor<32>(static_cast<uint32_t>(v))));
  v = min(v, static_cast<int>(lane_xor<16>(static_cast<uint32_t>(v))));
  v = min(v, static_cast<int>(lane_xor<8>(static_cast<uint32_t>(v))));
  v = min(v, static_cast<int>(lane_xor<4>(static_cast<uint32_t>(v))));
  v = min(v, static_cast<int>(lane_xor<2>(static_cast<uint32_t>(v))));
  return min(v, static_cast<int>(lane_xor<1>(static_cast<uint32_t>(v))));
}
// Inclusive scan over the 64 lanes in a fixed order: a Kogge-Stone scan inside each 16-lane row
// (DPP row shifts by 1, 2, 4, 8), then row r adds the totals of rows 0 .. r-1, summed from row
// 0 upwards. All 64 lanes must be active.
__device__ __forceinline__ double wave_inclusive_scan(double v, int lane) {
  v += row_shr_zero<1>(v);
  v += row_shr_zero<2>(v);
  v += row_shr_zero<4>(v);
  v += row_shr_zero<8>(v);
  const double r0 = read_lane(v, 15), r1 = read_lane(v, 31), r2 = read_lane(v, 47);
  const double r01 = r0 + r1, r012 = r01 + r2;
  const int row = lane >> 4;
  return row == 0 ? v : v + (row == 1 ? r0 : (row == 2 ? r01 : r012));
}
__device__ __forceinline__ int wave_inclusive_scan_int(int v, int lane) {
  v += static_cast<int>(row_shr_zero<1>(static_cast<uint32_t>(v)));
  v += static_cast<int>(row_shr_zero<2>(static_cast<uint32_t>(v)));
  v += static_cast<int>(row_shr_zero<4>(static_cast<uint32_t>(v)));
  v += static_cast<int>(row_shr_zero<8>(static_cast<uint32_t>(v)));
  const int r0 = read_lane(v, 15), r1 = read_lane(v, 31), r2 = read_lane(v, 47);
  const int row = lane >> 4;
  return v + (row == 0 ? 0 : (row == 1 ? r0 : (row == 2 ? r0 + r1 : r0 + r1 + r2)));
}
// Exclusive prefix from the inclusive scan `inc`: lane l - 1's value, 0 in lane 0.
__device__ __forceinline__ double wave_exclusive_of(double inc, int lane) {
  const double sh = row_shr_zero<1>(inc);
  const double p0 = read_lane(inc, 15), p1 = read_lane(inc, 31), p2 = read_lane(inc, 47);
  const int row = lane >> 4;
  if ((lane & 15) != 0) return sh;
  return row == 0 ? 0.0 : (row == 1 ? p0 : (row == 2 ? p1 : p2));
}

// ---- block reductions (blockDim.x = NT, a multiple of 64; `red` holds NT/64 slots) -------------
template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) m = fmaxf(m, red[i]);
  return m;
}
template <int NT>
__device__ __forceinline__ int block_max_int(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_max_int(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  int m = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) m = max(m, red[i]);
  return m;
}
template <int NT>
__device__ __forceinline__ int block_min_int(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_min_int(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  int m = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) m = min(m, red[i]);
  return m;
}
// The same reductions with LDS-only barriers (lds_barrier): global loads and LDS-DMA copies in
// flight stay in flight through them (a __syncthreads() waits for every one).
template <int NT>
__device__ __forceinline__ float block_max_lds(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_max(v);
  lds_barrier();
  if (lane == 0) red[w] = v;
  lds_barrier();
  float m = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) m = fmaxf(m, red[i]);
  return m;
}
template <int NT>
__device__ __forceinline__ int block_min_int_lds(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_min_int(v);
  lds_barrier();
  if (lane == 0) red[w] = v;
  lds_barrier();
  int m = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) m = min(m, red[i]);
  return m;
}
// Exclusive scan over the block; returns this thread's exclusive prefix, *total the sum.
template <int NT>
__device__ __forceinline__ double block_exclusive_scan(double v, double* red, double* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const double inc = wave_inclusive_scan(v, lane);
  const double exc = wave_exclusive_of(inc, lane);
  __syncthreads();
  if (lane == 63) red[w] = inc;
  __syncthreads();
  double before = 0.0, tot = 0.0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    if (i < w) before += red[i];
    tot += red[i];
  }
  *total = tot;
  return before + exc;
}
template <int NT>
__device__ __forceinline__ int block_exclusive_scan_int(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan_int(v, lane);
  __syncthreads();
  if (lane == 63) red[w] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    if (i < w) before += red[i];
    tot += red[i];
  }
  *total = tot;
  return before + (inc - v);
}

// The chunk holding a draw: chunks 0..n-1 carry masses mass(c) >= 0 (ascending token order);
// the draw is the first chunk whose cumulative mass exceeds the target (u * Z, Z = total mass).
// If rounding leaves the draw past the last positive chunk of the range that should hold it,
// that chunk is taken with take_last set (the caller then takes its last positive token).
struct Located {
  int chunk;        // -1 if the total mass is not positive and finite
  int take_last;
  double before;    // cumulative mass of the chunks before `chunk`
  double target;    // u * Z
  double total;     // Z
};

// A draw located by one wave, for blocks whose NT threads each own a contiguous range of
// `per` chunks (thread t: chunks t per .. t per + per - 1, clipped to n; per <= 64) and have
// written the sum of their range, added in chunk order, to ssum[t]; mass(c) must be readable by
// every lane (LDS). Three levels, each a wave scan and a ballot: the group of NT / 64 threads,
// the thread (the last with positive mass whose exclusive prefix is <= the target), and the
// chunk (the first whose inclusive prefix passes the target, else, when rounding leaves the draw
// past the thread's range, its last positive chunk with take_last set). The prefix of a thread
// is its group's prefix plus the sums before it in the group; the first positive thread of the
// chosen group has exactly its group's prefix, so the second level always finds one. All 64
// lanes of the wave must be active; every lane gets the result.
template <int NT, class MassFn, class TargetFn>
__device__ Located wave_locate(const double* ssum, int n, int per, TargetFn target_of,
                               MassFn mass) {
  constexpr int kG = NT / 64;
  const int lane = threadIdx.x & 63;
  double gs = 0.0;
#pragma unroll
  for (int i = 0; i < kG; ++i) gs += ssum[kG * lane + i];
  const double inc = wave_inclusive_scan(gs, lane);
  const double exc = wave_exclusive_of(inc, lane);
  Located r;
  r.total = read_lane(inc, kWave - 1);
  r.target = target_of(r.total);
  r.chunk = -1;
  r.take_last = 0;
  r.before = 0.0;
  const bool ok = (r.total > 0.0) && (r.total < __builtin_inf());
  const unsigned long long cand = __ballot(ok && gs > 0.0 && exc <= r.target);
  if (!cand) return r;
  const int g = 63 - __clzll(static_cast<long long>(cand));
  const double gbase = read_lane(exc, g);
  const double si = (lane < kG) ? ssum[kG * g + lane] : 0.0;
  const double tpre = gbase + wave_exclusive_of(wave_inclusive_scan(si, lane), lane);
  const unsigned long long cand2 = __ballot(lane < kG && si > 0.0 && tpre <= r.target);
  const int i2 = 63 - __clzll(static_cast<long long>(cand2));
  const int t = kG * g + i2;
  const double tbase = read_lane(tpre, i2);
  const int tc0 = min(n, t * per), tn = min(n, tc0 + per) - tc0;
  const double mi = (lane < tn) ? mass(tc0 + lane) : 0.0;
  const double mpre = tbase + wave_exclusive_of(wave_inclusive_scan(mi, lane), lane);
  const unsigned long long hit = __ballot(lane < tn && mpre + mi > r.target);
  int i3;
  if (hit) {
    i3 = __ffsll(static_cast<long long>(hit)) - 1;
  } else {
    const unsigned long long pos = __ballot(lane < tn && mi > 0.0);   // thread t has positive mass
    i3 = 63 - __clzll(static_cast<long long>(pos));
    r.take_last = 1;
  }
  r.chunk = tc0 + i3;
  r.before = read_lane(mpre, i3);
  return r;
}

// LDS slot of entry c in a staging array with one pad slot per 16 entries: a thread's
// contiguous 16-entry range then starts on a different bank than its neighbours'.
__host__ __device__ __forceinline__ int padded(int c) { return c + (c >> 4); }

// Mass of a partial (tile max m, fp32 sum s of exp(L - m)) relative to the row max M.
__device__ __forceinline__ double partial_mass(float m, double s, float M) {
  return (m == kNegInf) ? 0.0 : exp(static_cast<double>(m) - static_cast<double>(M)) * s;
}

}  // namespace dspark
