// RNN draft head, eq. (6) of [CSDN] deepseek.csdn.net (4.2, the two serial heads); [AIL]
// ailearn.mscapital.top "DSpark：..." (RNN head, optional):
//   z_k = [s_{k-1}; W1[x_{k-1}]; h_k],
//   s_k = sigma(W_g z_k) * s_{k-1} + (1 - sigma(W_g z_k)) * tanh(W_c z_k),
//   B_k = W2^T tanh(W_o z_k),
// with s_0 = 0 at the start of every block, the state of size r, no bias terms, and W_g, W_c,
// W_o stacked by rows into Wgco [3r][2r + d] whose columns follow z (state | embedding | hidden).
//
// Three kernels:
//   rnn_pre     the hidden-state block of Wgco applied to every h_k of the round (one bf16 MFMA
//               GEMM, B gamma x d x 3r, off the serial chain): P[split][B gamma][3r] in fp64.
//   rnn_state   one step: pre-activations P + Wgco[:, state] s_{k-1} + Wgco[:, emb] W1[x_{k-1}]
//               in fp64, the gates, s_k, and e_k = tanh(a_o), written as fp32 and as three bf16
//               terms (t1 = RN(e), t2 = RN(e - t1), t3 = RN(e - t1 - t2)) that the bias
//               contraction of the draft step consumes (their sum is the fp32 e).
//   split_bias  the same split of given fp32 vectors (the verify of an RNN draft).
#include <hip/hip_runtime.h>

#include "device.h"
#include "launch.h"
#include "tiles.h"

namespace dspark {
namespace {

// ---- rnn_pre: P = h . Wgco[:, hidden]^T ------------------------------------------------------
//
// A 256-thread workgroup computes a 64 (outputs n) x 64 (rows m = b gamma + k) tile over one
// half of the hidden dimension; wave w takes the 32 x 32 sub-tile (n: w & 1, m: w >> 1). The A
// operand is 8 consecutive bf16 of a Wgco row (output n = lane % 32), the B operand 8 of an h
// row (m = lane % 32), both 16-byte loads straight from global memory (the two waves sharing an
// operand meet in L1). Every 8 k-steps the fp32 MFMA sums are added into fp64 accumulators, so
// the fp32 part of the error covers 128 products at a time.
constexpr int kPreThreads = 256;
constexpr int kPreSplits = 2;
constexpr int kPreBatch = 8;   // k-steps per fp32 chunk

__device__ __forceinline__ u16x8_t load_or_zero(const uint16_t* row, int k, int d) {
  return (k < d) ? load_u16x8(row + k) : zero_u16x8();   // d % 8 == 0: chunks are whole
}

__global__ __launch_bounds__(kPreThreads) void rnn_pre_kernel(RnnPreArgs p) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int N = 3 * p.r, nz = 2 * p.r + p.d;
  const int ntn = (N + 63) / 64, ntm = (p.M + 63) / 64;
  const int tile = blockIdx.x % (ntn * ntm), split = blockIdx.x / (ntn * ntm);
  const int n0 = (tile % ntn) * 64 + 32 * (wave & 1);
  const int m0 = (tile / ntn) * 64 + 32 * (wave >> 1);
  // This split's k range, in whole 16-column steps.
  const int steps = (p.d + 15) / 16;
  const int s_lo = steps * split / kPreSplits, s_hi = steps * (split + 1) / kPreSplits;
  const uint16_t* arow = p.Wgco + static_cast<size_t>(min(n0 + col, N - 1)) * nz + 2 * p.r;
  const uint16_t* brow = p.h + static_cast<size_t>(min(m0 + col, p.M - 1)) * p.d;
  double acc64[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc64[j] = 0.0;
  for (int s0 = s_lo; s0 < s_hi; s0 += kPreBatch) {
    u16x8_t a[kPreBatch], b[kPreBatch];
#pragma unroll
    for (int i = 0; i < kPreBatch; ++i) {
      const int k = 16 * (s0 + i) + 8 * half;
      const bool in = s0 + i < s_hi;
      a[i] = in ? load_or_zero(arow, k, p.d) : zero_u16x8();
      b[i] = in ? load_or_zero(brow, k, p.d) : zero_u16x8();
    }
    f32x16_t acc = {};
#pragma unroll
    for (int i = 0; i < kPreBatch; ++i) acc = mfma_32x32x16(a[i], b[i], acc);
#pragma unroll
    for (int j = 0; j < 16; ++j) acc64[j] += static_cast<double>(acc[j]);
  }
  const int m = m0 + col;
  if (m < p.M) {
    double* out = p.P + (static_cast<size_t>(split) * p.M + m) * N;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int n = n0 + tile_token(j, half);
      if (n < N) out[n] = acc64[j];
    }
  }
}

// ---- rnn_state: one step of eq. (6) ----------------------------------------------------------
//
// Workgroup (request b, block of 64 state indices j); its four waves split the 2r columns of
// z's state and embedding blocks into quarters. Thread (j, quarter) forms the three partial
// dot products of rows j, r + j, 2r + j (W_g, W_c, W_o) over its quarter in fp64, z read from
// LDS (every lane of a wave reads the same element: a broadcast); the quarters are summed in
// fixed order with the two split-K parts of P.
constexpr int kStateThreads = 256;
constexpr int kStateJ = 64;

__device__ __forceinline__ double bf16_to_f64(uint16_t v) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(v) << 16));
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);   // x finite
}

__device__ __forceinline__ float bf16_value(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// The bf16 terms of a bias component, written to row[0], row[r], row[2r]: t1 = RN(e),
// t2 = RN(e - t1), t3 = RN(e - t1 - t2). Each difference is exact in fp32 (every term takes the
// leading 8 bits of what remains), so t1 + t2 + t3 = e for every finite fp32 e in (-1, 1).
__device__ __forceinline__ void split_terms(float e, uint16_t* row, int r) {
  static_assert(kRnnTerms == 3, "three terms");
  const uint16_t t1 = bf16_rne(e);
  const float rest1 = e - bf16_value(t1);
  const uint16_t t2 = bf16_rne(rest1);
  const float rest2 = rest1 - bf16_value(t2);
  row[0] = t1;
  row[r] = t2;
  row[2 * r] = bf16_rne(rest2);
}

__global__ __launch_bounds__(kStateThreads) void rnn_state_kernel(RnnStateArgs p) {
  extern __shared__ double zs[];              // [2r]: s_{k-1} | W1[x_{k-1}]
  __shared__ double part[3][3][kStateJ];      // quarters 1..3 of the three dot products
  const int tid = threadIdx.x, jl = tid & 63, quarter = tid >> 6;
  const int r = p.r, nz = 2 * r + p.d;
  const int nj = (r + kStateJ - 1) / kStateJ;
  const int b = blockIdx.x / nj, j0 = (blockIdx.x % nj) * kStateJ;
  const int32_t x = p.prev[static_cast<size_t>(b) * p.prev_stride];
  for (int i = tid; i < 2 * r; i += kStateThreads) {
    zs[i] = (i < r) ? (p.s_in ? p.s_in[static_cast<size_t>(b) * r + i] : 0.0)
                    : bf16_to_f64(p.W1[static_cast<size_t>(x) * r + (i - r)]);
  }
  __syncthreads();
  const int j = j0 + jl;
  const int jc = min(j, r - 1);               // rows past r are computed on row r - 1, not stored
  const int q = (2 * r) / 4, i0 = quarter * q;   // 2r is a multiple of 8
  const uint16_t* wg = p.Wgco + static_cast<size_t>(jc) * nz;
  const uint16_t* wc = p.Wgco + static_cast<size_t>(r + jc) * nz;
  const uint16_t* wo = p.Wgco + static_cast<size_t>(2 * r + jc) * nz;
  double ag = 0.0, ac = 0.0, ao = 0.0;
  for (int i = i0; i < i0 + q; i += 8) {
    const u16x8_t vg = load_u16x8(wg + i), vc = load_u16x8(wc + i), vo = load_u16x8(wo + i);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const double z = zs[i + t];
      ag += bf16_to_f64(vg[t]) * z;
      ac += bf16_to_f64(vc[t]) * z;
      ao += bf16_to_f64(vo[t]) * z;
    }
  }
  if (quarter > 0) {
    part[quarter - 1][0][jl] = ag;
    part[quarter - 1][1][jl] = ac;
    part[quarter - 1][2][jl] = ao;
  }
  __syncthreads();
  if (quarter != 0 || j >= r) return;
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    ag += part[t][0][jl];
    ac += part[t][1][jl];
    ao += part[t][2][jl];
  }
  const size_t m = static_cast<size_t>(b) * p.gamma + p.k;
  const int N = 3 * r;
  const double* P0 = p.P + m * N;
  const double* P1 = p.P + (static_cast<size_t>(p.B) * p.gamma + m) * N;
  ag += P0[j] + P1[j];
  ac += P0[r + j] + P1[r + j];
  ao += P0[2 * r + j] + P1[2 * r + j];
  const double gate = 1.0 / (1.0 + exp(-ag));
  const double s_prev = zs[j];
  p.s_out[static_cast<size_t>(b) * r + j] = gate * s_prev + (1.0 - gate) * tanh(ac);
  const float e = static_cast<float>(tanh(ao));
  p.e_out[m * r + j] = e;
  split_terms(e, p.E + m * (kRnnTerms * r) + j, r);
}

__global__ __launch_bounds__(256) void split_bias_kernel(SplitArgs p) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t n = static_cast<size_t>(p.n) * p.r;
  if (i >= n) return;
  const size_t m = i / p.r, j = i % p.r;
  split_terms(p.e[i], p.E + m * (kRnnTerms * p.r) + j, p.r);
}

}  // namespace

hipError_t launch_rnn_pre(const RnnPreArgs& a, hipStream_t s) {
  const int ntn = (3 * a.r + 63) / 64, ntm = (a.M + 63) / 64;
  hipLaunchKernelGGL(rnn_pre_kernel, dim3(ntn * ntm * kPreSplits), dim3(kPreThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rnn_state(const RnnStateArgs& a, hipStream_t s) {
  const int nj = (a.r + kStateJ - 1) / kStateJ;
  hipLaunchKernelGGL(rnn_state_kernel, dim3(a.B * nj), dim3(kStateThreads),
                     static_cast<size_t>(2 * a.r) * sizeof(double), s, a);
  return hipGetLastError();
}

hipError_t launch_split_bias(const SplitArgs& a, hipStream_t s) {
  const size_t n = static_cast<size_t>(a.n) * a.r;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(split_bias_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace dspark
