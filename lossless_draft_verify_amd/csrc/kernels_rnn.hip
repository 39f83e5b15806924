// RNN draft head, eq. (6) of [CSDN] deepseek.csdn.net (4.2, the two serial heads); [AIL]
// ailearn.mscapital.top "DSpark：..." (RNN head, optional):
//   z_k = [s_{k-1}; W1[x_{k-1}]; h_k],
//   s_k = sigma(W_g z_k) * s_{k-1} + (1 - sigma(W_g z_k)) * tanh(W_c z_k),
//   B_k = W2^T tanh(W_o z_k),
// with s_0 = 0 at the start of every block, the state of size r, no bias terms, and W_g, W_c,
// W_o stacked by rows into Wgco [3r][2r + d] whose columns follow z (state | embedding | hidden).
//
// Two kernels (the verify's target pass splits given bias vectors into the same terms):
//   rnn_pre     the hidden-state block of Wgco applied to every h_k of the round (one bf16 MFMA
//               GEMM, B gamma x d x 3r, off the serial chain): P[slice][B gamma][3r], the sums
//               over kRnnPreSplits slices of the hidden dimension (fp64 sums stored as fp32).
//   rnn_state   one step: pre-activations P + Wgco[:, state] s_{k-1} + Wgco[:, emb] W1[x_{k-1}]
//               in fp64, the gates, s_k, and e_k = tanh(a_o), written as fp32 and as three bf16
//               terms (t1 = RN(e), t2 = RN(e - t1), t3 = RN(e - t1 - t2)) that the bias
//               contraction of the draft step consumes (their sum is the fp32 e).
#include <hip/hip_runtime.h>

#include "device.h"
#include "dma.h"
#include "launch.h"
#include "tiles.h"

namespace dspark {
namespace {

// ---- rnn_pre: P = h . Wgco[:, hidden]^T ------------------------------------------------------
//
// A 256-thread workgroup computes a 64 (outputs n) x 64 (rows m = b gamma + k) tile over one
// of kRnnPreSplits slices of the hidden dimension; wave w takes the 32 x 32 sub-tile
// (n: w & 1, m: w >> 1). The slice is walked in chunks of 128 columns: the chunk's 64 Wgco rows
// and 64 h rows (256 B each) are copied into one of two LDS stages by LDS-DMA loads (whole 1 KB
// lines per instruction, the next chunk in flight while one is computed), XOR-swizzled in
// 16-byte pieces (piece c of row t at c ^ (t & 15)) so the 32 rows one ds_read_b128 touches fall
// on distinct banks. After every chunk (8 k-steps, 128 products) the fp32 MFMA sums are added
// into fp64 accumulators; each slice's sum is stored as fp32 (one rounding, about 6e-8
// relative) and the state step adds the slices in fp64. Columns past d read as zero.
constexpr int kPreThreads = 256;
constexpr int kPreChunk = 128;                        // columns per stage
constexpr int kPreRowBytes = kPreChunk * 2;           // 256 B: 16 pieces of 16 B
constexpr int kPreOperandBytes = 64 * kPreRowBytes;   // 16 KB per operand per stage
constexpr int kPreStageBytes = 2 * kPreOperandBytes;
constexpr int kPreCopies = kPreStageBytes / 1024 / (kPreThreads / 64);   // 8 per wave per chunk

__global__ __launch_bounds__(kPreThreads) void rnn_pre_kernel(RnnPreArgs p) {
  __shared__ __attribute__((aligned(1024))) unsigned char stage[2 * kPreStageBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int N = 3 * p.r, nz = 2 * p.r + p.d;
  const int ntn = (N + 63) / 64, ntm = (p.M + 63) / 64;
  const int tile = blockIdx.x % (ntn * ntm), split = blockIdx.x / (ntn * ntm);
  const int nb = (tile % ntn) * 64, mb = (tile / ntn) * 64;
  const int nchunks = (p.d + kPreChunk - 1) / kPreChunk;
  const int c_lo = nchunks * split / kRnnPreSplits, c_hi = nchunks * (split + 1) / kRnnPreSplits;
  const uint32_t stage_addr = lds_addr(stage);

  // This wave's copies of chunk c into stage st: instruction q covers 4 rows (64 pieces);
  // q < 16 fill the Wgco rows, the rest the h rows. Sources past d are clamped inside the row.
  auto issue = [&](int c, int st) {
#pragma unroll
    for (int i = 0; i < kPreCopies; ++i) {
      const int q = wave * kPreCopies + i;
      const int qq = q & 15;
      const int slot = 64 * qq + lane;
      const int row = slot >> 4;
      const int piece = (slot & 15) ^ (row & 15);
      const int k = min(c * kPreChunk + 8 * piece, p.d - 8);
      const uint16_t* src =
          (q < 16) ? p.Wgco + static_cast<size_t>(min(nb + row, N - 1)) * nz + 2 * p.r + k
                   : p.h + static_cast<size_t>(min(mb + row, p.M - 1)) * p.d + k;
      copy16_to_lds(src, stage_addr + st * kPreStageBytes + (q >> 4) * kPreOperandBytes +
                             1024 * qq);
    }
  };

  const int arow = 32 * (wave & 1) + col, brow = 32 * (wave >> 1) + col;
  double acc64[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc64[j] = 0.0;
  if (c_lo < c_hi) issue(c_lo, 0);
  for (int c = c_lo; c < c_hi; ++c) {
    if (c + 1 < c_hi) {
      issue(c + 1, (c + 1 - c_lo) & 1);
      wait_copies<kPreCopies>();
    } else {
      wait_copies<0>();
    }
    asm volatile("s_barrier" ::: "memory");
    const unsigned char* base = stage + ((c - c_lo) & 1) * kPreStageBytes;
    f32x16_t acc = {};
#pragma unroll
    for (int s = 0; s < kPreChunk / 16; ++s) {
      const int piece = 2 * s + half;
      const bool in = c * kPreChunk + 8 * piece < p.d;
      const u16x8_t a = *reinterpret_cast<const u16x8_t*>(
          base + arow * kPreRowBytes + 16 * (piece ^ (arow & 15)));
      const u16x8_t b = *reinterpret_cast<const u16x8_t*>(
          base + kPreOperandBytes + brow * kPreRowBytes + 16 * (piece ^ (brow & 15)));
      acc = mfma_32x32x16(b, in ? a : zero_u16x8(), acc);   // (rows m) x (outputs n)
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) acc64[j] += static_cast<double>(acc[j]);
    lds_barrier();   // the stage is free for chunk c + 2
  }
  // Lane col holds output n for the rows m of its half: each store writes two 128-byte row pieces.
  const int n = nb + 32 * (wave & 1) + col;
  if (n < N) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int m = mb + 32 * (wave >> 1) + tile_token(j, half);
      if (m < p.M) p.P[(static_cast<size_t>(split) * p.M + m) * N + n] = static_cast<float>(acc64[j]);
    }
  }
}

// ---- rnn_state: one step of eq. (6) ----------------------------------------------------------
//
// Workgroup (block of 16 state indices j, block of 8 requests), eight waves (two per SIMD, so
// that one's fp64 multiply-adds cover the other's latencies); the waves split the 2r columns of
// z's state and embedding blocks into eight slices (four at r = 16, the other four waves then
// add nothing). Each wave first copies its slice of the 48 weight rows it needs (rows j, r + j,
// 2r + j: W_g, W_c, W_o) into its own LDS region by LDS-DMA loads, all in flight at once
// (swizzled in 16-byte pieces like the other staged tiles); lane (j, request pair) then forms
// the six partial dot products with its two requests' z in fp64 (z from LDS, read by 16 lanes at
// once: broadcasts). Each weight element is read from L2 by 16 request blocks instead of 128
// requests. Every slice's sums go to LDS, and wave w finishes request w: the slices added in
// slice order, then the slices of P, then the gates.
constexpr int kStateThreads = 512;
constexpr int kStateWaves = kStateThreads / 64;
constexpr int kStateJ = 16;
constexpr int kStateB = 8;
static_assert(kStateJ * kStateB / 2 == 64 && kStateB == kStateWaves,
              "a lane per (state index, request pair); a wave per request in the tail");
constexpr int kStateRows = 3 * kStateJ;                              // 48 weight rows
constexpr int kStateSliceBytes = kStateRows * (2 * 256 / kStateWaves) * 2;   // r = 256: 6 KB

__device__ __forceinline__ double bf16_to_f64(uint16_t v) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(v) << 16));
}

// The terms of component j of request b's bias vector at position k, also in the MFMA operand
// layout of StepArgs::E2 (term t is k-step element t r + j).
__device__ __forceinline__ void split_terms_operand(float e, uint16_t* E2, int b, int k, int gamma,
                                                    int j, int r) {
  static_assert(kRnnTerms == 3, "three terms");
  const uint16_t t1 = bf16_rne(e);
  const float rest1 = e - bf16_value(t1);
  const uint16_t t2 = bf16_rne(rest1);
  const float rest2 = rest1 - bf16_value(t2);
  const uint16_t t[3] = {t1, t2, bf16_rne(rest2)};
  const size_t base = (static_cast<size_t>(b >> 5) * gamma + k) * (kRnnTerms * r / 16);
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const int i = q * r + j, s = i >> 4, h = (i >> 3) & 1;
    E2[((base + s) * 2 + h) * 256 + 8 * (b & 31) + (i & 7)] = t[q];
  }
}

__global__ __launch_bounds__(kStateThreads) void rnn_state_kernel(RnnStateArgs p) {
  extern __shared__ double zs[];                    // [kStateB][2r]: s_{k-1} | W1[x_{k-1}]
  __shared__ double part[kStateWaves][6][64];       // every slice's sums: (row, pair) x lane
  __shared__ __attribute__((aligned(1024))) unsigned char wst[kStateWaves * kStateSliceBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = p.r, nz = 2 * r + p.d;
  const int nj = (r + kStateJ - 1) / kStateJ;
  const int j0 = (blockIdx.x % nj) * kStateJ, b0 = (blockIdx.x / nj) * kStateB;
  const int ns = (2 * r >= 8 * kStateWaves) ? kStateWaves : 4;   // input slices (r = 16: four)
  const bool active = wave < ns;
  const int q = (2 * r) / ns, i0 = wave * q;         // q: a multiple of 8 inputs
  const int cpr = q / 8;                             // 16-byte pieces per row: 1, 2, 4 or 8
  const int swz = cpr - 1;
  // The previous tokens of the values this thread stages first, straight from memory (no
  // barrier), then their z loads; the weight copies (this wave's slice of the rows) and the
  // tail's pre-GEMM terms go out behind them.
  constexpr int kZPer = kStateB * 2 * 256 / kStateThreads;
  int32_t xt[kZPer];
#pragma unroll
  for (int u = 0; u < kZPer; ++u) {
    const int i = tid + u * kStateThreads;
    const int rb = min(i / (2 * r), kStateB - 1);
    xt[u] = clamp_token(p.prev[static_cast<size_t>(min(b0 + rb, p.B - 1)) * p.prev_stride], p.V);
  }
  double zv[kZPer];
#pragma unroll
  for (int u = 0; u < kZPer; ++u) {
    const int i = tid + u * kStateThreads;
    const int rb = min(i / (2 * r), kStateB - 1), c = i % (2 * r);
    const int b = min(b0 + rb, p.B - 1);
    const double sv = (p.s_in && c < r) ? p.s_in[static_cast<size_t>(b) * r + c] : 0.0;
    const double ev = bf16_to_f64(p.W1[static_cast<size_t>(xt[u]) * r + (c < r ? 0 : c - r)]);
    zv[u] = (c < r) ? sv : ev;
  }
  if (active) {
    const uint32_t wbase = lds_addr(wst) + wave * kStateSliceBytes;
    const int npieces = kStateRows * cpr;
    for (int t = 0; t * 64 < npieces; ++t) {
      const int slot = 64 * t + lane;
      if (slot < npieces) {
        const int row = slot / cpr;
        const int piece = (slot % cpr) ^ (row & swz);
        const int jr = min(j0 + row % kStateJ, r - 1);
        copy16_to_lds(
            p.Wgco + static_cast<size_t>((row / kStateJ) * r + jr) * nz + i0 + 8 * piece,
            wbase + 1024 * t);
      }
    }
  }
  // Tail of wave w: request b0 + w, lanes 0 .. kStateJ - 1 = state index j0 + lane; its
  // pre-GEMM terms (index clamped; pairs past B or r unused).
  const int tj = j0 + lane % kStateJ, tb = b0 + wave;
  const int N = 3 * r;
  const size_t M = static_cast<size_t>(p.B) * p.gamma;
  float pv[kRnnPreSplits][3];
  {
    const size_t m = static_cast<size_t>(min(tb, p.B - 1)) * p.gamma + p.k;
    const int jc = min(tj, r - 1);
#pragma unroll
    for (int sp = 0; sp < kRnnPreSplits; ++sp) {
      const float* P = p.P + (sp * M + m) * N;
      pv[sp][0] = P[jc];
      pv[sp][1] = P[r + jc];
      pv[sp][2] = P[2 * r + jc];
    }
  }
#pragma unroll
  for (int u = 0; u < kZPer; ++u) {
    const int i = tid + u * kStateThreads;
    if (i < kStateB * 2 * r) zs[i] = zv[u];
  }
  wait_copies<0>();
  __syncthreads();
  // Dot products: lane (state index j0 + jl, request pair rp) over this wave's inputs, for the
  // three gate rows and both requests of the pair.
  const int jl = lane % kStateJ, rp = lane / kStateJ;
  double acc[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};   // (g, c, o) x (request 2rp, 2rp + 1)
  if (active) {
    const unsigned char* wl = wst + wave * kStateSliceBytes;
    const double* z0 = zs + (2 * rp) * (2 * r) + i0;
    const double* z1 = z0 + 2 * r;
    for (int pc = 0; pc < cpr; ++pc) {
      u16x8_t w3[3];
#pragma unroll
      for (int m3 = 0; m3 < 3; ++m3) {
        const int row = m3 * kStateJ + jl;
        w3[m3] = *reinterpret_cast<const u16x8_t*>(wl + 16 * (row * cpr + (pc ^ (row & swz))));
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const double za = z0[8 * pc + t], zb = z1[8 * pc + t];
        const double g = bf16_to_f64(w3[0][t]), c = bf16_to_f64(w3[1][t]),
                     o = bf16_to_f64(w3[2][t]);
        // explicit fused multiply-adds (the build does not contract): one rounding per term
        acc[0] = fma(g, za, acc[0]);
        acc[1] = fma(c, za, acc[1]);
        acc[2] = fma(o, za, acc[2]);
        acc[3] = fma(g, zb, acc[3]);
        acc[4] = fma(c, zb, acc[4]);
        acc[5] = fma(o, zb, acc[5]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 6; ++t) part[wave][t][lane] = acc[t];
  __syncthreads();
  if (lane >= kStateJ || tj >= r || tb >= p.B) return;
  const int th = wave & 1;
  const int src = (wave >> 1) * kStateJ + lane;      // lane (state index, pair wave / 2) above
  double ag = part[0][3 * th][src], ac = part[0][3 * th + 1][src], ao = part[0][3 * th + 2][src];
#pragma unroll
  for (int w = 1; w < kStateWaves; ++w) {
    ag += part[w][3 * th][src];
    ac += part[w][3 * th + 1][src];
    ao += part[w][3 * th + 2][src];
  }
  const size_t m = static_cast<size_t>(tb) * p.gamma + p.k;
#pragma unroll
  for (int sp = 0; sp < kRnnPreSplits; ++sp) {
    ag += static_cast<double>(pv[sp][0]);
    ac += static_cast<double>(pv[sp][1]);
    ao += static_cast<double>(pv[sp][2]);
  }
  const double gate = 1.0 / (1.0 + exp(-ag));
  const double s_prev = zs[wave * (2 * r) + tj];
  p.s_out[static_cast<size_t>(tb) * r + tj] = gate * s_prev + (1.0 - gate) * tanh(ac);
  const float e = static_cast<float>(tanh(ao));
  p.e_out[m * r + tj] = e;
  split_terms(e, p.E + m * (kRnnTerms * r) + tj, r);
  if (p.E2) split_terms_operand(e, p.E2, tb, p.k, p.gamma, tj, r);
}

}  // namespace

hipError_t launch_rnn_pre(const RnnPreArgs& a, hipStream_t s) {
  const int ntn = (3 * a.r + 63) / 64, ntm = (a.M + 63) / 64;
  launch_kernel(rnn_pre_kernel, dim3(ntn * ntm * kRnnPreSplits), dim3(kPreThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rnn_state(const RnnStateArgs& a, hipStream_t s) {
  const int nj = (a.r + kStateJ - 1) / kStateJ;
  const int nb = (a.B + kStateB - 1) / kStateB;
  launch_kernel(rnn_state_kernel, dim3(nj * nb), dim3(kStateThreads),
                     static_cast<size_t>(kStateB * 2 * a.r) * sizeof(double), s, a);
  return hipGetLastError();
}

}  // namespace dspark
