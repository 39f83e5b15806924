// MFMA tile helpers shared by the draft step, the draft sampler and the residual kernels. All
// of them form a token tile's logits with the same instruction sequence, so a sampler that
// recomputes one tile reproduces the streaming pass bit for bit. Also the bias rows' layout and
// the split of an RNN bias component into its three bf16 terms.
#pragma once

#include "device.h"

namespace dspark {

// E rows in LDS are padded by 8 bf16 so the 32 rows a wave reads with one ds_read_b128 spread
// over the LDS banks.
template <int KS>
struct StepCfg {
  static constexpr int kR = KS * 16;
  static constexpr int kBG = (kR <= 256) ? 128 : 64;   // requests per LDS fill
  static constexpr int kLdsRow = kR + 8;
};

template <int KS>
__device__ __forceinline__ void load_w2_tile(u16x8_t (&a)[KS], const uint16_t* __restrict__ W2t,
                                             int tok, int V, int half) {
  constexpr int r = KS * 16;
  if (tok < V) {
    const uint16_t* p = W2t + static_cast<size_t>(tok) * r + 8 * half;
#pragma unroll
    for (int s = 0; s < KS; ++s) a[s] = load_u16x8(p + 16 * s);
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) a[s] = zero_u16x8();
  }
}

// Load four consecutive fp32 values v..v+3 of a row (those >= V read as 0).
__device__ __forceinline__ void load4(const float* __restrict__ row, int v, int V, bool vec4,
                                      float (&o)[4]) {
  if (vec4 && v + 3 < V) {
    const float4 t = *reinterpret_cast<const float4*>(row + v);
    o[0] = t.x;
    o[1] = t.y;
    o[2] = t.z;
    o[3] = t.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (v + i < V) ? row[v + i] : 0.0f;
  }
}

// Sixteen consecutive values row[v0 .. v0 + 15] (v0 a multiple of 4). With V % 4 == 0 the four
// 16-byte loads are unguarded, addresses past the row clamped to its last four values (the
// caller ignores those entries), so all four go out before the first is used: a guarded fallback
// in the same branch would make each load wait for the one before it. Otherwise per-element
// guarded loads (0 past V).
__device__ __forceinline__ void load16(const float* __restrict__ row, int v0, int V, bool vec4,
                                       float (&x)[16]) {
  if (vec4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 t = *reinterpret_cast<const float4*>(row + min(v0 + 4 * i, V - 4));
      x[4 * i + 0] = t.x;
      x[4 * i + 1] = t.y;
      x[4 * i + 2] = t.z;
      x[4 * i + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (v0 + i < V) ? row[v0 + i] : 0.0f;
  }
}

// Logits of the 16 accumulator slots a lane holds: L = U + bias (fp32 add), -inf past V.
__device__ __forceinline__ void tile_logits(const f32x16_t& acc, const float* __restrict__ Urow,
                                            int tok0, int V, int half, bool vec4, float (&L)[16]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int v = tok0 + 8 * g + 4 * half;
    float u[4];
    load4(Urow, v, V, vec4, u);
#pragma unroll
    for (int i = 0; i < 4; ++i) L[4 * g + i] = (v + i < V) ? (u[i] + acc[4 * g + i]) : kNegInf;
  }
}

__device__ __forceinline__ float sum16(const float (&t)[16]) {
  const float a = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
  const float b = ((t[8] + t[9]) + (t[10] + t[11])) + ((t[12] + t[13]) + (t[14] + t[15]));
  return a + b;
}

__device__ __forceinline__ float max16(const float (&L)[16]) {
  float m = L[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) m = fmaxf(m, L[j]);
  return m;
}

// The B-operand row of the bias contraction for one (request, position): the Markov
// embedding row W1[prev] (NT = 1, r bf16), or the RNN head's bias vector e of that position held
// as NT bf16 terms [t_1 | t_2 | t_3] (NT = kRnnTerms = 3, rows of 3r bf16 at E + pos * 3r):
// t_1 = RN(e), t_2 = RN(e - t_1), t_3 = RN(e - t_1 - t_2), whose sum carries the fp32 e to its
// 24 bits. The contraction runs over the NT terms in order, each over the r columns of W2, so
// every caller forms the same fp32 sums.
constexpr int kRnnTerms = 3;

template <int NT>
__device__ __forceinline__ const uint16_t* bias_row(const uint16_t* W1, const uint16_t* E, int r,
                                                    int32_t prev, int64_t pos) {
  if constexpr (NT == 1) {
    return W1 + static_cast<size_t>(prev) * r;
  } else {
    return E + static_cast<size_t>(pos) * (NT * r);
  }
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

// Recompute the logits of one 32-token tile for one request with exactly the instruction
// sequence of the streaming draft step (same k order: the NT terms in turn, each over the r
// columns; same operands; the request sits in every MFMA column, and column placement does not
// change the result). Called by a whole wave; the bias row (NT r bf16) is read from LDS one
// k-step at a time, and the tile's U values are loaded together with the W2 tile. Lanes 0 and 32
// hold the 32 logits, which are written to Ls[0..32).
template <int KS, int NT = 1>
__device__ void recompute_tile_lds(const uint16_t* Es, const uint16_t* __restrict__ W2t,
                                   const float* __restrict__ Urow, int tok0, int V, float* Ls) {
  const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
  u16x8_t a[KS];
  load_w2_tile<KS>(a, W2t, tok0 + col, V, half);
  float u[16];
  const bool vec4 = (V & 3) == 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float o[4];
    load4(Urow, tok0 + 8 * g + 4 * half, V, vec4, o);
#pragma unroll
    for (int i = 0; i < 4; ++i) u[4 * g + i] = o[i];
  }
  f32x16_t acc = {};
#pragma unroll
  for (int s = 0; s < NT * KS; ++s)
    acc = mfma_32x32x16(a[s % KS], *reinterpret_cast<const u16x8_t*>(Es + 16 * s + 8 * half), acc);
  if (col == 0) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int v = tok0 + tile_token(j, half);
      Ls[tile_token(j, half)] = (v < V) ? (u[j] + acc[j]) : kNegInf;
    }
  }
}

// Walk one tile in ascending token order on one wave: lane j < 32 holds the mass w of token j
// (0 past the vocabulary). Returns the first j with before + sum_{i<=j} w_i > target, or, if
// none (rounding) or take_last is set, the last j with w_j > 0 (0 if there is none).
__device__ __forceinline__ int walk_tile(double w, double before, double target, bool take_last) {
  const int lane = threadIdx.x & 63;
  const double cum = before + wave_inclusive_scan(w, lane);
  const unsigned long long hit = __ballot(!take_last && lane < 32 && cum > target);
  if (hit) return __ffsll(static_cast<long long>(hit)) - 1;
  const unsigned long long pos = __ballot(lane < 32 && w > 0.0);
  return pos ? 63 - __clzll(static_cast<long long>(pos)) : 0;
}

}  // namespace dspark
