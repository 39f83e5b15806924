// Markov-head draft and confidence head for gfx950.
//
// Sources: [V41] blog.javazero.top "DeepSeek-V4.1 模型结构（6）：解码，DSpark", "Markov head"
// (eqs. (4), (5), the serial loop) and "confidence head" (eq. (7)); [ZDS] zdszero.github.io
// spec_dspark, "在 SGLang 里" (sigmoid(raw / T) with per-position STS temperatures);
// [CSDN] deepseek.csdn.net DSpark walk-through, 4.1-4.2.
//
// One draft step k (the serial dependency: step k+1 needs every request's x_k):
//   markov_step  streams W2t and the U slice of position k once, forms
//                L = U_k + W1[x_{k-1}] . W2 tile by tile with bf16 MFMA (fp32 accumulate) and
//                writes, per request and 32-token tile, the tile max and the fp32 sum of
//                exp(L - tile max). The [B][V] logits are never written (unless asked for).
//   draft_sample one workgroup per request: combines the tile partials in fp64, finds the tile
//                that holds u * Z, recomputes that tile's 32 logits with the same MFMA sequence
//                (bit-identical), and walks them in fp64 to the drawn token.
#include "device.h"
#include "launch.h"
#include "tiles.h"

namespace dspark {

namespace {

template <int KS>
__global__ __launch_bounds__(kBlock, 2) void markov_step_kernel(StepArgs p) {
  using C = StepCfg<KS>;
  constexpr int r = C::kR;
  __shared__ __attribute__((aligned(16))) uint16_t E[C::kBG * C::kLdsRow];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int tok0 = blockIdx.x * (4 * kTileTokens) + wave * kTileTokens;
  const bool active = tok0 < p.V;
  const bool vec4 = (p.V & 3) == 0;

  u16x8_t a[KS];
  load_w2_tile<KS>(a, p.W2t, tok0 + col, p.V, half);

  for (int bg0 = 0; bg0 < p.B; bg0 += C::kBG) {
    const int nb = min(C::kBG, p.B - bg0);
    constexpr int kChunks = r / 8;  // 16-byte pieces per E row
    for (int c = threadIdx.x; c < C::kBG * kChunks; c += kBlock) {
      const int i = c / kChunks, q = c % kChunks;
      u16x8_t v = zero_u16x8();
      if (i < nb) {
        const int32_t row = p.prev[static_cast<size_t>(bg0 + i) * p.prev_stride];
        v = load_u16x8(p.W1 + static_cast<size_t>(row) * r + q * 8);
      }
      *reinterpret_cast<u16x8_t*>(&E[i * C::kLdsRow + q * 8]) = v;
    }
    __syncthreads();
    if (active) {
      for (int nt = 0; nt * 32 < nb; ++nt) {
        const uint16_t* erow = &E[(nt * 32 + col) * C::kLdsRow + 8 * half];
        f32x16_t acc = {};
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = mfma_32x32x16(a[s], load_u16x8(erow + 16 * s), acc);
        const int b = bg0 + nt * 32 + col;
        if (b < p.B) {
          const size_t urow = (static_cast<size_t>(b) * p.gamma + p.k) * p.V;
          float L[16];
          tile_logits(acc, p.U + urow, tok0, p.V, half, vec4, L);
          if (p.dbg) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int v = tok0 + 8 * g + 4 * half;
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (v + i < p.V) p.dbg[urow + v + i] = L[4 * g + i];
            }
          }
          float m = max16(L);
          m = fmaxf(m, __shfl_xor(m, 32, kWave));
          float t[16];
          tile_terms(L, m, t);
          float s = sum16(t);
          s = s + __shfl_xor(s, 32, kWave);
          if (half == 0) {
            const size_t o = static_cast<size_t>(b) * p.ntiles + tok0 / kTileTokens;
            p.pmax[o] = m;
            p.psum[o] = s;
          }
        }
      }
    }
    __syncthreads();
  }
}

template <int KS>
__global__ __launch_bounds__(kBlock) void draft_sample_kernel(SampleArgs p) {
  __shared__ double red_d[kBlock / 64];
  __shared__ float red_f[kBlock / 64];
  __shared__ int red_i[kBlock / 64];
  __shared__ Located loc;
  __shared__ float Ls[kTileTokens];
  __shared__ float Lc[kTileTokens];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t pbase = static_cast<size_t>(b) * p.ntiles;
  const size_t urow = (static_cast<size_t>(b) * p.gamma + p.k) * p.V;
  const int32_t prevtok = p.prev[static_cast<size_t>(b) * p.prev_stride];
  const size_t out = static_cast<size_t>(b) * p.gamma + p.k;

  // Row max over the tile maxima.
  float m = kNegInf;
  for (int c = tid; c < p.ntiles; c += kBlock) m = fmaxf(m, p.pmax[pbase + c]);
  const float M = block_max<kBlock>(m, red_f);

  const double u = static_cast<double>(p.uniforms[(static_cast<size_t>(b) * (p.gamma + 1) + p.k) * 3]);
  auto mass = [&](int c) {
    return partial_mass(p.pmax[pbase + c], static_cast<double>(p.psum[pbase + c]), M);
  };
  const Located L = locate_chunk<kBlock>(p.ntiles, u, mass, red_d, red_i, &loc);
  const double lse = static_cast<double>(M) + log(L.total);

  if (L.chunk < 0) {  // logits not finite: documented fallback
    if (tid == 0) {
      p.tokens[out] = 0;
      p.q[out] = __builtin_nanf("");
      p.lse[out] = __builtin_nan("");
    }
    return;
  }
  const int tok0 = L.chunk * kTileTokens;
  if (tid < 64) recompute_tile<KS>(p.W1, p.W2t, p.U + urow, prevtok, tok0, p.V, Ls);
  __syncthreads();
  int x = 0;
  __shared__ int s_x;
  if (tid == 0) {
    const float tm = p.pmax[pbase + L.chunk];
    const double f = exp(static_cast<double>(tm) - static_cast<double>(M));
    double cum = L.before;
    int found = -1, last = -1;
    for (int j = 0; j < kTileTokens && tok0 + j < p.V; ++j) {
      const float t = exp_term(Ls[j] - tm);
      if (t > 0.0f) last = j;
      if (!L.take_last) {
        cum += f * static_cast<double>(t);
        if (cum > L.target) {
          found = j;
          break;
        }
      }
    }
    s_x = tok0 + (found >= 0 ? found : (last >= 0 ? last : 0));
  }
  __syncthreads();
  x = s_x;
  // The token whose probability is reported (and that conditions the next position).
  const int32_t cond = p.force ? p.force[out] : x;
  const float* Lsrc = Ls;
  if (cond / kTileTokens != L.chunk) {
    if (tid < 64) recompute_tile<KS>(p.W1, p.W2t, p.U + urow, prevtok,
                                     (cond / kTileTokens) * kTileTokens, p.V, Lc);
    __syncthreads();
    Lsrc = Lc;
  }
  if (tid == 0) {
    const float lc = Lsrc[cond % kTileTokens];
    p.tokens[out] = x;
    p.q[out] = static_cast<float>(exp(static_cast<double>(lc) - lse));
    p.lse[out] = lse;
  }
}

// Confidence head: one wave per (request, position).
__global__ __launch_bounds__(kBlock) void confidence_kernel(ConfArgs p) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
  if (idx >= p.B * p.gamma) return;
  const int b = idx / p.gamma, k = idx % p.gamma;
  const int32_t prevtok = (k == 0) ? p.anchor[b] : p.tokens[static_cast<size_t>(b) * p.gamma + k - 1];
  double acc = 0.0;
  const uint16_t* hrow = p.h + static_cast<size_t>(idx) * p.d;
  for (int i = lane * 8; i < p.d; i += 64 * 8) {
    const u16x8_t hv = load_u16x8(hrow + i), wv = load_u16x8(p.w + i);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc += static_cast<double>(bf16_to_f32(hv[e]) * bf16_to_f32(wv[e]));  // exact product
  }
  const uint16_t* erow = p.W1 + static_cast<size_t>(prevtok) * p.r;
  for (int i = lane * 8; i < p.r; i += 64 * 8) {
    const u16x8_t ev = load_u16x8(erow + i), wv = load_u16x8(p.w + p.d + i);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc += static_cast<double>(bf16_to_f32(ev[e]) * bf16_to_f32(wv[e]));
  }
  const double z = wave_sum(acc);
  if (lane == 0) {
    const double c = 1.0 / (1.0 + exp(-z / static_cast<double>(p.T[k])));
    p.conf[idx] = static_cast<float>(c);
  }
}

}  // namespace

template <int KS>
static hipError_t launch_step_ks(const StepArgs& a, hipStream_t s) {
  const int grid = (a.V + 4 * kTileTokens - 1) / (4 * kTileTokens);
  hipLaunchKernelGGL(markov_step_kernel<KS>, dim3(grid), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}
template <int KS>
static hipError_t launch_sample_ks(const SampleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(draft_sample_kernel<KS>, dim3(a.B), dim3(kBlock), 0, s, a);
  return hipGetLastError();
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
hipError_t launch_draft_sample(const SampleArgs& a, int r, hipStream_t s) {
  DSPARK_DISPATCH_KS(r, launch_sample_ks, a, s)
}
hipError_t launch_confidence(const ConfArgs& a, hipStream_t s) {
  const int waves = a.B * a.gamma;
  const int grid = (waves + (kBlock / 64) - 1) / (kBlock / 64);
  hipLaunchKernelGGL(confidence_kernel, dim3(grid), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark
