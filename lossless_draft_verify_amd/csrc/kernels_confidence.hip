// Confidence head for gfx950: c_k = sigmoid(w . [h_k ; W1[x_{k-1}]] / T_k).
//
// Sources: [V41] blog.javazero.top "DeepSeek-V4.1 模型结构（6）：解码，DSpark", "confidence head"
// (eq. (7): the input holds x_{k-1}, not x_k; no bias term); [ZDS] zdszero.github.io
// spec_dspark, "在 SGLang 里" (sigmoid(raw / T) with per-position STS temperatures).
#include "device.h"
#include "launch.h"

namespace dspark {

namespace {

// Confidence head: one 256-thread block per (request, position). The previous token goes out
// first, then its embedding-row pieces and the hidden-state pieces together, before any product
// is summed. Products in fp64, summed per thread in piece order (hidden state, then
// embedding row), then across the block in a fixed order.
__global__ __launch_bounds__(kBlock) void confidence_kernel(ConfArgs p) {
  __shared__ double red[kBlock / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int idx = blockIdx.x;
  const int b = idx / p.gamma, k = idx % p.gamma;
  const uint16_t* hrow = p.h + static_cast<size_t>(idx) * p.d;
  const int32_t prevtok = clamp_token(
      (k == 0) ? p.anchor[b] : p.tokens[static_cast<size_t>(b) * p.gamma + k - 1], p.V);
  constexpr int kBatch = 4;   // pieces of 8 per thread per batch: 8192 elements per batch
  const int nh = p.d / 8;     // hidden-state pieces
  const int ne = p.r / 8;     // embedding-row pieces (<= 64, one per thread)
  const float Tk = p.T[k];
  u16x8_t xv[kBatch], ww[kBatch];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int c = min(c0 + q * kBlock + tid, nh - 1);
      xv[q] = load_u16x8(hrow + 8 * c);
      ww[q] = load_u16x8(p.w + 8 * c);
    }
  };
  double acc = 0.0;
  auto sum_batch = [&](int c0) {
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (c0 + q * kBlock + tid >= nh) break;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        acc += static_cast<double>(bf16_to_f32(xv[q][e]) * bf16_to_f32(ww[q][e]));   // exact
    }
  };
  // The first batch (the only one for d <= 8192) and the embedding-row pieces: every load is
  // issued at the barrier; without it the compiler moves each pair into the guarded sum, one
  // round trip at a time.
  load_batch(0);
  u16x8_t ev = zero_u16x8(), we = zero_u16x8();
  if (tid < ne) {
    ev = load_u16x8(p.W1 + static_cast<size_t>(prevtok) * p.r + 8 * tid);
    we = load_u16x8(p.w + p.d + 8 * tid);
  }
  asm volatile("" ::: "memory");
  sum_batch(0);
  for (int c0 = kBlock * kBatch; c0 < nh; c0 += kBlock * kBatch) {
    load_batch(c0);
    asm volatile("" ::: "memory");
    sum_batch(c0);
  }
  if (tid < ne) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += static_cast<double>(bf16_to_f32(ev[e]) * bf16_to_f32(we[e]));
  }
  acc = wave_sum(acc);
  if (lane == 0) red[wv] = acc;
  __syncthreads();
  if (tid == 0) {
    const double z = (red[0] + red[1]) + (red[2] + red[3]);
    p.conf[idx] = static_cast<float>(1.0 / (1.0 + exp(-z / static_cast<double>(Tk))));
  }
}

}  // namespace

hipError_t launch_confidence(const ConfArgs& a, hipStream_t s) {
  launch_kernel(confidence_kernel, dim3(a.B * a.gamma), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark
