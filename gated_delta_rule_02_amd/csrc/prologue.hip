// prologue.hip -- 4-tap causal depthwise convolution, SiLU and per-head L2
// normalisation in front of the gated delta rule ("Source notes" page, section
// "Linear attention", rows deltanet/kda: causal conv + SiLU, L2-normalised
// Q/K; "Frontier model atlas" entries 03/08: four-token causal convolution).
//
//   y_t = w0 x_{t-3} + w1 x_{t-2} + w2 x_{t-1} + w3 x_t      (zero history)
//   z_t = y_t sigmoid(y_t);   q, k rows: z / sqrt(sum z^2 + eps)
//
// HBM-bound: every input element is read once and every output written once.
// A head row of d channels is held by d/8 lanes, 8 channels each, so one load
// is 16 bytes (bf16) per lane and the lanes of a wave cover 64/(d/8) adjacent
// heads of one token: contiguous memory.  Each wave walks a span of tokens,
// keeping the last three inputs of its channels in registers (the 3-token
// halo is re-read once per span), and issues the loads of kU tokens before
// computing them.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kSpan = 64;  // tokens per wave
constexpr int kU = 4;      // tokens loaded ahead

template <typename TX, typename TO, int D, bool L2>
__global__ __launch_bounds__(kThreads) void prologue_kernel(const TX *__restrict__ x,
                                                            const float *__restrict__ w,
                                                            TO *__restrict__ y, int T, int H,
                                                            float eps) {
  constexpr int LPR = D / 8;               // lanes per head row
  constexpr int HPB = kThreads / LPR;      // heads per block
  const int nspan = (T + kSpan - 1) / kSpan;
  const int b = blockIdx.x / nspan;
  const int t0 = (blockIdx.x % nspan) * kSpan;
  const int head = blockIdx.y * HPB + threadIdx.x / LPR;
  if (head >= H) return;  // whole lane groups leave together
  const int c0 = (threadIdx.x % LPR) * 8;

  float w0[8], w1[8], w2[8], w3[8];
  {
    const float4 *wp = reinterpret_cast<const float4 *>(w + ((size_t)head * D + c0) * 4);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float4 t = wp[c];
      w0[c] = t.x; w1[c] = t.y; w2[c] = t.z; w3[c] = t.w;
    }
  }
  const size_t tok_stride = (size_t)H * D;
  const TX *xb = x + (size_t)b * T * tok_stride + (size_t)head * D + c0;
  TO *yb = y + (size_t)b * T * tok_stride + (size_t)head * D + c0;

  float xm3[8], xm2[8], xm1[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) xm3[c] = xm2[c] = xm1[c] = 0.f;
  if (t0 >= 3) load8(xb + (size_t)(t0 - 3) * tok_stride, xm3);
  if (t0 >= 2) load8(xb + (size_t)(t0 - 2) * tok_stride, xm2);
  if (t0 >= 1) load8(xb + (size_t)(t0 - 1) * tok_stride, xm1);

  const int t_end = min(T, t0 + kSpan);
  for (int t = t0; t < t_end; t += kU) {
    float xs[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (t + u < t_end) {
        load8(xb + (size_t)(t + u) * tok_stride, xs[u]);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) xs[u][c] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float z[8];
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float yv = w0[c] * xm3[c] + w1[c] * xm2[c] + w2[c] * xm1[c] + w3[c] * xs[u][c];
        z[c] = yv / (1.0f + __expf(-yv));
        ss += z[c] * z[c];
        xm3[c] = xm2[c];
        xm2[c] = xm1[c];
        xm1[c] = xs[u][c];
      }
      if constexpr (L2) {
        ss = group_sum<LPR>(ss);
        const float inv = rsqrtf(ss + eps);
#pragma unroll
        for (int c = 0; c < 8; ++c) z[c] *= inv;
      }
      if (t + u < t_end) store8(yb + (size_t)(t + u) * tok_stride, z);
    }
  }
}

template <typename TX, typename TO, int D>
hipError_t launch_d(const void *x, const float *w, void *y, int B, int T, int H, bool l2, float eps,
                    hipStream_t st) {
  constexpr int HPB = kThreads / (D / 8);
  const int nspan = (T + kSpan - 1) / kSpan;
  dim3 grid(B * nspan, (H + HPB - 1) / HPB);
  if (l2)
    hipLaunchKernelGGL((prologue_kernel<TX, TO, D, true>), grid, dim3(kThreads), 0, st,
                       (const TX *)x, w, (TO *)y, T, H, eps);
  else
    hipLaunchKernelGGL((prologue_kernel<TX, TO, D, false>), grid, dim3(kThreads), 0, st,
                       (const TX *)x, w, (TO *)y, T, H, eps);
  return hipGetLastError();
}

template <typename TX, typename TO>
hipError_t launch_xo(const void *x, const float *w, void *y, int B, int T, int H, int d, bool l2,
                     float eps, hipStream_t st) {
  switch (d) {
    case 16: return launch_d<TX, TO, 16>(x, w, y, B, T, H, l2, eps, st);
    case 32: return launch_d<TX, TO, 32>(x, w, y, B, T, H, l2, eps, st);
    case 64: return launch_d<TX, TO, 64>(x, w, y, B, T, H, l2, eps, st);
    case 128: return launch_d<TX, TO, 128>(x, w, y, B, T, H, l2, eps, st);
  }
  return hipErrorInvalidValue;
}

template <typename TX>
hipError_t launch_x(const void *x, const float *w, void *y, DType yt, int B, int T, int H, int d,
                    bool l2, float eps, hipStream_t st) {
  switch (yt) {
    case DType::F32: return launch_xo<TX, float>(x, w, y, B, T, H, d, l2, eps, st);
    case DType::BF16: return launch_xo<TX, bf16_t>(x, w, y, B, T, H, d, l2, eps, st);
    case DType::F16: return launch_xo<TX, f16_t>(x, w, y, B, T, H, d, l2, eps, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prologue(const void *x, DType xt, const float *w, void *y, DType yt, int B, int T,
                           int H, int d, bool l2, float eps, hipStream_t st) {
  if (xt == DType::BF16) return launch_x<bf16_t>(x, w, y, yt, B, T, H, d, l2, eps, st);
  if (xt == DType::F32) return launch_x<float>(x, w, y, yt, B, T, H, d, l2, eps, st);
  return hipErrorInvalidValue;
}

}  // namespace gdn
