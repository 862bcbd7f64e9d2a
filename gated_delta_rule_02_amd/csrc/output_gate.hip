// output_gate.hip -- the gated output norm that follows the state read of a
// Gated DeltaNet layer ("Source notes", section "Linear attention", row gdn:
// the read-out is RMS-normalised, scaled by a learned gain and multiplied by
// a SiLU gate; "Adopt vs. port", entry burn-rmsnorm: the RMS norm divides by
// the square root of the mean of squares plus eps and multiplies by the
// gain).  For every (batch, token, value head) row of o, of DV channels:
//
//     y_c = o_c / sqrt((1/DV) sum_c' o_c'^2 + eps) * gain_c * z_c sigmoid(z_c)
//
// HBM-bound: 4 B of o, one z and one y element per channel.  NL = DV / 8
// lanes hold a row, 8 channels each (two runs of 4), so a 256-thread block
// covers 256 / NL rows.
//
// Channel order.  For DV >= 32, lane j = 4 w + g of a row holds channels
// 32 w + 4 g .. + 3 and 32 w + 16 + 4 g .. + 3.  The row's sum of squares is
// formed in a fixed tree: the lane's 8 squares in order, then
// (p_0 + p_1) + (p_2 + p_3) over g within each w, then the w in order.  That
// is the order of the gate inside the sequential chunked pass (a compute
// wave w of 32 value rows, its lane groups g holding 4 rows each, two row
// tiles of 16), so the two give the same bits.
#include <hip/hip_runtime.h>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kGateThreads = 256;

template <int DV, typename TZ, typename TY>
__global__ __launch_bounds__(kGateThreads) void output_gate_kernel(
    const float *__restrict__ o, const TZ *__restrict__ z, const float *__restrict__ gain, float eps,
    TY *__restrict__ y, long rows) {
  constexpr int NL = DV / 8;                      // lanes per row
  constexpr int NWR = DV >= 32 ? DV / 32 : 1;     // 32-channel groups of the row
  const long row = (long)blockIdx.x * (kGateThreads / NL) + threadIdx.x / NL;
  const int j = threadIdx.x % NL;
  if (row >= rows) return;   // a row's lanes leave together
  // this lane's two runs of 4 channels
  const int c0 = DV >= 32 ? 32 * (j >> 2) + 4 * (j & 3) : 8 * j;
  const int c1 = DV >= 32 ? c0 + 16 : c0 + 4;
  const size_t base = (size_t)row * DV;
  float x[8], zz[8], gw[8];
  {
    float a[4], b[4];
    load4(o + base + c0, a);
    load4(o + base + c1, b);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
    load4(z + base + c0, a);
    load4(z + base + c1, b);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      zz[i] = a[i];
      zz[4 + i] = b[i];
    }
    load4(gain + c0, a);
    load4(gain + c1, b);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gw[i] = a[i];
      gw[4 + i] = b[i];
    }
  }
  float p = gate_sumsq8(x);
  if constexpr (NL >= 2) p = p + __shfl_xor(p, 1, 64);
  if constexpr (NL >= 4) p = p + __shfl_xor(p, 2, 64);
  // the 32-channel groups in order (lane 4 w of the row holds group w)
  const int lane0 = (threadIdx.x & 63) - j;
  float tot = __shfl(p, lane0, 64);
#pragma unroll
  for (int w = 1; w < NWR; ++w) tot = tot + __shfl(p, lane0 + 4 * w, 64);
  const float inv = gate_inv_rms<DV>(tot, eps);
  float ya[4], yb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ya[i] = gate_apply(x[i], inv, gw[i], zz[i]);
    yb[i] = gate_apply(x[4 + i], inv, gw[4 + i], zz[4 + i]);
  }
  store4(y + base + c0, ya);
  store4(y + base + c1, yb);
}

template <int DV, typename TZ>
hipError_t launch_gate_dv(const float *o, const void *z, const float *gain, float eps, void *y,
                          DType yt, long rows, hipStream_t s) {
  constexpr int RPB = kGateThreads / (DV / 8);
  const long blocks = (rows + RPB - 1) / RPB;
  if (blocks > 0x7FFFFFFFL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(kGateThreads);
  switch (yt) {
    case DType::F32:
      hipLaunchKernelGGL((output_gate_kernel<DV, TZ, float>), grid, block, 0, s, o, (const TZ *)z, gain,
                         eps, (float *)y, rows);
      break;
    case DType::BF16:
      hipLaunchKernelGGL((output_gate_kernel<DV, TZ, bf16_t>), grid, block, 0, s, o, (const TZ *)z,
                         gain, eps, (bf16_t *)y, rows);
      break;
    default:
      hipLaunchKernelGGL((output_gate_kernel<DV, TZ, f16_t>), grid, block, 0, s, o, (const TZ *)z, gain,
                         eps, (f16_t *)y, rows);
      break;
  }
  return hipGetLastError();
}

template <typename TZ>
hipError_t launch_gate_z(const float *o, const void *z, const float *gain, float eps, void *y, DType yt,
                         long rows, int dv, hipStream_t s) {
  switch (dv) {
    case 16: return launch_gate_dv<16, TZ>(o, z, gain, eps, y, yt, rows, s);
    case 32: return launch_gate_dv<32, TZ>(o, z, gain, eps, y, yt, rows, s);
    case 64: return launch_gate_dv<64, TZ>(o, z, gain, eps, y, yt, rows, s);
    case 128: return launch_gate_dv<128, TZ>(o, z, gain, eps, y, yt, rows, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_output_gate(const float *o, const void *z, DType zt, const float *gain, float eps,
                              void *y, DType yt, long rows, int dv, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  switch (zt) {
    case DType::F32: return launch_gate_z<float>(o, z, gain, eps, y, yt, rows, dv, s);
    case DType::BF16: return launch_gate_z<bf16_t>(o, z, gain, eps, y, yt, rows, dv, s);
    default: return launch_gate_z<f16_t>(o, z, gain, eps, y, yt, rows, dv, s);
  }
}

}  // namespace gdn
