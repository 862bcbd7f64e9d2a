// gdn_device.h -- device helpers shared by the gfx950 kernels: storage types,
// exact widening to fp32, round-to-nearest-even narrowing, vector loads and
// stores, wave-level sums over aligned lane groups, and the arithmetic of the
// convolution and of the gated output norm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Storage types.  bf16 is carried as its 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};
using f16_t = _Float16;

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(f16_t x) { return (float)x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float((uint32_t)x.bits << 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float x) { return (f16_t)x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  // round to nearest even (the gfx950 conversion instruction)
  bf16_t r;
  r.bits = __builtin_bit_cast(uint16_t, (__bf16)x);
  return r;
}

// Load 8 consecutive elements (16-byte aligned for 2-byte types, 32-byte for
// fp32) and widen to fp32.
__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const f16_t *p, float (&x)[8]) {
  const half8 h = *reinterpret_cast<const half8 *>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)h[i];
}
__device__ __forceinline__ void load8(const bf16_t *p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// Narrow 8 fp32 values and store them (16-byte aligned for 2-byte types).
__device__ __forceinline__ void store8(float *p, const float (&x)[8]) {
  *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4 *>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void store8(f16_t *p, const float (&x)[8]) {
  half8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (f16_t)x[i];
  *reinterpret_cast<half8 *>(p) = h;
}
__device__ __forceinline__ void store8(bf16_t *p, const float (&x)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)from_f32<bf16_t>(x[2 * i]).bits |
           ((uint32_t)from_f32<bf16_t>(x[2 * i + 1]).bits << 16);
  *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

// The token sequences of a call: B sequences of T tokens each (cu null), or
// B sequences packed one after another, sequence s being tokens
// cu[s] .. cu[s + 1] - 1 of the T.  The offsets are read on the device: each
// is clamped to [0, T] and a sequence whose end precedes its start is empty,
// so that no access leaves the tensors whatever the offsets hold.
struct Seqs {
  const int *cu;
  int B;
  const int *order = nullptr;   // the sequences, longest first (sequential pass)
};
__device__ __forceinline__ void seq_bounds(const Seqs &sq, int s, int T, int &start, int &len) {
  if (!sq.cu) {
    start = s * T;   // B * T < 2^31 (checked on the host)
    len = T;
    return;
  }
  const int a = min(max(sq.cu[s], 0), T), e = min(max(sq.cu[s + 1], a), T);
  start = a;
  len = e - a;
}
// Packed sequences keep the work units of G tokens of sequence s in the slots
// cu[s] / G + s + j, j < ceil(len / G): distinct for valid offsets, and below
// T / G + B for any.  seq_of_slot gives the sequence of a slot, its unit
// index and bounds, or -1 when no unit of any sequence is there.
__host__ __device__ __forceinline__ int packed_slots(int T, int B, int G) { return T / G + B; }
template <int G>
__device__ __forceinline__ int seq_of_slot(const Seqs &sq, int T, int slot, int &unit, int &start, int &len) {
  int lo = 0, hi = sq.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (min(max(sq.cu[mid], 0), T) / G + mid <= slot)
      lo = mid;
    else
      hi = mid - 1;
  }
  seq_bounds(sq, lo, T, start, len);
  unit = slot - (start / G + lo);
  return unit >= 0 && unit * G < len ? lo : -1;
}

// Workgroup barrier for hand-offs through LDS only: waits for this wave's
// LDS operations, then for the other waves.  Unlike __syncthreads(), it does
// not drain the wave's outstanding global loads and stores, so prefetches and
// output stores stay in flight across it.  Use it only where no other wave
// reads global memory this wave wrote.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// x plus the value of another lane of its 16-lane row, moved by DPP: ctrl is
// a gfx9 DPP control (quad permutation, row mirror, row half-mirror).
template <int CTRL> __device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over an aligned group of G lanes (G a power of two <= 64); every lane
// of the group receives the total.  Groups of up to 16 lanes reduce with DPP
// moves inside the row (quad swaps, then the half-row and row mirrors, each
// pairing lanes whose partial sums cover disjoint halves); wider groups add
// cross-row shuffles.
template <int G> __device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 2) x = dpp_add<0xB1>(x);    // quad_perm [1,0,3,2]
  if constexpr (G >= 4) x = dpp_add<0x4E>(x);    // quad_perm [2,3,0,1]
  if constexpr (G >= 8) x = dpp_add<0x141>(x);   // row_half_mirror
  if constexpr (G >= 16) x = dpp_add<0x140>(x);  // row_mirror
#pragma unroll
  for (int m = 16; m < G; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// x as computed in fp32.  The empty asm statement emits nothing; it only hides
// how x was made, so that the compiler cannot merge that operation with a
// narrowing conversion that follows (a mixed-precision fma rounds once where
// a product and a conversion round twice).  Every kernel then narrows the
// value the same way.
__device__ __forceinline__ float fp32_value(float x) {
  asm("" : "+v"(x));
  return x;
}

// Causal 4-tap depthwise convolution and SiLU of 8 channels at one token:
// x3, x2, x1 hold the inputs 3, 2 and 1 tokens back, x0 the current token's,
// w0..w3 the taps (w3 multiplies the current token).  Writes z = y sigmoid(y)
// and returns the sum of z^2 over the 8 channels.  Every kernel that applies
// the convolution calls this one function, every multiply-add in it is an
// explicit fma (the compiler may not choose which products to fuse) and z
// leaves it as an fp32 value, so they all round identically.
__device__ __forceinline__ float conv_silu8(const float (&w0)[8], const float (&w1)[8],
                                            const float (&w2)[8], const float (&w3)[8],
                                            const float (&x3)[8], const float (&x2)[8],
                                            const float (&x1)[8], const float (&x0)[8],
                                            float (&z)[8]) {
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float yv = __builtin_fmaf(w3[c], x0[c], __builtin_fmaf(w2[c], x1[c], __builtin_fmaf(w1[c], x2[c], w0[c] * x3[c])));
    z[c] = fp32_value(yv * __builtin_amdgcn_rcpf(1.0f + __expf(-yv)));   // SiLU; rcp is exact to 1 ulp
    ss = __builtin_fmaf(z[c], z[c], ss);
  }
  return ss;
}

// L2 normalisation of a head row of G * 8 channels held 8 per lane by an
// aligned group of G lanes: z / sqrt(sum z^2 + eps).
template <int G>
__device__ __forceinline__ void l2_scale8(float (&z)[8], float ss, float eps) {
  ss = group_sum<G>(ss);
  const float inv = rsqrtf(ss + eps);
#pragma unroll
  for (int c = 0; c < 8; ++c) z[c] = fp32_value(z[c] * inv);
}

// The gated output norm y = o / sqrt(mean(o^2) + eps) * gain * z sigmoid(z)
// over a row of DV channels, in the steps every kernel that applies it
// shares, so that they all round identically:
//  - gate_sumsq8: the sum of squares of 8 of the row's values, in a fixed
//    order (the caller combines such partial sums over lanes and waves in a
//    fixed tree);
//  - gate_inv_rms: 1 / sqrt(sum / DV + eps) from the row's sum of squares;
//  - gate_apply: ((o * inv) * gain) * silu(z), as an fp32 value.
__device__ __forceinline__ float gate_sumsq8(const float (&x)[8]) {
  float s = x[0] * x[0];
#pragma unroll
  for (int c = 1; c < 8; ++c) s = __builtin_fmaf(x[c], x[c], s);
  return s;
}
template <int DV> __device__ __forceinline__ float gate_inv_rms(float ss, float eps) {
  return rsqrtf(fp32_value(__builtin_fmaf(ss, 1.0f / DV, eps)));
}
__device__ __forceinline__ float gate_apply(float o, float inv, float gain, float z) {
  const float s = fp32_value(z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)));   // SiLU
  return fp32_value(fp32_value(fp32_value(o * inv) * gain) * s);
}

// Narrow 4 fp32 values and store them (16-byte aligned for fp32, 8-byte for
// 2-byte types).
__device__ __forceinline__ void store4(float *p, const float (&x)[4]) {
  *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store4(f16_t *p, const float (&x)[4]) {
  half4 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = (f16_t)x[i];
  *reinterpret_cast<half4 *>(p) = h;
}
__device__ __forceinline__ void store4(bf16_t *p, const float (&x)[4]) {
  uint32_t w[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    w[i] = (uint32_t)from_f32<bf16_t>(x[2 * i]).bits |
           ((uint32_t)from_f32<bf16_t>(x[2 * i + 1]).bits << 16);
  *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
}

// 4 fp32 values as 4 bf16 or fp16 (round to nearest even) in 8 bytes.
__device__ __forceinline__ uint2 pack4_bf16(const float (&x)[4]) {
  return make_uint2((uint32_t)from_f32<bf16_t>(x[0]).bits | ((uint32_t)from_f32<bf16_t>(x[1]).bits << 16),
                    (uint32_t)from_f32<bf16_t>(x[2]).bits | ((uint32_t)from_f32<bf16_t>(x[3]).bits << 16));
}
__device__ __forceinline__ uint2 pack4_f16(const float (&x)[4]) {
  const half4 h = {(f16_t)x[0], (f16_t)x[1], (f16_t)x[2], (f16_t)x[3]};
  return __builtin_bit_cast(uint2, h);
}

// Load 4 consecutive elements (8-byte aligned for 2-byte types, 16-byte for
// fp32) and widen to fp32.
__device__ __forceinline__ void load4(const float *p, float (&x)[4]) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}
__device__ __forceinline__ void load4(const f16_t *p, float (&x)[4]) {
  const half4 h = *reinterpret_cast<const half4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = (float)h[i];
}
__device__ __forceinline__ void load4(const bf16_t *p, float (&x)[4]) {
  const uint2 u = *reinterpret_cast<const uint2 *>(p);
  x[0] = __uint_as_float(u.x << 16);
  x[1] = __uint_as_float(u.x & 0xFFFF0000u);
  x[2] = __uint_as_float(u.y << 16);
  x[3] = __uint_as_float(u.y & 0xFFFF0000u);
}

// Inclusive prefix sum over the 64 lanes of a wave by DPP moves: shifts by
// 1, 2, 4, 8 within each 16-lane row (lanes shifted in from outside the row
// add zero), then the last lane of row 0 (row 2) is broadcast into row 1
// (row 3), and lane 31 into rows 2 and 3.  All lanes must be active.
template <int CTRL, int ROW_MASK, bool BOUND> __device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, BOUND));
}
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x += dpp_mov<0x111, 0xF, true>(x);   // row_shr:1
  x += dpp_mov<0x112, 0xF, true>(x);   // row_shr:2
  x += dpp_mov<0x114, 0xF, true>(x);   // row_shr:4
  x += dpp_mov<0x118, 0xF, true>(x);   // row_shr:8
  x += dpp_mov<0x142, 0xA, false>(x);  // row_bcast:15 -> rows 1, 3
  x += dpp_mov<0x143, 0xC, false>(x);  // row_bcast:31 -> rows 2, 3
  return x;
}

}  // namespace gdn
