// decode.hip -- one-token decode step of the gated delta rule on gfx950.
//
// Per (batch b, value head h) and state row i (the recurrence of the "Source
// notes" page, section "Linear attention", rows gdn / kda, with T = 1):
//     D_i = alpha S_i            (key-channel gate: S_i o alpha, alpha a dk-vector)
//     a   = D_i . k,  c = D_i . q
//     u   = beta (v_i - a)
//     S_i <- D_i + u k,    o_i = c + u (k . q)        (= S_i(new) . q)
// The new row's read o_i = S_i(new) . q is expanded so that both dot products
// are reduced from the old row in one pass: the state is read once and written
// once, which is all the HBM traffic this step needs.
//
// Mapping: a row of dk fp32 values is held by dk/8 lanes, 8 values each: lane
// j of the row holds columns 4j .. 4j+3 and dk/2 + 4j .. dk/2 + 4j+3, so each
// of its two 16-byte accesses is part of one contiguous run across the lanes.
// A 512-thread block covers 512/(dk/8) rows (32 at dk = 128, 16 lanes a row); many such
// blocks keep enough loads in flight (512 threads: 248 against 251 us per step at
// 256 threads and 250 at 1024 on the batched-decode workload).  The state is streamed with
// non-temporal loads and stores: it is touched once per step.  Row dot
// products are reduced across the dk/8 lanes of the row with xor shuffles.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kThreads = 512;

// Four consecutive values widened to fp32.
__device__ __forceinline__ void load4(const float *p, float *x) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}
__device__ __forceinline__ void load4(const f16_t *p, float *x) {
  const half4 h = *reinterpret_cast<const half4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = (float)h[i];
}
__device__ __forceinline__ void load4(const bf16_t *p, float *x) {
  const uint2 u = *reinterpret_cast<const uint2 *>(p);
  x[0] = __uint_as_float(u.x << 16); x[1] = __uint_as_float(u.x & 0xFFFF0000u);
  x[2] = __uint_as_float(u.y << 16); x[3] = __uint_as_float(u.y & 0xFFFF0000u);
}
// Columns c0 .. c0+3 and DK/2 + c0 .. DK/2 + c0+3 of a row.
template <int DK, typename T>
__device__ __forceinline__ void load_cols(const T *row, int c0, float (&x)[8]) {
  load4(row + c0, x);
  load4(row + DK / 2 + c0, x + 4);
}

template <typename TQ, typename TG, bool KEYGATE, int DK, int NR>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    const TQ *__restrict__ q, const TQ *__restrict__ k, const TQ *__restrict__ v,
    const TG *__restrict__ g, const TG *__restrict__ beta, float *__restrict__ S,
    float *__restrict__ o, int Hk, int Hv, int dv, int nodelta) {
  constexpr int LPR = DK / 8;          // lanes per state row
  constexpr int RPP = kThreads / LPR;  // rows per pass
  const int b = blockIdx.z, h = blockIdx.y;
  const int kh = h / (Hv / Hk);
  const int sub = threadIdx.x % LPR;
  const int c0 = sub * 4;
  const size_t bh = (size_t)b * Hv + h;

  float kk[8], qq[8], al[8];
  load_cols<DK>(k + ((size_t)b * Hk + kh) * DK, c0, kk);
  load_cols<DK>(q + ((size_t)b * Hk + kh) * DK, c0, qq);
  if constexpr (KEYGATE) {
    load_cols<DK>(g + bh * DK, c0, al);
#pragma unroll
    for (int j = 0; j < 8; ++j) al[j] = __expf(al[j]);
  } else {
    const float a = __expf(to_f32(g[bh]));
#pragma unroll
    for (int j = 0; j < 8; ++j) al[j] = a;
  }
  const float bt = to_f32(beta[bh]);
  float kq = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) kq += kk[j] * qq[j];
  kq = group_sum<LPR>(kq);

  const int row0 = blockIdx.x * (NR * RPP) + threadIdx.x / LPR;
  float *Sbh = S + bh * (size_t)dv * DK;
  float4v s[NR][2];
#pragma unroll
  for (int p = 0; p < NR; ++p) {
    const int i = row0 + p * RPP;
    if (i < dv) {
      const float *r = Sbh + (size_t)i * DK + c0;
      s[p][0] = __builtin_nontemporal_load(reinterpret_cast<const float4v *>(r));
      s[p][1] = __builtin_nontemporal_load(reinterpret_cast<const float4v *>(r + DK / 2));
    } else {
      s[p][0] = s[p][1] = float4v{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int p = 0; p < NR; ++p) {
    const int i = row0 + p * RPP;
    float a = 0.f, c = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = s[p][j >> 2][j & 3] * al[j];
      s[p][j >> 2][j & 3] = x;
      a += x * kk[j];
      c += x * qq[j];
    }
    a = group_sum<LPR>(a);
    c = group_sum<LPR>(c);
    if (i < dv) {
      // without the delta correction the write is beta v
      const float u = bt * (to_f32(v[bh * dv + i]) - (nodelta ? 0.f : a));
#pragma unroll
      for (int j = 0; j < 8; ++j) s[p][j >> 2][j & 3] += u * kk[j];
      float *r = Sbh + (size_t)i * DK + c0;
      __builtin_nontemporal_store(s[p][0], reinterpret_cast<float4v *>(r));
      __builtin_nontemporal_store(s[p][1], reinterpret_cast<float4v *>(r + DK / 2));
      if (sub == 0) o[bh * dv + i] = c + u * kq;
    }
  }
}

template <typename TQ, typename TG, bool KEYGATE, int DK>
hipError_t launch_dk(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                     const void *beta, float *S, float *o, hipStream_t st) {
  constexpr int NR = 1;
  constexpr int rows_per_block = NR * (kThreads / (DK / 8));
  dim3 grid((sh.dv + rows_per_block - 1) / rows_per_block, sh.Hv, sh.B);
  hipLaunchKernelGGL((decode_kernel<TQ, TG, KEYGATE, DK, NR>), grid, dim3(kThreads), 0, st,
                     (const TQ *)q, (const TQ *)k, (const TQ *)v, (const TG *)g, (const TG *)beta, S,
                     o, sh.Hk, sh.Hv, sh.dv, sh.no_delta ? 1 : 0);
  return hipGetLastError();
}

template <typename TQ, typename TG, bool KEYGATE>
hipError_t launch_gate(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                       const void *beta, float *S, float *o, hipStream_t st) {
  switch (sh.dk) {
    case 16: return launch_dk<TQ, TG, KEYGATE, 16>(sh, q, k, v, g, beta, S, o, st);
    case 32: return launch_dk<TQ, TG, KEYGATE, 32>(sh, q, k, v, g, beta, S, o, st);
    case 64: return launch_dk<TQ, TG, KEYGATE, 64>(sh, q, k, v, g, beta, S, o, st);
    case 128: return launch_dk<TQ, TG, KEYGATE, 128>(sh, q, k, v, g, beta, S, o, st);
  }
  return hipErrorInvalidValue;
}

template <typename TQ, typename TG>
hipError_t launch_tg(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                     const void *beta, float *S, float *o, hipStream_t st) {
  return sh.key_gate ? launch_gate<TQ, TG, true>(sh, q, k, v, g, beta, S, o, st)
                     : launch_gate<TQ, TG, false>(sh, q, k, v, g, beta, S, o, st);
}

template <typename TQ>
hipError_t launch_tq(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                     const void *beta, float *S, float *o, hipStream_t st) {
  return sh.gate_t == DType::F32 ? launch_tg<TQ, float>(sh, q, k, v, g, beta, S, o, st)
                                 : launch_tg<TQ, bf16_t>(sh, q, k, v, g, beta, S, o, st);
}

}  // namespace

hipError_t launch_decode(const Shape &sh, const void *q, const void *k, const void *v,
                         const void *g, const void *beta, float *S, float *o, hipStream_t st) {
  switch (sh.qkv) {
    case DType::F32: return launch_tq<float>(sh, q, k, v, g, beta, S, o, st);
    case DType::BF16: return launch_tq<bf16_t>(sh, q, k, v, g, beta, S, o, st);
    case DType::F16: return launch_tq<f16_t>(sh, q, k, v, g, beta, S, o, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
