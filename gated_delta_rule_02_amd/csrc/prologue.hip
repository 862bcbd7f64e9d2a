// prologue.hip -- 4-tap causal depthwise convolution, SiLU and per-head L2
// normalisation in front of the gated delta rule ("Source notes" page, section
// "Linear attention", rows deltanet/kda: causal conv + SiLU, L2-normalised
// Q/K; "Frontier model atlas" entries 03/08: four-token causal convolution).
//
//   y_t = w0 x_{t-3} + w1 x_{t-2} + w2 x_{t-1} + w3 x_t      (zero history)
//   z_t = y_t sigmoid(y_t);   q, k rows: z / sqrt(sum z^2 + eps)
//
// HBM-bound: every input element is read once (plus a 3-token halo per span)
// and every output written once.  One launch covers the q, k and v head rows
// together: a head row of d channels is held by d/8 lanes, 8 channels each,
// so one load is 16 bytes (bf16) per lane; each lane group walks a span of
// kSpan tokens of its head row, keeping the last three inputs in registers;
// the loads of the next kU tokens are in flight while the current ones are
// computed and stored.  Packed sequences of different lengths: a block takes
// a span of one sequence (the history before a sequence's first token is
// zero), found from the sequence offsets.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kSpan = 16;  // tokens per lane group
constexpr int kU = 4;      // tokens loaded ahead

struct ProTensor {
  const void *x;
  const float *w;  // [H*d][4]
  void *y;
  int H;
  bool l2;
  int choff;       // first channel in the concatenation q | k | v
};
struct ProArgs {
  ProTensor t[3];
  int B, T;
  float eps;
  Seqs sq;         // packed sequences (sq.cu), or B sequences of T tokens
  void *cs;        // convolution history [B][3][nch] (raw input type)
  int nch;         // channels of q | k | v
};

// Eight input channels as loaded (16 bytes of bf16, 32 of fp32), widened
// only where they are used, so that a load in flight holds no conversion.
template <typename TX>
struct Raw8 {
  uint4 v[sizeof(TX) / 2];
};
template <typename TX>
__device__ __forceinline__ Raw8<TX> load_raw8(const TX *p) {
  Raw8<TX> r;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(TX) / 2); ++i) r.v[i] = reinterpret_cast<const uint4 *>(p)[i];
  return r;
}
__device__ __forceinline__ void widen8(const Raw8<bf16_t> &r, float (&x)[8]) {
  const uint32_t w[4] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void widen8(const Raw8<float> &r, float (&x)[8]) {
  const uint32_t w[8] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w, r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w};
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = __uint_as_float(w[i]);
}

template <typename TX, typename TO, int D>
__global__ __launch_bounds__(kThreads) void prologue_kernel(ProArgs a) {
  constexpr int LPR = D / 8;                 // lanes per head row
  constexpr int RPB = kThreads / LPR;        // head rows per block
  // block -> (span, group of RPB rows of the concatenated q | k | v head
  // list); packed sequences: span slots, each a span of one sequence
  const int nspan = a.sq.cu ? packed_slots(a.T, a.B, kSpan) : (a.T + kSpan - 1) / kSpan;
  const int slot = blockIdx.x % nspan;
  const int bg = blockIdx.x / nspan;         // over B * ceil(rows / RPB), or ceil(rows / RPB)
  const int nrows = a.t[0].H + a.t[1].H + a.t[2].H;
  const int ngroups = (nrows + RPB - 1) / RPB;
  int b, span, start, T;
  if (a.sq.cu) {
    b = seq_of_slot<kSpan>(a.sq, a.T, slot, span, start, T);
    if (b < 0) return;
  } else {
    b = bg / ngroups;
    span = slot;
    seq_bounds(a.sq, b, a.T, start, T);
  }
  const int row = (bg % ngroups) * RPB + threadIdx.x / LPR;
  if (row >= nrows) return;  // whole lane groups leave together
  int ti = 0, head = row;
  if (head >= a.t[0].H) { head -= a.t[0].H; ti = 1; }
  if (ti == 1 && head >= a.t[1].H) { head -= a.t[1].H; ti = 2; }
  const ProTensor P = ti == 0 ? a.t[0] : (ti == 1 ? a.t[1] : a.t[2]);
  const int c0 = (threadIdx.x % LPR) * 8;
  const int t0 = span * kSpan;

  float w0[8], w1[8], w2[8], w3[8];
  {
    const float4 *wp = reinterpret_cast<const float4 *>(P.w + ((size_t)head * D + c0) * 4);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float4 t = wp[c];
      w0[c] = t.x; w1[c] = t.y; w2[c] = t.z; w3[c] = t.w;
    }
  }
  const size_t tok_stride = (size_t)P.H * D;
  const TX *xb = reinterpret_cast<const TX *>(P.x) + (size_t)start * tok_stride + (size_t)head * D + c0;
  TO *yb = reinterpret_cast<TO *>(P.y) + (size_t)start * tok_stride + (size_t)head * D + c0;

  float xm3[8], xm2[8], xm1[8];
  if (t0 >= 3 && t0 + kSpan <= T) {
    // A whole span with its whole history: the loads of the next kU tokens
    // are issued before the current ones are computed and stored, and every
    // store is unconditional, so each wait is for loads alone (one counter
    // tracks loads and stores in issue order).
    widen8(load_raw8(xb + (size_t)(t0 - 3) * tok_stride), xm3);
    widen8(load_raw8(xb + (size_t)(t0 - 2) * tok_stride), xm2);
    widen8(load_raw8(xb + (size_t)(t0 - 1) * tok_stride), xm1);
    Raw8<TX> cur[kU], nxt[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) cur[u] = load_raw8(xb + (size_t)(t0 + u) * tok_stride);
#pragma unroll
    for (int it = 0; it < kSpan / kU; ++it) {
      const int t = t0 + it * kU;
      if (it + 1 < kSpan / kU) {
#pragma unroll
        for (int u = 0; u < kU; ++u) nxt[u] = load_raw8(xb + (size_t)(t + kU + u) * tok_stride);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        float x0[8], z[8];
        widen8(cur[u], x0);
        const float ss = conv_silu8(w0, w1, w2, w3, xm3, xm2, xm1, x0, z);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          xm3[c] = xm2[c];
          xm2[c] = xm1[c];
          xm1[c] = x0[c];
        }
        if (P.l2) l2_scale8<LPR>(z, ss, a.eps);
        store8(yb + (size_t)(t + u) * tok_stride, z);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) cur[u] = nxt[u];
    }
    return;
  }
  // the first span of a sequence, or its last when it is cut short
#pragma unroll
  for (int c = 0; c < 8; ++c) xm3[c] = xm2[c] = xm1[c] = 0.f;
  if (t0 >= 3) load8(xb + (size_t)(t0 - 3) * tok_stride, xm3);
  if (t0 >= 2) load8(xb + (size_t)(t0 - 2) * tok_stride, xm2);
  if (t0 >= 1) load8(xb + (size_t)(t0 - 1) * tok_stride, xm1);

  const int t_end = min(T, t0 + kSpan);
  for (int t = t0; t < t_end; t += kU) {
    float xs[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u) load8(xb + (size_t)min(t + u, t_end - 1) * tok_stride, xs[u]);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float z[8];
      const float ss = conv_silu8(w0, w1, w2, w3, xm3, xm2, xm1, xs[u], z);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        xm3[c] = xm2[c];
        xm2[c] = xm1[c];
        xm1[c] = xs[u][c];
      }
      if (P.l2) l2_scale8<LPR>(z, ss, a.eps);
      if (t + u < t_end) store8(yb + (size_t)(t + u) * tok_stride, z);
    }
  }
}

// One token per sequence continuing from a convolution history: the
// history cs[b][j] holds the raw inputs of tokens t - 3 + j.  The token's
// q, k, v are made exactly as the prologue makes them (the same functions),
// and the history moves on by one token (each lane owns its 8 channels).
template <typename TX, typename TO, int D>
__global__ __launch_bounds__(kThreads) void decode_prologue_kernel(ProArgs a) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kThreads / LPR;
  const int nrows = a.t[0].H + a.t[1].H + a.t[2].H;
  const int ngroups = (nrows + RPB - 1) / RPB;
  const int b = blockIdx.x / ngroups;
  const int row = (blockIdx.x % ngroups) * RPB + threadIdx.x / LPR;
  if (row >= nrows) return;  // whole lane groups leave together
  int ti = 0, head = row;
  if (head >= a.t[0].H) { head -= a.t[0].H; ti = 1; }
  if (ti == 1 && head >= a.t[1].H) { head -= a.t[1].H; ti = 2; }
  const ProTensor P = ti == 0 ? a.t[0] : (ti == 1 ? a.t[1] : a.t[2]);
  const int c0 = (threadIdx.x % LPR) * 8;
  float w0[8], w1[8], w2[8], w3[8];
  {
    const float4 *wp = reinterpret_cast<const float4 *>(P.w + ((size_t)head * D + c0) * 4);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float4 t = wp[c];
      w0[c] = t.x; w1[c] = t.y; w2[c] = t.z; w3[c] = t.w;
    }
  }
  TX *cs = reinterpret_cast<TX *>(a.cs) + (size_t)b * 3 * a.nch + P.choff + (size_t)head * D + c0;
  const size_t at = ((size_t)b * P.H + head) * D + c0;
  const Raw8<TX> h3 = load_raw8(cs), h2 = load_raw8(cs + a.nch), h1 = load_raw8(cs + 2 * a.nch);
  const Raw8<TX> xr = load_raw8(reinterpret_cast<const TX *>(P.x) + at);
  float xm3[8], xm2[8], xm1[8], x0[8], z[8];
  widen8(h3, xm3);
  widen8(h2, xm2);
  widen8(h1, xm1);
  widen8(xr, x0);
  const float ss = conv_silu8(w0, w1, w2, w3, xm3, xm2, xm1, x0, z);
  if (P.l2) l2_scale8<LPR>(z, ss, a.eps);
  store8(reinterpret_cast<TO *>(P.y) + at, z);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(TX) / 2); ++i) {
    reinterpret_cast<uint4 *>(cs)[i] = h2.v[i];
    reinterpret_cast<uint4 *>(cs + a.nch)[i] = h1.v[i];
    reinterpret_cast<uint4 *>(cs + 2 * a.nch)[i] = xr.v[i];
  }
}

// The convolution history after the last token of each sequence: the raw
// inputs of its last three tokens (zero before its first).
template <typename TX, int D>
__global__ __launch_bounds__(kThreads) void conv_state_kernel(ProArgs a) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kThreads / LPR;
  const int nrows = a.t[0].H + a.t[1].H + a.t[2].H;
  const int ngroups = (nrows + RPB - 1) / RPB;
  const int b = blockIdx.x / ngroups;
  const int row = (blockIdx.x % ngroups) * RPB + threadIdx.x / LPR;
  if (row >= nrows) return;
  int ti = 0, head = row;
  if (head >= a.t[0].H) { head -= a.t[0].H; ti = 1; }
  if (ti == 1 && head >= a.t[1].H) { head -= a.t[1].H; ti = 2; }
  const ProTensor P = ti == 0 ? a.t[0] : (ti == 1 ? a.t[1] : a.t[2]);
  const int c0 = (threadIdx.x % LPR) * 8;
  int start, T;
  seq_bounds(a.sq, b, a.T, start, T);
  TX *cs = reinterpret_cast<TX *>(a.cs) + (size_t)b * 3 * a.nch + P.choff + (size_t)head * D + c0;
  const TX *xb = reinterpret_cast<const TX *>(P.x) + (size_t)start * P.H * D + (size_t)head * D + c0;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int t = T - 3 + j;
    Raw8<TX> r;
    if (t >= 0) {
      r = load_raw8(xb + (size_t)t * P.H * D);
    } else {
#pragma unroll
      for (int i = 0; i < (int)(sizeof(TX) / 2); ++i) r.v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < (int)(sizeof(TX) / 2); ++i) reinterpret_cast<uint4 *>(cs + (size_t)j * a.nch)[i] = r.v[i];
  }
}

template <typename TX, typename TO, int D>
hipError_t launch_d(const ProArgs &a, hipStream_t st) {
  constexpr int RPB = kThreads / (D / 8);
  const int nspan = a.sq.cu ? packed_slots(a.T, a.B, kSpan) : (a.T + kSpan - 1) / kSpan;
  const int nrows = a.t[0].H + a.t[1].H + a.t[2].H;
  const long blocks = (long)nspan * (a.sq.cu ? 1 : a.B) * ((nrows + RPB - 1) / RPB);
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prologue_kernel<TX, TO, D>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <typename TX, typename TO>
hipError_t launch_xo(const ProArgs &a, int d, hipStream_t st) {
  switch (d) {
    case 16: return launch_d<TX, TO, 16>(a, st);
    case 32: return launch_d<TX, TO, 32>(a, st);
    case 64: return launch_d<TX, TO, 64>(a, st);
    case 128: return launch_d<TX, TO, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename TX>
hipError_t launch_x(const ProArgs &a, DType yt, int d, hipStream_t st) {
  switch (yt) {
    case DType::F32: return launch_xo<TX, float>(a, d, st);
    case DType::BF16: return launch_xo<TX, bf16_t>(a, d, st);
    case DType::F16: return launch_xo<TX, f16_t>(a, d, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_one(const ProArgs &a, DType xt, DType yt, int d, hipStream_t st) {
  if (xt == DType::BF16) return launch_x<bf16_t>(a, yt, d, st);
  if (xt == DType::F32) return launch_x<float>(a, yt, d, st);
  return hipErrorInvalidValue;
}

// Launch one of the per-sequence kernels (decode_prologue_kernel or
// conv_state_kernel) for head dim d over B sequences.
template <int D>
int blocks_per_seq(const ProArgs &a) {
  constexpr int RPB = kThreads / (D / 8);
  return (a.t[0].H + a.t[1].H + a.t[2].H + RPB - 1) / RPB;
}
template <typename TX, typename TO, int D>
hipError_t launch_dec_d(const ProArgs &a, bool state_only, hipStream_t st) {
  const dim3 grid((unsigned)(a.B * blocks_per_seq<D>(a)));
  if (state_only)
    hipLaunchKernelGGL((conv_state_kernel<TX, D>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((decode_prologue_kernel<TX, TO, D>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}
template <typename TX, typename TO>
hipError_t launch_dec_xo(const ProArgs &a, int d, bool state_only, hipStream_t st) {
  switch (d) {
    case 16: return launch_dec_d<TX, TO, 16>(a, state_only, st);
    case 32: return launch_dec_d<TX, TO, 32>(a, state_only, st);
    case 64: return launch_dec_d<TX, TO, 64>(a, state_only, st);
    case 128: return launch_dec_d<TX, TO, 128>(a, state_only, st);
  }
  return hipErrorInvalidValue;
}
template <typename TX>
hipError_t launch_dec_x(const ProArgs &a, DType yt, int d, bool state_only, hipStream_t st) {
  switch (yt) {
    case DType::F32: return launch_dec_xo<TX, float>(a, d, state_only, st);
    case DType::BF16: return launch_dec_xo<TX, bf16_t>(a, d, state_only, st);
    case DType::F16: return launch_dec_xo<TX, f16_t>(a, d, state_only, st);
  }
  return hipErrorInvalidValue;
}
hipError_t launch_dec(ProArgs a, DType xt, DType yt, int dk, int dv, bool state_only, hipStream_t st) {
  auto one = [&](const ProArgs &x, int d) {
    if (xt == DType::BF16) return launch_dec_x<bf16_t>(x, yt, d, state_only, st);
    if (xt == DType::F32) return launch_dec_x<float>(x, yt, d, state_only, st);
    return hipErrorInvalidValue;
  };
  if (dk == dv) return one(a, dk);
  ProArgs av = a;   // different head dims: q and k in one launch, v in another
  a.t[2].H = 0;
  av.t[0].H = 0;
  av.t[1].H = 0;
  const hipError_t e = one(a, dk);
  return e != hipSuccess ? e : one(av, dv);
}

ProArgs dec_args(const void *xq, const void *xk, const void *xv, const float *w, void *cs, void *q,
                 void *k, void *v, int B, int T, int Hk, int Hv, int dk, int dv, float eps, const int *cu) {
  const size_t nw = (size_t)Hk * dk * 4;
  ProArgs a;
  a.B = B;
  a.T = T;
  a.eps = eps;
  a.sq = Seqs{cu, B};
  a.cs = cs;
  a.nch = 2 * Hk * dk + Hv * dv;
  a.t[0] = ProTensor{xq, w, q, Hk, true, 0};
  a.t[1] = ProTensor{xk, w ? w + nw : nullptr, k, Hk, true, Hk * dk};
  a.t[2] = ProTensor{xv, w ? w + 2 * nw : nullptr, v, Hv, false, 2 * Hk * dk};
  return a;
}

}  // namespace

hipError_t launch_decode_prologue(const void *xq, const void *xk, const void *xv, DType xt, const float *w,
                                  void *cs, void *q, void *k, void *v, DType yt, int B, int Hk, int Hv,
                                  int dk, int dv, float eps, hipStream_t st) {
  return launch_dec(dec_args(xq, xk, xv, w, cs, q, k, v, B, 1, Hk, Hv, dk, dv, eps, nullptr), xt, yt, dk, dv,
                    false, st);
}

hipError_t launch_conv_state(const void *xq, const void *xk, const void *xv, DType xt, void *cs, int B,
                             int T, int Hk, int Hv, int dk, int dv, const int *cu, hipStream_t st) {
  return launch_dec(dec_args(xq, xk, xv, nullptr, cs, nullptr, nullptr, nullptr, B, T, Hk, Hv, dk, dv, 0.f,
                             cu),
                    xt, DType::F32, dk, dv, true, st);
}

hipError_t launch_prologue(const void *xq, const void *xk, const void *xv, DType xt, const float *w,
                           void *q, void *k, void *v, DType yt, int B, int T, int Hk, int Hv, int dk,
                           int dv, float eps, hipStream_t st, const int *cu) {
  const size_t nw = (size_t)Hk * dk * 4;   // conv_w rows of q, then of k, then of v
  ProArgs a;
  a.B = B;
  a.T = T;
  a.eps = eps;
  a.sq = Seqs{cu, B};
  a.t[0] = ProTensor{xq, w, q, Hk, true, 0};
  a.t[1] = ProTensor{xk, w + nw, k, Hk, true, Hk * dk};
  a.t[2] = ProTensor{xv, w + 2 * nw, v, Hv, false, 2 * Hk * dk};
  if (dk == dv) return launch_one(a, xt, yt, dk, st);
  // different head dims: q and k in one launch, v in another
  ProArgs av = a;
  a.t[2].H = 0;
  av.t[0].H = 0;
  av.t[1].H = 0;
  hipError_t e = launch_one(a, xt, yt, dk, st);
  if (e != hipSuccess) return e;
  return launch_one(av, xt, yt, dv, st);
}

}  // namespace gdn
