// chunk_bwd.hip -- the backward of the gated delta rule with the per-head
// gate, in chunks of C = 64 tokens on the fp32 matrix cores (16x16x4).
// ("Source notes", Linear attention, row kda: the first-order backward; the
// "SinkProbe" page: the exact chunkwise form of the recurrence.)
//
// Per (batch, value head) and chunk, with S0 the state before the chunk,
// gamma_i the gate's log summed over the chunk's tokens up to i, Gam =
// diag(e^gamma), M_ij = e^(gamma_i - gamma_j) (i >= j), and T = (I + A)^-1,
// A_ij = beta_i M_ij k_i.k_j (i > j), the forward is
//   X = beta (V - Gam K S0^T),  U = T X,  O = Gam Q S0^T + P U  (P = M o Q K^T),
//   S_C = e^gamma_C S0 + U^T Kt  (Kt_j = e^(gamma_C - gamma_j) k_j).
// For dO (of O) and dS_C (of S_C), its backward is
//   dU = P^T dO + Kt dS_C^T,  E = T^T dU (= dX),  dv = beta E,
//   dS0 = e^gamma_C dS_C + dO^T Gam Q - (beta Gam E)^T K,
//   dP = dO U^T,  dA = -E U^T,
//   dq = Gam dO S0 + (M o dP) K,
//   dk = (M o dP)^T Q + Kt-weighted U dS_C - beta Gam E S0 + beta (B K) + (beta B)^T K,  B = M o dA,
//   dbeta = rows of E . (V - Gam K S0^T) + rows of K . (B K),
// and the gradient of each gamma_i collects the same products as row dots
// with q_i and k_i (plus <dS_C, S_C> at the chunk's last token); dg is its
// sum over the chunk's later tokens.
//
// Four launches, the three passes after the first working from its output:
//  - prep, per (chunk, value head): gamma, beta, T and P^T;
//  - forward pass, per (batch, value head, 32 state rows), over the chunks in
//    order: the state before each chunk and U;
//  - backward pass, per (batch, value head, 32 state rows), over the chunks
//    in reverse: the state gradient after each chunk, E, dv and dS0;
//  - gradients, per (chunk, key head) over the key head's value heads: dq,
//    dk (summed over the value heads), dg, dbeta.
// The two passes are independent of each other.  All arithmetic is fp32.
#include <hip/hip_runtime.h>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int C = 64;       // tokens per chunk
constexpr int R = 32;       // state rows of a workgroup in the two passes
constexpr int LC = C + 4;   // LDS row strides (4 mod 32 floats: conflict-free row and column reads)
constexpr int LR = R + 4;

struct CbArgs {
  const void *q, *k, *v, *g, *beta;
  const float *S0, *dO, *dST;
  float *dq, *dk, *dv, *dg, *dbeta, *dS0;
  // workspace, per (batch, value head, chunk): T [C][C], P^T [C][C], gamma [C], beta [C],
  // state before the chunk [dv][dk], state gradient after it [dv][dk], U [C][dv], E [C][dv]
  float *Tm, *Pt, *gam, *bet, *S0s, *dSC, *Um, *Em;
  int T, Hk, Hv, dv_dim, nc;
};

__device__ __forceinline__ float4v mma(float a, float b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Four consecutive entries of a row, and four consecutive rows of a column.
__device__ __forceinline__ float4v row4(const float *p) { return *reinterpret_cast<const float4v *>(p); }
__device__ __forceinline__ float4v col4(const float *p, int ld) { return float4v{p[0], p[ld], p[2 * ld], p[3 * ld]}; }

// acc += A B^T over k in [0, K) on a 16x16 tile.  fa(k) gives the lane's
// A entries (i0 + ln, k .. k + 3), fb(k) its B entries (j0 + ln, k .. k + 3);
// the lane's k are k0 + 4 g4 + e.  The lane (g4, ln) holds (i0 + 4 g4 + e, j0 + ln).
template <int K, typename FA, typename FB>
__device__ __forceinline__ void mm(float4v &acc, const FA &fa, const FB &fb, int g4) {
#pragma unroll
  for (int k = 0; k < K; k += 16) {
    const float4v x = fa(k + 4 * g4), y = fb(k + 4 * g4);
    acc = mma(x[0], y[0], acc);
    acc = mma(x[1], y[1], acc);
    acc = mma(x[2], y[2], acc);
    acc = mma(x[3], y[3], acc);
  }
}

// rows of a chunk of q or k (zeros past the sequence's end) into LDS, fp32 [C][DK + 4]
template <typename TQ, int DK>
__device__ __forceinline__ void load_rows(float *dst, const TQ *src, size_t row0, int stride, int len, int tid) {
  constexpr int LK = DK + 4;
  for (int u = tid; u < C * DK / 8; u += 256) {
    const int t = u / (DK / 8), c = (u % (DK / 8)) * 8;
    float x[8];
    if (t < len) {
      load8(src + (row0 + (size_t)t * stride) * DK + c, x);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    *reinterpret_cast<float4v *>(dst + t * LK + c) = float4v{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<float4v *>(dst + t * LK + c + 4) = float4v{x[4], x[5], x[6], x[7]};
  }
}

// a [C][C] matrix of the workspace into LDS [C][LC]
__device__ __forceinline__ void load_cc(float *dst, const float *src, int tid) {
  for (int u = tid; u < C * C / 4; u += 256) {
    const int i = u / (C / 4), j = (u % (C / 4)) * 4;
    *reinterpret_cast<float4v *>(dst + i * LC + j) = *reinterpret_cast<const float4v *>(src + i * C + j);
  }
}

// the chunk's gate factors: e^gamma_t, e^(gamma_C - gamma_t), beta_t (and gamma_t if sg)
__device__ __forceinline__ void load_gates(float *sEg, float *sEc, float *sb, const CbArgs &a, size_t cn, int tid,
                                           float *sg = nullptr) {
  if (tid < C) {
    const float gm = a.gam[cn * C + tid], gC = a.gam[cn * C + C - 1];
    if (sg) sg[tid] = gm;
    sEg[tid] = __expf(gm);
    sEc[tid] = __expf(gC - gm);
    sb[tid] = a.bet[cn * C + tid];
  }
}

// ---------------------------------------------------------------------------
// prep: gamma (inclusive prefix sum of g over the chunk, zero past the end),
// beta, P^T and T = (I + A)^-1 by forward substitution.
template <typename TQ, typename TG, int DK>
__global__ __launch_bounds__(256) void cb_prep_kernel(CbArgs a) {
  constexpr int LK = DK + 4;
  extern __shared__ float4v smem4[];
  float *smem = reinterpret_cast<float *>(smem4);
  float *sK = smem, *sQ = sK + C * LK, *sA = sQ + C * LK, *sg = sA + C * LC, *sb = sg + C;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 15, g4 = lane >> 4;
  const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int T = a.T, Hk = a.Hk, Hv = a.Hv, kh = h / (Hv / Hk);
  const int t0 = n * C, len = min(C, T - t0);
  const size_t cn = ((size_t)b * Hv + h) * a.nc + n;
  const size_t row0 = (size_t)b * T + t0;
  load_rows<TQ, DK>(sK, (const TQ *)a.k, row0 * Hk + kh, Hk, len, tid);
  load_rows<TQ, DK>(sQ, (const TQ *)a.q, row0 * Hk + kh, Hk, len, tid);
  if (w == 0) {
    const TG *g = (const TG *)a.g, *be = (const TG *)a.beta;
    const float gt = lane < len ? to_f32(g[(row0 + lane) * Hv + h]) : 0.f;
    const float bt = lane < len ? to_f32(be[(row0 + lane) * Hv + h]) : 0.f;
    const float gm = wave_prefix_sum(gt);
    sg[lane] = gm;
    sb[lane] = bt;
    a.gam[cn * C + lane] = gm;
    a.bet[cn * C + lane] = bt;
  }
  __syncthreads();
  // wave w: block row w (tokens 16 w ..); the lane holds i = 16 w + 4 g4 + e, j = 16 J + ln
  float *Ptg = a.Pt + cn * C * C;
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    float4v kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
    if (J <= w) {
      mm<DK>(kk, [&](int k) { return row4(sK + (16 * w + ln) * LK + k); },
             [&](int k) { return row4(sK + (16 * J + ln) * LK + k); }, g4);
      mm<DK>(qk, [&](int k) { return row4(sQ + (16 * w + ln) * LK + k); },
             [&](int k) { return row4(sK + (16 * J + ln) * LK + k); }, g4);
    }
    const int j = 16 * J + ln;
    float4v pt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + 4 * g4 + e;
      const float m = i >= j ? __expf(sg[i] - sg[j]) : 0.f;
      sA[i * LC + j] = i > j ? sb[i] * m * kk[e] : 0.f;
      pt[e] = m * qk[e];
    }
    *reinterpret_cast<float4v *>(Ptg + j * C + 16 * w + 4 * g4) = pt;   // P^T[j][i]
  }
  __syncthreads();
  if (w == 0) {
    // column c = lane of T: T[i][c] = [i == c] - sum_{j < i} A[i][j] T[j][c]
    float tc[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < i; ++j) s = __builtin_fmaf(sA[i * LC + j], tc[j], s);
      tc[i] = (i == lane ? 1.f : 0.f) - s;
    }
    float *Tg = a.Tm + cn * C * C;
#pragma unroll
    for (int i = 0; i < C; ++i) Tg[i * C + lane] = tc[i];
  }
}

// ---------------------------------------------------------------------------
// forward pass: 32 state rows r0 .. of one (batch, value head) over the
// chunks in order.  Wave w holds the state tiles of row block w & 1 and
// column blocks (w >> 1) NCT/2 .. ; of the [32][C] products, row block w & 1
// and column blocks 2 (w >> 1), 2 (w >> 1) + 1.
template <typename TQ, int DK>
__global__ __launch_bounds__(256) void cb_fwd_kernel(CbArgs a) {
  constexpr int LK = DK + 4, NST = DK / 32;
  extern __shared__ float4v smem4[];
  float *smem = reinterpret_cast<float *>(smem4);
  float *sK = smem, *sT = sK + C * LK, *sS = sT + C * LC, *sX = sS + R * LK, *sU = sX + R * LC;
  float *sEg = sU + R * LC, *sEc = sEg + C, *sb = sEc + C;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 15, g4 = lane >> 4;
  const int sl = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int T = a.T, Hk = a.Hk, Hv = a.Hv, DV = a.dv_dim, nc = a.nc, kh = h / (Hv / Hk), r0 = sl * R;
  const int rt = w & 1, ct0 = (w >> 1) * NST, zc0 = (w >> 1) * 2;
  const size_t bh = (size_t)b * Hv + h;
  const TQ *v = (const TQ *)a.v;
  float4v S[NST];
#pragma unroll
  for (int s = 0; s < NST; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[s][e] = a.S0 ? a.S0[(bh * DV + r0 + 16 * rt + 4 * g4 + e) * DK + 16 * (ct0 + s) + ln] : 0.f;
  for (int n = 0; n < nc; ++n) {
    const int t0 = n * C, len = min(C, T - t0);
    const size_t cn = bh * nc + n, row0 = (size_t)b * T + t0;
    load_rows<TQ, DK>(sK, (const TQ *)a.k, row0 * Hk + kh, Hk, len, tid);
    load_cc(sT, a.Tm + cn * C * C, tid);
    load_gates(sEg, sEc, sb, a, cn, tid);
    float *S0g = a.S0s + (cn * DV + r0) * DK;
#pragma unroll
    for (int s = 0; s < NST; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * g4 + e, c = 16 * (ct0 + s) + ln;
        sS[r * LK + c] = S[s][e];
        S0g[r * DK + c] = S[s][e];
      }
    __syncthreads();
    // X^T[r][t] = beta_t (v_t[r] - e^gamma_t (S k_t)[r])
#pragma unroll
    for (int z = 0; z < 2; ++z) {
      const int t = 16 * (zc0 + z) + ln;
      float4v acc = {0.f, 0.f, 0.f, 0.f};
      mm<DK>(acc, [&](int k) { return row4(sS + (16 * rt + ln) * LK + k); },
             [&](int k) { return row4(sK + t * LK + k); }, g4);
      float vx[4] = {0.f, 0.f, 0.f, 0.f};
      if (t < len) load4(v + (row0 + t) * Hv * DV + (size_t)h * DV + r0 + 16 * rt + 4 * g4, vx);
      const float eg = sEg[t], bt = sb[t];
#pragma unroll
      for (int e = 0; e < 4; ++e) sX[(16 * rt + 4 * g4 + e) * LC + t] = bt * (vx[e] - eg * acc[e]);
    }
    __syncthreads();
    // U^T[r][i] = sum_j X^T[r][j] T[i][j]; U to the workspace, U^T e^(gamma_C - gamma_i) to LDS
#pragma unroll
    for (int z = 0; z < 2; ++z) {
      const int i = 16 * (zc0 + z) + ln;
      float4v u = {0.f, 0.f, 0.f, 0.f};
      mm<C>(u, [&](int k) { return row4(sX + (16 * rt + ln) * LC + k); },
            [&](int k) { return row4(sT + i * LC + k); }, g4);
      *reinterpret_cast<float4v *>(a.Um + (cn * C + i) * DV + r0 + 16 * rt + 4 * g4) = u;
      const float ec = sEc[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) sU[(16 * rt + 4 * g4 + e) * LC + i] = u[e] * ec;
    }
    __syncthreads();
    // S <- e^gamma_C S + sum_j U~^T[r][j] k_j
    const float eC = sEg[C - 1];
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int c = 16 * (ct0 + s) + ln;
      S[s] *= eC;
      mm<C>(S[s], [&](int k) { return row4(sU + (16 * rt + ln) * LC + k); },
            [&](int k) { return col4(sK + k * LK + c, LK); }, g4);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// backward pass: the state gradient of 32 rows r0 .. of one (batch, value
// head) over the chunks in reverse, with the same tiles as the forward pass.
template <typename TQ, int DK>
__global__ __launch_bounds__(256) void cb_bwd_kernel(CbArgs a) {
  constexpr int LK = DK + 4, NST = DK / 32;
  extern __shared__ float4v smem4[];
  float *smem = reinterpret_cast<float *>(smem4);
  float *sK = smem, *sQ = sK + C * LK, *sT = sQ + C * LK, *sP = sT + C * LC, *sO = sP + C * LC;
  float *sS = sO + C * LR, *sD = sS + R * LK, *sE = sD + R * LC;
  float *sEg = sE + R * LC, *sEc = sEg + C, *sb = sEc + C;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 15, g4 = lane >> 4;
  const int sl = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int T = a.T, Hk = a.Hk, Hv = a.Hv, DV = a.dv_dim, nc = a.nc, kh = h / (Hv / Hk), r0 = sl * R;
  const int rt = w & 1, ct0 = (w >> 1) * NST, zc0 = (w >> 1) * 2;
  const size_t bh = (size_t)b * Hv + h;
  float4v dS[NST];
#pragma unroll
  for (int s = 0; s < NST; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dS[s][e] = a.dST ? a.dST[(bh * DV + r0 + 16 * rt + 4 * g4 + e) * DK + 16 * (ct0 + s) + ln] : 0.f;
  for (int n = nc - 1; n >= 0; --n) {
    const int t0 = n * C, len = min(C, T - t0);
    const size_t cn = bh * nc + n, row0 = (size_t)b * T + t0;
    load_rows<TQ, DK>(sK, (const TQ *)a.k, row0 * Hk + kh, Hk, len, tid);
    load_rows<TQ, DK>(sQ, (const TQ *)a.q, row0 * Hk + kh, Hk, len, tid);
    load_cc(sT, a.Tm + cn * C * C, tid);
    load_cc(sP, a.Pt + cn * C * C, tid);
    load_gates(sEg, sEc, sb, a, cn, tid);
    for (int u = tid; u < C * R / 4; u += 256) {
      const int t = u / (R / 4), r = (u % (R / 4)) * 4;
      *reinterpret_cast<float4v *>(sO + t * LR + r) =
          t < len ? *reinterpret_cast<const float4v *>(a.dO + ((row0 + t) * Hv + h) * DV + r0 + r)
                  : float4v{0.f, 0.f, 0.f, 0.f};
    }
    float *dSg = a.dSC + (cn * DV + r0) * DK;
#pragma unroll
    for (int s = 0; s < NST; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * g4 + e, c = 16 * (ct0 + s) + ln;
        sS[r * LK + c] = dS[s][e];
        dSg[r * DK + c] = dS[s][e];
      }
    __syncthreads();
    // dU^T[r][i] = e^(gamma_C - gamma_i) (dS k_i)[r] + sum_j dO[j][r] P[j][i]
#pragma unroll
    for (int z = 0; z < 2; ++z) {
      const int i = 16 * (zc0 + z) + ln;
      float4v acc = {0.f, 0.f, 0.f, 0.f};
      mm<DK>(acc, [&](int k) { return row4(sS + (16 * rt + ln) * LK + k); },
             [&](int k) { return row4(sK + i * LK + k); }, g4);
      acc *= sEc[i];
      mm<C>(acc, [&](int k) { return col4(sO + k * LR + 16 * rt + ln, LR); },
            [&](int k) { return row4(sP + i * LC + k); }, g4);
#pragma unroll
      for (int e = 0; e < 4; ++e) sD[(16 * rt + 4 * g4 + e) * LC + i] = acc[e];
    }
    __syncthreads();
    // E^T[r][i] = sum_j dU^T[r][j] T[j][i]; dv = beta E; -beta e^gamma E^T to LDS
#pragma unroll
    for (int z = 0; z < 2; ++z) {
      const int i = 16 * (zc0 + z) + ln;
      float4v E = {0.f, 0.f, 0.f, 0.f};
      mm<C>(E, [&](int k) { return row4(sD + (16 * rt + ln) * LC + k); },
            [&](int k) { return col4(sT + k * LC + i, LC); }, g4);
      const float bi = sb[i];
      if (i < len)
        *reinterpret_cast<float4v *>(a.dv + ((row0 + i) * Hv + h) * DV + r0 + 16 * rt + 4 * g4) = E * bi;
      *reinterpret_cast<float4v *>(a.Em + (cn * C + i) * DV + r0 + 16 * rt + 4 * g4) = E;
      const float f = -bi * sEg[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) sE[(16 * rt + 4 * g4 + e) * LC + i] = E[e] * f;
    }
    __syncthreads();
    // dS <- e^gamma_C dS + sum_t dO[t][r] e^gamma_t q_t - sum_t beta_t e^gamma_t E[t][r] k_t
    const float eC = sEg[C - 1];
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int c = 16 * (ct0 + s) + ln;
      dS[s] *= eC;
      mm<C>(dS[s], [&](int k) { return col4(sO + k * LR + 16 * rt + ln, LR) * row4(sEg + k); },
            [&](int k) { return col4(sQ + k * LK + c, LK); }, g4);
      mm<C>(dS[s], [&](int k) { return row4(sE + (16 * rt + ln) * LC + k); },
            [&](int k) { return col4(sK + k * LK + c, LK); }, g4);
    }
    __syncthreads();
  }
#pragma unroll
  for (int s = 0; s < NST; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      a.dS0[(bh * DV + r0 + 16 * rt + 4 * g4 + e) * DK + 16 * (ct0 + s) + ln] = dS[s][e];
}

// ---------------------------------------------------------------------------
// gradients of one (chunk, key head): for each value head of the key head,
// the products over the value rows in slices of 32 (dP = dO U^T, E U^T,
// dO S0, E S0, U dS_C), then the products with the masked C x C matrices
// and the row dots; dq and dk summed over the value heads.  Wave w holds
// token block w of every [C][.] product.
template <typename TQ, typename TG, int DK>
__global__ __launch_bounds__(256) void cb_grads_kernel(CbArgs a) {
  constexpr int LK = DK + 4, NCT = DK / 16;
  constexpr int SLICE = 3 * C * LR + 2 * R * LK, MASKS = 2 * C * LC;
  constexpr int REGION = SLICE > MASKS ? SLICE : MASKS;
  extern __shared__ float4v smem4[];
  float *smem = reinterpret_cast<float *>(smem4);
  float *sK = smem, *sQ = sK + C * LK, *rg = sQ + C * LK;
  float *sO = rg, *sU = sO + C * LR, *sE = sU + C * LR, *sS0 = sE + C * LR, *sdS = sS0 + R * LK;
  float *sdP = rg, *sB = sdP + C * LC;
  float *sEg = rg + REGION, *sEc = sEg + C, *sb = sEc + C, *sGam = sb + C, *sBet = sGam + C, *sBx = sBet + C;
  float *sg = sBx + C, *sRed = sg + C;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 15, g4 = lane >> 4;
  const int n = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int T = a.T, Hk = a.Hk, Hv = a.Hv, DV = a.dv_dim, nc = a.nc, grp = Hv / Hk;
  const int t0 = n * C, len = min(C, T - t0);
  const size_t row0 = (size_t)b * T + t0;
  const TQ *v = (const TQ *)a.v;
  load_rows<TQ, DK>(sK, (const TQ *)a.k, row0 * Hk + kh, Hk, len, tid);
  load_rows<TQ, DK>(sQ, (const TQ *)a.q, row0 * Hk + kh, Hk, len, tid);
  float4v dQa[NCT], dKa[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) dQa[c] = dKa[c] = float4v{0.f, 0.f, 0.f, 0.f};
  for (int hh = 0; hh < grp; ++hh) {
    const int h = kh * grp + hh;
    const size_t cn = ((size_t)b * Hv + h) * nc + n;
    __syncthreads();   // the previous head's last reads of LDS are done
    load_gates(sEg, sEc, sb, a, cn, tid, sg);
    if (tid < 2) sRed[tid] = 0.f;
    float4v dPa[4], dAa[4], Q1[NCT], ES[NCT], UD[NCT];
#pragma unroll
    for (int J = 0; J < 4; ++J) dPa[J] = dAa[J] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCT; ++c) Q1[c] = ES[c] = UD[c] = float4v{0.f, 0.f, 0.f, 0.f};
    float dbx = 0.f, sdot = 0.f;
    for (int r0 = 0; r0 < DV; r0 += R) {
      __syncthreads();
      for (int u = tid; u < C * R / 4; u += 256) {
        const int t = u / (R / 4), r = (u % (R / 4)) * 4;
        *reinterpret_cast<float4v *>(sO + t * LR + r) =
            t < len ? *reinterpret_cast<const float4v *>(a.dO + ((row0 + t) * Hv + h) * DV + r0 + r)
                    : float4v{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<float4v *>(sU + t * LR + r) =
            *reinterpret_cast<const float4v *>(a.Um + (cn * C + t) * DV + r0 + r);
        *reinterpret_cast<float4v *>(sE + t * LR + r) =
            *reinterpret_cast<const float4v *>(a.Em + (cn * C + t) * DV + r0 + r);
      }
      for (int u = tid; u < R * DK / 4; u += 256) {
        const int r = u / (DK / 4), c = (u % (DK / 4)) * 4;
        *reinterpret_cast<float4v *>(sS0 + r * LK + c) =
            *reinterpret_cast<const float4v *>(a.S0s + (cn * DV + r0 + r) * DK + c);
        *reinterpret_cast<float4v *>(sdS + r * LK + c) =
            *reinterpret_cast<const float4v *>(a.dSC + (cn * DV + r0 + r) * DK + c);
      }
      __syncthreads();
      {
        // E . v over the slice for token tid / 4
        const int t = tid >> 2, rr = (tid & 3) * 8;
        if (t < len) {
          float vx[8];
          load8(v + ((row0 + t) * Hv + h) * DV + r0 + rr, vx);
#pragma unroll
          for (int e = 0; e < 8; ++e) dbx = __builtin_fmaf(sE[t * LR + rr + e], vx[e], dbx);
        }
      }
      for (int u = tid; u < R * DK; u += 256) {
        const int r = u / DK, c = u % DK;
        sdot = __builtin_fmaf(sS0[r * LK + c], sdS[r * LK + c], sdot);
      }
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        mm<R>(dPa[J], [&](int k) { return row4(sO + (16 * w + ln) * LR + k); },
              [&](int k) { return row4(sU + (16 * J + ln) * LR + k); }, g4);
        mm<R>(dAa[J], [&](int k) { return row4(sE + (16 * w + ln) * LR + k); },
              [&](int k) { return row4(sU + (16 * J + ln) * LR + k); }, g4);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int c = 16 * ct + ln;
        mm<R>(Q1[ct], [&](int k) { return row4(sO + (16 * w + ln) * LR + k); },
              [&](int k) { return col4(sS0 + k * LK + c, LK); }, g4);
        mm<R>(ES[ct], [&](int k) { return row4(sE + (16 * w + ln) * LR + k); },
              [&](int k) { return col4(sS0 + k * LK + c, LK); }, g4);
        mm<R>(UD[ct], [&](int k) { return row4(sU + (16 * w + ln) * LR + k); },
              [&](int k) { return col4(sdS + k * LK + c, LK); }, g4);
      }
    }
    __syncthreads();
    // M o dP and B = M o dA = -(M o E U^T) into LDS (over the slices' space)
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      const int j = 16 * J + ln;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * w + 4 * g4 + e;
        const float m = i >= j ? __expf(sg[i] - sg[j]) : 0.f;
        sdP[i * LC + j] = m * dPa[J][e];
        sB[i * LC + j] = i > j ? -m * dAa[J][e] : 0.f;
      }
    }
    // E . v and <dS_C, S0> over the workgroup
    dbx = group_sum<4>(dbx);
    if ((tid & 3) == 0) sBx[tid >> 2] = dbx;
    sdot = group_sum<64>(sdot);
    if (lane == 0) atomicAdd(&sRed[1], sdot);
    __syncthreads();
    float gp[4] = {0.f, 0.f, 0.f, 0.f}, bp[4] = {0.f, 0.f, 0.f, 0.f}, cp = 0.f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int c = 16 * ct + ln;
      float4v q2 = {0.f, 0.f, 0.f, 0.f}, k1 = q2, f1 = q2, f2 = q2;
      mm<C>(q2, [&](int k) { return row4(sdP + (16 * w + ln) * LC + k); },
            [&](int k) { return col4(sK + k * LK + c, LK); }, g4);
      mm<C>(k1, [&](int k) { return col4(sdP + k * LC + 16 * w + ln, LC); },
            [&](int k) { return col4(sQ + k * LK + c, LK); }, g4);
      mm<C>(f1, [&](int k) { return row4(sB + (16 * w + ln) * LC + k); },
            [&](int k) { return col4(sK + k * LK + c, LK); }, g4);
      mm<C>(f2, [&](int k) { return col4(sB + k * LC + 16 * w + ln, LC) * row4(sb + k); },
            [&](int k) { return col4(sK + k * LK + c, LK); }, g4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * w + 4 * g4 + e;
        const float eg = sEg[t], bt = sb[t];
        const float dq = __builtin_fmaf(eg, Q1[ct][e], q2[e]);
        const float f1m = __builtin_fmaf(-eg, ES[ct][e], f1[e]);   // (B k)_t - e^gamma_t (E S0)_t
        const float d4 = sEc[t] * UD[ct][e];
        const float g1 = k1[e] + d4 + f2[e];
        dQa[ct][e] += dq;
        dKa[ct][e] += __builtin_fmaf(bt, f1m, g1);
        const float qv = sQ[t * LK + c], kv = sK[t * LK + c];
        gp[e] += qv * dq - kv * g1 + kv * bt * f1m;
        bp[e] += kv * f1m;
        cp = __builtin_fmaf(kv, d4, cp);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gp[e] = group_sum<16>(gp[e]);
      bp[e] = group_sum<16>(bp[e]);
    }
    if (ln == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sGam[16 * w + 4 * g4 + e] = gp[e];
        sBet[16 * w + 4 * g4 + e] = bp[e];
      }
    }
    cp = group_sum<64>(cp);
    if (lane == 0) atomicAdd(&sRed[0], cp);
    __syncthreads();
    if (w == 0) {
      // dg_t = sum over the chunk's tokens i >= t of the gradient of gamma_i; the
      // last token also carries <dS_C, S_C> = e^gamma_C <dS_C, S0> + sum_j k_j . dk4_j
      const int t = C - 1 - lane;
      const float x = sGam[t] + (t == C - 1 ? __builtin_fmaf(sEg[C - 1], sRed[1], sRed[0]) : 0.f);
      const float s = wave_prefix_sum(x);
      if (t < len) {
        a.dg[(row0 + t) * Hv + h] = s;
        a.dbeta[(row0 + t) * Hv + h] = sBet[t] + sBx[t];
      }
    }
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * w + 4 * g4 + e;
      if (t < len) {
        a.dq[((row0 + t) * Hk + kh) * DK + 16 * ct + ln] = dQa[ct][e];
        a.dk[((row0 + t) * Hk + kh) * DK + 16 * ct + ln] = dKa[ct][e];
      }
    }
}

template <int DK>
struct CbSmem {
  static constexpr int LK = DK + 4;
  static constexpr int prep = (2 * C * LK + C * LC + 2 * C) * 4;
  static constexpr int fwd = (C * LK + C * LC + R * LK + 2 * R * LC + 3 * C) * 4;
  static constexpr int bwd = (2 * C * LK + 2 * C * LC + C * LR + R * LK + 2 * R * LC + 3 * C) * 4;
  static constexpr int slice = 3 * C * LR + 2 * R * LK, masks = 2 * C * LC;
  static constexpr int grads = (2 * C * LK + (slice > masks ? slice : masks) + 7 * C + 4) * 4;
};

template <typename F>
hipError_t set_smem(F *kern, int bytes) {
  return hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <typename TQ, typename TG, int DK>
hipError_t launch_cb_t(const Shape &sh, const CbArgs &a, hipStream_t st) {
  using Sm = CbSmem<DK>;
  static_assert(Sm::bwd <= 160 * 1024 && Sm::grads <= 160 * 1024 && Sm::prep <= 160 * 1024, "LDS");
  hipError_t e;
  if ((e = set_smem(cb_prep_kernel<TQ, TG, DK>, Sm::prep)) != hipSuccess) return e;
  if ((e = set_smem(cb_fwd_kernel<TQ, DK>, Sm::fwd)) != hipSuccess) return e;
  if ((e = set_smem(cb_bwd_kernel<TQ, DK>, Sm::bwd)) != hipSuccess) return e;
  if ((e = set_smem(cb_grads_kernel<TQ, TG, DK>, Sm::grads)) != hipSuccess) return e;
  hipLaunchKernelGGL((cb_prep_kernel<TQ, TG, DK>), dim3(a.nc, sh.Hv, sh.B), dim3(256), Sm::prep, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((cb_fwd_kernel<TQ, DK>), dim3(sh.dv / R, sh.Hv, sh.B), dim3(256), Sm::fwd, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((cb_bwd_kernel<TQ, DK>), dim3(sh.dv / R, sh.Hv, sh.B), dim3(256), Sm::bwd, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((cb_grads_kernel<TQ, TG, DK>), dim3(a.nc, sh.Hk, sh.B), dim3(256), Sm::grads, st, a);
  return hipGetLastError();
}

template <typename TQ, typename TG>
hipError_t launch_cb_d(const Shape &sh, const CbArgs &a, hipStream_t st) {
  switch (sh.dk) {
    case 32: return launch_cb_t<TQ, TG, 32>(sh, a, st);
    case 64: return launch_cb_t<TQ, TG, 64>(sh, a, st);
    case 128: return launch_cb_t<TQ, TG, 128>(sh, a, st);
  }
  return hipErrorInvalidValue;
}

// floats of each workspace array per (batch, value head, chunk)
struct CbSizes {
  size_t cc, c, st, cv;
  explicit CbSizes(const Shape &sh) : cc((size_t)C * C), c(C), st((size_t)sh.dv * sh.dk), cv((size_t)C * sh.dv) {}
  size_t per_chunk() const { return 2 * cc + 2 * c + 2 * st + 2 * cv; }
};

}  // namespace

size_t chunk_backward_workspace(const Shape &sh) {
  const size_t nc = (size_t)(sh.T + C - 1) / C;
  return (size_t)sh.B * sh.Hv * nc * CbSizes(sh).per_chunk() * 4;
}

hipError_t launch_chunk_backward(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                                 const void *beta, const float *S0, const float *dO, const float *dST, float *dq,
                                 float *dk, float *dv, float *dg, float *dbeta, float *dS0, void *ws,
                                 hipStream_t st) {
  CbArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.S0 = S0;
  a.dO = dO;
  a.dST = dST;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dg = dg;
  a.dbeta = dbeta;
  a.dS0 = dS0;
  a.T = sh.T;
  a.Hk = sh.Hk;
  a.Hv = sh.Hv;
  a.dv_dim = sh.dv;
  a.nc = (sh.T + C - 1) / C;
  const size_t units = (size_t)sh.B * sh.Hv * a.nc;
  const CbSizes z(sh);
  float *p = (float *)ws;
  a.Tm = p;
  p += units * z.cc;
  a.Pt = p;
  p += units * z.cc;
  a.gam = p;
  p += units * z.c;
  a.bet = p;
  p += units * z.c;
  a.S0s = p;
  p += units * z.st;
  a.dSC = p;
  p += units * z.st;
  a.Um = p;
  p += units * z.cv;
  a.Em = p;
  if (sh.qkv == DType::F32)
    return sh.gate_t == DType::F32 ? launch_cb_d<float, float>(sh, a, st) : launch_cb_d<float, bf16_t>(sh, a, st);
  if (sh.qkv == DType::BF16)
    return sh.gate_t == DType::F32 ? launch_cb_d<bf16_t, float>(sh, a, st) : launch_cb_d<bf16_t, bf16_t>(sh, a, st);
  return sh.gate_t == DType::F32 ? launch_cb_d<f16_t, float>(sh, a, st) : launch_cb_d<f16_t, bf16_t>(sh, a, st);
}

}  // namespace gdn
