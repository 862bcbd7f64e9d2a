// chunk_bwd.hip -- the backward of the gated delta rule, per-head and
// per-key-channel gates, in chunks of C = 64 tokens on the fp32 matrix cores
// (16x16x4).
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
// with q_i and k_i (plus <dS_C, S_C> at the chunk's last token); dg_t is the
// sum of those over the chunk's tokens i >= t.  The gate is taken to decay
// (g <= 0), so every factor e^(gamma_i - gamma_j) with i >= j is at most 1.
//
// Per-key-channel gate: gamma_i is a vector over the key channels and every
// decay acts channel by channel: A_ij = beta_i sum_c k_ic k_jc e^(gamma_ic -
// gamma_jc) and P likewise with q_i; X = beta (V - (K o e^gamma) S0^T);
// S_C = S0 diag(e^gamma_C) + U^T (K o e^(gamma_C - gamma)); dU takes
// K o e^(gamma_C - gamma) and dS0 = dS_C diag(e^gamma_C) + dO^T (Q o e^gamma)
// - (beta E)^T (K o e^gamma).  The masked products, (M o dP) K and the like,
// become sums over j of dP_ij k_j o e^(gamma_i - gamma_j): in 16-token blocks,
// off the diagonal through a reference token between i and j (both factors
// at most 1), on the diagonal term by term.  The gradient of gamma, and dg,
// are per channel.
//
// Four launches, the three passes after the first working from its output:
//  - prep, per (chunk, key head) over the key head's value heads: gamma,
//    beta, T and P^T (per-key-channel gate: also K o e^gamma, Q o e^gamma
//    and K o e^(gamma_C - gamma), for the passes);
//  - forward pass, per (batch, value head, 32 state rows), over the chunks in
//    order: the state before each chunk and U;
//  - backward pass, per (batch, value head, 32 state rows), over the chunks
//    in reverse: the state gradient after each chunk, E, dv and dS0;
//  - gradients, per (chunk, key head) over the key head's value heads: dq,
//    dk (summed over the value heads), dg, dbeta.
// The two passes are independent of each other.  All arithmetic is fp32.
// With a workspace too small for every chunk's arrays, the sequence runs in
// segments of consecutive chunks, last first: T, gamma, beta are made for
// all chunks, a forward pass keeps only the states at the segment starts,
// and each segment then runs P^T, its forward pass, its backward pass (the
// state gradient carried in dS0) and its gradients; the results are the same
// bits as with one segment.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int C = 64;       // tokens per chunk
constexpr int R = 32;       // state rows of a workgroup in the two passes
constexpr int LC = C + 4;   // LDS row strides (4 mod 32 floats: conflict-free row and column reads)
constexpr int LR = R + 4;

// flags of a launch
constexpr int kPrepT = 1, kPrepP = 2;   // prep: T, gamma, beta; P^T
constexpr int kStatesOnly = 4;          // forward pass: only the states at segment starts
// Per-key-channel gate: a 16-token block whose decay over its tokens, gamma at
// its first token minus gamma at its last, is at most kWide in every channel
// goes through the matrix cores with one reference token for the whole block
// (one factor at most 1, the other at most e^kWide, finite however the
// products are masked); a wider block is summed term by term.
constexpr float kWide = 60.f;

struct CbArgs {
  const void *q, *k, *v, *g, *beta;
  const float *S0, *dO;
  const float *dS_in;   // the state gradient after the last chunk of the launch's range (null: zeros)
  float *dq, *dk, *dv, *dg, *dbeta, *dS0;
  // workspace.  For every (batch, value head, chunk): T [C][C], gamma [C], beta [C].
  // For the chunks of one segment (ncs of them per (batch, value head), from chunk
  // sc0): P^T [C][C], the state before the chunk [dv][dk], the state gradient after
  // it [dv][dk], U [C][dv], E [C][dv].  With several segments, the state before
  // each segment's first chunk, [B Hv][nseg][dv][dk].
  float *Tm, *gam, *bet, *Pt, *S0s, *dSC, *Um, *Em, *Sseg;
  // per-key-channel gate, for every chunk: gamma is [C][dk], and the decayed
  // operands K o e^gamma, Q o e^gamma, K o e^(gamma_C - gamma), [C][dk] each
  float *Kh, *Qh, *Kt;
  int T, Hk, Hv, dv_dim, nc;
  int c0, c1;         // the launch's chunks
  int sc0, ncs, nseg;
  int flags;
  int nd;             // the update without the delta correction: A = 0 (T = I), X = beta V
};

// index of (batch-head bh, chunk n) in the all-chunk arrays and in the segment arrays
__device__ __forceinline__ size_t gch(const CbArgs &a, size_t bh, int n) { return bh * a.nc + n; }
__device__ __forceinline__ size_t sch(const CbArgs &a, size_t bh, int n) { return bh * a.ncs + (n - a.sc0); }

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

// Four consecutive input values as raw bits, and as fp32.
template <typename TQ> struct Quad { using type = uint2; };
template <> struct Quad<float> { using type = float4v; };
template <typename TQ>
__device__ __forceinline__ typename Quad<TQ>::type quad_load(const TQ *p) {
  return *reinterpret_cast<const typename Quad<TQ>::type *>(p);
}
__device__ __forceinline__ float4v quad_f32(float4v x) { return x; }
__device__ __forceinline__ float4v quad_f32(uint2 x, bf16_t) {
  return float4v{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xFFFF0000u), __uint_as_float(x.y << 16),
                 __uint_as_float(x.y & 0xFFFF0000u)};
}
__device__ __forceinline__ float4v quad_f32(uint2 x, f16_t) {
  const half4 h = __builtin_bit_cast(half4, x);
  return float4v{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}
template <typename TQ>
__device__ __forceinline__ float4v quad_to_f32(typename Quad<TQ>::type x) {
  if constexpr (sizeof(TQ) == 4) return quad_f32(x);
  else return quad_f32(x, TQ{});
}

// rows of a chunk of q or k (zeros past the sequence's end) into LDS, fp32 [C][DK + 4]
// (a 256-thread workgroup).  Every load is issued before the first is used: a row
// past the end reads the chunk's last row in its place and is zeroed after, so that
// no load sits in a branch of its own and waits there.
template <typename TQ, int DK>
__device__ __forceinline__ void load_rows(float *dst, const TQ *src, size_t row0, int stride, int len, int tid) {
  constexpr int LK = DK + 4, NU = C * DK / 8 / 256;
  typename Quad<TQ>::type x[NU][2];
#pragma unroll
  for (int i = 0; i < NU; ++i) {
    const int u = tid + 256 * i, t = min(u / (DK / 8), len - 1), c = (u % (DK / 8)) * 8;
    const TQ *p = src + (row0 + (size_t)t * stride) * DK + c;
    x[i][0] = quad_load(p);
    x[i][1] = quad_load(p + 4);
  }
#pragma unroll
  for (int i = 0; i < NU; ++i) {
    const int u = tid + 256 * i, t = u / (DK / 8), c = (u % (DK / 8)) * 8;
    const float4v z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<float4v *>(dst + t * LK + c) = t < len ? quad_to_f32<TQ>(x[i][0]) : z;
    *reinterpret_cast<float4v *>(dst + t * LK + c + 4) = t < len ? quad_to_f32<TQ>(x[i][1]) : z;
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
// beta, P^T and T = (I + A)^-1 in 16 x 16 blocks: the diagonal blocks by
// forward substitution (one wave each), then the blocks below them, one block
// diagonal at a time, as T_IJ = -T_II sum_{J <= K < I} A_IK T_KJ.
constexpr int LX = 20;   // stride of the prep's 16 x 16 staging tiles
// the prep's first LDS region: k rows [C][DK + 4], later T [C][LC] and four staging tiles
__host__ __device__ constexpr int prep_region(int DK) {
  return C * (DK + 4) > C * LC + 4 * 16 * LX ? C * (DK + 4) : C * LC + 4 * 16 * LX;
}

// T = (I + A)^-1 for the strictly lower A in LDS [C][LC], into sT [C][LC] and
// Tg [C][C]: the 16 x 16 diagonal blocks by forward substitution (wave w the
// block w), then the blocks below them one block diagonal at a time as
// T_IJ = -T_II sum_{J <= K < I} A_IK T_KJ (sX: the wave's 16 x 16 staging
// tile).  The caller has synchronised the workgroup after writing A.
__device__ __forceinline__ void solve_T(const float *sA, float *sT, float *sX, float *Tg, int tid) {
  const int w = tid >> 6, lane = tid & 63, ln = lane & 15, g4 = lane >> 4;
  {
    // diagonal block w: lane (c, q) = (lane / 4, lane % 4) holds T[b + 4 m + q][b + c]
    // (b = 16 w); T[i][c] = [i == c] - sum_{j < i} A[i][j] T[j][c], the sum over
    // j = 4 m + q in the lane and over q in the quad (A is zero on and above the diagonal)
    const int c = lane >> 2, q = lane & 3, bw = 16 * w;
    float t4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) s = __builtin_fmaf(sA[(bw + i) * LC + bw + 4 * m + q], t4[m], s);
      s = group_sum<4>(s);
      const float val = (i == c ? 1.f : 0.f) - s;
      t4[i >> 2] = q == (i & 3) ? val : t4[i >> 2];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) sT[(bw + 4 * m + q) * LC + bw + c] = t4[m];
    // blocks above the diagonal are zero
    for (int J = w + 1; J < 4; ++J)
#pragma unroll
      for (int m = 0; m < 4; ++m) sT[(bw + 4 * m + q) * LC + 16 * J + c] = 0.f;
  }
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    lds_barrier();
    if (w < 4 - d) {
      const int I = w + d, J = w;
      float4v x = {0.f, 0.f, 0.f, 0.f};
      for (int K = J; K < I; ++K)
        mm<16>(x, [&](int k) { return row4(sA + (16 * I + ln) * LC + 16 * K + k); },
               [&](int k) { return col4(sT + (16 * K + k) * LC + 16 * J + ln, LC); }, g4);
#pragma unroll
      for (int e = 0; e < 4; ++e) sX[(4 * g4 + e) * LX + ln] = x[e];
      float4v y = {0.f, 0.f, 0.f, 0.f};
      mm<16>(y, [&](int k) { return row4(sT + (16 * I + ln) * LC + 16 * I + k); },
             [&](int k) { return col4(sX + k * LX + ln, LX); }, g4);
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[(16 * I + 4 * g4 + e) * LC + 16 * J + ln] = -y[e];
    }
  }
  lds_barrier();
  for (int u = tid; u < C * C / 4; u += 256) {
    const int i = u / (C / 4), j = (u % (C / 4)) * 4;
    *reinterpret_cast<float4v *>(Tg + i * C + j) = row4(sT + i * LC + j);
  }
}

template <typename TQ, typename TG, int DK>
__global__ __launch_bounds__(256) void cb_prep_kernel(CbArgs a) {
  constexpr int LK = DK + 4;
  extern __shared__ float4v smem4[];
  float *smem = reinterpret_cast<float *>(smem4);
  float *sK = smem, *sA = sK + prep_region(DK), *sg = sA + C * LC, *sb = sg + C;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 15, g4 = lane >> 4;
  const int n = a.c0 + blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int T = a.T, Hk = a.Hk, Hv = a.Hv, grp = Hv / Hk;
  const int t0 = n * C, len = min(C, T - t0);
  const size_t row0 = (size_t)b * T + t0;
  const bool doT = a.flags & kPrepT, doP = a.flags & kPrepP;
  load_rows<TQ, DK>(sK, (const TQ *)a.k, row0 * Hk + kh, Hk, len, tid);
  // the lane's q entries of token 16 w + ln as matrix-core operands (zeros past the end)
  float4v qa[DK / 16];
  {
    const int t = 16 * w + ln, tc = min(t, len - 1);   // past the end: the last row, zeroed
    typename Quad<TQ>::type qr[DK / 16];
#pragma unroll
    for (int kb = 0; kb < DK / 16; ++kb) qr[kb] = quad_load((const TQ *)a.q + ((row0 + tc) * Hk + kh) * DK + 16 * kb + 4 * g4);
#pragma unroll
    for (int kb = 0; kb < DK / 16; ++kb) qa[kb] = t < len ? quad_to_f32<TQ>(qr[kb]) : float4v{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  // K K^T and Q K^T of the key head, once for its value heads: wave w holds the
  // tiles of block row w (tokens 16 w ..) left of and on the diagonal; the lane
  // holds i = 16 w + 4 g4 + e, j = 16 J + ln
  float4v kk[4], qk[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    kk[J] = qk[J] = float4v{0.f, 0.f, 0.f, 0.f};
    if (J <= w && doT && !a.nd)   // without the delta correction A = 0, so T = I
      mm<DK>(kk[J], [&](int k) { return row4(sK + (16 * w + ln) * LK + k); },
             [&](int k) { return row4(sK + (16 * J + ln) * LK + k); }, g4);
    if (J <= w && doP)
      mm<DK>(qk[J], [&](int k) { return qa[k >> 4]; }, [&](int k) { return row4(sK + (16 * J + ln) * LK + k); },
             g4);
  }
  // T over the k rows' space; a 16 x 16 staging tile per wave after it
  float *sT = sK, *sX = sK + C * LC + w * 16 * LX;
  for (int hh = 0; hh < grp; ++hh) {
    const int h = kh * grp + hh;
    const size_t bh = (size_t)b * Hv + h, cn = gch(a, bh, n);
    __syncthreads();   // the k rows (first head) or the previous head's T are read
    if (w == 0) {
      const TG *g = (const TG *)a.g, *be = (const TG *)a.beta;
      const int tl = min(lane, len - 1);   // past the end: the last token's, zeroed
      const TG gr = g[(row0 + tl) * Hv + h], br = be[(row0 + tl) * Hv + h];
      const float gt = lane < len ? to_f32(gr) : 0.f, bt = lane < len ? to_f32(br) : 0.f;
      const float gm = wave_prefix_sum(gt);
      sg[lane] = gm;
      sb[lane] = bt;
      if (doT) {
        a.gam[cn * C + lane] = gm;
        a.bet[cn * C + lane] = bt;
      }
    }
    __syncthreads();
    float *Ptg = a.Pt + sch(a, bh, n) * C * C;
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      const int j = 16 * J + ln;
      float4v pt;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * w + 4 * g4 + e;
        const float m = i >= j ? __expf(sg[i] - sg[j]) : 0.f;
        sA[i * LC + j] = i > j ? sb[i] * m * kk[J][e] : 0.f;
        pt[e] = m * qk[J][e];
      }
      if (doP) *reinterpret_cast<float4v *>(Ptg + j * C + 16 * w + 4 * g4) = pt;   // P^T[j][i]
    }
    if (!doT) continue;
    __syncthreads();
    solve_T(sA, sT, sX, a.Tm + cn * C * C, tid);
  }
}

// ---------------------------------------------------------------------------
// prep, per-key-channel gate: per (chunk, key head), for each value head of
// the key head: gamma [C][dk] (the prefix sums of g over the chunk, channel by
// channel), beta, the decayed operands K o e^gamma, Q o e^gamma and
// K o e^(gamma_C - gamma), A and P, P^T and T.  A_ij = beta_i sum_c k_ic k_jc
// e^(gamma_ic - gamma_jc) and P_ij = sum_c q_ic k_jc e^(...): in 16 x 16
// blocks about the row block's first token p, as products of
// (k_i o e^(gamma_i - gamma_p)) and (k_j o e^(gamma_p - gamma_j)), both
// factors at most 1 below the diagonal (j < p <= i) and the second at most
// e^kWide on it; a diagonal block whose decay is wider in some channel is
// summed term by term, each factor e^(gamma_ic - gamma_jc) at most 1.
template <typename TQ, typename TG, int DK>
__global__ __launch_bounds__(256) void cb_prep_key_kernel(CbArgs a) {
  constexpr int LK = DK + 4;
  extern __shared__ float4v smem4[];
  float *smem = reinterpret_cast<float *>(smem4);
  float *sK = smem, *sQ = sK + C * LK, *sG = sQ + C * LK, *sA = sG + C * LK, *sT = sA + C * LC;
  float *sb = sT + C * LC;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 15, g4 = lane >> 4;
  float *sX = sb + C + w * 16 * LX;
  const int n = a.c0 + blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int T = a.T, Hk = a.Hk, Hv = a.Hv, grp = Hv / Hk;
  const int t0 = n * C, len = min(C, T - t0);
  const size_t row0 = (size_t)b * T + t0;
  const bool doT = a.flags & kPrepT, doP = a.flags & kPrepP;
  load_rows<TQ, DK>(sK, (const TQ *)a.k, row0 * Hk + kh, Hk, len, tid);
  load_rows<TQ, DK>(sQ, (const TQ *)a.q, row0 * Hk + kh, Hk, len, tid);
  const TG *g = (const TG *)a.g, *be = (const TG *)a.beta;
  for (int hh = 0; hh < grp; ++hh) {
    const int h = kh * grp + hh;
    const size_t bh = (size_t)b * Hv + h, cn = gch(a, bh, n);
    __syncthreads();   // the rows are loaded, or the previous head's reads are done
    if (tid < DK) {
      // gamma_tc = sum_{s <= t} g_sc over the chunk (zero past the end): every
      // token's g requested first (past the end the last token's), then summed
      TG x[C];
#pragma unroll
      for (int t = 0; t < C; ++t) x[t] = g[((row0 + min(t, len - 1)) * Hv + h) * DK + tid];
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < C; ++t) {
        sum += t < len ? to_f32(x[t]) : 0.f;
        sG[t * LK + tid] = sum;
      }
    }
    if (tid < C) {
      const TG bx = be[(row0 + min(tid, len - 1)) * Hv + h];
      sb[tid] = tid < len ? to_f32(bx) : 0.f;
    }
    __syncthreads();
    if (doT) {
      float *gg = a.gam + cn * C * DK, *kh_ = a.Kh + cn * C * DK, *qh_ = a.Qh + cn * C * DK, *kt_ = a.Kt + cn * C * DK;
      for (int u = tid; u < C * DK / 4; u += 256) {
        const int t = u / (DK / 4), c = (u % (DK / 4)) * 4;
        const float4v gm = row4(sG + t * LK + c), gC = row4(sG + (C - 1) * LK + c);
        const float4v kv = row4(sK + t * LK + c), qv = row4(sQ + t * LK + c);
        float4v e1, e2;
#pragma unroll
        for (int e = 0; e < 4; ++e) e1[e] = __expf(gm[e]), e2[e] = __expf(gC[e] - gm[e]);
        *reinterpret_cast<float4v *>(gg + t * DK + c) = gm;
        *reinterpret_cast<float4v *>(kh_ + t * DK + c) = kv * e1;
        *reinterpret_cast<float4v *>(qh_ + t * DK + c) = qv * e1;
        *reinterpret_cast<float4v *>(kt_ + t * DK + c) = kv * e2;
      }
      if (tid < C) a.bet[cn * C + tid] = sb[tid];
    }
    float *Ptg = a.Pt + sch(a, bh, n) * C * C;
    // blocks (w, J <= w): about token p = 16 w; the lane holds i = 16 w + 4 g4 + e, j = 16 J + ln.
    // The diagonal block too unless its decay is wide in some channel.  Channels outer,
    // so that the row side k_i o e^(gamma_i - gamma_p) is formed once for all J.
    const int p = 16 * w;
    float rng = 0.f;
    for (int c = lane; c < DK; c += 64) rng = fmaxf(rng, sG[p * LK + c] - sG[(p + 15) * LK + c]);
    const bool wide = __any(rng > kWide);
    const int nb = wide ? w : w + 1;   // the blocks J < nb go through the matrix cores
    float4v kk[4], qk[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) kk[J] = qk[J] = float4v{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < DK; k += 16) {
      const int kb = k + 4 * g4;
      const float4v gi = row4(sG + (16 * w + ln) * LK + kb), gp = row4(sG + p * LK + kb);
      const float4v ki = row4(sK + (16 * w + ln) * LK + kb), qi = row4(sQ + (16 * w + ln) * LK + kb);
      float4v xk, xq;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float fi = __expf(gi[e] - gp[e]);
        xk[e] = ki[e] * fi;
        xq[e] = qi[e] * fi;
      }
#pragma unroll
      for (int J = 0; J < 4; ++J)
        if (J < nb) {
          const int j = 16 * J + ln;
          const float4v gj = row4(sG + j * LK + kb), kj = row4(sK + j * LK + kb);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float y = kj[e] * __expf(gp[e] - gj[e]);
            if (!a.nd) kk[J] = mma(xk[e], y, kk[J]);   // without the delta correction A = 0, so T = I
            qk[J] = mma(xq[e], y, qk[J]);
          }
        }
    }
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J == w && wide) continue;   // a wide diagonal block is written below
      const int j = 16 * J + ln;
      float4v pt;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * w + 4 * g4 + e;
        sA[i * LC + j] = i > j ? sb[i] * kk[J][e] : 0.f;
        pt[e] = i >= j ? qk[J][e] : 0.f;
      }
      if (doP) *reinterpret_cast<float4v *>(Ptg + j * C + 16 * w + 4 * g4) = pt;   // P^T[j][i]; zero above
    }
    // a wide diagonal block w, term by term: pair m = (i, j) of the block, four per lane
    if (wide) {
      for (int m = lane; m < 256; m += 64) {
        const int il = m >> 4, jl = m & 15, i = 16 * w + il, j = 16 * w + jl;
        float av = 0.f, pv = 0.f;
        if (jl <= il) {
          for (int c = 0; c < DK; c += 4) {
            const float4v gi = row4(sG + i * LK + c), gj = row4(sG + j * LK + c);
            const float4v ki = row4(sK + i * LK + c), qi = row4(sQ + i * LK + c), kj = row4(sK + j * LK + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float f = kj[e] * __expf(gi[e] - gj[e]);
              av = __builtin_fmaf(ki[e], f, av);
              pv = __builtin_fmaf(qi[e], f, pv);
            }
          }
        }
        sA[i * LC + j] = jl < il && !a.nd ? sb[i] * av : 0.f;
        if (doP) Ptg[j * C + i] = pv;
      }
    }
    if (!doT) continue;
    __syncthreads();
    solve_T(sA, sT, sX, a.Tm + cn * C * C, tid);
  }
}

// ---------------------------------------------------------------------------
// The two passes.  A workgroup of NW waves holds 32 state rows r0 .. of one
// (batch, value head), fp32 [32][dk] in matrix-core tiles: wave w the tiles
// w NS .. w NS + NS - 1 (row block id / NCT, column block id % NCT); of the
// [32][C] products, the tiles w ZT .. (row block id / 4, column block id % 4).
// The next chunk's inputs are loaded into registers while the current one is
// worked on, and staged into LDS at the start of the next.
template <typename TQ, int DK>
struct PassCfg {
  static constexpr int NW = DK == 128 ? 8 : 4, NT = 64 * NW;
  static constexpr int LK = DK + 16 / (int)sizeof(TQ);   // q, k rows in LDS, input type
  static constexpr int LS = DK + 4;                        // state rows in LDS, fp32
  static constexpr int NCT = DK / 16, NS = 2 * NCT / NW, ZT = 8 / NW;
};

// f(std::integral_constant<int, zc>) for a 16-token block zc in 0..3 known only
// at run time: one copy of f per block, so that ranges depending on it are
// fixed at compile time
template <typename F>
__device__ __forceinline__ void with_block(int zc, F &&f) {
  switch (zc) {
    case 0: f(std::integral_constant<int, 0>{}); break;
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    default: f(std::integral_constant<int, 3>{}); break;
  }
}

// as mm, over the k blocks lo <= k / 16 < hi only (the rest of A or B is zero)
template <int K, typename FA, typename FB>
__device__ __forceinline__ void mmr(float4v &acc, const FA &fa, const FB &fb, int g4, int lo, int hi) {
#pragma unroll
  for (int k = 0; k < K; k += 16) {
    if (k / 16 < lo || k / 16 >= hi) continue;
    const float4v x = fa(k + 4 * g4), y = fb(k + 4 * g4);
    acc = mma(x[0], y[0], acc);
    acc = mma(x[1], y[1], acc);
    acc = mma(x[2], y[2], acc);
    acc = mma(x[3], y[3], acc);
  }
}

// The task (row slice, value head, batch) of a pass's workgroup.  Workgroups
// go round-robin over the 8 XCDs by their linear index; the row slices of
// one (batch, value head) read the same per-chunk matrices and inputs, so
// each XCD takes a contiguous range of tasks and the slices of a head share
// its L2 (numbered as the grid, x fastest, they would sit on four XCDs and
// fetch those matrices from HBM once each).
__device__ __forceinline__ void pass_task(int &sl, int &h, int &b) {
  const int ns = gridDim.x, nh = gridDim.y, total = ns * nh * gridDim.z;
  const int lin = blockIdx.x + ns * (blockIdx.y + nh * blockIdx.z);
  const int xcd = lin & 7, idx = lin >> 3, per = total >> 3, rem = total & 7;
  const int task = xcd * per + min(xcd, rem) + idx;
  sl = task % ns;
  h = task / ns % nh;
  b = task / ns / nh;
}

// the column block of [32][C] tile z of wave w (row block (w ZT + z) / 4): blocks
// zc and 3 - zc go to waves that share a SIMD (eight waves) or to one wave (four),
// so products over the triangular T and P^T weigh the same on every SIMD
template <int NW, int ZT>
__device__ __forceinline__ int pass_block(int w, int z) {
  const int id = w * ZT + z, rt = id / 4, p = id % 4;
  if constexpr (NW == 8) return rt == 0 ? p : 3 - p;
  else return p == 0 ? 0 : p == 1 ? 3 : p == 2 ? 1 : 2;
}

// C rows of DK elements of q or k (zeros past the sequence's end), raw, in
// 16-byte units spread over the NT threads.
template <typename TQ, int DK, int NT>
struct RowsReg {
  static constexpr int UPR = DK * (int)sizeof(TQ) / 16, NU = C * UPR / NT;
  uint4 u[NU];
  __device__ __forceinline__ void load(const TQ *row0, size_t stride, int len, int tid) {
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int x = tid + i * NT, t = x / UPR, cu = x % UPR;
      u[i] = t < len ? *reinterpret_cast<const uint4 *>(row0 + (size_t)t * stride + cu * (16 / sizeof(TQ)))
                     : uint4{0u, 0u, 0u, 0u};
    }
  }
  template <int LK>
  __device__ __forceinline__ void store(TQ *s, int tid) const {
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int x = tid + i * NT, t = x / UPR, cu = x % UPR;
      *reinterpret_cast<uint4 *>(s + t * LK + cu * (16 / sizeof(TQ))) = u[i];
    }
  }
};

// a [C][C] fp32 matrix of the workspace
template <int NT>
struct CcReg {
  static constexpr int NU = C * C / 4 / NT;
  float4v u[NU];
  __device__ __forceinline__ void load(const float *src, int tid) {
#pragma unroll
    for (int i = 0; i < NU; ++i) u[i] = *reinterpret_cast<const float4v *>(src + 4 * (tid + i * NT));
  }
  __device__ __forceinline__ void store(float *s, int tid) const {
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int x = tid + i * NT;
      *reinterpret_cast<float4v *>(s + (x / (C / 4)) * LC + (x % (C / 4)) * 4) = u[i];
    }
  }
};

// four consecutive input elements, raw until used
// LDS reads of input-type rows: four consecutive entries, four rows of a column
template <typename TQ>
__device__ __forceinline__ float4v rowq(const TQ *p) {
  float x[4];
  load4(p, x);
  return float4v{x[0], x[1], x[2], x[3]};
}
template <typename TQ>
__device__ __forceinline__ float4v colq(const TQ *p, int ld) {
  return float4v{to_f32(p[0]), to_f32(p[ld]), to_f32(p[2 * ld]), to_f32(p[3 * ld])};
}

// the chunk's gate inputs (thread t < C: gamma_t, gamma_C, beta_t), and their LDS form
struct GateReg {
  float g, gC, b;
  __device__ __forceinline__ void load(const CbArgs &a, size_t cn, int tid) {
    if (tid < C) {
      g = a.gam[cn * C + tid];
      gC = a.gam[cn * C + C - 1];
      b = a.bet[cn * C + tid];
    }
  }
  __device__ __forceinline__ void store(float *sEg, float *sEc, float *sb, int tid) const {
    if (tid < C) {
      sEg[tid] = __expf(g);
      sEc[tid] = __expf(gC - g);
      sb[tid] = b;
    }
  }
};

// a [C][DK] fp32 matrix of the workspace (the key gate's decayed operands), into
// LDS rows of DK + 4
template <int DK, int NT>
struct CkReg {
  static constexpr int NU = C * DK / 4 / NT;
  float4v u[NU];
  __device__ __forceinline__ void load(const float *src, int tid) {
#pragma unroll
    for (int i = 0; i < NU; ++i) u[i] = *reinterpret_cast<const float4v *>(src + 4 * (tid + i * NT));
  }
  __device__ __forceinline__ void store(float *s, int tid) const {
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int x = tid + i * NT;
      *reinterpret_cast<float4v *>(s + (x / (DK / 4)) * (DK + 4) + (x % (DK / 4)) * 4) = u[i];
    }
  }
};

// the key gate's chunk scalars: beta_t (thread t < C) and e^gamma_C per channel (thread c < DK)
template <int DK>
struct KeyGateReg {
  float b, gC;
  __device__ __forceinline__ void load(const CbArgs &a, size_t cn, int tid) {
    if (tid < C) b = a.bet[cn * C + tid];
    if (tid < DK) gC = a.gam[(cn * C + C - 1) * DK + tid];
  }
  __device__ __forceinline__ void store(float *sb, float *sEC, int tid) const {
    if (tid < C) sb[tid] = b;
    if (tid < DK) sEC[tid] = __expf(gC);
  }
};

// forward pass, over the chunks in order: the state before each chunk and U.
// Key gate (KEY): K o e^gamma and K o e^(gamma_C - gamma) from the prep in
// place of k, and the state's columns decay by e^gamma_C,c.
template <typename TQ, int DK, bool KEY>
__global__ __launch_bounds__((PassCfg<TQ, DK>::NT)) void cb_fwd_kernel(CbArgs a) {
  using P = PassCfg<TQ, DK>;
  constexpr int LK = P::LK, LS = P::LS, NCT = P::NCT, NS = P::NS, ZT = P::ZT, NT = P::NT;
  extern __shared__ float4v smem4[];
  TQ *sK = reinterpret_cast<TQ *>(smem4);
  float *sKh = reinterpret_cast<float *>(smem4), *sKt = sKh + C * LS;   // key gate
  float *sT = KEY ? sKt + C * LS : reinterpret_cast<float *>(sK + C * LK);
  float *sS = sT + C * LC, *sX = sS + R * LS, *sU = sX + R * LC;
  float *sEg = sU + R * LC, *sEc = sEg + C, *sb = sEc + C, *sEC = sb + C;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 15, g4 = lane >> 4;
  int sl, h, b;
  pass_task(sl, h, b);
  const int T = a.T, Hk = a.Hk, Hv = a.Hv, DV = a.dv_dim, kh = h / (Hv / Hk), r0 = sl * R;
  const size_t bh = (size_t)b * Hv + h;
  const TQ *k = (const TQ *)a.k, *v = (const TQ *)a.v;
  int srt[NS], sct[NS], zrt[ZT], zcc[ZT];
#pragma unroll
  for (int s = 0; s < NS; ++s) srt[s] = (w * NS + s) / NCT, sct[s] = (w * NS + s) % NCT;
#pragma unroll
  for (int z = 0; z < ZT; ++z) zrt[z] = (w * ZT + z) / 4, zcc[z] = pass_block<P::NW, ZT>(w, z);
  const bool so = a.flags & kStatesOnly;
  // the state before the range: S0, or the kept state of the segment that starts it
  const float *Sin = a.c0 == 0 ? a.S0 : a.Sseg + (bh * a.nseg + a.c0 / a.ncs) * DV * DK;
  float4v S[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[s][e] = Sin ? Sin[(r0 + 16 * srt[s] + 4 * g4 + e) * DK + 16 * sct[s] + ln + (a.c0 == 0 ? bh * DV * DK : 0)]
                    : 0.f;
  auto keep_state = [&](int sg) {   // the state before segment sg's first chunk
    float *Sg = a.Sseg + (bh * a.nseg + sg) * DV * DK;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) Sg[(r0 + 16 * srt[s] + 4 * g4 + e) * DK + 16 * sct[s] + ln] = S[s][e];
  };
  RowsReg<TQ, DK, NT> kr;
  CkReg<DK, NT> khr, ktr;
  CcReg<NT> tr;
  GateReg gr;
  KeyGateReg<DK> kgr;
  typename Quad<TQ>::type vq[ZT];
  auto fetch = [&](int n) {
    const int t0 = n * C, len = min(C, T - t0);
    const size_t cn = gch(a, bh, n), row0 = (size_t)b * T + t0;
    if constexpr (KEY) {
      khr.load(a.Kh + cn * C * DK, tid);
      ktr.load(a.Kt + cn * C * DK, tid);
      kgr.load(a, cn, tid);
    } else {
      kr.load(k + (row0 * Hk + kh) * DK, (size_t)Hk * DK, len, tid);
      gr.load(a, cn, tid);
    }
    tr.load(a.Tm + cn * C * C, tid);
#pragma unroll
    for (int z = 0; z < ZT; ++z) {
      const int t = 16 * zcc[z] + ln;
      vq[z] = t < len ? quad_load(v + ((row0 + t) * Hv + h) * DV + r0 + 16 * zrt[z] + 4 * g4)
                      : typename Quad<TQ>::type{};
    }
  };
  fetch(a.c0);
  for (int n = a.c0; n < a.c1; ++n) {
    if constexpr (KEY) {
      khr.store(sKh, tid);
      ktr.store(sKt, tid);
      kgr.store(sb, sEC, tid);
    } else {
      kr.template store<LK>(sK, tid);
      gr.store(sEg, sEc, sb, tid);
    }
    tr.store(sT, tid);
    float4v vx[ZT];
#pragma unroll
    for (int z = 0; z < ZT; ++z) vx[z] = quad_to_f32<TQ>(vq[z]);
    if (so && n > 0 && n % a.ncs == 0) keep_state(n / a.ncs);
    float *S0g = a.S0s + (sch(a, bh, n) * DV + r0) * DK;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * srt[s] + 4 * g4 + e, c = 16 * sct[s] + ln;
        sS[r * LS + c] = S[s][e];
        if (!so) S0g[r * DK + c] = S[s][e];
      }
    lds_barrier();
    if (n + 1 < a.c1) fetch(n + 1);
    // X^T[r][t] = beta_t (v_t[r] - e^gamma_t (S k_t)[r])
#pragma unroll
    for (int z = 0; z < ZT; ++z) {
      const int rt = zrt[z], t = 16 * zcc[z] + ln;
      float4v acc = {0.f, 0.f, 0.f, 0.f};
      if (!a.nd)
        mm<DK>(acc, [&](int kk) { return row4(sS + (16 * rt + ln) * LS + kk); },
               [&](int kk) {
                 if constexpr (KEY) return row4(sKh + t * LS + kk);   // (k o e^gamma)_t
                 else return rowq(sK + t * LK + kk);
               }, g4);
      const float eg = KEY ? 1.f : sEg[t], bt = sb[t];
#pragma unroll
      for (int e = 0; e < 4; ++e) sX[(16 * rt + 4 * g4 + e) * LC + t] = bt * (vx[z][e] - eg * acc[e]);
    }
    lds_barrier();
    // U^T[r][i] = sum_j X^T[r][j] T[i][j]; U to the workspace, U^T e^(gamma_C - gamma_i) to LDS
#pragma unroll
    for (int z = 0; z < ZT; ++z) {
      const int rt = zrt[z], i = 16 * zcc[z] + ln;
      float4v u = {0.f, 0.f, 0.f, 0.f};
      // T[i][j] is zero for j > i: key blocks up to i's
      with_block(zcc[z], [&](auto ZC) {
        mmr<C>(u, [&](int kk) { return row4(sX + (16 * rt + ln) * LC + kk); },
               [&](int kk) { return row4(sT + i * LC + kk); }, g4, 0, decltype(ZC)::value + 1);
      });
      if (!so) *reinterpret_cast<float4v *>(a.Um + (sch(a, bh, n) * C + i) * DV + r0 + 16 * rt + 4 * g4) = u;
      const float ec = KEY ? 1.f : sEc[i];   // the key gate's decay is in K o e^(gamma_C - gamma)
#pragma unroll
      for (int e = 0; e < 4; ++e) sU[(16 * rt + 4 * g4 + e) * LC + i] = u[e] * ec;
    }
    lds_barrier();
    // S <- e^gamma_C S + sum_j U~^T[r][j] k_j (key gate: S diag(e^gamma_C) + U^T (K o e^(gamma_C - gamma)))
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int rt = srt[s], c = 16 * sct[s] + ln;
      S[s] *= KEY ? sEC[c] : sEg[C - 1];
      mm<C>(S[s], [&](int kk) { return row4(sU + (16 * rt + ln) * LC + kk); },
            [&](int kk) {
              if constexpr (KEY) return col4(sKt + kk * LS + c, LS);
              else return colq(sK + kk * LK + c, LK);
            }, g4);
    }
    lds_barrier();
  }
  if (so) keep_state(a.c1 / a.ncs);
}

// backward pass, over the chunks in reverse: the state gradient after each
// chunk, E, dv, and dS0 at the end.  Key gate (KEY): K o e^(gamma_C - gamma)
// in place of the decayed k of dU, K o e^gamma and Q o e^gamma in place of
// the decayed k and q of the state gradient's update; K o e^(gamma_C - gamma)
// is read only before the first barrier of a chunk, so Q o e^gamma is written
// over it after that barrier (and its next chunk loaded after that).
template <typename TQ, int DK, bool KEY>
__global__ __launch_bounds__((PassCfg<TQ, DK>::NT)) void cb_bwd_kernel(CbArgs a) {
  using P = PassCfg<TQ, DK>;
  constexpr int LK = P::LK, LS = P::LS, NCT = P::NCT, NS = P::NS, ZT = P::ZT, NT = P::NT;
  extern __shared__ float4v smem4[];
  TQ *sK = reinterpret_cast<TQ *>(smem4), *sQ = sK + C * LK;
  float *sKtQ = reinterpret_cast<float *>(smem4), *sKh = sKtQ + C * LS;   // key gate
  float *sT = KEY ? sKh + C * LS : reinterpret_cast<float *>(sQ + C * LK);
  float *sP = sT + C * LC, *sO = sP + C * LC, *sS = sO + C * LR, *sD = sS + R * LS, *sE = sD + R * LC;
  float *sEg = sE + R * LC, *sEc = sEg + C, *sb = sEc + C, *sEC = sb + C;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 15, g4 = lane >> 4;
  int sl, h, b;
  pass_task(sl, h, b);
  const int T = a.T, Hk = a.Hk, Hv = a.Hv, DV = a.dv_dim, kh = h / (Hv / Hk), r0 = sl * R;
  const size_t bh = (size_t)b * Hv + h;
  const TQ *k = (const TQ *)a.k, *q = (const TQ *)a.q;
  int srt[NS], sct[NS], zrt[ZT], zcc[ZT];
#pragma unroll
  for (int s = 0; s < NS; ++s) srt[s] = (w * NS + s) / NCT, sct[s] = (w * NS + s) % NCT;
#pragma unroll
  for (int z = 0; z < ZT; ++z) zrt[z] = (w * ZT + z) / 4, zcc[z] = pass_block<P::NW, ZT>(w, z);
  float4v dS[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dS[s][e] = a.dS_in ? a.dS_in[(bh * DV + r0 + 16 * srt[s] + 4 * g4 + e) * DK + 16 * sct[s] + ln] : 0.f;
  RowsReg<TQ, DK, NT> kr, qr;
  CkReg<DK, NT> ktr, khr, qhr;
  CcReg<NT> tr, pr;
  GateReg gr;
  KeyGateReg<DK> kgr;
  constexpr int NO = C * R / 4 / NT;   // dO: 16-byte units per thread
  float4v orr[NO];
  auto fetch = [&](int n) {   // all but the key gate's Q o e^gamma
    const int t0 = n * C, len = min(C, T - t0);
    const size_t cn = gch(a, bh, n), row0 = (size_t)b * T + t0;
    if constexpr (KEY) {
      ktr.load(a.Kt + cn * C * DK, tid);
      khr.load(a.Kh + cn * C * DK, tid);
      kgr.load(a, cn, tid);
    } else {
      kr.load(k + (row0 * Hk + kh) * DK, (size_t)Hk * DK, len, tid);
      qr.load(q + (row0 * Hk + kh) * DK, (size_t)Hk * DK, len, tid);
      gr.load(a, cn, tid);
    }
    tr.load(a.Tm + cn * C * C, tid);
    pr.load(a.Pt + sch(a, bh, n) * C * C, tid);
#pragma unroll
    for (int i = 0; i < NO; ++i) {
      const int x = tid + i * NT, t = x / (R / 4), r = (x % (R / 4)) * 4;
      orr[i] = t < len ? *reinterpret_cast<const float4v *>(a.dO + ((row0 + t) * Hv + h) * DV + r0 + r)
                       : float4v{0.f, 0.f, 0.f, 0.f};
    }
  };
  fetch(a.c1 - 1);
  if constexpr (KEY) qhr.load(a.Qh + gch(a, bh, a.c1 - 1) * C * DK, tid);
  for (int n = a.c1 - 1; n >= a.c0; --n) {
    const int t0 = n * C, len = min(C, T - t0);
    const size_t cn = sch(a, bh, n), row0 = (size_t)b * T + t0;
    if constexpr (KEY) {
      ktr.store(sKtQ, tid);
      khr.store(sKh, tid);
      kgr.store(sb, sEC, tid);
    } else {
      kr.template store<LK>(sK, tid);
      qr.template store<LK>(sQ, tid);
      gr.store(sEg, sEc, sb, tid);
    }
    tr.store(sT, tid);
    pr.store(sP, tid);
#pragma unroll
    for (int i = 0; i < NO; ++i) {
      const int x = tid + i * NT;
      *reinterpret_cast<float4v *>(sO + (x / (R / 4)) * LR + (x % (R / 4)) * 4) = orr[i];
    }
    float *dSg = a.dSC + (cn * DV + r0) * DK;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * srt[s] + 4 * g4 + e, c = 16 * sct[s] + ln;
        sS[r * LS + c] = dS[s][e];
        dSg[r * DK + c] = dS[s][e];
      }
    lds_barrier();
    if (n > a.c0) fetch(n - 1);
    // dU^T[r][i] = e^(gamma_C - gamma_i) (dS k_i)[r] + sum_j dO[j][r] P[j][i]
#pragma unroll
    for (int z = 0; z < ZT; ++z) {
      const int rt = zrt[z], i = 16 * zcc[z] + ln;
      float4v acc = {0.f, 0.f, 0.f, 0.f};
      mm<DK>(acc, [&](int kk) { return row4(sS + (16 * rt + ln) * LS + kk); },
             [&](int kk) {
               if constexpr (KEY) return row4(sKtQ + i * LS + kk);   // (k o e^(gamma_C - gamma))_i
               else return rowq(sK + i * LK + kk);
             }, g4);
      if constexpr (!KEY) acc *= sEc[i];
      // P[j][i] is zero for j < i: token blocks from i's
      with_block(zcc[z], [&](auto ZC) {
        mmr<C>(acc, [&](int kk) { return col4(sO + kk * LR + 16 * rt + ln, LR); },
               [&](int kk) { return row4(sP + i * LC + kk); }, g4, decltype(ZC)::value, 4);
      });
#pragma unroll
      for (int e = 0; e < 4; ++e) sD[(16 * rt + 4 * g4 + e) * LC + i] = acc[e];
    }
    lds_barrier();
    if constexpr (KEY) {   // Q o e^gamma over K o e^(gamma_C - gamma), then the next chunk's
      qhr.store(sKtQ, tid);
      if (n > a.c0) qhr.load(a.Qh + gch(a, bh, n - 1) * C * DK, tid);
    }
    // E^T[r][i] = sum_j dU^T[r][j] T[j][i]; dv = beta E; -beta e^gamma E^T to LDS
#pragma unroll
    for (int z = 0; z < ZT; ++z) {
      const int rt = zrt[z], i = 16 * zcc[z] + ln;
      float4v E = {0.f, 0.f, 0.f, 0.f};
      // T[j][i] is zero for j < i: token blocks from i's
      with_block(zcc[z], [&](auto ZC) {
        mmr<C>(E, [&](int kk) { return row4(sD + (16 * rt + ln) * LC + kk); },
               [&](int kk) { return col4(sT + kk * LC + i, LC); }, g4, decltype(ZC)::value, 4);
      });
      const float bi = sb[i];
      if (i < len)
        *reinterpret_cast<float4v *>(a.dv + ((row0 + i) * Hv + h) * DV + r0 + 16 * rt + 4 * g4) = E * bi;
      *reinterpret_cast<float4v *>(a.Em + (cn * C + i) * DV + r0 + 16 * rt + 4 * g4) = E;
      const float f = KEY ? -bi : -bi * sEg[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) sE[(16 * rt + 4 * g4 + e) * LC + i] = E[e] * f;
    }
    lds_barrier();
    // dS <- e^gamma_C dS + sum_t dO[t][r] e^gamma_t q_t - sum_t beta_t e^gamma_t E[t][r] k_t
    // (key gate: dS diag(e^gamma_C) + dO^T (Q o e^gamma) - (beta E)^T (K o e^gamma))
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int rt = srt[s], c = 16 * sct[s] + ln;
      if constexpr (KEY) {
        dS[s] *= sEC[c];
        mm<C>(dS[s], [&](int kk) { return col4(sO + kk * LR + 16 * rt + ln, LR); },
              [&](int kk) { return col4(sKtQ + kk * LS + c, LS); }, g4);
        if (!a.nd)
          mm<C>(dS[s], [&](int kk) { return row4(sE + (16 * rt + ln) * LC + kk); },
                [&](int kk) { return col4(sKh + kk * LS + c, LS); }, g4);
      } else {
        dS[s] *= sEg[C - 1];
        mm<C>(dS[s], [&](int kk) { return col4(sO + kk * LR + 16 * rt + ln, LR) * row4(sEg + kk); },
              [&](int kk) { return colq(sQ + kk * LK + c, LK); }, g4);
        if (!a.nd)   // X = beta V does not depend on the state without the delta correction
          mm<C>(dS[s], [&](int kk) { return row4(sE + (16 * rt + ln) * LC + kk); },
                [&](int kk) { return colq(sK + kk * LK + c, LK); }, g4);
      }
    }
    lds_barrier();
  }
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      a.dS0[(bh * DV + r0 + 16 * srt[s] + 4 * g4 + e) * DK + 16 * sct[s] + ln] = dS[s][e];
}

// ---------------------------------------------------------------------------
// gradients of one (chunk, key head): for each value head of the key head,
// the products over the value rows in slices of 32 (dP = dO U^T, E U^T,
// dO S0, E S0, U dS_C), then the products with the masked C x C matrices
// and the row dots; dq and dk summed over the value heads.  Eight waves
// (four for dk < 128 and for the key gate): wave w holds token block w & 3 of every [C][.]
// product, and half w >> 2 of its column blocks.  The next slice is loaded
// into registers while the current one is worked on.
template <typename TQ, int DK, bool KEY = false>
struct GradCfg {
  // the key gate runs four waves at dk 128 too, one per SIMD, so that each
  // has the whole register file: its per-channel terms spill 352 bytes per
  // lane with four waves against 448 with eight (backward 4.42 vs 4.49 ms)
  static constexpr int NW = DK == 128 && !KEY ? 8 : 4, NT = 64 * NW, NH = NW / 4;   // column halves
  static constexpr int LK = DK + 4, NCT = DK / 16, HCT = NCT / NH, HJ = 4 / NH;
  // the key gate keeps gamma [C][dk] after the two masked matrices
  static constexpr int SLICE = 3 * C * LR + 2 * R * LK, MASKS = 2 * C * LC + (KEY ? C * LK : 0);
  static constexpr int REGION = SLICE > MASKS ? SLICE : MASKS;
  static constexpr int NC4 = C * R / 4 / NT, NS4 = R * DK / 4 / NT;   // 16-byte units per thread
  static constexpr int NV = 8 * C / NT;                                 // (token, 4 rows) units of E . v
  static constexpr int smem = (2 * C * LK + REGION + (4 + 3 * NH) * C + 2 * NW + (KEY ? (NW + 4) * DK : 0)) * 4;
};

// acc1 += A1 B^T, acc2 += A2 B^T (one read of B), over the k blocks lo <= k / 16 < hi
template <int K, typename FA1, typename FA2, typename FB>
__device__ __forceinline__ void mm2r(float4v &acc1, float4v &acc2, const FA1 &fa1, const FA2 &fa2, const FB &fb,
                                     int g4, int lo, int hi) {
#pragma unroll
  for (int k = 0; k < K; k += 16) {
    if (k / 16 < lo || k / 16 >= hi) continue;
    const float4v x1 = fa1(k + 4 * g4), x2 = fa2(k + 4 * g4), y = fb(k + 4 * g4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc1 = mma(x1[e], y[e], acc1);
      acc2 = mma(x2[e], y[e], acc2);
    }
  }
}

// acc1 += A1 B^T, acc2 += A2 B^T (one read of B)
template <int K, typename FA1, typename FA2, typename FB>
__device__ __forceinline__ void mm2(float4v &acc1, float4v &acc2, const FA1 &fa1, const FA2 &fa2, const FB &fb,
                                    int g4) {
#pragma unroll
  for (int k = 0; k < K; k += 16) {
    const float4v x1 = fa1(k + 4 * g4), x2 = fa2(k + 4 * g4), y = fb(k + 4 * g4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc1 = mma(x1[e], y[e], acc1);
      acc2 = mma(x2[e], y[e], acc2);
    }
  }
}

// The masked products of a diagonal 16-token block p .. p + 15 in channel c, term
// by term (each factor e^(gamma_i - gamma_j), i >= j, at most 1; masked entries
// are zero and their factor is clamped to 1): rows p + 4 g4 + e of
// sum_j dP_ij k_j e^.., sum_j B_ij k_j e^.., and of the transposed sums with q_i
// and beta_i k_i.  Out of line: only blocks whose decay is too wide for the
// matrix-core form take it.
struct Diag4 {
  float4v q2, f1, k1, f2;
};
template <int LK>
__device__ __noinline__ Diag4 wide_diagonal(const float *sdP, const float *sB, const float *sK, const float *sQ,
                                            const float *sG, const float *sb, int p, int c, int g4) {
  float gi[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) gi[e] = sG[(p + 4 * g4 + e) * LK + c];
  Diag4 d;
  d.q2 = d.f1 = d.k1 = d.f2 = float4v{0.f, 0.f, 0.f, 0.f};
  for (int j = p; j < p + 16; ++j) {
    const float kj = sK[j * LK + c], gj = sG[j * LK + c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = p + 4 * g4 + e;
      const float f = kj * __expf(fminf(gi[e] - gj, 0.f));
      d.q2[e] = __builtin_fmaf(sdP[i * LC + j], f, d.q2[e]);
      d.f1[e] = __builtin_fmaf(sB[i * LC + j], f, d.f1[e]);
    }
  }
  for (int i = p; i < p + 16; ++i) {
    const float qi = sQ[i * LK + c], ki = sK[i * LK + c] * sb[i], gv = sG[i * LK + c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = p + 4 * g4 + e;
      const float f = __expf(fminf(gv - gi[e], 0.f));
      d.k1[e] = __builtin_fmaf(sdP[i * LC + j], qi * f, d.k1[e]);
      d.f2[e] = __builtin_fmaf(sB[i * LC + j], ki * f, d.f2[e]);
    }
  }
  return d;
}

template <typename TQ, typename TG, int DK, bool ND, bool KEY>
__global__ __launch_bounds__((GradCfg<TQ, DK, KEY>::NT)) void cb_grads_kernel(CbArgs a) {
  using G = GradCfg<TQ, DK, KEY>;
  constexpr int LK = G::LK, NT = G::NT, NH = G::NH, HCT = G::HCT, HJ = G::HJ, NC4 = G::NC4, NS4 = G::NS4;
  constexpr int NV = G::NV;
  extern __shared__ float4v smem4[];
  float *smem = reinterpret_cast<float *>(smem4);
  float *sK = smem, *sQ = sK + C * LK, *rg = sQ + C * LK;
  float *sO = rg, *sU = sO + C * LR, *sE = sU + C * LR, *sS0 = sE + C * LR, *sdS = sS0 + R * LK;
  float *sdP = rg, *sB = sdP + C * LC;
  float *sEg = rg + G::REGION, *sEc = sEg + C, *sb = sEc + C, *sg = sb + C;
  float *sGam = sg + C, *sBet = sGam + NH * C, *sBx = sBet + NH * C, *sRed = sBx + NH * C;
  // key gate: gamma [C][dk] after the masked matrices, and the per-channel gradient of
  // gamma over them once they are read; per-wave channel sums of dS_C o S0 and of k o dk4
  float *sG = sB + C * LC, *sGp = rg, *sSd = sRed + 2 * G::NW, *sKd = sSd + G::NW * DK;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 15, g4 = lane >> 4;
  const int tw = w & 3, hw = w >> 2, ct0 = hw * HCT, J0 = hw * HJ;
  const int n = a.c0 + blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int T = a.T, Hk = a.Hk, Hv = a.Hv, DV = a.dv_dim, grp = Hv / Hk;
  const int t0 = n * C, len = min(C, T - t0);
  const size_t row0 = (size_t)b * T + t0;
  const TQ *v = (const TQ *)a.v;
  {   // k and q rows, fp32; every load issued first (past the end the last row's, zeroed)
    constexpr int NU = C * DK / 8 / NT;
    static_assert(C * DK / 8 % NT == 0, "whole units per thread");
    typename Quad<TQ>::type x[NU][4];
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = tid + i * NT, t = min(u / (DK / 8), len - 1), c = (u % (DK / 8)) * 8;
      const size_t o = ((row0 + t) * Hk + kh) * DK + c;
      x[i][0] = quad_load((const TQ *)a.k + o);
      x[i][1] = quad_load((const TQ *)a.k + o + 4);
      x[i][2] = quad_load((const TQ *)a.q + o);
      x[i][3] = quad_load((const TQ *)a.q + o + 4);
    }
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = tid + i * NT, t = u / (DK / 8), c = (u % (DK / 8)) * 8;
      const float4v z = {0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<float4v *>(sK + t * LK + c) = t < len ? quad_to_f32<TQ>(x[i][0]) : z;
      *reinterpret_cast<float4v *>(sK + t * LK + c + 4) = t < len ? quad_to_f32<TQ>(x[i][1]) : z;
      *reinterpret_cast<float4v *>(sQ + t * LK + c) = t < len ? quad_to_f32<TQ>(x[i][2]) : z;
      *reinterpret_cast<float4v *>(sQ + t * LK + c + 4) = t < len ? quad_to_f32<TQ>(x[i][3]) : z;
    }
  }
  // slice registers: dO, U, E [C][32] and S0, dS_C [32][dk], and v for E . v; the
  // loads take a uniform base per (head, slice) and 32-bit offsets per thread
  float4v ro[NC4], ru[NC4], re[NC4], rs[NS4], rd[NS4];
  typename Quad<TQ>::type rv[NV];
  // E . v: unit tid + i NT is token (tid + i NT) / 8, rows 4 ((tid + i NT) % 8) ..
  auto vtok = [&](int i) { return (tid + i * NT) >> 3; };
  const int vr = (tid & 7) * 4;
  auto fetch = [&](int h, int r0) {
    const size_t cn = sch(a, (size_t)b * Hv + h, n);
    const float *pO = a.dO + (row0 * Hv + h) * DV + r0, *pU = a.Um + cn * C * DV + r0, *pE = a.Em + cn * C * DV + r0;
    const float *pS = a.S0s + (cn * DV + r0) * DK, *pD = a.dSC + (cn * DV + r0) * DK;
#pragma unroll
    for (int i = 0; i < NC4; ++i) {
      const int x = tid + i * NT, t = x / (R / 4), r = (x % (R / 4)) * 4;
      ro[i] = t < len ? *reinterpret_cast<const float4v *>(pO + (t * Hv * DV + r)) : float4v{0.f, 0.f, 0.f, 0.f};
      ru[i] = *reinterpret_cast<const float4v *>(pU + (t * DV + r));
      re[i] = *reinterpret_cast<const float4v *>(pE + (t * DV + r));
    }
#pragma unroll
    for (int i = 0; i < NS4; ++i) {
      const int x = tid + i * NT;
      rs[i] = *reinterpret_cast<const float4v *>(pS + 4 * x);
      rd[i] = *reinterpret_cast<const float4v *>(pD + 4 * x);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (vtok(i) < len) rv[i] = quad_load(v + (row0 * Hv + h) * DV + r0 + (vtok(i) * Hv * DV + vr));
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < NC4; ++i) {
      const int x = tid + i * NT, t = x / (R / 4), r = (x % (R / 4)) * 4;
      *reinterpret_cast<float4v *>(sO + t * LR + r) = ro[i];
      *reinterpret_cast<float4v *>(sU + t * LR + r) = ru[i];
      *reinterpret_cast<float4v *>(sE + t * LR + r) = re[i];
    }
#pragma unroll
    for (int i = 0; i < NS4; ++i) {
      const int x = tid + i * NT, r = x / (DK / 4), c = (x % (DK / 4)) * 4;
      *reinterpret_cast<float4v *>(sS0 + r * LK + c) = rs[i];
      *reinterpret_cast<float4v *>(sdS + r * LK + c) = rd[i];
    }
  };
  float4v dQa[HCT], dKa[HCT];
#pragma unroll
  for (int c = 0; c < HCT; ++c) dQa[c] = dKa[c] = float4v{0.f, 0.f, 0.f, 0.f};
  const int nsl = DV / R;
  fetch(kh * grp, 0);
  for (int hh = 0; hh < grp; ++hh) {
    const int h = kh * grp + hh;
    const size_t cn = gch(a, (size_t)b * Hv + h, n);
    float4v dPa[HJ], dAa[HJ], Q1[HCT], ES[HCT], UD[HCT];
#pragma unroll
    for (int J = 0; J < HJ; ++J) dPa[J] = dAa[J] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < HCT; ++c) Q1[c] = ES[c] = UD[c] = float4v{0.f, 0.f, 0.f, 0.f};
    float dbx[NV], sdot = 0.f;
    float4v sd4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NV; ++i) dbx[i] = 0.f;
    for (int si = 0; si < nsl; ++si) {
      lds_barrier();   // the previous slice's (or head's) reads of the region are done
      stage();
      float4v vx[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) vx[i] = quad_to_f32<TQ>(rv[i]);
      if (si == 0) {
        if constexpr (KEY) {
          if (tid < C) sb[tid] = a.bet[cn * C + tid];
        } else {
          load_gates(sEg, sEc, sb, a, cn, tid, sg);
        }
      }
      lds_barrier();
      // the next slice, or the next head's first
      if (si + 1 < nsl)
        fetch(h, (si + 1) * R);
      else if (hh + 1 < grp)
        fetch(h + 1, 0);
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (vtok(i) < len) {
          const float4v ev = row4(sE + vtok(i) * LR + vr);
          dbx[i] += ev[0] * vx[i][0] + ev[1] * vx[i][1] + ev[2] * vx[i][2] + ev[3] * vx[i][3];
        }
#pragma unroll
      for (int i = 0; i < NS4; ++i) {
        const int x = tid + i * NT, r = x / (DK / 4), c = (x % (DK / 4)) * 4;
        const float4v p = row4(sS0 + r * LK + c) * row4(sdS + r * LK + c);
        if constexpr (KEY) sd4 += p;   // the thread's channels are the same in every unit
        else sdot += (p[0] + p[1]) + (p[2] + p[3]);
      }
      // without the delta correction A and X do not depend on k or the state: no E U^T, no E S0
#pragma unroll
      for (int J = 0; J < HJ; ++J) {
        if constexpr (ND)
          mm<R>(dPa[J], [&](int k) { return row4(sO + (16 * tw + ln) * LR + k); },
                [&](int k) { return row4(sU + (16 * (J0 + J) + ln) * LR + k); }, g4);
        else
          mm2<R>(dPa[J], dAa[J], [&](int k) { return row4(sO + (16 * tw + ln) * LR + k); },
                 [&](int k) { return row4(sE + (16 * tw + ln) * LR + k); },
                 [&](int k) { return row4(sU + (16 * (J0 + J) + ln) * LR + k); }, g4);
      }
#pragma unroll
      for (int ct = 0; ct < HCT; ++ct) {
        const int c = 16 * (ct0 + ct) + ln;
        if constexpr (ND)
          mm<R>(Q1[ct], [&](int k) { return row4(sO + (16 * tw + ln) * LR + k); },
                [&](int k) { return col4(sS0 + k * LK + c, LK); }, g4);
        else
          mm2<R>(Q1[ct], ES[ct], [&](int k) { return row4(sO + (16 * tw + ln) * LR + k); },
                 [&](int k) { return row4(sE + (16 * tw + ln) * LR + k); },
                 [&](int k) { return col4(sS0 + k * LK + c, LK); }, g4);
        mm<R>(UD[ct], [&](int k) { return row4(sU + (16 * tw + ln) * LR + k); },
              [&](int k) { return col4(sdS + k * LK + c, LK); }, g4);
        __builtin_amdgcn_sched_barrier(0);   // one tile's operands live at a time
      }
    }
    if constexpr (KEY) {
      lds_barrier();
      int kln = ln, kg4 = g4;   // opaque per head: no lane address is hoisted out of the head loop
      asm volatile("" : "+v"(kln), "+v"(kg4));
      // dP and B = dA = -E U^T, masked only: the decay is per channel, in the
      // products below; gamma [C][dk] of the head after them
#pragma unroll
      for (int J = 0; J < HJ; ++J) {
        const int j = 16 * (J0 + J) + kln;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * tw + 4 * kg4 + e;
          sdP[i * LC + j] = i >= j ? dPa[J][e] : 0.f;
          sB[i * LC + j] = i > j ? -dAa[J][e] : 0.f;
        }
      }
      for (int u = tid; u < C * DK / 4; u += NT)
        *reinterpret_cast<float4v *>(sG + (u / (DK / 4)) * LK + (u % (DK / 4)) * 4) =
            *reinterpret_cast<const float4v *>(a.gam + cn * C * DK + 4 * u);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const float x = group_sum<8>(dbx[i]);
        if ((tid & 7) == 0) sBx[vtok(i)] = x;
      }
      // <dS_C, S0> per channel: lanes of one lane % (dk / 4) hold the same four channels
#pragma unroll
      for (int m = DK / 4; m < 64; m <<= 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) sd4[e] += __shfl_xor(sd4[e], m, 64);
      if (lane < DK / 4) *reinterpret_cast<float4v *>(sSd + w * DK + 4 * lane) = sd4;
      lds_barrier();
      // the slice products' shares of dq, dk, the gradient of gamma and dbeta, with
      // their per-channel factors, so that they are not held through the products:
      // dq = e^gamma o (dO S0) + q2, dk = g1 + beta f1m with f1m = f1 - e^gamma o (E S0)
      // and g1 = k1 + f2 + dk4, dk4 = e^(gamma_C - gamma) o (U dS_C)
      float bp[4] = {0.f, 0.f, 0.f, 0.f}, gpk[HCT][4], kdx[HCT];
#pragma unroll
      for (int ct = 0; ct < HCT; ++ct) {
        const int c = 16 * (ct0 + ct) + kln;
        const float gC = sG[(C - 1) * LK + c];
        float kd = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * tw + 4 * kg4 + e;
          const float gt = sG[t * LK + c], eg = __expf(gt), bt = sb[t];
          const float dq1 = eg * Q1[ct][e], x1 = -eg * ES[ct][e], d4 = __expf(gC - gt) * UD[ct][e];
          const float qv = sQ[t * LK + c], kv = sK[t * LK + c];
          dQa[ct][e] += dq1;
          dKa[ct][e] += __builtin_fmaf(bt, x1, d4);
          gpk[ct][e] = qv * dq1 - kv * d4 + kv * bt * x1;
          bp[e] += kv * x1;
          kd = __builtin_fmaf(kv, d4, kd);
        }
        kdx[ct] = kd;
      }
      // token block TW of the rows (q2, f1: sums over keys j <= i) and of the columns
      // (k1, f2: sums over rows i >= j).  The blocks go through the matrix cores
      // about a reference token: the rows' first token p for the keys up to the
      // block, the columns' last token pe for the rows from it, so that both
      // factors of e^(gamma_i - gamma_j) = e^(gamma_i - gamma_ref) e^(gamma_ref -
      // gamma_j) are at most 1 off the diagonal and one at most e^kWide on it; a
      // diagonal block whose decay is wider in the wave's channels term by term.
      // adds a tile's masked products to dq, dk, the gradient of gamma and dbeta
      auto combine = [&](int ct, const float4v &q2, const float4v &f1, const float4v &k1, const float4v &f2) {
        const int c = 16 * (ct0 + ct) + kln;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * tw + 4 * kg4 + e;
          const float bt = sb[t], qv = sQ[t * LK + c], kv = sK[t * LK + c];
          const float g1 = k1[e] + f2[e];
          dQa[ct][e] += q2[e];
          dKa[ct][e] += __builtin_fmaf(bt, f1[e], g1);
          gpk[ct][e] += qv * q2[e] - kv * g1 + kv * bt * f1[e];
          bp[e] += kv * f1[e];
        }
      };
      unsigned wmask = 0;   // the wave's column tiles whose diagonal block is wide
      auto products = [&](auto TWc) {
        constexpr int TW = decltype(TWc)::value, p = 16 * TW, pe = p + 15;
#pragma unroll
        for (int ct = 0; ct < HCT; ++ct) {
          const int c = 16 * (ct0 + ct) + kln;
          const float gp = sG[p * LK + c], gl = sG[pe * LK + c];
          float gi[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) gi[e] = sG[(p + 4 * kg4 + e) * LK + c];
          float4v q2 = {0.f, 0.f, 0.f, 0.f}, f1 = q2, k1 = q2, f2 = q2;
          // the decay over the block in the wave's channels decides whether the
          // diagonal block joins the matrix-core products
          const bool wide = __any(gp - gl > kWide);
          // the keys of the blocks [LO, HI) about token p (into q2, f1), the rows of the
          // blocks [LO, HI) about token pe (into k1, f2); one block's operands at a time
          auto rows = [&](auto LO, auto HI, float4v &acc1, float4v &acc2, float cap) {
#pragma unroll
            for (int k0 = 16 * decltype(LO)::value; k0 < 16 * decltype(HI)::value; k0 += 16) {
              const int k = k0 + 4 * kg4;
              const float4v kv = col4(sK + k * LK + c, LK), gv = col4(sG + k * LK + c, LK);
              const float4v x1 = row4(sdP + (p + kln) * LC + k), x2 = row4(sB + (p + kln) * LC + k);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float y = kv[e] * __expf(fminf(gp - gv[e], cap));
                acc1 = mma(x1[e], y, acc1);
                if constexpr (!ND) acc2 = mma(x2[e], y, acc2);   // B = 0 without the delta correction
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          };
          auto cols = [&](auto LO, auto HI, float4v &acc1, float4v &acc2, float cap) {
#pragma unroll
            for (int k0 = 16 * decltype(LO)::value; k0 < 16 * decltype(HI)::value; k0 += 16) {
              const int k = k0 + 4 * kg4;
              const float4v gv = col4(sG + k * LK + c, LK), qv = col4(sQ + k * LK + c, LK);
              const float4v kv = col4(sK + k * LK + c, LK) * row4(sb + k);
              const float4v x1 = col4(sdP + k * LC + p + kln, LC), x2 = col4(sB + k * LC + p + kln, LC);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float f = __expf(fminf(gv[e] - gl, cap));
                acc1 = mma(x1[e], qv[e] * f, acc1);
                if constexpr (!ND) acc2 = mma(x2[e], kv[e] * f, acc2);
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          };
          using I0 = std::integral_constant<int, 0>;
          using IT = std::integral_constant<int, TW>;
          using IT1 = std::integral_constant<int, TW + 1>;
          using I4 = std::integral_constant<int, 4>;
          rows(I0{}, IT{}, q2, f1, 0.f);
          cols(IT1{}, I4{}, k1, f2, 0.f);
          {   // the diagonal block (masked entries are zero); a wide one's finite values are dropped
            float4v d1 = {0.f, 0.f, 0.f, 0.f}, d2 = d1, d3 = d1, d4 = d1;
            rows(IT{}, IT1{}, d1, d2, kWide);
            cols(IT{}, IT1{}, d3, d4, kWide);
            const float keep = wide ? 0.f : 1.f;
            q2 += d1 * keep;
            f1 += d2 * keep;
            k1 += d3 * keep;
            f2 += d4 * keep;
            if (wide) wmask |= 1u << ct;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float fr = __expf(gi[e] - gp), fc = __expf(gl - gi[e]);
            q2[e] *= fr;
            f1[e] *= fr;
            k1[e] *= fc;
            f2[e] *= fc;
          }
          combine(ct, q2, f1, k1, f2);
          asm volatile("" ::: "memory");
        }
      };
      switch (tw) {
        case 0: products(std::integral_constant<int, 0>{}); break;
        case 1: products(std::integral_constant<int, 1>{}); break;
        case 2: products(std::integral_constant<int, 2>{}); break;
        default: products(std::integral_constant<int, 3>{}); break;
      }
      // wide diagonal blocks, term by term (each factor e^(gamma_i - gamma_j), i >= j,
      // at most 1; masked entries are zero and their factor is clamped to 1)
      if (wmask) {
#pragma unroll
        for (int ct = 0; ct < HCT; ++ct)
          if (wmask & (1u << ct)) {
            const Diag4 d = wide_diagonal<LK>(sdP, sB, sK, sQ, sG, sb, 16 * tw, 16 * (ct0 + ct) + kln, kg4);
            combine(ct, d.q2, d.f1, d.k1, d.f2);
          }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) bp[e] = group_sum<16>(bp[e]);
      if (kln == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sBet[hw * C + 16 * tw + 4 * kg4 + e] = bp[e];
      }
#pragma unroll
      for (int ct = 0; ct < HCT; ++ct) {   // sum of k o dk4 over the wave's tokens, per channel
        float x = kdx[ct];
        x += __shfl_xor(x, 16, 64);
        x += __shfl_xor(x, 32, 64);
        if (kg4 == 0) sKd[tw * DK + 16 * (ct0 + ct) + kln] = x;
      }
      lds_barrier();   // the products' reads of the masked matrices are done
#pragma unroll
      for (int ct = 0; ct < HCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) sGp[(16 * tw + 4 * kg4 + e) * LK + 16 * (ct0 + ct) + kln] = gpk[ct][e];
      lds_barrier();
      // dg_tc = sum over the chunk's tokens s >= t of the gradient of gamma_sc; the last
      // token also carries <dS_C, S_C>_c = e^gamma_Cc <dS_C, S0>_c + sum_j k_jc dk4_jc
      for (int c = tid; c < DK; c += NT) {
        float sd = 0.f, kd = 0.f;
        for (int u = 0; u < G::NW; ++u) sd += sSd[u * DK + c];
        for (int u = 0; u < 4; ++u) kd += sKd[u * DK + c];
        float s = __builtin_fmaf(__expf(sG[(C - 1) * LK + c]), sd, kd);
        for (int t = C - 1; t >= 0; --t) {
          s += sGp[t * LK + c];
          if (t < len) a.dg[((row0 + t) * Hv + h) * DK + c] = s;
        }
      }
      if (w == G::NW - 1) {
        float y = sBet[lane] + sBx[lane];
#pragma unroll
        for (int u = 1; u < NH; ++u) y += sBet[u * C + lane];
        if (lane < len) a.dbeta[(row0 + lane) * Hv + h] = y;
      }
    } else {
      lds_barrier();
      // M o dP and B = M o dA = -(M o E U^T) into LDS (over the slices' space)
#pragma unroll
      for (int J = 0; J < HJ; ++J) {
        const int j = 16 * (J0 + J) + ln;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * tw + 4 * g4 + e;
          const float m = i >= j ? __expf(sg[i] - sg[j]) : 0.f;
          sdP[i * LC + j] = m * dPa[J][e];
          sB[i * LC + j] = i > j ? -m * dAa[J][e] : 0.f;
        }
      }
      // E . v (eight threads per token) and <dS_C, S0> over the workgroup
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const float x = group_sum<8>(dbx[i]);
        if ((tid & 7) == 0) sBx[vtok(i)] = x;
      }
      sdot = group_sum<64>(sdot);
      if (lane == 0) sRed[G::NW + w] = sdot;   // one slot per wave: a fixed order of the sum
      lds_barrier();
      float gp[4] = {0.f, 0.f, 0.f, 0.f}, bp[4] = {0.f, 0.f, 0.f, 0.f}, cp = 0.f;
      // M o dP and B are zero above the diagonal (B on it too): token block TW's rows
      // need the key blocks up to TW, its columns the token blocks from TW (the tiles
      // above the diagonal are never read).  One copy of the products per TW, so
      // that every range is fixed at compile time.
      auto products = [&](auto TWc) {
        constexpr int TW = decltype(TWc)::value;
#pragma unroll
        for (int ct = 0; ct < HCT; ++ct) {
          const int c = 16 * (ct0 + ct) + ln;
          float4v q2 = {0.f, 0.f, 0.f, 0.f}, k1 = q2, f1 = q2, f2 = q2;
          if constexpr (ND) {   // B = 0 without the delta correction
            mmr<C>(q2, [&](int k) { return row4(sdP + (16 * TW + ln) * LC + k); },
                   [&](int k) { return col4(sK + k * LK + c, LK); }, g4, 0, TW + 1);
          } else {
            mm2r<C>(q2, f1, [&](int k) { return row4(sdP + (16 * TW + ln) * LC + k); },
                    [&](int k) { return row4(sB + (16 * TW + ln) * LC + k); },
                    [&](int k) { return col4(sK + k * LK + c, LK); }, g4, 0, TW + 1);
          }
          mmr<C>(k1, [&](int k) { return col4(sdP + k * LC + 16 * TW + ln, LC); },
                 [&](int k) { return col4(sQ + k * LK + c, LK); }, g4, TW, 4);
          if constexpr (!ND)
            mmr<C>(f2, [&](int k) { return col4(sB + k * LC + 16 * TW + ln, LC) * row4(sb + k); },
                   [&](int k) { return col4(sK + k * LK + c, LK); }, g4, TW, 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 16 * TW + 4 * g4 + e;
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
          // the next tile reads its operands again rather than keep them in registers
          asm volatile("" ::: "memory");
        }
      };
      switch (tw) {
        case 0: products(std::integral_constant<int, 0>{}); break;
        case 1: products(std::integral_constant<int, 1>{}); break;
        case 2: products(std::integral_constant<int, 2>{}); break;
        default: products(std::integral_constant<int, 3>{}); break;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gp[e] = group_sum<16>(gp[e]);
        bp[e] = group_sum<16>(bp[e]);
      }
      if (ln == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sGam[hw * C + 16 * tw + 4 * g4 + e] = gp[e];
          sBet[hw * C + 16 * tw + 4 * g4 + e] = bp[e];
        }
      }
      cp = group_sum<64>(cp);
      if (lane == 0) sRed[w] = cp;
      lds_barrier();
      if (w == 0) {
        // dg_t = sum over the chunk's tokens i >= t of the gradient of gamma_i; the
        // last token also carries <dS_C, S_C> = e^gamma_C <dS_C, S0> + sum_j k_j . dk4_j
        const int t = C - 1 - lane;
        float x = sGam[t], y = sBet[t] + sBx[t];
#pragma unroll
        for (int u = 1; u < NH; ++u) x += sGam[u * C + t], y += sBet[u * C + t];
        if (t == C - 1) {
          float c4 = 0.f, sd = 0.f;
#pragma unroll
          for (int u = 0; u < G::NW; ++u) c4 += sRed[u], sd += sRed[G::NW + u];
          x += __builtin_fmaf(sEg[C - 1], sd, c4);
        }
        const float s = wave_prefix_sum(x);
        if (t < len) {
          a.dg[(row0 + t) * Hv + h] = s;
          a.dbeta[(row0 + t) * Hv + h] = y;
        }
      }
    }
  }
  float *pq = a.dq + (row0 * Hk + kh) * DK, *pk = a.dk + (row0 * Hk + kh) * DK;
#pragma unroll
  for (int ct = 0; ct < HCT; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * tw + 4 * g4 + e, o = t * Hk * DK + 16 * (ct0 + ct) + ln;
      if (t < len) {
        pq[o] = dQa[ct][e];
        pk[o] = dKa[ct][e];
      }
    }
}

template <typename TQ, int DK, bool KEY>
struct CbSmem {
  static constexpr int LK = DK + 4;
  static constexpr int QK = PassCfg<TQ, DK>::LK * (int)sizeof(TQ), LS = DK + 4;
  // the key gate's passes hold two fp32 [C][dk] operands in place of the rows of k
  // (and q), and e^gamma_C per channel
  static constexpr int OP1 = KEY ? 2 * C * LS * 4 : C * QK, OP2 = KEY ? 2 * C * LS * 4 : 2 * C * QK;
  static constexpr int EC = KEY ? DK : 0;
  static constexpr int fwd = OP1 + (C * LC + R * LS + 2 * R * LC + 3 * C + EC) * 4;
  static constexpr int bwd = OP2 + (2 * C * LC + C * LR + R * LS + 2 * R * LC + 3 * C + EC) * 4;
  static constexpr int prep = KEY ? (3 * C * LK + 2 * C * LC + C + 4 * 16 * LX) * 4
                                  : (prep_region(DK) + C * LC + 2 * C) * 4;
  static constexpr int grads = GradCfg<TQ, DK, KEY>::smem;
};

template <typename F>
hipError_t set_smem(F *kern, int bytes) {
  return hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

// The workspace of one call: how many segments, and where each array starts.
// Floats per (batch, value head): T, gamma, beta for every chunk (the key
// gate: gamma [C][dk], and K o e^gamma, Q o e^gamma, K o e^(gamma_C - gamma)
// too); P^T, S0, dS_C, U, E for the chunks of one segment.  One segment is the fastest; with
// more, a forward pass over the chunks before the last segment first keeps
// the states at the segment starts, and each segment then runs its own
// forward pass.

struct CbPlan {
  int nc, nseg, ncs;
  size_t units, sunits;   // (batch, value head, chunk) for all chunks and for one segment
  size_t f_T, f_g, f_b, f_Kh, f_Qh, f_Kt, f_Sseg, f_P, f_S0, f_dS, f_U, f_E, floats;
  CbPlan(const Shape &sh, int want) {
    nc = (sh.T + C - 1) / C;
    ncs = (nc + want - 1) / want;
    nseg = (nc + ncs - 1) / ncs;
    const size_t bh = (size_t)sh.B * sh.Hv, st = (size_t)sh.dv * sh.dk, cv = (size_t)C * sh.dv;
    units = bh * nc;
    sunits = bh * ncs;
    const size_t ck = sh.key_gate ? (size_t)C * sh.dk : 0;   // a key gate's [C][dk] arrays
    size_t o = 0;
    f_T = o, o += units * C * C;
    f_g = o, o += sh.key_gate ? units * ck : units * C;
    f_b = o, o += units * C;
    f_Kh = o, o += units * ck;
    f_Qh = o, o += units * ck;
    f_Kt = o, o += units * ck;
    f_Sseg = o, o += nseg > 1 ? bh * nseg * st : 0;
    f_P = o, o += sunits * C * C;
    f_S0 = o, o += sunits * st;
    f_dS = o, o += sunits * st;
    f_U = o, o += sunits * cv;
    f_E = o, o += sunits * cv;
    floats = o;
  }
  size_t bytes() const { return floats * 4; }
};

// the plan with the fewest segments whose workspace fits in `bytes`, else the
// plan with the smallest workspace (more segments keep more segment-start
// states, so the smallest is not the one with the most segments)
inline CbPlan plan_for(const Shape &sh, size_t bytes) {
  const int nc = (sh.T + C - 1) / C;
  CbPlan best(sh, 1);
  for (int want = 1; want <= nc; ++want) {
    CbPlan p(sh, want);
    if (p.bytes() <= bytes) return p;
    if (p.bytes() < best.bytes()) best = p;
  }
  return best;
}

template <typename TQ, typename TG, int DK, bool KEY>
hipError_t launch_cb_t(const Shape &sh, const CbPlan &pl, CbArgs a, const float *dST, hipStream_t st) {
  using Sm = CbSmem<TQ, DK, KEY>;
  constexpr int NTP = PassCfg<TQ, DK>::NT, NTG = GradCfg<TQ, DK, KEY>::NT;
  static_assert(Sm::fwd <= 160 * 1024 && Sm::bwd <= 160 * 1024 && Sm::grads <= 160 * 1024 &&
                    Sm::prep <= 160 * 1024,
                "LDS");
  constexpr auto prep_k = KEY ? cb_prep_key_kernel<TQ, TG, DK> : cb_prep_kernel<TQ, TG, DK>;
  hipError_t e;
  if ((e = set_smem(prep_k, Sm::prep)) != hipSuccess) return e;
  if ((e = set_smem(cb_fwd_kernel<TQ, DK, KEY>, Sm::fwd)) != hipSuccess) return e;
  if ((e = set_smem(cb_bwd_kernel<TQ, DK, KEY>, Sm::bwd)) != hipSuccess) return e;
  if ((e = set_smem(cb_grads_kernel<TQ, TG, DK, false, KEY>, Sm::grads)) != hipSuccess) return e;
  if ((e = set_smem(cb_grads_kernel<TQ, TG, DK, true, KEY>, Sm::grads)) != hipSuccess) return e;
  const dim3 pass(sh.dv / R, sh.Hv, sh.B);
  auto prep = [&](int flags) {
    a.flags = flags;
    hipLaunchKernelGGL(prep_k, dim3(a.c1 - a.c0, sh.Hk, sh.B), dim3(256), Sm::prep, st, a);
    return hipGetLastError();
  };
  auto fwd = [&](int flags) {
    a.flags = flags;
    hipLaunchKernelGGL((cb_fwd_kernel<TQ, DK, KEY>), pass, dim3(NTP), Sm::fwd, st, a);
    return hipGetLastError();
  };
  auto segment = [&]() {   // the chunks [c0, c1) of one segment, from their P^T to their gradients
    hipError_t r = fwd(0);
    if (r != hipSuccess) return r;
    hipLaunchKernelGGL((cb_bwd_kernel<TQ, DK, KEY>), pass, dim3(NTP), Sm::bwd, st, a);
    if ((r = hipGetLastError()) != hipSuccess) return r;
    const dim3 grid(a.c1 - a.c0, sh.Hk, sh.B);
    if (a.nd)
      hipLaunchKernelGGL((cb_grads_kernel<TQ, TG, DK, true, KEY>), grid, dim3(NTG), Sm::grads, st, a);
    else
      hipLaunchKernelGGL((cb_grads_kernel<TQ, TG, DK, false, KEY>), grid, dim3(NTG), Sm::grads, st, a);
    return hipGetLastError();
  };
  a.nseg = pl.nseg;
  a.ncs = pl.ncs;
  if (pl.nseg == 1) {
    a.c0 = a.sc0 = 0, a.c1 = pl.nc;
    a.dS_in = dST;
    if ((e = prep(kPrepT | kPrepP)) != hipSuccess) return e;
    return segment();
  }
  // T, gamma, beta of every chunk; the states at the segment starts; then the
  // segments from the last, the state gradient carried in dS0
  a.c0 = a.sc0 = 0, a.c1 = pl.nc;
  if ((e = prep(kPrepT)) != hipSuccess) return e;
  a.c1 = (pl.nseg - 1) * pl.ncs;
  if ((e = fwd(kStatesOnly)) != hipSuccess) return e;
  for (int sg = pl.nseg - 1; sg >= 0; --sg) {
    a.c0 = a.sc0 = sg * pl.ncs;
    a.c1 = std::min(pl.nc, a.c0 + pl.ncs);
    a.dS_in = sg == pl.nseg - 1 ? dST : a.dS0;
    if ((e = prep(kPrepP)) != hipSuccess) return e;
    if ((e = segment()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename TQ, typename TG>
hipError_t launch_cb_d(const Shape &sh, const CbPlan &pl, const CbArgs &a, const float *dST, hipStream_t st) {
  const bool key = sh.key_gate;
  switch (sh.dk) {
    case 32:
      return key ? launch_cb_t<TQ, TG, 32, true>(sh, pl, a, dST, st)
                 : launch_cb_t<TQ, TG, 32, false>(sh, pl, a, dST, st);
    case 64:
      return key ? launch_cb_t<TQ, TG, 64, true>(sh, pl, a, dST, st)
                 : launch_cb_t<TQ, TG, 64, false>(sh, pl, a, dST, st);
    case 128:
      return key ? launch_cb_t<TQ, TG, 128, true>(sh, pl, a, dST, st)
                 : launch_cb_t<TQ, TG, 128, false>(sh, pl, a, dST, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t backward_workspace(const Shape &sh, size_t cap) { return plan_for(sh, cap).bytes(); }

hipError_t launch_backward(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                           const void *beta, const float *S0, const float *dO, const float *dST, float *dq,
                           float *dk, float *dv, float *dg, float *dbeta, float *dS0, void *ws, size_t ws_bytes,
                           hipStream_t st) {
  const CbPlan pl = plan_for(sh, ws_bytes);
  CbArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.S0 = S0;
  a.dO = dO;
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
  a.nc = pl.nc;
  a.nd = sh.no_delta ? 1 : 0;
  float *w = (float *)ws;
  a.Tm = w + pl.f_T;
  a.gam = w + pl.f_g;
  a.bet = w + pl.f_b;
  a.Sseg = w + pl.f_Sseg;
  a.Pt = w + pl.f_P;
  a.S0s = w + pl.f_S0;
  a.dSC = w + pl.f_dS;
  a.Um = w + pl.f_U;
  a.Em = w + pl.f_E;
  a.Kh = w + pl.f_Kh;
  a.Qh = w + pl.f_Qh;
  a.Kt = w + pl.f_Kt;
  if (sh.qkv == DType::F32)
    return sh.gate_t == DType::F32 ? launch_cb_d<float, float>(sh, pl, a, dST, st)
                                   : launch_cb_d<float, bf16_t>(sh, pl, a, dST, st);
  if (sh.qkv == DType::BF16)
    return sh.gate_t == DType::F32 ? launch_cb_d<bf16_t, float>(sh, pl, a, dST, st)
                                   : launch_cb_d<bf16_t, bf16_t>(sh, pl, a, dST, st);
  return sh.gate_t == DType::F32 ? launch_cb_d<f16_t, float>(sh, pl, a, dST, st)
                                 : launch_cb_d<f16_t, bf16_t>(sh, pl, a, dST, st);
}

}  // namespace gdn
