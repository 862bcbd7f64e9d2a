// backward.hip -- the backward of the gated delta rule token by token: the
// first-order backward over the state history ("Source notes", section
// "Linear attention", row kda: the backward keeps the whole state history),
// here kept for every kHist-th token and recomputed in between.  For the
// loss gradients dO (of o) and dS_T (of S_T) it gives dq, dk, dv, dg, dbeta
// and dS0, in fp32.  It serves the per-key-channel gate (launch_backward
// sends the per-head gate to the chunked backward); the kernels are written
// for both gates.
//
// Per (batch, value head) and token t, with D = alpha S_{t-1} (key-channel
// gate: S_{t-1} diag(alpha)), a = D k, u = beta (v - a), S_t = D + u k^T,
// o_t = S_t q and G the gradient with respect to S_t, in reverse order:
//   G += dO_t q^T;   dq_t = S_t^T dO_t
//   du = G k;   dv_t = beta du;   dbeta_t = du . (v - a);   dk_t = G^T u - beta D^T du
//   dD = G - beta du k^T;   dg_t = <dD, D> (per key channel: column sums of dD o D)
//   G <- alpha dD (per key channel: dD diag(alpha))
// and dS0 = G at the end.  Rows of S evolve independently in both passes:
// every row-local quantity (a, u, du, dv, dD) needs only the row, and the
// rest (dq, dk, dbeta, dg) are sums over rows.
//
// Three launches:
//  - history: one wave per ROWS state rows of a (batch, value head) runs
//    the forward recurrence and stores the state before every kHist-th token
//    (fp32, [B,Hv,ceil(T / kHist),dv,dk]);
//  - backward: workgroups of kSlice / ROWS such waves run the tokens
//    backwards in blocks of kHist, recomputing the block's states from the
//    stored one into LDS first; they write dv and dS0, and per token the
//    partial sums over their kSlice rows of dq, dk, dbeta and dg;
//  - reduce: the partial sums over the row slices (and, for dq and dk, over
//    the value heads of a key head).
// The history is written once and read once (dv dk 4 bytes per kHist tokens
// and value head each way); the recomputation costs one forward step per
// token but the first of each block.
//
// Lane layout: CG = dk / 8 lanes hold a row, 8 key channels each; a wave
// holds 64 / CG rows at a time and RL = CG / 2 such row sets, rows
// m (64 / CG) + lane / CG, so every access of a row set is one contiguous run.
#include <hip/hip_runtime.h>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kSlice = 32;  // state rows of a backward workgroup (dv is a multiple of it)
constexpr int kHist = 4;    // the history keeps the state before every kHist-th token

template <int DK>
struct BwdCfg {
  static constexpr int CG = DK / 8;                 // lanes per row
  static constexpr int RS = 64 / CG;                // rows per row set
  static constexpr int ROWS = RS > 8 ? RS : 8;      // state rows per wave
  static constexpr int RL = ROWS / RS;              // row sets (rows per lane)
  static constexpr int WAVES = kSlice / ROWS;       // waves of a backward workgroup
};

// Sum over the lanes holding the same key channels (one per row of a row set).
template <int CG>
__device__ __forceinline__ float rows_sum(float x) {
#pragma unroll
  for (int m = CG; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <typename T>
__device__ __forceinline__ void load8f(const T *p, float (&x)[8]) {
  load8(p, x);
}

// Per-token inputs of a wave: k (and q) at the lane's 8 channels, v (and dO)
// at the lane's rows, the decay and beta.
template <typename TQ, typename TG, bool KEY, int DK, bool BWD>
struct TokIn {
  float k[8], q[BWD ? 8 : 1], al[KEY ? 8 : 1], v[BwdCfg<DK>::RL], dO[BWD ? BwdCfg<DK>::RL : 1], beta;
};

template <typename TQ, typename TG, bool KEY, int DK, bool BWD>
__device__ __forceinline__ void load_tok(TokIn<TQ, TG, KEY, DK, BWD> &in, const TQ *q, const TQ *k, const TQ *v,
                                         const TG *g, const TG *beta, const float *dO, size_t bt, int Hk,
                                         int Hv, int DV, int kh, int h, int cg, int rbase) {
  using Cfg = BwdCfg<DK>;
  load8f(k + (bt * Hk + kh) * DK + 8 * cg, in.k);
  if constexpr (BWD) load8f(q + (bt * Hk + kh) * DK + 8 * cg, in.q);
  if constexpr (KEY) {
    float gg[8];
    load8f(g + (bt * Hv + h) * DK + 8 * cg, gg);
#pragma unroll
    for (int c = 0; c < 8; ++c) in.al[c] = __expf(gg[c]);
  } else {
    in.al[0] = __expf(to_f32(g[bt * Hv + h]));
  }
  in.beta = to_f32(beta[bt * Hv + h]);
#pragma unroll
  for (int m = 0; m < Cfg::RL; ++m) {
    const size_t at = (bt * Hv + h) * DV + rbase + m * Cfg::RS;
    in.v[m] = to_f32(v[at]);
    if constexpr (BWD) in.dO[m] = dO[at];
  }
}

struct BwdArgs {
  const void *q, *k, *v, *g, *beta;
  const float *S0, *dO, *dST;
  float *hist, *part, *dv, *dS0;
  int T, Hk, Hv, dv_dim;
};

// One token of the forward recurrence on the wave's rows: S <- alpha S, then
// S <- S + beta (v - S k) k^T.  The history pass and the backward's
// recomputation both take this function, so they agree bit for bit.
template <typename TQ, typename TG, bool KEY, int DK, bool BWD>
__device__ __forceinline__ void fwd_step(float (&S)[BwdCfg<DK>::RL][8], const TokIn<TQ, TG, KEY, DK, BWD> &in) {
  using Cfg = BwdCfg<DK>;
#pragma unroll
  for (int m = 0; m < Cfg::RL; ++m) {
    float p = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      S[m][c] *= KEY ? in.al[c] : in.al[0];
      p = __builtin_fmaf(S[m][c], in.k[c], p);
    }
    p = group_sum<Cfg::CG>(p);
    const float u = in.beta * (in.v[m] - p);
#pragma unroll
    for (int c = 0; c < 8; ++c) S[m][c] = __builtin_fmaf(u, in.k[c], S[m][c]);
  }
}

template <typename TQ, typename TG, bool KEY, int DK>
__global__ __launch_bounds__(64) void bwd_history_kernel(BwdArgs a) {
  using Cfg = BwdCfg<DK>;
  const int lane = threadIdx.x, cg = lane % Cfg::CG, rs = lane / Cfg::CG;
  const int slice = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Hv = a.Hv, DV = a.dv_dim, T = a.T, kh = h / (Hv / a.Hk);
  const int rbase = slice * Cfg::ROWS + rs;
  const size_t bh = (size_t)b * Hv + h;
  float S[Cfg::RL][8];
#pragma unroll
  for (int m = 0; m < Cfg::RL; ++m) {
    if (a.S0)
      load8f(a.S0 + (bh * DV + rbase + m * Cfg::RS) * DK + 8 * cg, S[m]);
    else
#pragma unroll
      for (int c = 0; c < 8; ++c) S[m][c] = 0.f;
  }
  const int nh = (T + kHist - 1) / kHist;
  float *hb = a.hist + (bh * nh * DV + rbase) * DK + 8 * cg;
  TokIn<TQ, TG, KEY, DK, false> cur, nxt;
  if (T > 0)
    load_tok(cur, (const TQ *)a.q, (const TQ *)a.k, (const TQ *)a.v, (const TG *)a.g, (const TG *)a.beta,
             nullptr, (size_t)b * T, a.Hk, Hv, DV, kh, h, cg, rbase);
  for (int t = 0; t < T; ++t) {
    if (t + 1 < T)
      load_tok(nxt, (const TQ *)a.q, (const TQ *)a.k, (const TQ *)a.v, (const TG *)a.g, (const TG *)a.beta,
               nullptr, (size_t)b * T + t + 1, a.Hk, Hv, DV, kh, h, cg, rbase);
    if (t % kHist == 0) {
      float *ht = hb + (size_t)(t / kHist) * DV * DK;
#pragma unroll
      for (int m = 0; m < Cfg::RL; ++m) store8(ht + (size_t)m * Cfg::RS * DK, S[m]);
    }
    fwd_step(S, cur);
    cur = nxt;
  }
}

// partial sums per (batch, value head, slice of kSlice rows, token): dq[DK], dk[DK], dbeta, dg[KEY ? DK : 1]
template <bool KEY, int DK>
__host__ __device__ constexpr int part_width() {
  return 2 * DK + 1 + (KEY ? DK : 1);
}

// LDS of a backward workgroup: per wave the kHist - 1 recomputed states
// (lane-interleaved, [slot][m][c][lane]), then the partial sums of waves
// 1 .. WAVES - 1 for wave 0 to add.
template <bool KEY, int DK>
constexpr int bwd_smem() {
  using Cfg = BwdCfg<DK>;
  return (Cfg::WAVES * (kHist - 1) * Cfg::RL * 8 * 64 + (Cfg::WAVES - 1) * part_width<KEY, DK>()) * 4;
}

// WAVES waves, ROWS state rows each, walk the tokens backwards in blocks
// of kHist: from the state kept before the block's first token they
// recompute the states before its other tokens into LDS (forward), then run
// the block's tokens backwards.  The next token's inputs are loaded one step
// ahead, the next block's kept state during this block's backward steps.
// Per token, waves 1 .. WAVES - 1 hand their partial sums to wave 0 through
// LDS, and wave 0 writes the slice's sums.
template <typename TQ, typename TG, bool KEY, int DK>
__global__ __launch_bounds__(64 * BwdCfg<DK>::WAVES) void bwd_kernel(BwdArgs a) {
  using Cfg = BwdCfg<DK>;
  constexpr int PW = part_width<KEY, DK>();
  constexpr int NF = Cfg::RL * 8;   // state values per lane
  extern __shared__ float smem[];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, cg = lane % Cfg::CG, rs = lane / Cfg::CG;
  float *sH = smem + wv * (kHist - 1) * NF * 64;
  float *sRed = smem + Cfg::WAVES * (kHist - 1) * NF * 64;   // [WAVES - 1][PW]
  const int slice = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Hv = a.Hv, DV = a.dv_dim, T = a.T, kh = h / (Hv / a.Hk);
  const int nsl = DV / kSlice;
  const int rbase = slice * kSlice + wv * Cfg::ROWS + rs;
  const size_t bh = (size_t)b * Hv + h;
  float G[Cfg::RL][8];
#pragma unroll
  for (int m = 0; m < Cfg::RL; ++m) {
    if (a.dST)
      load8f(a.dST + (bh * DV + rbase + m * Cfg::RS) * DK + 8 * cg, G[m]);
    else
#pragma unroll
      for (int c = 0; c < 8; ++c) G[m][c] = 0.f;
  }
  const int nh = (T + kHist - 1) / kHist;
  const float *hb = a.hist + (bh * nh * DV + rbase) * DK + 8 * cg;
  float *pb = a.part + ((bh * nsl + slice) * T) * PW;
  auto load_hist = [&](float (&X)[Cfg::RL][8], int j) {
#pragma unroll
    for (int m = 0; m < Cfg::RL; ++m) load8f(hb + (size_t)j * DV * DK + (size_t)m * Cfg::RS * DK, X[m]);
  };
  auto put = [&](int slot, const float (&X)[Cfg::RL][8]) {
#pragma unroll
    for (int m = 0; m < Cfg::RL; ++m)
#pragma unroll
      for (int c = 0; c < 8; ++c) sH[(slot * NF + m * 8 + c) * 64 + lane] = X[m][c];
  };
  auto get = [&](int slot, float (&X)[Cfg::RL][8]) {
#pragma unroll
    for (int m = 0; m < Cfg::RL; ++m)
#pragma unroll
      for (int c = 0; c < 8; ++c) X[m][c] = sH[(slot * NF + m * 8 + c) * 64 + lane];
  };
  // the token of op i of block j: the recomputation of tokens t0 .. t1 - 2,
  // then the backward of t1 - 1 .. t0
  auto op_tok = [&](int j, int i) {
    const int t0 = j * kHist, t1 = min(t0 + kHist, T), nr = t1 - t0 - 1;
    return i < nr ? t0 + i : t1 - 1 - (i - nr);
  };
  auto load_op = [&](TokIn<TQ, TG, KEY, DK, true> &in, int t) {
    load_tok(in, (const TQ *)a.q, (const TQ *)a.k, (const TQ *)a.v, (const TG *)a.g, (const TG *)a.beta, a.dO,
             (size_t)b * T + t, a.Hk, Hv, DV, kh, h, cg, rbase);
  };
  TokIn<TQ, TG, KEY, DK, true> cur, nxt;
  float H0[Cfg::RL][8], Hn[Cfg::RL][8];
  if (T > 0) {
    load_hist(H0, nh - 1);
    load_op(cur, op_tok(nh - 1, 0));
  }
  for (int j = nh - 1; j >= 0; --j) {
    const int t0 = j * kHist, t1 = min(t0 + kHist, T), nr = t1 - t0 - 1, no = 2 * (t1 - t0) - 1;
    // the next op's inputs: this block's op i + 1, or the first op of block j - 1
    auto prefetch = [&](int i) {
      if (i + 1 < no)
        load_op(nxt, op_tok(j, i + 1));
      else if (j > 0)
        load_op(nxt, op_tok(j - 1, 0));
    };
    {
      float S[Cfg::RL][8];
#pragma unroll
      for (int m = 0; m < Cfg::RL; ++m)
#pragma unroll
        for (int c = 0; c < 8; ++c) S[m][c] = H0[m][c];
      for (int i = 0; i < nr; ++i) {   // S: the state before token t0 + i + 1
        prefetch(i);
        fwd_step(S, cur);
        put(i, S);
        cur = nxt;
      }
    }
    if (j > 0) load_hist(Hn, j - 1);
    for (int i = nr; i < no; ++i) {
      prefetch(i);
      const int t = t1 - 1 - (i - nr);
      float P[Cfg::RL][8];   // the state before token t
      if (t == t0) {
#pragma unroll
        for (int m = 0; m < Cfg::RL; ++m)
#pragma unroll
          for (int c = 0; c < 8; ++c) P[m][c] = H0[m][c];
      } else {
        get(t - t0 - 1, P);
      }
      float dq[8] = {}, dk[8] = {}, dgk[8] = {}, dbeta = 0.f, dgh = 0.f;
#pragma unroll
      for (int m = 0; m < Cfg::RL; ++m) {
        float D[8], p = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          D[c] = P[m][c] * (KEY ? cur.al[c] : cur.al[0]);
          p = __builtin_fmaf(D[c], cur.k[c], p);
        }
        p = group_sum<Cfg::CG>(p);                     // a = D k
        const float u = cur.beta * (cur.v[m] - p);
        const float dOm = cur.dO[m];
        float gk = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float st = __builtin_fmaf(u, cur.k[c], D[c]);   // S_t
          dq[c] = __builtin_fmaf(dOm, st, dq[c]);
          G[m][c] = __builtin_fmaf(dOm, cur.q[c], G[m][c]);
          gk = __builtin_fmaf(G[m][c], cur.k[c], gk);
        }
        const float du = group_sum<Cfg::CG>(gk);       // du = G k
        if (cg == 0) a.dv[(((size_t)b * T + t) * Hv + h) * DV + rbase + m * Cfg::RS] = cur.beta * du;
        dbeta = __builtin_fmaf(du, cur.v[m] - p, dbeta);
        const float bdu = cur.beta * du;
        float gd = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          dk[c] = __builtin_fmaf(u, G[m][c], dk[c]);
          dk[c] = __builtin_fmaf(-bdu, D[c], dk[c]);
          const float dd = __builtin_fmaf(-bdu, cur.k[c], G[m][c]);
          if constexpr (KEY)
            dgk[c] = __builtin_fmaf(dd, D[c], dgk[c]);
          else
            gd = __builtin_fmaf(dd, D[c], gd);
          G[m][c] = dd * (KEY ? cur.al[c] : cur.al[0]);
        }
        if constexpr (!KEY) dgh += gd;
      }
      // sums over the wave's rows: channels over the row sets, scalars also over the row's lanes
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        dq[c] = rows_sum<Cfg::CG>(dq[c]);
        dk[c] = rows_sum<Cfg::CG>(dk[c]);
        if constexpr (KEY) dgk[c] = rows_sum<Cfg::CG>(dgk[c]);
      }
      dbeta = rows_sum<Cfg::CG>(dbeta);              // every lane of a row holds the row's value
      if constexpr (!KEY) dgh = rows_sum<Cfg::CG>(group_sum<Cfg::CG>(dgh));
      // the other waves' sums to wave 0
      float *red = sRed + (wv - 1) * PW;
      if (wv > 0 && rs == 0) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          red[8 * cg + c] = dq[c];
          red[DK + 8 * cg + c] = dk[c];
          if constexpr (KEY) red[2 * DK + 1 + 8 * cg + c] = dgk[c];
        }
        if (cg == 0) {
          red[2 * DK] = dbeta;
          if constexpr (!KEY) red[2 * DK + 1] = dgh;
        }
      }
      lds_barrier();
      if (wv == 0 && rs == 0) {
        float *pt = pb + (size_t)t * PW;
        auto total = [&](float x, int at) {   // this wave's, then waves 1, 2, .. in order
#pragma unroll
          for (int u = 0; u < Cfg::WAVES - 1; ++u) x += sRed[u * PW + at];
          return x;
        };
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          pt[8 * cg + c] = total(dq[c], 8 * cg + c);
          pt[DK + 8 * cg + c] = total(dk[c], DK + 8 * cg + c);
          if constexpr (KEY) pt[2 * DK + 1 + 8 * cg + c] = total(dgk[c], 2 * DK + 1 + 8 * cg + c);
        }
        if (cg == 0) {
          pt[2 * DK] = total(dbeta, 2 * DK);
          if constexpr (!KEY) pt[2 * DK + 1] = total(dgh, 2 * DK + 1);
        }
      }
      lds_barrier();   // wave 0 has read the sums before the next token's
      if (i + 1 < no || j > 0) cur = nxt;
    }
    if (j > 0) {
#pragma unroll
      for (int m = 0; m < Cfg::RL; ++m)
#pragma unroll
        for (int c = 0; c < 8; ++c) H0[m][c] = Hn[m][c];
    }
  }
#pragma unroll
  for (int m = 0; m < Cfg::RL; ++m) store8(a.dS0 + (bh * DV + rbase + m * Cfg::RS) * DK + 8 * cg, G[m]);
}

// dq, dk per (batch, token, key head): the partial sums over the slices of
// every value head of the group; dbeta, dg per (batch, token, value head).
template <bool KEY, int DK>
__global__ __launch_bounds__(DK) void bwd_reduce_kernel(const float *part, float *dq, float *dk, float *dg,
                                                         float *dbeta, int T, int Hk, int Hv, int nsl) {
  constexpr int PW = part_width<KEY, DK>();
  const int j = threadIdx.x;
  const int kh = blockIdx.y;
  const size_t bt = blockIdx.x;   // b * T + t
  const int b = (int)(bt / T), t = (int)(bt % T);
  const int grp = Hv / Hk;
  float sq = 0.f, sk = 0.f;
  for (int hh = 0; hh < grp; ++hh) {
    const int h = kh * grp + hh;
    float sb = 0.f, sg = 0.f;
    for (int s = 0; s < nsl; ++s) {
      const float *pt = part + ((((size_t)b * Hv + h) * nsl + s) * T + t) * PW;
      sq += pt[j];
      sk += pt[DK + j];
      if (KEY) sg += pt[2 * DK + 1 + j];
      if (j == 0) {
        sb += pt[2 * DK];
        if (!KEY) sg += pt[2 * DK + 1];
      }
    }
    if (KEY) dg[(bt * Hv + h) * DK + j] = sg;
    if (j == 0) {
      dbeta[bt * Hv + h] = sb;
      if (!KEY) dg[bt * Hv + h] = sg;
    }
  }
  dq[(bt * Hk + kh) * DK + j] = sq;
  dk[(bt * Hk + kh) * DK + j] = sk;
}

template <typename TQ, typename TG, bool KEY, int DK>
hipError_t launch_bwd_t(const Shape &sh, const BwdArgs &a, float *dq, float *dk, float *dg, float *dbeta,
                        hipStream_t st) {
  using Cfg = BwdCfg<DK>;
  const int nsl = sh.dv / kSlice;
  hipLaunchKernelGGL((bwd_history_kernel<TQ, TG, KEY, DK>), dim3(Cfg::WAVES * nsl, sh.Hv, sh.B), dim3(64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int smem = bwd_smem<KEY, DK>();
  static_assert(smem <= 64 * 1024, "LDS");
  hipLaunchKernelGGL((bwd_kernel<TQ, TG, KEY, DK>), dim3(nsl, sh.Hv, sh.B), dim3(64 * Cfg::WAVES), smem, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_reduce_kernel<KEY, DK>), dim3((unsigned)((size_t)sh.B * sh.T), sh.Hk), dim3(DK), 0,
                     st, a.part, dq, dk, dg, dbeta, sh.T, sh.Hk, sh.Hv, nsl);
  return hipGetLastError();
}

template <typename TQ, typename TG, bool KEY>
hipError_t launch_bwd_k(const Shape &sh, const BwdArgs &a, float *dq, float *dk, float *dg, float *dbeta,
                        hipStream_t st) {
  switch (sh.dk) {
    case 32: return launch_bwd_t<TQ, TG, KEY, 32>(sh, a, dq, dk, dg, dbeta, st);
    case 64: return launch_bwd_t<TQ, TG, KEY, 64>(sh, a, dq, dk, dg, dbeta, st);
    case 128: return launch_bwd_t<TQ, TG, KEY, 128>(sh, a, dq, dk, dg, dbeta, st);
  }
  return hipErrorInvalidValue;
}

template <typename TQ, typename TG>
hipError_t launch_bwd_g(const Shape &sh, const BwdArgs &a, float *dq, float *dk, float *dg, float *dbeta,
                        hipStream_t st) {
  return launch_bwd_k<TQ, TG, true>(sh, a, dq, dk, dg, dbeta, st);
}

// Bytes of the kept states (the partial sums per slice of kSlice rows and
// token follow them in the workspace).
inline size_t history_bytes(const Shape &sh) {
  return (size_t)sh.B * sh.Hv * ((sh.T + kHist - 1) / kHist) * sh.dv * sh.dk * 4;
}

}  // namespace

size_t backward_workspace(const Shape &sh, size_t cap) {
  if (!sh.key_gate) return chunk_backward_workspace(sh, cap);
  const size_t pw = 2 * (size_t)sh.dk + 1 + (sh.key_gate ? sh.dk : 1);
  const size_t part = (size_t)sh.B * sh.Hv * (sh.dv / kSlice) * sh.T * pw * 4;
  return ((history_bytes(sh) + 255) & ~(size_t)255) + part;
}

hipError_t launch_backward(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                           const void *beta, const float *S0, const float *dO, const float *dST, float *dq,
                           float *dk, float *dv, float *dg, float *dbeta, float *dS0, void *ws, size_t ws_bytes,
                           hipStream_t st) {
  if (!sh.key_gate)
    return launch_chunk_backward(sh, q, k, v, g, beta, S0, dO, dST, dq, dk, dv, dg, dbeta, dS0, ws, ws_bytes, st);
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.S0 = S0;
  a.dO = dO;
  a.dST = dST;
  a.hist = (float *)ws;
  a.part = (float *)((char *)ws + ((history_bytes(sh) + 255) & ~(size_t)255));
  a.dv = dv;
  a.dS0 = dS0;
  a.T = sh.T;
  a.Hk = sh.Hk;
  a.Hv = sh.Hv;
  a.dv_dim = sh.dv;
  if (sh.qkv == DType::F32)
    return sh.gate_t == DType::F32 ? launch_bwd_g<float, float>(sh, a, dq, dk, dg, dbeta, st)
                                   : launch_bwd_g<float, bf16_t>(sh, a, dq, dk, dg, dbeta, st);
  if (sh.qkv == DType::BF16)
    return sh.gate_t == DType::F32 ? launch_bwd_g<bf16_t, float>(sh, a, dq, dk, dg, dbeta, st)
                                   : launch_bwd_g<bf16_t, bf16_t>(sh, a, dq, dk, dg, dbeta, st);
  return sh.gate_t == DType::F32 ? launch_bwd_g<f16_t, float>(sh, a, dq, dk, dg, dbeta, st)
                                 : launch_bwd_g<f16_t, bf16_t>(sh, a, dq, dk, dg, dbeta, st);
}

}  // namespace gdn
