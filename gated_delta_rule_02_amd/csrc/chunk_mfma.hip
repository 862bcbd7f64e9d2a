// chunk_mfma.hip -- chunked forward of the gated delta rule (scalar per-head
// decay) on the gfx950 matrix cores: dk = dv = 128, chunk C = 64, fp16 MFMA
// operands, fp32 accumulation, fp32 state.
//
// Method: the recurrence of the "Source notes" page ("Linear attention", row
// gdn; decay before the delta update, read after the write, scale 1) computed
// in exact chunkwise form (as the attention-sink study page, "SinkProbe",
// does for its delta-rule layer).  The pages do not print the chunk algebra;
// for one (batch, value head), a chunk of n <= C tokens, entering state S
// (dv x dk), in-chunk prefix gamma_r = g_1 + ... + g_r and Gamma_r = e^{gamma_r}:
//
//   A = strict_lower(diag(beta) L o K K^T),    L[r][s] = e^{gamma_r - gamma_s}
//   T = (I + A)^{-1}                           (unit lower triangular)
//   X = diag(beta) V - diag(beta Gamma) K S^T
//   N = T X                                    (the chunk's new values)
//   O = diag(Gamma) Q S^T + (L o Q K^T)_incl N
//   S <- Gamma_n S + (diag(e^{gamma_n - gamma}) N)^T K
//
// Applying T to X (rather than forming W = T diag(beta Gamma) K and
// U = T diag(beta) V) saves one C x C x d product per chunk.  Every exponent is
// of a non-positive number, so nothing overflows.  The "Backend and numerical
// limits" section records the prior art's precision model (fp32 carry and
// accumulation, 16-bit operands, TF32 triangular inversion); here operands are
// fp16 (three more mantissa bits than bf16 at the same matrix-core rate), the
// triangular inverse has fp32 16 x 16 diagonal blocks and fp16-MFMA
// off-diagonal blocks, and the state is carried in fp32 accumulators.
//
// Work decomposition: the rows of the state evolve independently, so one
// 256-thread workgroup (4 waves) owns the DVS = 32 state rows [i0, i0 + 32)
// of one (batch, value head) and walks the chunks in order; its fp32 state
// slice stays in MFMA accumulator registers for the whole sequence.  Blocks
// are numbered so that the 4 slices and the 3 value heads that share a
// key/query head land on the same XCD (the shared K/Q and the 64-byte V rows
// then hit in that XCD's L2).  LDS is 77.6 KB, so two workgroups run per CU and
// one's vector-ALU phases overlap the other's matrix phases.  The next
// chunk's global loads are issued at the top of the current chunk into
// registers and land in LDS at its end.
//
// Per chunk (w = wave 0..3, tiles are 16 x 16; "R" = row block of the chunk):
//   phase 1  G = K K^T row w, P0 = Q K^T row 3-w, K S^T and Q S^T rows w
//   epi 1    A (off-diagonal fp16, diagonal fp32), P = masked decayed P0,
//            X^T, O accumulator = Gamma Q S^T
//   phase 2  T: diagonal 16 x 16 blocks by forward substitution (wave w ->
//            block w); off-diagonal blocks column by column (wave w ->
//            column w) with 16x16x16 MFMAs: T_RS = -T_RR sum_M A_RM T_MS
//   phase 3  N = T X rows w  ->  N^T and (diag(e^{gamma_n - gamma}) N)^T
//   phase 4  O += P N rows w -> HBM;  S^T tiles (2w, 2w+1) update -> fp16 copy
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int DK = 128, DV = 128, C = 64;
constexpr int DVS = 32;             // state rows per workgroup
constexpr int NS = DV / DVS;        // slices per head
constexpr int NI = DVS / 16;        // 16-wide value tiles per slice

// LDS strides (in elements)
constexpr int KST = DK + 8;         // sK, sQ, sS rows (fp16)
constexpr int CST = C + 8;          // sKt, sT, sP, sAo, sXN, sNd rows (fp16)
constexpr int VST = DVS + 8;        // sV rows (fp16)
constexpr int DST = 17;             // sAd rows (fp32)

// LDS map (bytes)
constexpr int OFF_KT = 0;                                 // [DK][CST] fp16
constexpr int OFF_S = OFF_KT + DK * CST * 2;              // [DVS][KST] fp16
constexpr int OFF_V = OFF_S + DVS * KST * 2;              // [C][VST] fp16
constexpr int OFF_XN = OFF_V + C * VST * 2;               // [DVS][CST] fp16: X^T, then N^T
constexpr int OFF_ND = OFF_XN + DVS * CST * 2;            // [DVS][CST] fp16: decayed N^T
constexpr int OFF_SC = OFF_ND + DVS * CST * 2;            // 5 x [C] fp32
constexpr int OFF_U = OFF_SC + 5 * C * 4;                 // union region
constexpr int OFF_K = OFF_U;                              // phase 1: [C][KST] fp16
constexpr int OFF_Q = OFF_U + C * KST * 2;                // phase 1: [C][KST] fp16
constexpr int OFF_T = OFF_U;                              // later: [C][CST] fp16
constexpr int OFF_P = OFF_T + C * CST * 2;                // later: [C][CST] fp16
constexpr int OFF_AO = OFF_P + C * CST * 2;               // later: [C][CST] fp16
constexpr int OFF_AD = OFF_AO + C * CST * 2;              // later: [4][16][DST] fp32
constexpr int U_BYTES_1 = 2 * C * KST * 2;
constexpr int U_BYTES_2 = 3 * C * CST * 2 + 4 * 16 * DST * 4;
constexpr int SMEM = OFF_U + (U_BYTES_1 > U_BYTES_2 ? U_BYTES_1 : U_BYTES_2);
static_assert(SMEM <= 80 * 1024, "two workgroups per CU need <= 80 KB of LDS each");

__device__ __forceinline__ float4v mfma32(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4v mfma16(half4 a, half4 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 to_half8(uint4 u, bf16_t) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  half8 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[2 * i] = (_Float16)__uint_as_float(w[i] << 16);
    h[2 * i + 1] = (_Float16)__uint_as_float(w[i] & 0xFFFF0000u);
  }
  return h;
}
__device__ __forceinline__ half8 to_half8(uint4 u, f16_t) {
  half8 h;
  __builtin_memcpy(&h, &u, 16);
  return h;
}

template <typename TQ, typename TG>
struct Fetch {
  uint4 k[4], q[4], v;
  float g, beta;
};

template <typename TQ, typename TG>
__device__ __forceinline__ void fetch_chunk(Fetch<TQ, TG> &f, const TQ *__restrict__ q,
                                            const TQ *__restrict__ k, const TQ *__restrict__ v,
                                            const TG *__restrict__ g, const TG *__restrict__ beta,
                                            int tid, size_t bt0, int n, int Hk, int Hv, int kh, int h,
                                            int i0) {
  const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = (tid >> 4) + 16 * it;
    const size_t off = ((bt0 + row) * Hk + kh) * DK + (tid & 15) * 8;
    f.k[it] = row < n ? *reinterpret_cast<const uint4 *>(k + off) : z;
    f.q[it] = row < n ? *reinterpret_cast<const uint4 *>(q + off) : z;
  }
  {
    const int row = tid >> 2;
    const size_t off = ((bt0 + row) * Hv + h) * DV + i0 + (tid & 3) * 8;
    f.v = row < n ? *reinterpret_cast<const uint4 *>(v + off) : z;
  }
  if (tid < C) {
    const bool ok = tid < n;
    f.g = ok ? to_f32(g[(bt0 + tid) * Hv + h]) : 0.f;
    f.beta = ok ? to_f32(beta[(bt0 + tid) * Hv + h]) : 0.f;
  }
}

template <typename TQ, typename TG>
__device__ __forceinline__ void commit_chunk(const Fetch<TQ, TG> &f, unsigned char *smem, int tid) {
  _Float16 *sK = reinterpret_cast<_Float16 *>(smem + OFF_K);
  _Float16 *sQ = reinterpret_cast<_Float16 *>(smem + OFF_Q);
  _Float16 *sKt = reinterpret_cast<_Float16 *>(smem + OFF_KT);
  _Float16 *sV = reinterpret_cast<_Float16 *>(smem + OFF_V);
  float *sc = reinterpret_cast<float *>(smem + OFF_SC);
  const int c8 = (tid & 15) * 8;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = (tid >> 4) + 16 * it;
    const half8 hk = to_half8(f.k[it], TQ{});
    const half8 hq = to_half8(f.q[it], TQ{});
    *reinterpret_cast<half8 *>(sK + row * KST + c8) = hk;
    *reinterpret_cast<half8 *>(sQ + row * KST + c8) = hq;
#pragma unroll
    for (int j = 0; j < 8; ++j) sKt[(c8 + j) * CST + row] = hk[j];
  }
  *reinterpret_cast<half8 *>(sV + (tid >> 2) * VST + (tid & 3) * 8) = to_half8(f.v, TQ{});
  if (tid < C) {
    // inclusive prefix of the log decay over the chunk (wave 0, one token per lane)
    float x = f.g;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      if (tid >= off) x += y;
    }
    const float gC = __shfl(x, 63, 64);
    const float eg = __expf(x);
    sc[0 * C + tid] = x;                 // gamma_r
    sc[1 * C + tid] = eg;                // Gamma_r
    sc[2 * C + tid] = f.beta;            // beta_r
    sc[3 * C + tid] = f.beta * eg;       // beta_r Gamma_r
    sc[4 * C + tid] = __expf(gC - x);    // e^{gamma_n - gamma_r}
  }
}

template <typename TQ, typename TG>
__global__ __launch_bounds__(kThreads, 2) void chunk_mfma_kernel(
    const TQ *__restrict__ q, const TQ *__restrict__ k, const TQ *__restrict__ v,
    const TG *__restrict__ g, const TG *__restrict__ beta, const float *__restrict__ S0,
    float *__restrict__ o, float *__restrict__ ST, int T, int Hk, int Hv, int ntasks) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  _Float16 *sKt = reinterpret_cast<_Float16 *>(smem + OFF_KT);
  _Float16 *sS = reinterpret_cast<_Float16 *>(smem + OFF_S);
  _Float16 *sV = reinterpret_cast<_Float16 *>(smem + OFF_V);
  _Float16 *sXN = reinterpret_cast<_Float16 *>(smem + OFF_XN);
  _Float16 *sNd = reinterpret_cast<_Float16 *>(smem + OFF_ND);
  const float *sGam = reinterpret_cast<const float *>(smem + OFF_SC);
  const float *sEg = sGam + C;
  const float *sB = sGam + 2 * C;
  const float *sBG = sGam + 3 * C;
  const float *sDec = sGam + 4 * C;
  _Float16 *sK = reinterpret_cast<_Float16 *>(smem + OFF_K);
  _Float16 *sQ = reinterpret_cast<_Float16 *>(smem + OFF_Q);
  _Float16 *sT = reinterpret_cast<_Float16 *>(smem + OFF_T);
  _Float16 *sP = reinterpret_cast<_Float16 *>(smem + OFF_P);
  _Float16 *sAo = reinterpret_cast<_Float16 *>(smem + OFF_AO);
  float *sAd = reinterpret_cast<float *>(smem + OFF_AD);

  // ---- task: blocks round-robin over the 8 XCDs; give each XCD a contiguous
  // range of tasks so the slices/heads that share K and Q share an L2 ----
  const int bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3;
  const int per = ntasks >> 3, rem = ntasks & 7;
  const int task = xcd * per + min(xcd, rem) + idx;
  const int slice = task % NS;
  const int bh = task / NS;  // b * Hv + h
  const int h = bh % Hv, b = bh / Hv;
  const int kh = h / (Hv / Hk);
  const int i0 = slice * DVS;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g4 = l >> 4, ln = l & 15;
  const size_t bT = (size_t)b * T;

  // ---- entering state: S^T tiles (J = 2w + jj, I) in accumulators ----
  float4v accS[2][NI];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int I = 0; I < NI; ++I) {
      const int j0 = 16 * (2 * w + jj) + 4 * g4;
      const int il = 16 * I + ln;
      float4v s = {0.f, 0.f, 0.f, 0.f};
      if (S0) {
        const float4 t = *reinterpret_cast<const float4 *>(S0 + ((size_t)bh * DV + i0 + il) * DK + j0);
        s[0] = t.x; s[1] = t.y; s[2] = t.z; s[3] = t.w;
      }
      accS[jj][I] = s;
      half4 hs;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) hs[ii] = (_Float16)s[ii];
      *reinterpret_cast<half4 *>(sS + il * KST + j0) = hs;
    }

  const int nchunks = (T + C - 1) / C;
  Fetch<TQ, TG> f;
  fetch_chunk(f, q, k, v, g, beta, tid, bT, min(C, T), Hk, Hv, kh, h, i0);
  commit_chunk(f, smem, tid);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * C;
    if (c + 1 < nchunks)
      fetch_chunk(f, q, k, v, g, beta, tid, bT + t0 + C, min(C, T - t0 - C), Hk, Hv, kh, h, i0);

    // ================= phase 1: G row w, P0 row 3-w, K S^T and Q S^T rows w
    float4v accG[4], accP[4], accDK[NI], accDQ[NI];
    const int Rp = 3 - w;
    {
      half8 ak[4], aq[4], ap[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        ak[kk] = *reinterpret_cast<const half8 *>(sK + (16 * w + ln) * KST + 32 * kk + 8 * g4);
        aq[kk] = *reinterpret_cast<const half8 *>(sQ + (16 * w + ln) * KST + 32 * kk + 8 * g4);
        ap[kk] = *reinterpret_cast<const half8 *>(sQ + (16 * Rp + ln) * KST + 32 * kk + 8 * g4);
      }
#pragma unroll
      for (int S = 0; S < 4; ++S) {
        float4v ag = {0.f, 0.f, 0.f, 0.f}, apv = {0.f, 0.f, 0.f, 0.f};
        if (S <= w || S <= Rp) {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const half8 bk =
                *reinterpret_cast<const half8 *>(sK + (16 * S + ln) * KST + 32 * kk + 8 * g4);
            if (S <= w) ag = mfma32(ak[kk], bk, ag);
            if (S <= Rp) apv = mfma32(ap[kk], bk, apv);
          }
        }
        accG[S] = ag;
        accP[S] = apv;
      }
#pragma unroll
      for (int I = 0; I < NI; ++I) {
        float4v dk_ = {0.f, 0.f, 0.f, 0.f}, dq_ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const half8 bs =
              *reinterpret_cast<const half8 *>(sS + (16 * I + ln) * KST + 32 * kk + 8 * g4);
          dk_ = mfma32(ak[kk], bs, dk_);
          dq_ = mfma32(aq[kk], bs, dq_);
        }
        accDK[I] = dk_;
        accDQ[I] = dq_;
      }
    }
    __syncthreads();  // sK / sQ are dead from here: their space becomes T, P, A

    // ================= epilogue 1
    float4v accO[NI];
    {
      // A from G: off-diagonal blocks fp16, diagonal blocks fp32 (strictly lower)
#pragma unroll
      for (int S = 0; S < 4; ++S) {
        if (S <= w) {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int r = 16 * w + 4 * g4 + ii, s = 16 * S + ln;
            const float a = sB[r] * __expf(sGam[r] - sGam[s]) * accG[S][ii];
            if (S < w)
              sAo[r * CST + s] = (_Float16)a;
            else
              sAd[(w * 16 + (r - 16 * w)) * DST + (s - 16 * w)] = s < r ? a : 0.f;
          }
        }
        if (S <= Rp) {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int r = 16 * Rp + 4 * g4 + ii, s = 16 * S + ln;
            const float p = s <= r ? __expf(sGam[r] - sGam[s]) * accP[S][ii] : 0.f;
            sP[r * CST + s] = (_Float16)p;
          }
        }
      }
      // zero the upper blocks that the K = 32 products read: P_01, P_23, T_01, T_23
      {
        const int rr = tid >> 4, cc = tid & 15;
        sP[rr * CST + 16 + cc] = (_Float16)0.f;
        sP[(32 + rr) * CST + 48 + cc] = (_Float16)0.f;
        sT[rr * CST + 16 + cc] = (_Float16)0.f;
        sT[(32 + rr) * CST + 48 + cc] = (_Float16)0.f;
      }
      // X^T and the O accumulator
#pragma unroll
      for (int I = 0; I < NI; ++I) {
        const int r0 = 16 * w + 4 * g4, il = 16 * I + ln;
        half4 xv;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = r0 + ii;
          const float x = sB[r] * (float)sV[r * VST + il] - sBG[r] * accDK[I][ii];
          xv[ii] = (_Float16)x;
          accO[I][ii] = sEg[r] * accDQ[I][ii];
        }
        *reinterpret_cast<half4 *>(sXN + il * CST + r0) = xv;
      }
    }
    __syncthreads();

    // ================= phase 2a: diagonal blocks of T by forward substitution
    {
      const int cc = l >> 2, sub = l & 3;
      const float *Ad = sAd + w * 16 * DST;
      float t[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) t[j] = (4 * j + sub == cc) ? 1.f : 0.f;
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = 4 * j + sub;
          if (m < r) part += Ad[r * DST + m] * t[j];
        }
        part += __shfl_xor(part, 1, 64);
        part += __shfl_xor(part, 2, 64);
        const float val = (r == cc) ? 1.f : -part;
        if ((r & 3) == sub) t[r >> 2] = val;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) sT[(16 * w + 4 * j + sub) * CST + 16 * w + cc] = (_Float16)t[j];
    }
    __syncthreads();

    // ================= phase 2b: off-diagonal blocks, column S = w (waves 0..2)
    if (w < 3) {
      const int S = w;
      half4 tcol[4];
#pragma unroll
      for (int M = 0; M < 4; ++M) {
        if (M == S) {
#pragma unroll
          for (int j = 0; j < 4; ++j) tcol[M][j] = sT[(16 * S + 4 * g4 + j) * CST + 16 * S + ln];
        }
      }
#pragma unroll
      for (int R = 1; R < 4; ++R) {
        if (R > S) {
          float4v y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int M = 0; M < 3; ++M) {
            if (M >= S && M < R) {
              const half4 a =
                  *reinterpret_cast<const half4 *>(sAo + (16 * R + ln) * CST + 16 * M + 4 * g4);
              y = mfma16(a, tcol[M], y);
            }
          }
          half4 yb;
#pragma unroll
          for (int j = 0; j < 4; ++j) yb[j] = (_Float16)y[j];
          const half4 trr =
              *reinterpret_cast<const half4 *>(sT + (16 * R + ln) * CST + 16 * R + 4 * g4);
          const float4v zero = {0.f, 0.f, 0.f, 0.f};
          const float4v tr = mfma16(trr, yb, zero);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            tcol[R][j] = (_Float16)(-tr[j]);
            sT[(16 * R + 4 * g4 + j) * CST + 16 * S + ln] = tcol[R][j];
          }
        }
      }
    }
    __syncthreads();

    // ================= phase 3: N = T X, rows w
    float4v accN[NI];
#pragma unroll
    for (int I = 0; I < NI; ++I) {
      float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk == 0 || w >= 2) {
          const half8 a = *reinterpret_cast<const half8 *>(sT + (16 * w + ln) * CST + 32 * kk + 8 * g4);
          const half8 bx =
              *reinterpret_cast<const half8 *>(sXN + (16 * I + ln) * CST + 32 * kk + 8 * g4);
          acc = mfma32(a, bx, acc);
        }
      }
      accN[I] = acc;
    }
    __syncthreads();  // X^T fully read: its space takes N^T
#pragma unroll
    for (int I = 0; I < NI; ++I) {
      const int r0 = 16 * w + 4 * g4, il = 16 * I + ln;
      half4 nv, nd;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        nv[ii] = (_Float16)accN[I][ii];
        nd[ii] = (_Float16)(accN[I][ii] * sDec[r0 + ii]);
      }
      *reinterpret_cast<half4 *>(sXN + il * CST + r0) = nv;
      *reinterpret_cast<half4 *>(sNd + il * CST + r0) = nd;
    }
    __syncthreads();

    // ================= phase 4: O += P N (rows w) and the state update
#pragma unroll
    for (int I = 0; I < NI; ++I) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk == 0 || w >= 2) {
          const half8 a = *reinterpret_cast<const half8 *>(sP + (16 * w + ln) * CST + 32 * kk + 8 * g4);
          const half8 bn =
              *reinterpret_cast<const half8 *>(sXN + (16 * I + ln) * CST + 32 * kk + 8 * g4);
          accO[I] = mfma32(a, bn, accO[I]);
        }
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 16 * w + 4 * g4 + ii;
        if (t0 + r < T) o[((bT + t0 + r) * Hv + h) * DV + i0 + 16 * I + ln] = accO[I][ii];
      }
    }
    {
      const float gC = sEg[C - 1];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int J = 2 * w + jj;
        half8 a[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          a[kk] = *reinterpret_cast<const half8 *>(sKt + (16 * J + ln) * CST + 32 * kk + 8 * g4);
#pragma unroll
        for (int I = 0; I < NI; ++I) {
          float4v acc = accS[jj][I];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) acc[ii] *= gC;
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const half8 bn =
                *reinterpret_cast<const half8 *>(sNd + (16 * I + ln) * CST + 32 * kk + 8 * g4);
            acc = mfma32(a[kk], bn, acc);
          }
          accS[jj][I] = acc;
          half4 hs;
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) hs[ii] = (_Float16)acc[ii];
          *reinterpret_cast<half4 *>(sS + (16 * I + ln) * KST + 16 * J + 4 * g4) = hs;
        }
      }
    }
    __syncthreads();
    if (c + 1 < nchunks) {
      commit_chunk(f, smem, tid);
      __syncthreads();
    }
  }

  // ---- final state ----
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int I = 0; I < NI; ++I) {
      const int j0 = 16 * (2 * w + jj) + 4 * g4;
      const int il = 16 * I + ln;
      const float4v s = accS[jj][I];
      *reinterpret_cast<float4 *>(ST + ((size_t)bh * DV + i0 + il) * DK + j0) =
          make_float4(s[0], s[1], s[2], s[3]);
    }
}

template <typename TQ, typename TG>
hipError_t launch_t(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                    const void *beta, const float *S0, float *o, float *ST, hipStream_t st) {
  auto kern = chunk_mfma_kernel<TQ, TG>;
  hipError_t e =
      hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, SMEM);
  if (e != hipSuccess) return e;
  const int ntasks = sh.B * sh.Hv * NS;
  hipLaunchKernelGGL(kern, dim3(ntasks), dim3(kThreads), SMEM, st, (const TQ *)q, (const TQ *)k,
                     (const TQ *)v, (const TG *)g, (const TG *)beta, S0, o, ST, sh.T, sh.Hk, sh.Hv,
                     ntasks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_mfma(const Shape &sh, const void *q, const void *k, const void *v,
                             const void *g, const void *beta, const float *S0, float *o, float *ST,
                             hipStream_t st) {
  if (sh.qkv == DType::BF16)
    return sh.gate_t == DType::F32 ? launch_t<bf16_t, float>(sh, q, k, v, g, beta, S0, o, ST, st)
                                   : launch_t<bf16_t, bf16_t>(sh, q, k, v, g, beta, S0, o, ST, st);
  return sh.gate_t == DType::F32 ? launch_t<f16_t, float>(sh, q, k, v, g, beta, S0, o, ST, st)
                                 : launch_t<f16_t, bf16_t>(sh, q, k, v, g, beta, S0, o, ST, st);
}

}  // namespace gdn
