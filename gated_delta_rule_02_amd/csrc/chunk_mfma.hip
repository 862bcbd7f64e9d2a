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
//   S <- Gamma_n S + N^T diag(e^{gamma_n - gamma}) K
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
// Two kernels.
//  * chunk_prep (every chunk in parallel): for one (batch, key head, chunk)
//    G = K K^T once, then for each value head of the group A and
//    T = (I + A)^{-1}: the 16 x 16 diagonal blocks by forward substitution in
//    fp32 (wave w -> block w), the off-diagonal blocks column by column with
//    16x16x16 MFMAs (wave w -> column w), T_RS = -T_RR sum_M A_RM T_MS.  T is
//    written to the workspace as the six MFMA A-operand fragments the
//    sequential kernel consumes (6 KB per chunk and value head).
//  * chunk_seq (the chunks of one sequence in order): one 256-thread
//    workgroup owns DVS = 32 rows of the state of one (batch, value head)
//    (rows evolve independently) and keeps them in fp32 accumulators.  Per
//    chunk only the state-dependent products remain on its path:
//      phase 1  K S^T -> X^T (LDS);  S Q^T (the read, kept transposed so a
//               lane holds 4 adjacent value channels of one token);
//               (Q K^T)^T tiles -> decayed, masked P kept in registers
//      phase 2  N = T X  -> N^T, (diag(e^{gamma_n-gamma}) N)^T (LDS)
//      phase 3  O^T = Gamma (S Q^T) + N^T P^T -> HBM (16-byte stores);
//               S = Gamma_n S + N^T diag(..) K  (K columns read from LDS)
//    P never touches LDS: the MFMA only needs A and B to agree on the order
//    of the contraction index, so the P fragment packs the two (Q K^T)^T
//    tiles of a 32-wide step as {4 g..4 g+3, 16+4 g..16+4 g+3} and N^T is
//    read in the same order.  Q and T go straight from memory into MFMA
//    registers.  LDS is 46 KB.  Blocks are numbered so that the 4 slices and
//    the value heads sharing a key head land on one XCD (shared K/Q and the
//    64-byte V rows then hit in its L2).  The next chunk's loads are issued
//    into registers during the current chunk and land in LDS at its end;
//    the workgroup barriers wait for LDS traffic only, so those loads and the
//    output stores stay in flight across them.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int DK = 128, DV = 128, C = 64;
constexpr int DVS = 32;             // state rows per sequential workgroup
constexpr int NS = DV / DVS;        // slices per head
constexpr int NI = DVS / 16;        // 16-wide value tiles per slice
constexpr int NFRAG = 6;            // T fragments per chunk: (R,kk) = (0,0),(1,0),(2,0),(2,1),(3,0),(3,1)
constexpr size_t T_BYTES = NFRAG * 64 * 16;   // per (chunk, value head)

// LDS strides (elements)
constexpr int KST = DK + 8;         // sK, sS rows (fp16)
constexpr int CST = C + 8;          // sT, sAo, sXt, sNt, sNd rows (fp16)
constexpr int VST = DVS + 8;        // sV rows (fp16)
constexpr int DST = 17;             // sAd rows (fp32)

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
__device__ __forceinline__ half8 to_half8(uint4 u, f16_t) { return __builtin_bit_cast(half8, u); }

__device__ __forceinline__ int frag_index(int R, int kk) { return R < 2 ? R : 2 * R - 2 + kk; }

// Inclusive prefix of the chunk's log decay (wave 0: lane = token) and the
// per-token scalars: gamma, Gamma = e^gamma, beta, beta Gamma, e^{gamma_n - gamma}.
__device__ __forceinline__ void chunk_scalars(float g, float beta, float *sc, int lane) {
  float x = g;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  const float gC = __shfl(x, 63, 64);
  const float eg = __expf(x);
  sc[0 * C + lane] = x;
  sc[1 * C + lane] = eg;
  sc[2 * C + lane] = beta;
  sc[3 * C + lane] = beta * eg;
  sc[4 * C + lane] = __expf(gC - x);
}

// ============================================================================
// chunk_prep: T = (I + A)^{-1} per (chunk, value head)
// ============================================================================
constexpr int P_OFF_K = 0;                              // [C][KST] fp16
constexpr int P_OFF_T = P_OFF_K + C * KST * 2;          // [C][CST] fp16
constexpr int P_OFF_AO = P_OFF_T + C * CST * 2;         // [C][CST] fp16
constexpr int P_OFF_AD = P_OFF_AO + C * CST * 2;        // [4][16][DST] fp32
constexpr int P_OFF_SC = P_OFF_AD + 4 * 16 * DST * 4;   // 5 x [C] fp32
constexpr int P_SMEM = P_OFF_SC + 5 * C * 4;

template <typename TQ, typename TG>
__global__ __launch_bounds__(kThreads, 2) void chunk_prep_kernel(
    const TQ *__restrict__ k, const TG *__restrict__ g, const TG *__restrict__ beta,
    uint4 *__restrict__ Tws, int T, int Hk, int Hv, int nchunks) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[P_SMEM];
  _Float16 *sK = reinterpret_cast<_Float16 *>(smem + P_OFF_K);
  _Float16 *sT = reinterpret_cast<_Float16 *>(smem + P_OFF_T);
  _Float16 *sAo = reinterpret_cast<_Float16 *>(smem + P_OFF_AO);
  float *sAd = reinterpret_cast<float *>(smem + P_OFF_AD);
  float *sc = reinterpret_cast<float *>(smem + P_OFF_SC);
  const float *sGam = sc;
  const float *sB = sc + 2 * C;

  const int c = blockIdx.x;
  const int b = blockIdx.y / Hk, kh = blockIdx.y % Hk;
  const int grp = Hv / Hk;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g4 = l >> 4, ln = l & 15;
  const int t0 = c * C, n = min(C, T - t0);
  const size_t bt0 = (size_t)b * T + t0;

  // K tile (fp16)
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = (tid >> 4) + 16 * it;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (row < n) u = *reinterpret_cast<const uint4 *>(k + ((bt0 + row) * Hk + kh) * DK + (tid & 15) * 8);
    *reinterpret_cast<half8 *>(sK + row * KST + (tid & 15) * 8) = to_half8(u, TQ{});
  }
  lds_barrier();

  // G row w, tiles (w, w - d)
  float4v accG[4];
  {
    const _Float16 *kw = sK + (16 * w + ln) * KST + 8 * g4;
    half8 ak[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) ak[kk] = *reinterpret_cast<const half8 *>(kw + 32 * kk);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float4v ag = {0.f, 0.f, 0.f, 0.f};
      if (d <= w) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          ag = mfma32(ak[kk], *reinterpret_cast<const half8 *>(kw - 16 * d * KST + 32 * kk), ag);
      }
      accG[d] = ag;
    }
  }

  for (int hv = 0; hv < grp; ++hv) {
    const int h = kh * grp + hv;
    lds_barrier();  // previous head's T fully written out
    if (tid < C) {
      const bool ok = tid < n;
      const float gv = ok ? to_f32(g[(bt0 + tid) * Hv + h]) : 0.f;
      const float bv = ok ? to_f32(beta[(bt0 + tid) * Hv + h]) : 0.f;
      chunk_scalars(gv, bv, sc, tid);
    }
    lds_barrier();
    // A: diagonal blocks fp32 (strictly lower), off-diagonal blocks fp16
    {
      const int r0 = 16 * w + 4 * g4;
      float gr[4], br[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        gr[ii] = sGam[r0 + ii];
        br[ii] = sB[r0 + ii];
      }
      float *ad = sAd + (w * 16 + 4 * g4) * DST + ln;
      _Float16 *ao = sAo + r0 * CST + 16 * w + ln;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        if (d <= w) {
          const float gs = sGam[16 * (w - d) + ln];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            if (d == 0) {
              const bool keep = ln < 4 * g4 + ii;
              const float a = br[ii] * __expf(keep ? gr[ii] - gs : 0.f) * accG[0][ii];
              ad[ii * DST] = keep ? a : 0.f;
            } else {
              ao[ii * CST - 16 * d] = (_Float16)(br[ii] * __expf(gr[ii] - gs) * accG[d][ii]);
            }
          }
        }
      }
      // the upper blocks inside the fragments are zero
      const int rr = tid >> 4, cc = tid & 15;
      sT[rr * CST + 16 + cc] = (_Float16)0.f;
      sT[(32 + rr) * CST + 48 + cc] = (_Float16)0.f;
    }
    lds_barrier();
    // diagonal blocks of T by forward substitution (wave w -> block w):
    // lane = (column cc, sub); the lane keeps T[4j + sub][cc], j = 0..3
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
    lds_barrier();
    // off-diagonal blocks, column S = w (waves 0..2); block (S+e, S) = tc[e]
    if (w < 3) {
      const int S = w;
      half4 tc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) tc[0][j] = sT[(16 * S + 4 * g4 + j) * CST + 16 * S + ln];
#pragma unroll
      for (int e = 1; e < 4; ++e) {
        if (S + e <= 3) {
          const int R = S + e;
          float4v y = {0.f, 0.f, 0.f, 0.f};
          const _Float16 *arow = sAo + (16 * R + ln) * CST + 16 * S + 4 * g4;
#pragma unroll
          for (int f = 0; f < e; ++f)
            y = mfma16(*reinterpret_cast<const half4 *>(arow + 16 * f), tc[f], y);
          half4 yb;
#pragma unroll
          for (int j = 0; j < 4; ++j) yb[j] = (_Float16)y[j];
          const half4 trr =
              *reinterpret_cast<const half4 *>(sT + (16 * R + ln) * CST + 16 * R + 4 * g4);
          const float4v zero = {0.f, 0.f, 0.f, 0.f};
          const float4v tr = mfma16(trr, yb, zero);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            tc[e][j] = (_Float16)(-tr[j]);
            sT[(16 * R + 4 * g4 + j) * CST + 16 * S + ln] = tc[e][j];
          }
        }
      }
    }
    lds_barrier();
    // T as A-operand fragments: wave w writes row block w
    {
      uint4 *dst = Tws + (((size_t)b * Hv + h) * nchunks + c) * (NFRAG * 64);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk == 0 || w >= 2) {
          const uint4 fr = *reinterpret_cast<const uint4 *>(sT + (16 * w + ln) * CST + 32 * kk + 8 * g4);
          dst[frag_index(w, kk) * 64 + l] = fr;
        }
      }
    }
  }
}

// ============================================================================
// chunk_seq: the sequential pass over the chunks of one sequence
// ============================================================================
constexpr int S_OFF_K = 0;                              // [C][KST] fp16
constexpr int S_OFF_S = S_OFF_K + C * KST * 2;          // [DVS][KST] fp16
constexpr int S_OFF_V = S_OFF_S + DVS * KST * 2;        // [C][VST] fp16
constexpr int S_OFF_XT = S_OFF_V + C * VST * 2;         // [DVS][CST] fp16
constexpr int S_OFF_NT = S_OFF_XT + DVS * CST * 2;      // [DVS][CST] fp16
constexpr int S_OFF_ND = S_OFF_NT + DVS * CST * 2;      // [DVS][CST] fp16
constexpr int S_OFF_SC = S_OFF_ND + DVS * CST * 2;      // 5 x [C] fp32
constexpr int S_SMEM = S_OFF_SC + 5 * C * 4;
static_assert(S_SMEM <= 64 * 1024, "static LDS");

// The next chunk's raw loads.  Every load is unconditional (rows past the end
// of the sequence re-read its last row) and nothing is converted here, so no
// instruction needs the data before the chunk is committed: the loads stay in
// flight through the current chunk's work.
template <typename TQ, typename TG>
struct SeqFetch {
  uint4 k[4], q[4], v, t0, t1;
  TG g, beta;
  int n;  // valid rows of the fetched chunk
};

template <typename TQ, typename TG>
__device__ __forceinline__ void seq_fetch(SeqFetch<TQ, TG> &f, const TQ *__restrict__ q,
                                          const TQ *__restrict__ k, const TQ *__restrict__ v,
                                          const TG *__restrict__ g, const TG *__restrict__ beta,
                                          const uint4 *__restrict__ Tc, int tid, int w, int l,
                                          size_t bt0, int n, int Hk, int Hv, int kh, int h, int i0) {
  f.n = n;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = min((tid >> 4) + 16 * it, n - 1);
    f.k[it] = *reinterpret_cast<const uint4 *>(k + ((bt0 + row) * Hk + kh) * DK + (tid & 15) * 8);
  }
  {
    // Q fragments of row block w: lane (g4, ln) -> Q[16 w + ln][32 kk + 8 g4 ..]
    const int row = min(16 * w + (l & 15), n - 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      f.q[kk] = *reinterpret_cast<const uint4 *>(q + ((bt0 + row) * Hk + kh) * DK + 32 * kk + 8 * (l >> 4));
  }
  {
    const int row = min(tid >> 2, n - 1);
    f.v = *reinterpret_cast<const uint4 *>(v + ((bt0 + row) * Hv + h) * DV + i0 + (tid & 3) * 8);
  }
  f.t0 = Tc[frag_index(w, 0) * 64 + l];
  f.t1 = Tc[frag_index(w, w >= 2 ? 1 : 0) * 64 + l];
  const int row = min(tid & 63, n - 1);
  f.g = g[(bt0 + row) * Hv + h];
  f.beta = beta[(bt0 + row) * Hv + h];
}

// Land a fetched chunk: K and V tiles into LDS (rows past the end as zeros),
// Q and T fragments into registers, the per-token scalars into LDS.
template <typename TQ, typename TG>
__device__ __forceinline__ void seq_commit(const SeqFetch<TQ, TG> &f, _Float16 *sK, _Float16 *sV,
                                           float *sc, half8 (&qf)[4], half8 (&tf)[2], int tid,
                                           int w, int l) {
  const int c8 = (tid & 15) * 8;
  const half8 hz = {};
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = (tid >> 4) + 16 * it;
    *reinterpret_cast<half8 *>(sK + row * KST + c8) = row < f.n ? to_half8(f.k[it], TQ{}) : hz;
  }
  *reinterpret_cast<half8 *>(sV + (tid >> 2) * VST + (tid & 3) * 8) =
      (tid >> 2) < f.n ? to_half8(f.v, TQ{}) : hz;
  const bool qok = 16 * w + (l & 15) < f.n;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qf[kk] = qok ? to_half8(f.q[kk], TQ{}) : hz;
  tf[0] = __builtin_bit_cast(half8, f.t0);
  tf[1] = __builtin_bit_cast(half8, f.t1);
  if (tid < C) {
    const bool ok = tid < f.n;
    chunk_scalars(ok ? to_f32(f.g) : 0.f, ok ? to_f32(f.beta) : 0.f, sc, tid);
  }
}

template <typename TQ, typename TG>
__global__ __launch_bounds__(kThreads, 2) void chunk_seq_kernel(
    const TQ *__restrict__ q, const TQ *__restrict__ k, const TQ *__restrict__ v,
    const TG *__restrict__ g, const TG *__restrict__ beta, const uint4 *__restrict__ Tws,
    const float *__restrict__ S0, float *__restrict__ o, float *__restrict__ ST, int T, int Hk,
    int Hv, int ntasks, int nchunks) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[S_SMEM];
  _Float16 *sK = reinterpret_cast<_Float16 *>(smem + S_OFF_K);
  _Float16 *sS = reinterpret_cast<_Float16 *>(smem + S_OFF_S);
  _Float16 *sV = reinterpret_cast<_Float16 *>(smem + S_OFF_V);
  _Float16 *sXt = reinterpret_cast<_Float16 *>(smem + S_OFF_XT);
  _Float16 *sNt = reinterpret_cast<_Float16 *>(smem + S_OFF_NT);
  _Float16 *sNd = reinterpret_cast<_Float16 *>(smem + S_OFF_ND);
  float *sc = reinterpret_cast<float *>(smem + S_OFF_SC);
  const float *sGam = sc, *sEg = sc + C, *sB = sc + 2 * C, *sBG = sc + 3 * C, *sDec = sc + 4 * C;

  // blocks go round-robin over the 8 XCDs: give each XCD a contiguous task range
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
  const uint4 *Tbh = Tws + (size_t)bh * nchunks * (NFRAG * 64);

  // entering state: tiles (I, J = 2 w + jj), lane holds S[16 I + 4 g4 + ii][16 J + ln]
  float4v accS[2][NI];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int I = 0; I < NI; ++I) {
      const int j = 16 * (2 * w + jj) + ln;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int il = 16 * I + 4 * g4 + ii;
        const float s = S0 ? S0[((size_t)bh * DV + i0 + il) * DK + j] : 0.f;
        accS[jj][I][ii] = s;
        sS[il * KST + j] = (_Float16)s;
      }
    }

  SeqFetch<TQ, TG> f;
  half8 qf[4];
  half8 tf[2];
  seq_fetch(f, q, k, v, g, beta, Tbh, tid, w, l, bT, min(C, T), Hk, Hv, kh, h, i0);
  seq_commit(f, sK, sV, sc, qf, tf, tid, w, l);
  lds_barrier();

  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * C;
    if (c + 1 < nchunks)
      seq_fetch(f, q, k, v, g, beta, Tbh + (size_t)(c + 1) * (NFRAG * 64), tid, w, l, bT + t0 + C,
                min(C, T - t0 - C), Hk, Hv, kh, h, i0);

    // ================= phase 1
    float4v accDK[NI], accO[NI], accPt[4];
    {
      const _Float16 *kw = sK + (16 * w + ln) * KST + 8 * g4;
      half8 ak[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) ak[kk] = *reinterpret_cast<const half8 *>(kw + 32 * kk);
#pragma unroll
      for (int I = 0; I < NI; ++I) {
        float4v dk_ = {0.f, 0.f, 0.f, 0.f}, so_ = {0.f, 0.f, 0.f, 0.f};
        const _Float16 *srow = sS + (16 * I + ln) * KST + 8 * g4;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const half8 s8 = *reinterpret_cast<const half8 *>(srow + 32 * kk);
          dk_ = mfma32(ak[kk], s8, dk_);   // (K S^T)[16 w + 4 g4 + ii][16 I + ln]
          so_ = mfma32(s8, qf[kk], so_);   // (S Q^T)[16 I + 4 g4 + ii][16 w + ln]
        }
        accDK[I] = dk_;
        accO[I] = so_;
      }
      // (Q K^T)^T tiles (S', w) for S' <= w: lane holds P0[16 w + ln][16 S' + 4 g4 + ii]
#pragma unroll
      for (int Sp = 0; Sp < 4; ++Sp) {
        float4v acc = {0.f, 0.f, 0.f, 0.f};
        if (Sp <= w) {
          const _Float16 *krow = sK + (16 * Sp + ln) * KST + 8 * g4;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            acc = mfma32(*reinterpret_cast<const half8 *>(krow + 32 * kk), qf[kk], acc);
        }
        accPt[Sp] = acc;
      }
    }

    // ================= epilogue 1: X^T to LDS, O scaled, P in registers
    half8 pf[2];
    {
      const int r0 = 16 * w + 4 * g4;
#pragma unroll
      for (int I = 0; I < NI; ++I) {
        const int il = 16 * I + ln;
        half4 xv;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = r0 + ii;
          xv[ii] = (_Float16)(sB[r] * (float)sV[r * VST + il] - sBG[r] * accDK[I][ii]);
        }
        *reinterpret_cast<half4 *>(sXt + il * CST + r0) = xv;
      }
      const int rq = 16 * w + ln;        // this lane's token in the read
      const float gq = sGam[rq], eq = sEg[rq];
#pragma unroll
      for (int I = 0; I < NI; ++I)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) accO[I][ii] *= eq;
#pragma unroll
      for (int Sp = 0; Sp < 4; ++Sp) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int s = 16 * Sp + 4 * g4 + ii;
          const bool keep = s <= rq;
          const float p = keep ? __expf(gq - sGam[s]) * accPt[Sp][ii] : 0.f;
          pf[Sp >> 1][(Sp & 1) * 4 + ii] = (_Float16)p;
        }
      }
    }
    lds_barrier();

    // ================= phase 2: N = T X (rows 16 w ..)
    {
      const int r0 = 16 * w + 4 * g4;
#pragma unroll
      for (int I = 0; I < NI; ++I) {
        float4v acc = {0.f, 0.f, 0.f, 0.f};
        const _Float16 *xrow = sXt + (16 * I + ln) * CST + 8 * g4;
        acc = mfma32(tf[0], *reinterpret_cast<const half8 *>(xrow), acc);
        if (w >= 2) acc = mfma32(tf[1], *reinterpret_cast<const half8 *>(xrow + 32), acc);
        const int il = 16 * I + ln;
        half4 nv, nd;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          nv[ii] = (_Float16)acc[ii];
          nd[ii] = (_Float16)(acc[ii] * sDec[r0 + ii]);
        }
        *reinterpret_cast<half4 *>(sNt + il * CST + r0) = nv;
        *reinterpret_cast<half4 *>(sNd + il * CST + r0) = nd;
      }
    }
    lds_barrier();

    // ================= phase 3: O^T += N^T P^T -> HBM; state update
    {
      const int rq = t0 + 16 * w + ln;
#pragma unroll
      for (int I = 0; I < NI; ++I) {
        const _Float16 *nrow = sNt + (16 * I + ln) * CST + 4 * g4;
        float4v acc = accO[I];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk == 0 || w >= 2) {
            const half4 lo = *reinterpret_cast<const half4 *>(nrow + 32 * kk);
            const half4 hi = *reinterpret_cast<const half4 *>(nrow + 32 * kk + 16);
            const half8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc = mfma32(a, pf[kk], acc);
          }
        }
        if (rq < T)
          *reinterpret_cast<float4 *>(o + ((bT + rq) * Hv + h) * DV + i0 + 16 * I + 4 * g4) =
              make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
      const float gC = sEg[C - 1];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int J = 2 * w + jj;
        half8 kc[2];  // K[32 kk + 8 g4 + j][16 J + ln]
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int j = 0; j < 8; ++j) kc[kk][j] = sK[(32 * kk + 8 * g4 + j) * KST + 16 * J + ln];
#pragma unroll
        for (int I = 0; I < NI; ++I) {
          float4v acc = accS[jj][I];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) acc[ii] *= gC;
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            acc = mfma32(*reinterpret_cast<const half8 *>(sNd + (16 * I + ln) * CST + 32 * kk + 8 * g4),
                         kc[kk], acc);
          accS[jj][I] = acc;
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) sS[(16 * I + 4 * g4 + ii) * KST + 16 * J + ln] = (_Float16)acc[ii];
        }
      }
    }
    lds_barrier();
    if (c + 1 < nchunks) {
      seq_commit(f, sK, sV, sc, qf, tf, tid, w, l);
      lds_barrier();
    }
  }

  // final state
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int I = 0; I < NI; ++I) {
      const int j = 16 * (2 * w + jj) + ln;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        ST[((size_t)bh * DV + i0 + 16 * I + 4 * g4 + ii) * DK + j] = accS[jj][I][ii];
    }
}

template <typename TQ, typename TG>
hipError_t launch_t(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                    const void *beta, const float *S0, float *o, float *ST, void *ws, hipStream_t st) {
  const int nchunks = (sh.T + C - 1) / C;
  hipLaunchKernelGGL((chunk_prep_kernel<TQ, TG>), dim3(nchunks, sh.B * sh.Hk), dim3(kThreads), 0, st,
                     (const TQ *)k, (const TG *)g, (const TG *)beta, (uint4 *)ws, sh.T, sh.Hk, sh.Hv,
                     nchunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ntasks = sh.B * sh.Hv * NS;
  hipLaunchKernelGGL((chunk_seq_kernel<TQ, TG>), dim3(ntasks), dim3(kThreads), 0, st, (const TQ *)q,
                     (const TQ *)k, (const TQ *)v, (const TG *)g, (const TG *)beta,
                     (const uint4 *)ws, S0, o, ST, sh.T, sh.Hk, sh.Hv, ntasks, nchunks);
  return hipGetLastError();
}

}  // namespace

size_t chunk_mfma_workspace(const Shape &sh) {
  const size_t nchunks = (size_t)(sh.T + C - 1) / C;
  return (size_t)sh.B * sh.Hv * nchunks * T_BYTES;
}

hipError_t launch_chunk_mfma(const Shape &sh, const void *q, const void *k, const void *v,
                             const void *g, const void *beta, const float *S0, float *o, float *ST,
                             void *ws, hipStream_t st) {
  if (sh.qkv == DType::BF16)
    return sh.gate_t == DType::F32
               ? launch_t<bf16_t, float>(sh, q, k, v, g, beta, S0, o, ST, ws, st)
               : launch_t<bf16_t, bf16_t>(sh, q, k, v, g, beta, S0, o, ST, ws, st);
  return sh.gate_t == DType::F32 ? launch_t<f16_t, float>(sh, q, k, v, g, beta, S0, o, ST, ws, st)
                                 : launch_t<f16_t, bf16_t>(sh, q, k, v, g, beta, S0, o, ST, ws, st);
}

}  // namespace gdn
