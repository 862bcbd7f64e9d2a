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
// Fragments.  A 16x16x32 MFMA only needs its A and B operands to agree on the
// order of the 32 contraction indices a lane group holds.  Here lane group g
// (lanes 16 g .. 16 g + 15) of step kk holds the indices
//     kset(g, kk) = {32 kk + 4 g + e, 32 kk + 16 + 4 g + e : e = 0..3},
// which are exactly the rows an accumulator tile pair (16 rows each) leaves in
// that lane group.  So an MFMA result can feed the next MFMA as an operand
// without leaving the lane that computed it.
//
// Two kernels.
//  * chunk_prep (every chunk in parallel), per (batch, key head, chunk):
//    G = K K^T and P0 = masked Q K^T once; then per value head of the group
//    A and T = (I + A)^{-1} (16 x 16 diagonal blocks by forward substitution
//    in fp32, wave w -> block w; off-diagonal blocks column by column with
//    16x16x16 MFMAs, wave w -> column w: T_RS = -T_RR sum_M A_RM T_MS), and
//    P = L o P0.  T and P (per value head) go to the workspace as 64 x 64
//    lower-triangular matrices in fragment order: six 1 KB fragments each,
//    lane (g, l) of fragment (R, kk) holding row 16 R + l at columns kset(g, kk).
//  * chunk_seq (the chunks of one sequence in order): a workgroup owns 32,
//    64 or 128 value rows of the state of one (batch, value head); each of
//    its compute waves owns 16 or 32 of them (rows evolve independently) for
//    all 64 rows of a chunk, in fp32 accumulators.  Its whole chain stays in
//    registers:
//        S (fp32) -> S fragments (fp16)                    [no data movement]
//        X = beta V - beta Gamma K S^T                     (K from LDS)
//        N = T X,  N~ = diag(e^{gamma_n - gamma}) N        (T from LDS)
//        O^T = Gamma (S Q^T) + N^T P^T -> HBM              (Q, P from LDS)
//        S^T <- Gamma_n S^T + K^T N~                       (K columns from LDS)
//    so the compute waves share only the chunk's K, Q, V tiles, T, P and
//    gate scalars, double-buffered in LDS: one barrier per chunk.  Four
//    more waves (one per SIMD) do all the loading: chunk c + 2 is fetched
//    and chunk c + 1 written to LDS while chunk c is computed (with the
//    prologue inside and fp16 q, k: K and Q of chunk c + 1 go straight from
//    global memory to LDS instead).  Blocks are numbered so that workgroups
//    sharing a key head run on one XCD (shared K and Q then hit in its L2).
#include <algorithm>
#include <map>
#include <mutex>
#include <type_traits>
#include <vector>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int DK = 128, DV = 128, C = 64;
constexpr int NFRAG = 6;                      // fragments (R, kk): (0,0),(1,0),(2,0),(2,1),(3,0),(3,1)

// LDS strides (elements)
constexpr int KST = DK + 8;                   // K, Q rows (fp16)
constexpr int CST = C + 8;                    // 64 x 64 fp16 matrices
constexpr int DST = 17;                       // fp32 16 x 16 diagonal blocks

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
__device__ __forceinline__ half4 to_half4(uint2 u, bf16_t) {
  return half4{(_Float16)__uint_as_float(u.x << 16), (_Float16)__uint_as_float(u.x & 0xFFFF0000u),
               (_Float16)__uint_as_float(u.y << 16), (_Float16)__uint_as_float(u.y & 0xFFFF0000u)};
}
__device__ __forceinline__ half4 to_half4(uint2 u, f16_t) { return __builtin_bit_cast(half4, u); }

// Eight fp32 values narrowed to a 16-bit type, as stored to memory.
__device__ __forceinline__ uint4 pack8(const float (&x)[8], f16_t) {
  half8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (f16_t)x[i];
  return __builtin_bit_cast(uint4, h);
}
// Eight bf16 values of a 16-byte piece, widened (row zero when `zero`).
__device__ __forceinline__ void unpack8(uint4 u, bool zero, float (&x)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = zero ? 0.f : __uint_as_float(w[i] << 16);
    x[2 * i + 1] = zero ? 0.f : __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// Raw inputs of the convolution prologue when it runs inside the chunked
// forward: the prep kernel convolves q and k (and writes them out for the
// sequential pass), the sequential pass convolves v as it loads it.
struct ConvIn {
  const bf16_t *xq, *xk, *xv;   // raw q, k [B,T,Hk,dk] and v [B,T,Hv,dv]
  const float *wq, *wk, *wv;    // their taps, [channels][4]
  void *q, *k;                  // q and k after the prologue, qkv dtype [B,T,Hk,dk]
  float eps;
};

// Workspace index of chunk 0 of (sequence b, value head h): per (b, h) runs of
// nchunks chunks, or, for packed sequences, per value head runs of nchunks
// slots (the sequence's chunks from slot start / C + b).
__device__ __forceinline__ size_t ws_chain(const Seqs &sq, int b, int h, int Hv, int nchunks, int start) {
  return sq.cu ? (size_t)h * nchunks + start / C + b : ((size_t)b * Hv + h) * nchunks;
}

__device__ __forceinline__ int frag_index(int R, int kk) { return R < 2 ? R : 2 * R - 2 + kk; }

// LDS transpose read of gfx950 (ds_read_b64_tr_b16).  Within each group of 16
// lanes, every lane reads 8 bytes (four fp16) and lane j receives element j % 4
// of the reads of lanes 4 e + j / 4, e = 0..3.  So if lane i of the group reads
// row r0 + i / 4, columns c0 + 4 (i % 4) .. + 3 of a row-major matrix, lane j
// receives rows r0 .. r0 + 3 of column c0 + j: a column gather in one read.
typedef short short4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ half4 lds_read_tr(const _Float16 *p) {
  return __builtin_bit_cast(
      half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v *)p));
}

// One row of a row-major fp16 matrix at the columns kset(g4, kk).
__device__ __forceinline__ half8 perm_row(const _Float16 *M, int st, int row, int kk, int g4) {
  const _Float16 *p = M + row * st + 32 * kk + 4 * g4;
  const half4 lo = *reinterpret_cast<const half4 *>(p);
  const half4 hi = *reinterpret_cast<const half4 *>(p + 16);
  return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Two accumulator tiles (rows 16 (2 kk) + 4 g4 + ii and 16 (2 kk + 1) + 4 g4 + ii)
// packed as one fragment in kset order.
__device__ __forceinline__ half8 pack_pair(float4v a, float4v b) {
  return half8{(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3],
               (_Float16)b[0], (_Float16)b[1], (_Float16)b[2], (_Float16)b[3]};
}

// Inclusive prefix of the chunk's log decay (one full wave: lane = token) and
// the per-token scalars: gamma, Gamma = e^gamma, beta, beta Gamma, e^{gamma_n - gamma}.
__device__ __forceinline__ void chunk_scalars(float g, float beta, float *sc, int lane) {
  const float x = wave_prefix_sum(g);
  const float gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
  const float eg = __expf(x);
  sc[0 * C + lane] = x;
  sc[1 * C + lane] = eg;
  sc[2 * C + lane] = beta;
  sc[3 * C + lane] = beta * eg;
  sc[4 * C + lane] = __expf(gC - x);
}

// fp16 high and low parts of x: x = hi + lo to about 22 bits.
// The low part is x - hi (exact in fp32) rounded to fp16 by one mixed-precision
// fma (hi read as fp16, -1 and x as fp32), written out as the instruction:
// the compiler otherwise widens hi, subtracts and narrows again.
__device__ __forceinline__ void split16(float x, _Float16 &hi, _Float16 &lo) {
  hi = (_Float16)x;
  const uint32_t h = __builtin_bit_cast(uint16_t, hi);
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(x));
  lo = __builtin_bit_cast(_Float16, (uint16_t)r);
}

// T = (I + A)^{-1} for a 64 x 64 unit lower-triangular I + A, then T (and,
// NP >= 1, P after it; NP = 2, P as high part sP and low part sPl) stored as
// fragments at dst.  On entry the strictly
// lower 16 x 16 diagonal blocks of A are in sAd (fp32), its blocks below the
// diagonal in sAo (fp16), and sT (and sP) have zero blocks (0,1) and (2,3)
// (the fragments read them).  Called by all 256 threads; wave w owns block
// row w.
//
// Diagonal blocks: forward substitution in fp32 (wave w -> block w).  Blocks
// below: column by column, T_RS = -T_RR sum_M A_RM T_MS, on 16x16x16 MFMAs.
template <int NP>
__device__ __forceinline__ void invert_store(const float *sAd, const _Float16 *sAo, _Float16 *sT,
                                             const _Float16 *sP, const _Float16 *sPl, uint4 *__restrict__ dst,
                                             int w, int l) {
  const int g4 = l >> 4, ln = l & 15;
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
      part = group_sum<4>(part);
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
  {
    // T (then P): NFRAG fragments each
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      if (kk == 0 || w >= 2) {
        dst[frag_index(w, kk) * 64 + l] = __builtin_bit_cast(uint4, perm_row(sT, CST, 16 * w + ln, kk, g4));
        if constexpr (NP >= 1)
          dst[(NFRAG + frag_index(w, kk)) * 64 + l] =
              __builtin_bit_cast(uint4, perm_row(sP, CST, 16 * w + ln, kk, g4));
        if constexpr (NP == 2)
          dst[(2 * NFRAG + frag_index(w, kk)) * 64 + l] =
              __builtin_bit_cast(uint4, perm_row(sPl, CST, 16 * w + ln, kk, g4));
      }
  }
}

// Workspace of the key-channel gate per (batch, value head, chunk), in
// 16-byte units: T and P fragments; K o e^gamma, Q o e^gamma and
// K o e^{gamma_n - gamma} (fp16, 64 x 128 row-major, rows past the end of the
// sequence zero); beta[64] and Gamma_n[128] (fp32).
// Workspace of the head gate per (batch, value head, chunk): T fragments,
// then the per-token scalars of chunk_scalars (5 x 64 fp32); P is formed in
// the sequential pass.  With at most 64 chains (the sequential pass then
// runs two compute waves per workgroup and is bound by its chain of chunks)
// the prep also forms P and stores its high and low parts after T.
constexpr int GDN_SC = NFRAG * 64;
constexpr int GDN_CHUNK_U4 = GDN_SC + 5 * C / 4;
constexpr int GDN_SC_P = 3 * NFRAG * 64;
constexpr int GDN_CHUNK_U4_P = GDN_SC_P + 5 * C / 4;
constexpr int KDA_KG = 2 * NFRAG * 64;
constexpr int KDA_QG = KDA_KG + C * DK / 8;
constexpr int KDA_KD = KDA_QG + C * DK / 8;
constexpr int KDA_SC = KDA_KD + C * DK / 8;
constexpr int KDA_NSC = (C + DK) / 4;
constexpr int KDA_CHUNK_U4 = (KDA_SC + KDA_NSC + 15) / 16 * 16;

// ============================================================================
// chunk_prep: per (chunk, key head) G = K K^T; per (chunk, value head) T = (I + A)^{-1}
// ============================================================================
// K is only read before the value-head loop (into the G accumulators); the
// per-head matrices then reuse its space.  After K and Q (Q: with the
// convolution, whose q this kernel makes for the sequential pass): the gate
// and beta of the group's heads (2 x grp x C fp32), then the five per-token
// scalars of the current head, which (convolution) first hold the taps of k
// and q: the two are never live together.
constexpr int P_OFF_K = 0;                              // [C][KST] fp16
constexpr int P_OFF_Q = P_OFF_K + C * KST * 2;          // [C][KST] fp16
constexpr int P_OFF_T = 0;                              // [C][CST] fp16 (over K)
constexpr int P_OFF_AO = P_OFF_T + C * CST * 2;         // [C][CST] fp16
constexpr int P_OFF_AD = P_OFF_AO + C * CST * 2;        // [4][16][DST] fp32
constexpr int P_OFF_GB = P_OFF_Q + C * KST * 2;         // then 2 x grp x C fp32
constexpr int P_SC_BYTES = 5 * C * 4, P_TAP_BYTES = 2 * DK * 16;
static_assert(P_OFF_AD + 4 * 16 * DST * 4 <= P_OFF_GB, "per-head matrices overlap the gates");
// PW (P to the workspace): its high and low parts after the inverse's
// matrices (over Q, which is read only before the head loop), and the gates
// after them
constexpr int P_OFF_PH = P_OFF_AD + 4 * 16 * DST * 4;   // [C][CST] fp16
constexpr int P_OFF_PL = P_OFF_PH + C * CST * 2;        // [C][CST] fp16
constexpr int P_OFF_GB_P = P_OFF_PL + C * CST * 2;
inline size_t prep_smem(int grp, bool conv, bool pw) {
  return (pw ? P_OFF_GB_P : P_OFF_GB) + (size_t)2 * grp * C * 4 + (conv ? P_TAP_BYTES : P_SC_BYTES);
}

// CONV: q and k are computed here from the raw inputs of cv (convolution,
// SiLU, L2 normalisation) and written to cv.q and cv.k for the sequential
// pass; the q and k arguments are not read.  PW: P = L o Q K^T with the
// decays too, once per key head as P0 = masked Q K^T, then scaled per value
// head; its high and low parts go to the workspace after T.
template <typename TQ, typename TG, bool CONV, bool PW>
__global__ __launch_bounds__(kThreads, 4) void chunk_prep_kernel(
    const TQ *__restrict__ q, const TQ *__restrict__ k, const TG *__restrict__ g,
    const TG *__restrict__ beta, uint4 *__restrict__ Tws, int Tall, int Hk, int Hv, int nchunks, int c0,
    ConvIn cv, Seqs sq) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  _Float16 *sK = reinterpret_cast<_Float16 *>(smem + P_OFF_K);
  _Float16 *sT = reinterpret_cast<_Float16 *>(smem + P_OFF_T);
  _Float16 *sAo = reinterpret_cast<_Float16 *>(smem + P_OFF_AO);
  float *sAd = reinterpret_cast<float *>(smem + P_OFF_AD);
  _Float16 *sQ = reinterpret_cast<_Float16 *>(smem + P_OFF_Q);
  _Float16 *sPh = reinterpret_cast<_Float16 *>(smem + P_OFF_PH);   // PW: P, high part
  _Float16 *sPl = reinterpret_cast<_Float16 *>(smem + P_OFF_PL);   // ... and low part
  float *sGB = reinterpret_cast<float *>(smem + (PW ? P_OFF_GB_P : P_OFF_GB));   // [2][grp][C]: gate, beta per head
  float *sc = sGB + 2 * (Hv / Hk) * C;
  const float *sGam = sc;
  const float *sB = sc + 2 * C;
  float4 *sTap = reinterpret_cast<float4 *>(sc);   // CONV: taps of k, then q (before the head loop)

  // block -> (chunk c of sequence b, key head kh); packed sequences: blockIdx.x
  // is a chunk slot (nchunks = the slot count)
  const int kh = blockIdx.y % Hk;
  int c, b, start, T;
  if (sq.cu) {
    b = seq_of_slot<C>(sq, Tall, blockIdx.x, c, start, T);
    if (b < 0) return;
  } else {
    c = c0 + blockIdx.x;
    b = blockIdx.y / Hk;
    seq_bounds(sq, b, Tall, start, T);
  }
  const int grp = Hv / Hk;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g4 = l >> 4, ln = l & 15;
  const int t0 = c * C, n = min(C, T - t0);
  const size_t bt0 = (size_t)start + t0;

  // CONV: this lane's rows of K and Q in the qkv type, stored to cv.k, cv.q
  // once the loads have all landed
  uint4 ky[CONV ? 4 : 1], qy[CONV ? 4 : 1];
  const int rb = tid >> 4, ch = (tid & 15) * 8;
  // The K tile (fp16), rows past the end zero; all loads are in flight
  // before the first is converted.  CONV: lane group rb = tid / 16 makes rows
  // 4 rb .. 4 rb + 3 of K and Q from the raw rows 4 rb - 3 .. 4 rb + 3 (zero
  // before the sequence start) at the lane's 8 channels.
  {
    constexpr int NL = CONV ? 7 : 4;
    uint4 uk[NL], uq[(CONV || PW) ? NL : 1];
    if constexpr (CONV) {
#pragma unroll
      for (int j = 0; j < 7; ++j) {
        const int tt = min(max(t0 + 4 * rb - 3 + j, 0), T - 1);
        const size_t off = (((size_t)start + tt) * Hk + kh) * DK + ch;
        uk[j] = *reinterpret_cast<const uint4 *>(cv.xk + off);
        uq[j] = *reinterpret_cast<const uint4 *>(cv.xq + off);
      }
      // the taps of k (threads 0..127) and q (128..255), one channel each
      sTap[tid] = *reinterpret_cast<const float4 *>((tid < DK ? cv.wk : cv.wq) + ((size_t)kh * DK + (tid & (DK - 1))) * 4);
    } else {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int row = (tid >> 4) + 16 * it;
        const size_t off = ((bt0 + min(row, n - 1)) * Hk + kh) * DK + ch;
        uk[it] = *reinterpret_cast<const uint4 *>(k + off);
        if constexpr (PW) uq[it] = *reinterpret_cast<const uint4 *>(q + off);
      }
    }
    // gate and beta of every value head of the group, [head][token] in LDS
    // past the fixed layout, all requested before anything is stored: one
    // counter tracks loads and stores, so waiting for a load issued after a
    // store would also wait for that store.
    {
      TG graw[2], braw[2];
      for (int e0 = 0; e0 < grp * C; e0 += 2 * kThreads) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int e = min(e0 + u * kThreads + tid, grp * C - 1);
          const int tok = min(e / grp, n - 1), hh = kh * grp + e % grp;
          graw[u] = g[(bt0 + tok) * Hv + hh];
          braw[u] = beta[(bt0 + tok) * Hv + hh];
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int e = e0 + u * kThreads + tid;
          if (e < grp * C) {
            const int tok = e / grp, hv = e % grp;
            sGB[hv * C + tok] = tok < n ? to_f32(graw[u]) : 0.f;
            sGB[(grp + hv) * C + tok] = tok < n ? to_f32(braw[u]) : 0.f;
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    const half8 hz = {};
    if constexpr (CONV) {
      lds_barrier();   // the taps are in LDS
      // the prologue's arithmetic, rounded to the qkv type as it stores it
      auto conv_rows = [&](const uint4 (&x)[7], const float4 *taps, _Float16 *sX, uint4 (&y)[4]) {
        float w[4][8];
#pragma unroll
        for (int c8 = 0; c8 < 8; ++c8) {
          const float4 t4 = taps[ch + c8];
          w[0][c8] = t4.x; w[1][c8] = t4.y; w[2][c8] = t4.z; w[3][c8] = t4.w;
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int row = 4 * rb + it;
          float x3[8], x2[8], x1[8], x0[8], z[8];
          unpack8(x[it], t0 + row - 3 < 0, x3);
          unpack8(x[it + 1], t0 + row - 2 < 0, x2);
          unpack8(x[it + 2], t0 + row - 1 < 0, x1);
          unpack8(x[it + 3], false, x0);
          const float ss = conv_silu8(w[0], w[1], w[2], w[3], x3, x2, x1, x0, z);
          l2_scale8<16>(z, ss, cv.eps);
          y[it] = pack8(z, TQ{});
          *reinterpret_cast<half8 *>(sX + row * KST + ch) = row < n ? to_half8(y[it], TQ{}) : hz;
        }
      };
      conv_rows(uk, sTap, sK, ky);
      // q's rows go to LDS too (without PW nothing reads them there, but
      // without these stores the compiler's schedule of this kernel spills
      // registers)
      conv_rows(uq, sTap + DK, sQ, qy);
    } else {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int row = (tid >> 4) + 16 * it;
        *reinterpret_cast<half8 *>(sK + row * KST + ch) = row < n ? to_half8(uk[it], TQ{}) : hz;
        if constexpr (PW)
          *reinterpret_cast<half8 *>(sQ + row * KST + ch) = row < n ? to_half8(uq[it], TQ{}) : hz;
      }
    }
  }
  lds_barrier();

  // G row w (tiles (w, w - d))
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
  // PW: P0 row w (tiles (w, w - d)) = Q rows 16 w .. times K rows 16 (w - d) ..
  float4v accP[PW ? 4 : 1];
  if constexpr (PW) {
    const _Float16 *qw = sQ + (16 * w + ln) * KST + 8 * g4;
    const _Float16 *kw = sK + (16 * w + ln) * KST + 8 * g4;
    half8 aq[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) aq[kk] = *reinterpret_cast<const half8 *>(qw + 32 * kk);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float4v ap = {0.f, 0.f, 0.f, 0.f};
      if (d <= w) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          ap = mfma32(aq[kk], *reinterpret_cast<const half8 *>(kw - 16 * d * KST + 32 * kk), ap);
      }
      accP[d] = ap;
    }
  }
  // All loads so far have landed (nothing is stored yet): said explicitly so
  // that the head loop does not wait on them again behind its own stores.
  // (gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15.)
  __builtin_amdgcn_s_waitcnt(0x0F70);
  if constexpr (CONV) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = 4 * rb + it;
      if (row < n) {
        const size_t off = ((bt0 + row) * Hk + kh) * DK + ch;
        *reinterpret_cast<uint4 *>(reinterpret_cast<TQ *>(cv.k) + off) = ky[it];
        *reinterpret_cast<uint4 *>(reinterpret_cast<TQ *>(cv.q) + off) = qy[it];
      }
    }
  }
  for (int hv = 0; hv < grp; ++hv) {
    const int h = kh * grp + hv;
    lds_barrier();  // K, or the previous head's T, has been read out
    if (tid < C) chunk_scalars(sGB[hv * C + tid], sGB[(grp + hv) * C + tid], sc, tid);
    lds_barrier();
    uint4 *wch = Tws + (ws_chain(sq, b, h, Hv, nchunks, start) + c) * (PW ? GDN_CHUNK_U4_P : GDN_CHUNK_U4);
    if (tid < 5 * C / 4) wch[(PW ? GDN_SC_P : GDN_SC) + tid] = reinterpret_cast<const uint4 *>(sc)[tid];
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
      const int rr = tid >> 4, cc = tid & 15;
      sT[rr * CST + 16 + cc] = (_Float16)0.f;
      sT[(32 + rr) * CST + 48 + cc] = (_Float16)0.f;
      if constexpr (PW) {
        // P = P0 e^{gamma_r - gamma_s} (s <= r), high and low parts
        _Float16 *ph = sPh + r0 * CST + 16 * w + ln, *pl = sPl + r0 * CST + 16 * w + ln;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          if (d <= w) {
            const float gs = sGam[16 * (w - d) + ln];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
              const bool keep = d > 0 || ln <= 4 * g4 + ii;
              _Float16 hi, lo;
              split16(keep ? __expf(gr[ii] - gs) * accP[d][ii] : 0.f, hi, lo);
              ph[ii * CST - 16 * d] = hi;
              pl[ii * CST - 16 * d] = lo;
            }
          }
        }
        sPh[rr * CST + 16 + cc] = (_Float16)0.f;
        sPh[(32 + rr) * CST + 48 + cc] = (_Float16)0.f;
        sPl[rr * CST + 16 + cc] = (_Float16)0.f;
        sPl[(32 + rr) * CST + 48 + cc] = (_Float16)0.f;
      }
    }
    invert_store<PW ? 2 : 0>(sAd, sAo, sT, sPh, sPl, wch, w, l);
  }
}

// ============================================================================
// chunk_seq: the sequential pass over the chunks of one sequence
// ============================================================================
// NW compute waves hold the state, 16 RT value rows each; four more waves
// load the next chunks and write them to LDS, so the compute waves issue no
// loads at all (their only memory traffic is LDS reads and the output
// stores, and a wait for a load never waits for stores).
//
// Two barriers per chunk c.  Before the first (B1) the compute waves read the
// chunk's V and form its P (the decayed masked Q K^T) from the K and Q
// fragments they read for K S^T and S Q^T; after B1 they read P for the
// output product while the loading waves write V of chunk c + 1 (complete at
// the second barrier, B2), so V and P need one LDS buffer each.  K, Q, T and
// the per-token scalars of chunk c + 1 are written during chunk c into the
// other of two buffers and are complete at B2.
//
// Precision: X, N (as the operand of the output product) and P are each
// split into an fp16 high part and an fp16 low part (x = hi + lo with
// |lo| <= 2^-11 |x|), and their products take the three terms
// hi*hi + lo*hi + hi*lo; with the prologue inside, v stays fp32 (V^T in LDS)
// up to X.  An fp16 operand alone rounds each of these to 11 bits, which on
// the conv-prefill workload costs up to 2e-2 of
// rms(o) over a whole output tensor; the splits bring that below 1e-2.
template <int NW, int RT, bool KDA, bool VLO>
struct SeqCfg {
  static constexpr int LW = 4;                 // loading waves
  static constexpr int CT = 64 * NW;           // compute threads
  static constexpr int THREADS = 64 * (NW + LW);
  static constexpr int LT = 64 * LW;           // loading threads
  static constexpr int WGC = 16 * NW * RT;     // value rows per workgroup
  static constexpr int NS = DV / WGC;          // workgroups per (batch, value head)
  static constexpr int VST = WGC + 8;          // sV row stride
  static constexpr int NKQ = (C * DK / 8) / LT;     // 16-byte K (and Q) pieces per loading thread
  static constexpr int NV = (C * WGC / 8) / LT;     // 16-byte V pieces per loading thread
  // head gate with two compute waves: P (high and low) comes from the workspace
  static constexpr bool PWS = !KDA && NW == 2;
  // fragments from the workspace: T (key gate: T, P; PWS: T, P high, P low)
  static constexpr int NFR = KDA ? 2 * NFRAG : PWS ? 3 * NFRAG : NFRAG;
  static constexpr int NTP = (NFR * 64 + LT - 1) / LT;  // their pieces per loading thread
  static constexpr int NSC = KDA ? C + DK : 5 * C;       // fp32 scalars per chunk
  static constexpr int SC_U4 = KDA ? KDA_SC : PWS ? GDN_SC_P : GDN_SC;   // their offset in the chunk's workspace
  static constexpr int CHUNK_U4 = KDA ? KDA_CHUNK_U4 : PWS ? GDN_CHUNK_U4_P : GDN_CHUNK_U4;   // workspace per chunk
  static constexpr int TPS_U4 = NFR * 64 + NSC / 4;        // fragments, then the scalars (16 B units)
  static constexpr int OFF_K = 0;                          // 2 x [C][KST] fp16
  static constexpr int OFF_Q = OFF_K + 2 * C * KST * 2;    // 2 x [C][KST] fp16
  static constexpr int OFF_KD = OFF_Q + 2 * C * KST * 2;   // 2 x [C][KST] fp16 (key gate)
  // V (one buffer): [C][VST] fp16; VLO: fp32 and transposed, [WGC][VTS]
  static constexpr int VTS = C + 4;
  static constexpr int OFF_V = OFF_KD + (KDA ? 2 * C * KST * 2 : 0);
  static constexpr int OFF_TP = OFF_V + (VLO ? WGC * VTS * 4 : C * VST * 2);   // 2 x [TPS_U4] x 16 B
  static constexpr int OFF_P = OFF_TP + 2 * TPS_U4 * 16;   // head gate: P high, then low fragments
  static constexpr int OFF_W = OFF_P + (KDA || PWS ? 0 : 2 * NFRAG * 1024);   // VLO: v taps, [WGC][4] fp32
  static constexpr int SMEM = OFF_W + (VLO ? WGC * 16 : 0);
  // with the output gate: the row sums of squares of two chunks, [2][C][NW] fp32
  static constexpr int OFF_SS = SMEM;
  static constexpr int SMEM_GATE = OFF_SS + 2 * C * NW * 4;
  static_assert(SMEM_GATE <= 160 * 1024, "LDS");
  static_assert((C * DK / 8) % LT == 0 && (C * WGC / 8) % LT == 0, "loads per thread");
  static_assert(LT >= NSC / 4, "one scalar piece per loading thread");
  static_assert(NSC % 4 == 0 && (C * (KST / 8)) % 64 == 0, "16-byte pieces");
};

// Wave load g of a chunk's K and Q tiles straight into LDS (g < NK: K, then
// Q): 64 pieces of 16 bytes, KP to a tile row of KST halves (the last piece
// of a row is padding, which repeats the row's first).  Rows past n repeat
// row n - 1.  Returns this lane's source, the wave's LDS destination, the
// lane's row and its piece in the row (-1: padding).  Everything is selected
// as a value (a function of the arguments), so that no variable has to stay
// in memory for the choice.
template <typename TQ>
struct TilePiece {
  const TQ *src;
  _Float16 *dst;
  int row, pc;
};
template <int NK, int KP, typename TQ>
__device__ __forceinline__ TilePiece<TQ> tile_piece(int g, int n, size_t t0, int lane, const TQ *kb,
                                                    const TQ *qb, int rs, _Float16 *tk, _Float16 *tq) {
  const bool isK = g < NK;
  const int i = isK ? g : g - NK;
  const int e = 64 * i + lane;
  const int row = e / KP, pc = e - row * KP;
  return TilePiece<TQ>{(isK ? kb : qb) + (t0 + min(row, n - 1)) * rs + (pc < KP - 1 ? 8 * pc : 0),
                       (isK ? tk : tq) + 8 * 64 * i, row, pc < KP - 1 ? pc : -1};
}

// One 16-byte piece per lane from global memory straight into LDS (the
// gfx950 global_load_lds_dwordx4): lane i of the wave writes its piece to
// dst + 16 i, dst being the same for the whole wave.  The wave's load counter
// covers the write to LDS.
__device__ __forceinline__ void lds_load16(const void *src, void *dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
}

// A chunk's loads into registers.  Nothing is converted here, so no
// instruction needs the data before it is committed to LDS.  CONV: the raw v
// rows of the lane's NV output rows and the three before (K and Q go
// straight to LDS).
template <int NW, int RT, bool KDA, bool CONV>
struct SeqFetch {
  using Cfg = SeqCfg<NW, RT, KDA, CONV>;
  static constexpr int NKQ = CONV ? 1 : Cfg::NKQ;
  uint4 k[NKQ], q[NKQ], kd[KDA ? Cfg::NKQ : 1], v[CONV ? Cfg::NV + 3 : Cfg::NV], tp[Cfg::NTP], sc;
  int n, t0;
};

// KDA false: head gate; K, Q, V, g, beta are read from the inputs and T from
// the workspace, P is formed here.  KDA true: key-channel gate; the decayed
// K, Q, the state-update K, T, P, beta and Gamma_n come from the workspace
// (q, k, g, beta are not read) and the state decays per key channel.  CONV:
// v is computed from the raw rows cv.xv as it is loaded (convolution and
// SiLU, kept to fp32 as high and low fp16 parts) and K, Q (fp16, after the
// prologue) go from global memory straight to LDS; v is not read.  GATE (a
// whole value head per workgroup): the gated output norm is applied to the
// chunk's outputs and y is written instead of o (which is not used).  ND:
// the update without the delta correction: N = beta V (no K S^T term, the
// workspace's T is not read).
template <typename TQ, typename TG, int NW, int RT, bool KDA, bool CONV, bool GATE, bool ND>
__global__ __launch_bounds__(64 * (NW + 4), 1) void chunk_seq_kernel(
    const TQ *__restrict__ q, const TQ *__restrict__ k, const TQ *__restrict__ v,
    const TG *__restrict__ g, const TG *__restrict__ beta, const uint4 *__restrict__ ws,
    const float *__restrict__ S0, float *__restrict__ o, float *__restrict__ ST, int Tall, int Hk,
    int Hv, int ntasks, int nchunks, int c_begin, int c_end, ConvIn cv, GateArgs ga, Seqs sq) {
  static_assert(!CONV || (std::is_same<TQ, f16_t>::value && !KDA), "the prologue inside: fp16 q, k, head gate");
  using Cfg = SeqCfg<NW, RT, KDA, CONV>;
  constexpr int NSC = Cfg::NSC, LW = Cfg::LW;
  constexpr int LT = Cfg::LT, WGC = Cfg::WGC, NS = Cfg::NS, VST = Cfg::VST;
  constexpr int NKQ = Cfg::NKQ, NV = Cfg::NV, NTP = Cfg::NTP, NFR = Cfg::NFR;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  // Blocks go round-robin over the 8 XCDs.  Sequences of one length: each XCD
  // takes a contiguous task range.  Packed sequences: the tasks of one
  // (sequence, key head) group stay on one XCD (its value heads share K and
  // Q in that L2), group j goes to XCD j % 8 and the groups come longest
  // sequence first, so that every XCD gets an even share of the chunks and
  // the longest chains start first.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3;
  int slice, h, b;
  if (sq.cu) {
    const int G = Hv / Hk * NS;   // tasks per group
    const int j = idx / G * 8 + xcd, m = idx % G;
    if (j >= sq.B * Hk) return;   // the grid rounds the groups up to a multiple of 8
    b = sq.order ? sq.order[j / Hk] : j / Hk;
    h = j % Hk * (Hv / Hk) + m / NS;
    slice = m % NS;
  } else {
    const int per = ntasks >> 3, rem = ntasks & 7;
    const int task = xcd * per + min(xcd, rem) + idx;
    slice = task % NS;
    h = task / NS % Hv;
    b = task / NS / Hv;
  }
  const int bh = b * Hv + h;
  const int kh = h / (Hv / Hk);
  int start, T;   // the sequence's first token and length
  seq_bounds(sq, b, Tall, start, T);
  if (sq.cu) {    // packed sequences: all of the sequence's chunks
    c_begin = 0;
    c_end = (T + C - 1) / C;
  }
  if (c_begin >= c_end) {   // an empty sequence: the state passes through
    if (threadIdx.x < Cfg::CT)
      for (int e = threadIdx.x; e < WGC * DK; e += Cfg::CT) {
        const size_t at = ((size_t)bh * DV + slice * WGC + e / DK) * DK + e % DK;
        ST[at] = S0 ? S0[at] : 0.f;
      }
    return;
  }

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int l = tid & 63, g4 = l >> 4, ln = l & 15;
  const int ltid = tid - Cfg::CT;                           // index among the loading threads

  // Per-sequence bases (uniform) and per-thread load offsets (fixed for all chunks).
  const int kq_rs = Hk * DK, v_rs = Hv * DV;        // row strides of q/k and v (elements)
  const TQ *kb = k + ((size_t)start * Hk + kh) * DK;
  const TQ *qb = q + ((size_t)start * Hk + kh) * DK;
  const TQ *vb = v + ((size_t)start * Hv + h) * DV + slice * WGC;
  const uint4 *wsbh = ws + ws_chain(sq, b, h, Hv, nchunks, start) * Cfg::CHUNK_U4;

  _Float16 *const sKb = reinterpret_cast<_Float16 *>(smem + Cfg::OFF_K);
  _Float16 *const sQb = reinterpret_cast<_Float16 *>(smem + Cfg::OFF_Q);
  _Float16 *const sKdb = reinterpret_cast<_Float16 *>(smem + Cfg::OFF_KD);
  _Float16 *const sV = reinterpret_cast<_Float16 *>(smem + Cfg::OFF_V);
  float *const sVt = reinterpret_cast<float *>(smem + Cfg::OFF_V);   // CONV: V^T, fp32
  // V^T element (value row c, token t) sits at token slot t ^ 4 (c / 8 mod 16):
  // the loading waves write 4 tokens of 8 rows 8 apart per lane, which with
  // any 16-byte aligned row stride would all fall on the same banks.  The
  // swizzle keeps groups of 4 tokens together.
  auto vt_at = [&](int c, int t) __attribute__((always_inline)) {
    return sVt + c * Cfg::VTS + (t ^ (4 * ((c >> 3) & 15)));
  };
  uint4 *const sTPb = reinterpret_cast<uint4 *>(smem + Cfg::OFF_TP);   // buffer b at b TPS_U4
  uint4 *const sPh = reinterpret_cast<uint4 *>(smem + Cfg::OFF_P);     // head gate: P high fragments
  uint4 *const sPl = sPh + NFRAG * 64;                                  // ... and low
  constexpr int TPS_U4 = Cfg::TPS_U4, SC_AT = NFR * 64;   // the scalars follow the fragments

  using Fetch = SeqFetch<NW, RT, KDA, CONV>;
  // CONV: loading thread -> value channels 8 ch8 .. + 7 of the slice at the
  // chunk rows NV rb .. NV rb + NV - 1 (a row's channels on consecutive lanes)
  const int vrb = ltid / (WGC / 8), vch8 = ltid % (WGC / 8);
  const bf16_t *xvb = cv.xv + ((size_t)start * Hv + h) * DV + slice * WGC + vch8 * 8;
  // parts: K and Q (and the key gate's state-update K), V, and the T (and P)
  // fragments with the scalars
  constexpr int FKQ = 1, FV = 2, FTP = 4, FALL = 7;
  auto fetch = [&](Fetch &f, int c, int part) {
    const int n = min(C, T - c * C);
    f.n = n;
    const size_t t0 = (size_t)c * C;
    f.t0 = (int)t0;
    const uint4 *wc = wsbh + (size_t)c * Cfg::CHUNK_U4;
    if constexpr (!CONV) {
      if (part & FKQ) {
        if constexpr (KDA) {
          // rows past the end of the sequence are zero in the workspace
#pragma unroll
          for (int it = 0; it < NKQ; ++it) {
            const int e = ltid + LT * it;
            f.k[it] = wc[KDA_KG + e];
            f.q[it] = wc[KDA_QG + e];
            f.kd[it] = wc[KDA_KD + e];
          }
        } else {
          // rows past the end of the sequence (last chunk) re-read its last row
          const TQ *kc = kb + t0 * kq_rs, *qc = qb + t0 * kq_rs;
#pragma unroll
          for (int it = 0; it < NKQ; ++it) {
            const int e = ltid + LT * it;
            const int off = min(e >> 4, n - 1) * kq_rs + (e & 15) * 8;
            f.k[it] = *reinterpret_cast<const uint4 *>(kc + off);
            f.q[it] = *reinterpret_cast<const uint4 *>(qc + off);
          }
        }
      }
    }
    if (part & FV) {
      if constexpr (CONV) {
#pragma unroll
        for (int j = 0; j < NV + 3; ++j) {
          const int tt = min(max((int)t0 + NV * vrb - 3 + j, 0), T - 1);
          f.v[j] = *reinterpret_cast<const uint4 *>(xvb + (size_t)tt * v_rs);
        }
      } else {
        const TQ *vc = vb + t0 * v_rs;
#pragma unroll
        for (int it = 0; it < NV; ++it) {
          const int e = ltid + LT * it;
          f.v[it] = *reinterpret_cast<const uint4 *>(vc + min(e / (WGC / 8), n - 1) * v_rs +
                                                     (e % (WGC / 8)) * 8);
        }
      }
    }
    if (part & FTP) {
#pragma unroll
      for (int it = 0; it < NTP; ++it) f.tp[it] = wc[min(ltid + LT * it, NFR * 64 - 1)];
      f.sc = wc[Cfg::SC_U4 + min(ltid, NSC / 4 - 1)];
    }
  };
  // The fragments and scalars of f into T/P buffer `buf`.
  auto commit_tp = [&](const Fetch &f, int buf) {
#pragma unroll
    for (int it = 0; it < NTP; ++it) {
      const int e = ltid + LT * it;
      if (e < NFR * 64) sTPb[buf * TPS_U4 + e] = f.tp[it];
    }
    if (ltid < NSC / 4) sTPb[buf * TPS_U4 + SC_AT + ltid] = f.sc;
  };
  // K and Q (and the state-update K) of f into buffer `buf` (register path)
  auto commit_kq = [&](const Fetch &f, int buf) {
    if constexpr (!CONV) {
      _Float16 *k_ = sKb + buf * C * KST, *q_ = sQb + buf * C * KST;
      // K and Q (and the state-update K) are fp16 in the workspace of the key gate
      using TK = typename std::conditional<KDA, f16_t, TQ>::type;
      const half8 hz = {};
#pragma unroll
      for (int it = 0; it < NKQ; ++it) {
        const int e = ltid + LT * it;
        // last chunk of a ragged sequence: rows past its end are zero
        const bool ok = KDA || (e >> 4) < f.n;
        const int off = (e >> 4) * KST + (e & 15) * 8;
        *reinterpret_cast<half8 *>(k_ + off) = ok ? to_half8(f.k[it], TK{}) : hz;
        *reinterpret_cast<half8 *>(q_ + off) = ok ? to_half8(f.q[it], TK{}) : hz;
        if constexpr (KDA) *reinterpret_cast<half8 *>(sKdb + buf * C * KST + off) = to_half8(f.kd[it], f16_t{});
      }
    }
  };
  // V of f into the V buffer (register path; rows past the sequence end zero)
  auto commit_v = [&](const Fetch &f) {
    if constexpr (!CONV) {
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        const int e = ltid + LT * it;
        const int row = e / (WGC / 8);
        *reinterpret_cast<half8 *>(sV + row * VST + (e % (WGC / 8)) * 8) =
            row < f.n ? to_half8(f.v[it], TQ{}) : half8{};
      }
    }
  };

  // The chunk's P = L o Q K^T (head gate), formed by the compute waves before
  // B1 from the K and Q fragments they read for K S^T and S Q^T: block (R, S),
  // S <= R, is computed as P^T = K_S Q_R^T, so that lane (g4, ln) holds
  // P[16 R + ln][16 S + 4 g4 + ii]: four consecutive elements of its own slot
  // in the fragment (R, S / 2) that the output product reads.  p_store scales
  // them by the decays, writes their high and low parts, and zeroes the upper
  // halves of the diagonal fragments (blocks (0, 1) and (2, 3)).
  auto p_store = [&](int R, int S, float4v acc, const float *sc) __attribute__((always_inline)) {
    const float gr = sc[16 * R + ln];
    const float4 gs = *reinterpret_cast<const float4 *>(sc + 16 * S + 4 * g4);
    const float gsv[4] = {gs.x, gs.y, gs.z, gs.w};
    half4 ph, pl;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const bool keep = S < R || 4 * g4 + ii <= ln;
      _Float16 hi, lo;
      split16(keep ? __expf(gr - gsv[ii]) * acc[ii] : 0.f, hi, lo);
      ph[ii] = hi;
      pl[ii] = lo;
    }
    const int at = frag_index(R, S >> 1) * 64 + l;
    half4 *dh = reinterpret_cast<half4 *>(sPh + at) + (S & 1);
    half4 *dl = reinterpret_cast<half4 *>(sPl + at) + (S & 1);
    *dh = ph;
    *dl = pl;
    if (S == R && !(R & 1)) {   // the block right of the diagonal in the same fragment
      dh[1] = half4{};
      dl[1] = half4{};
    }
  };
  if (w >= NW) {
    if constexpr (CONV) {
      // Loading waves, the prologue inside: K and Q (fp16, made by the prep
      // kernel) of chunk c + 1 go from global memory straight into the other
      // LDS buffer while chunk c is computed; the raw v rows with the T
      // fragments and the scalars of chunk c + 1, fetched into registers one
      // chunk earlier (fa, fb alternate), are convolved before B1 and
      // written after it.  Each wave waits for its own loads before B2.
      const int lw = w - NW;
      // NK wave loads a tile; wave lw issues loads lw, lw + LW, .., NPER of
      // them, the last ones repeating one of its own (so every wave issues the
      // same number and its waits have a fixed count).  Rows past n repeat
      // row n - 1 (in bounds) and are zeroed once they have landed, each wave
      // over the pieces it loaded itself.
      constexpr int KP = KST / 8, NK = C * KP / 64, NTOT = 2 * NK, NPER = (NTOT + LW - 1) / LW;
      static_assert(NTOT >= LW, "loads per wave");
      // the taps of the lane's 8 channels, read back from LDS by every
      // convolution: each lane writes the taps it reads (lanes sharing
      // channels write the same values), so no other wave is waited for
      float4 *const sW = reinterpret_cast<float4 *>(smem + Cfg::OFF_W);
#pragma unroll
      for (int c8 = 0; c8 < 8; ++c8)
        sW[vch8 * 8 + c8] =
            *reinterpret_cast<const float4 *>(cv.wv + ((size_t)h * DV + slice * WGC + vch8 * 8 + c8) * 4);
      auto piece = [&](int j, int n, size_t t0, int buf) __attribute__((always_inline)) {
        int gi = lw + LW * j;
        if (gi >= NTOT) gi -= LW;
        return tile_piece<NK, KP>(gi, n, t0, l, kb, qb, kq_rs, sKb + buf * C * KST, sQb + buf * C * KST);
      };
      auto issue_kq = [&](int c, int buf) __attribute__((always_inline)) {
        const int n = min(C, T - c * C);
#pragma unroll
        for (int j = 0; j < NPER; ++j) {
          const auto pt = piece(j, n, (size_t)c * C, buf);
          lds_load16(pt.src, pt.dst);
        }
      };
      // after the wave's loads have landed: zero the rows past a ragged end
      auto zero_tail = [&](int c, int buf) __attribute__((always_inline)) {
        const int n = min(C, T - c * C);
        if (n < C) {
          for (int j = 0; j < NPER; ++j) {
            const auto pt = piece(j, n, (size_t)c * C, buf);
            if (pt.row >= n && pt.pc >= 0) *reinterpret_cast<half8 *>(pt.dst + 8 * l) = half8{};
          }
        }
      };
      // v of the lane's rows from the raw rows of f, with the prologue's
      // arithmetic, into z (fp32; rows past the end zero)
      auto conv_v = [&](const Fetch &f, float (&z)[NV][8]) __attribute__((always_inline)) {
        float wv[4][8];
#pragma unroll
        for (int c8 = 0; c8 < 8; ++c8) {
          const float4 t4 = sW[vch8 * 8 + c8];
          wv[0][c8] = t4.x; wv[1][c8] = t4.y; wv[2][c8] = t4.z; wv[3][c8] = t4.w;
        }
        float x[NV + 3][8];
#pragma unroll
        for (int j = 0; j < NV + 3; ++j) unpack8(f.v[j], j < 3 && f.t0 + NV * vrb - 3 + j < 0, x[j]);
#pragma unroll
        for (int it = 0; it < NV; ++it) {
          const int row = NV * vrb + it;
          (void)conv_silu8(wv[0], wv[1], wv[2], wv[3], x[it], x[it + 1], x[it + 2], x[it + 3], z[it]);
#pragma unroll
          for (int e = 0; e < 8; ++e) z[it][e] = row < f.n ? z[it][e] : 0.f;
        }
      };
      // z into the V buffer, transposed: channel-major, the lane's NV
      // consecutive rows of a channel in one write.  The writes are written
      // out as instructions: the compiler would otherwise make them wait for
      // the K, Q loads into LDS issued before them (it cannot tell that they
      // touch other LDS), which take until the end of the chunk; the loads'
      // own wait comes before the next barrier, and the writes are complete
      // at the barrier (its wait for this wave's LDS operations).
      auto write_v = [&](const float (&z)[NV][8]) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // the LDS address (offset in the workgroup's LDS) of the write
          const uint32_t dst = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float *)(
              vt_at(vch8 * 8 + e, NV * vrb));
          if constexpr (NV == 4) {
            const float4v x = {z[0][e], z[1][e], z[2][e], z[3][e]};
            asm volatile("ds_write_b128 %0, %1" ::"v"(dst), "v"(x));
          }
          if constexpr (NV == 2) {
            const float2 x = make_float2(z[0][e], z[1][e]);
            asm volatile("ds_write_b64 %0, %1" ::"v"(dst), "v"(x));
          }
          if constexpr (NV == 1) asm volatile("ds_write_b32 %0, %1" ::"v"(dst), "v"(z[0][e]));
        }
      };
      Fetch fa, fb;
      // chunk c_begin: everything in LDS before the first barrier
      fetch(fa, c_begin, FV | FTP);
      issue_kq(c_begin, 0);
      fetch(fb, min(c_begin + 1, c_end - 1), FV | FTP);
      commit_tp(fa, 0);
      {
        float z[NV][8];
        conv_v(fa, z);
        write_v(z);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt 0: this wave's K and Q pieces are in LDS
      zero_tail(c_begin, 0);
      lds_barrier();
      // chunk c: fb holds chunk c + 1's registers, fa takes chunk c + 2's
      auto lstep = [&](int c, Fetch &fn, Fetch &fc) __attribute__((always_inline)) {
        const int buf = (c + 1 - c_begin) & 1;
        const bool more = c + 1 < c_end;
        float z[NV][8];
        // fc's registers landed during the previous chunk: they are written
        // out and convolved before new loads are issued, so that no wait for
        // them covers the new ones
        if (more) {
          commit_tp(fc, buf);
          conv_v(fc, z);
        }
        if (more) issue_kq(c + 1, buf);
        fetch(fn, min(c + 2, c_end - 1), FV | FTP);
        lds_barrier();   // B1: the compute waves have read V of chunk c
        if (more) write_v(z);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt 0
        if (more) zero_tail(c + 1, buf);
        lds_barrier();   // B2
      };
      for (int c = c_begin; c < c_end; c += 2) {
        lstep(c, fa, fb);
        if (c + 1 < c_end) lstep(c + 1, fb, fa);
      }
    } else {
      // Loading waves, register path: chunk c + 2 is loaded while chunk c is
      // computed, and chunk c + 1, loaded one chunk earlier, is written to
      // the other LDS buffer (K, Q, T, scalars before B1, V after it).  These
      // waves issue no stores, so each wait for a chunk's loads is exact.
      Fetch fa, fb;
      fetch(fa, c_begin, FALL);
      commit_kq(fa, 0);
      commit_tp(fa, 0);
      commit_v(fa);
      fetch(fb, min(c_begin + 1, c_end - 1), FALL);
      lds_barrier();
      auto lstep = [&](int c, Fetch &fn, Fetch &fc) __attribute__((always_inline)) {
        const int buf = (c + 1 - c_begin) & 1;
        const bool more = c + 1 < c_end;
        // fc's registers landed during the previous chunk: write them out
        // before new loads are issued, so that no wait covers the new ones
        if (more) {
          commit_kq(fc, buf);
          commit_tp(fc, buf);
        }
        fetch(fn, min(c + 2, c_end - 1), FALL);
        lds_barrier();   // B1: the compute waves have read V of chunk c
        if (more) commit_v(fc);
        lds_barrier();   // B2
      };
      for (int c = c_begin; c < c_end; c += 2) {
        lstep(c, fa, fb);
        if (c + 1 < c_end) lstep(c + 1, fb, fa);
      }
    }
    return;
  }

  const int ic = w * 16 * RT;             // this wave's first value row within the workgroup
  const int iw0 = slice * WGC + ic;       // ... within the head
  float *ob = GATE ? nullptr : o + ((size_t)start * Hv + h) * DV + iw0 + 4 * g4;

  // state: row tile t (value rows iw0 + 16 t ..), tiles J of S^T; the lane
  // holds S[iw0 + 16 t + ln][16 J + 4 g4 + ii]
  float4v accS[RT][8];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int J = 0; J < 8; ++J) {
      float4v s = {0.f, 0.f, 0.f, 0.f};
      if (S0) {
        const float4 t4 = *reinterpret_cast<const float4 *>(
            S0 + ((size_t)bh * DV + iw0 + 16 * t + ln) * DK + 16 * J + 4 * g4);
        s[0] = t4.x; s[1] = t4.y; s[2] = t4.z; s[3] = t4.w;
      }
      accS[t][J] = s;
    }

  // The gated output norm: the row sums of squares of a chunk's outputs are
  // combined over the compute waves through LDS (written before the chunk's
  // last barrier, read after it), so the outputs of chunk c are normalised
  // and stored just after that barrier.  The lane's gain values are loaded
  // with the entering state and its z values at the start of each chunk
  // (rows past the end of the sequence re-read the last one).
  static_assert(!GATE || (NS == 1 && RT == 2 && NW == 4 && !KDA), "the gate needs a whole value head");
  float gw[RT][4];
  const bf16_t *zb = nullptr;
  // z and y move as 16 bytes per lane: lanes of lane groups g4 and g4 ^ 1
  // hold the 8 rows 8 (g4 >> 1) .. + 7 of a tile for one token each (row
  // block 2 p + (g4 & 1)), exchanged with __shfl_xor(., 16)
  const bool godd = g4 & 1;
  const size_t yoff = ((size_t)start * Hv + h) * DV + iw0 + 8 * (g4 >> 1);
  if constexpr (GATE) {
#pragma unroll
    for (int t = 0; t < RT; ++t) load4(ga.gain + iw0 + 16 * t + 4 * g4, gw[t]);
    zb = (const bf16_t *)ga.z + yoff;
  }
  uint4 zl[RT][2];   // z of a chunk as loaded: [tile][row block pair]
  uint2 yp[RT][4];   // y of a chunk, 16-bit, this lane's 4 rows per (tile, row block)

  // The arithmetic of chunk c before B1 (buffer (c - c_begin) & 1): K S^T and
  // S Q^T, X, N and the state update; accO gets S Q^T, and nh, nl the high
  // and low parts of N for the output product after B1.
  float4v accO[RT][4];
  half8 nh[RT][2], nl[RT][2];
  auto compute_a = [&](int c, auto &&mid) {
    const int buf = (c - c_begin) & 1;
    const _Float16 *cK = sKb + buf * C * KST, *cQ = sQb + buf * C * KST;
    const uint4 *cT = sTPb + buf * TPS_U4;
    const float *sc = reinterpret_cast<const float *>(cT + SC_AT);
    // transpose-read bases: lane (g4, i) reads row 4 g4 + i / 4, columns 4 (i % 4) .. + 3
    const _Float16 *kT = cK + (4 * g4 + (ln >> 2)) * KST + 4 * (ln & 3);
    const int vto = (4 * g4 + (ln >> 2)) * VST + ic + 4 * (ln & 3);
    // the K whose columns update the state: K itself, or K o e^{gamma_n - gamma} for the key gate
    const _Float16 *uT = KDA ? sKdb + buf * C * KST + (4 * g4 + (ln >> 2)) * KST + 4 * (ln & 3) : kT;

    half8 kk0[4], kk1[4];   // kept K fragments: of row w (and, with two waves, of row w + 2)
    if constexpr (GATE) {
      const int R0 = w == 0 ? 1 : w == 1 ? 2 : 3;   // the rows of the off-diagonal blocks (R0.., S = w)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kk0[kk] = perm_row(cK, KST, 16 * w + ln, kk, g4);
#pragma unroll
      for (int R = 1; R < 4; ++R) {
        if (w < 3 && R >= R0) {
          float4v a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) a = mfma32(kk0[kk], perm_row(cQ, KST, 16 * R + ln, kk, g4), a);
          p_store(R, w, a, sc);
        }
      }
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        const bool diag = (w == 1 && R == 0) || (w == 2 && R == 1) || (w == 3 && R >= 2);
        if (diag) {
          float4v a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            a = mfma32(perm_row(cK, KST, 16 * R + ln, kk, g4), perm_row(cQ, KST, 16 * R + ln, kk, g4), a);
          p_store(R, R, a, sc);
        }
      }
    }

    // S fragments (fp16) in kset order over the key channels
    half8 sf[RT][4];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) sf[t][kk] = pack_pair(accS[t][2 * kk], accS[t][2 * kk + 1]);

    // K S^T (rows r = 16 R + 4 g4 + ii, value row ln) and S Q^T (transposed read);
    // each K and Q fragment serves every row tile of the wave.  With them,
    // the wave's blocks of P (head gate): the block (R, R) from this row's
    // fragments, and (R, S) for S < R from the K fragments of row S that the
    // wave kept.  Blocks per wave (as if there were four compute waves;
    // with two, wave w also takes wave w + 2's): wave 0 keeps K_0 for (1,0)
    // (2,0) (3,0); wave 1 keeps K_1 for (2,1) (3,1) and makes (0,0); wave 2
    // keeps K_2 for (3,2) and makes (1,1); wave 3 makes (2,2) (3,3).  (With
    // the output gate, whose registers leave no room for the kept fragments,
    // the wave forms the same blocks first, from fragments it reads for them.)
    float4v accX[RT][4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      half8 kf[4], qf[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        kf[kk] = perm_row(cK, KST, 16 * R + ln, kk, g4);
        qf[kk] = perm_row(cQ, KST, 16 * R + ln, kk, g4);
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        float4v ax = {0.f, 0.f, 0.f, 0.f}, ao = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          if constexpr (!ND) ax = mfma32(kf[kk], sf[t][kk], ax);
          ao = mfma32(sf[t][kk], qf[kk], ao);
        }
        accX[t][R] = ax;
        accO[t][R] = ao;
      }
      if constexpr (!KDA && !GATE && !Cfg::PWS) {
        // virtual wave vw in [0, 4): this wave's own w, and w + 2 with two waves
#pragma unroll
        for (int vw = 0; vw < 4; ++vw) {
          if (vw % NW != w) continue;
          half8 (&kp)[4] = vw < NW ? kk0 : kk1;
          if (vw < 3 && R == vw) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) kp[kk] = kf[kk];
          }
          if (vw < 3 && R > vw) {
            float4v a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) a = mfma32(kp[kk], qf[kk], a);
            p_store(R, vw, a, sc);
          }
          const bool diag = (vw == 1 && R == 0) || (vw == 2 && R == 1) || (vw == 3 && R >= 2);
          if (diag) {
            float4v a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) a = mfma32(kf[kk], qf[kk], a);
            p_store(R, R, a, sc);
          }
        }
      }
    }

    if constexpr (RT == 1 && !ND && (KDA || Cfg::PWS)) {
      // the K and Q fragments of row block R + 1 are read while the eight
      // products of block R run
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    mid();

    // X = beta V - beta Gamma (K S^T) as fp32 (V rows 16 R + 4 g4 .. + 3 at
    // this lane's value column, by transpose reads of the high and low
    // parts), then its high and low fp16 parts, as fragments over the chunk
    // rows.  Without the delta correction this is N itself.
    half8 xh[RT][2], xl[RT][2];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      const int r0 = 16 * R + 4 * g4;
      // beta and beta Gamma (key gate: Gamma is inside the decayed K)
      const float4 bb = *reinterpret_cast<const float4 *>(sc + (KDA ? 0 : 2 * C) + r0);
      const float4 bg = KDA ? bb : *reinterpret_cast<const float4 *>(sc + 3 * C + r0);
      const float bv[4] = {bb.x, bb.y, bb.z, bb.w}, gv[4] = {bg.x, bg.y, bg.z, bg.w};
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        float vx4[4];
        if constexpr (CONV) {
          const float4 vv = *reinterpret_cast<const float4 *>(vt_at(ic + 16 * t + ln, r0));
          vx4[0] = vv.x; vx4[1] = vv.y; vx4[2] = vv.z; vx4[3] = vv.w;
        } else {
          const half4 vv = lds_read_tr(sV + vto + 16 * t + 16 * R * VST);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) vx4[ii] = (float)vv[ii];
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float vx = vx4[ii];
          const float x = ND ? bv[ii] * vx : bv[ii] * vx - gv[ii] * accX[t][R][ii];
          _Float16 hi, lo;
          split16(x, hi, lo);
          xh[t][R >> 1][(R & 1) * 4 + ii] = hi;
          xl[t][R >> 1][(R & 1) * 4 + ii] = lo;
        }
      }
    }

    // N = T X (from both parts of X), its high and low parts for the output
    // product and N~ = diag(e^{gamma_n - gamma}) N for the state update
    half8 ndf[RT][2];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      const half8 t0f = ND ? half8{} : __builtin_bit_cast(half8, cT[frag_index(R, 0) * 64 + l]);
      const half8 t1f = (ND || R < 2) ? half8{} : __builtin_bit_cast(half8, cT[frag_index(R, 1) * 64 + l]);
      const float4 dd = KDA ? make_float4(1.f, 1.f, 1.f, 1.f)
                            : *reinterpret_cast<const float4 *>(sc + 4 * C + 16 * R + 4 * g4);
      const float dv4[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        float4v acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (ND) {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            acc[ii] = (float)xh[t][R >> 1][(R & 1) * 4 + ii] + (float)xl[t][R >> 1][(R & 1) * 4 + ii];
        } else {
          acc = mfma32(t0f, xh[t][0], acc);
          acc = mfma32(t0f, xl[t][0], acc);
          if (R >= 2) {
            acc = mfma32(t1f, xh[t][1], acc);
            acc = mfma32(t1f, xl[t][1], acc);
          }
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          _Float16 hi, lo;
          split16(acc[ii], hi, lo);
          nh[t][R >> 1][(R & 1) * 4 + ii] = hi;
          nl[t][R >> 1][(R & 1) * 4 + ii] = lo;
          ndf[t][R >> 1][(R & 1) * 4 + ii] = (_Float16)(acc[ii] * dv4[ii]);
        }
      }
    }

    // S^T <- Gamma_n S^T + K^T N~  (K columns 16 J + ln at the chunk rows kset)
    {
      const float gC = KDA ? 1.f : sc[C + C - 1];
#pragma unroll
      for (int J = 0; J < 8; ++J) {
        half8 kc[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const half4 lo = lds_read_tr(uT + 32 * kk * KST + 16 * J);
          const half4 hi = lds_read_tr(uT + (32 * kk + 16) * KST + 16 * J);
          kc[kk] = half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        float sj[4];
        if constexpr (KDA) {
          // per key channel 16 J + 4 g4 + ii
          const float4 gn = *reinterpret_cast<const float4 *>(sc + C + 16 * J + 4 * g4);
          sj[0] = gn.x; sj[1] = gn.y; sj[2] = gn.z; sj[3] = gn.w;
        } else {
          sj[0] = sj[1] = sj[2] = sj[3] = gC;
        }
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          float4v acc = accS[t][J];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) acc[ii] *= sj[ii];
          acc = mfma32(kc[0], ndf[t][0], acc);
          acc = mfma32(kc[1], ndf[t][1], acc);
          accS[t][J] = acc;
        }
      }
    }
  };

  // After B1: O^T = Gamma (S Q^T) + N^T P^T with the three terms of the high
  // and low parts (key gate: P, from the workspace, has one part).  Row
  // r = 16 R + ln of this lane.
  auto compute_b = [&](int c, auto &&emit) {
    const int buf = (c - c_begin) & 1;
    const uint4 *cT = sTPb + buf * TPS_U4;
    const float *sc = reinterpret_cast<const float *>(cT + SC_AT);
    if constexpr (RT == 1) {
      // One row tile per wave (32- and 64-row workgroups): the four row
      // blocks' accumulators take each term in turn, so that four
      // independent products are in flight where one chain of up to six
      // dependent ones was (long prefill 2.49 -> 2.35 ms); each accumulator
      // still takes its terms in the same order.  With two row tiles the
      // per-block order below keeps fewer fragments live and is faster.
      const uint4 *ph = KDA || Cfg::PWS ? cT + NFRAG * 64 : sPh;
      const uint4 *pl = Cfg::PWS ? cT + 2 * NFRAG * 64 : sPl;
      half8 p0h[4], p1h[4], p0l[4], p1l[4];
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        p0h[R] = __builtin_bit_cast(half8, ph[frag_index(R, 0) * 64 + l]);
        p1h[R] = R >= 2 ? __builtin_bit_cast(half8, ph[frag_index(R, 1) * 64 + l]) : half8{};
        p0l[R] = half8{};
        p1l[R] = half8{};
        if constexpr (!KDA) {
          p0l[R] = __builtin_bit_cast(half8, pl[frag_index(R, 0) * 64 + l]);
          if (R >= 2) p1l[R] = __builtin_bit_cast(half8, pl[frag_index(R, 1) * 64 + l]);
          const float er = sc[C + 16 * R + ln];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) accO[0][R][ii] *= er;
        }
      }
#pragma unroll
      for (int R = 0; R < 4; ++R) accO[0][R] = mfma32(nh[0][0], p0h[R], accO[0][R]);
#pragma unroll
      for (int R = 0; R < 4; ++R) accO[0][R] = mfma32(nl[0][0], p0h[R], accO[0][R]);
      if constexpr (!KDA) {
#pragma unroll
        for (int R = 0; R < 4; ++R) accO[0][R] = mfma32(nh[0][0], p0l[R], accO[0][R]);
      }
      emit(0);
      emit(1);
#pragma unroll
      for (int R = 2; R < 4; ++R) accO[0][R] = mfma32(nh[0][1], p1h[R], accO[0][R]);
#pragma unroll
      for (int R = 2; R < 4; ++R) accO[0][R] = mfma32(nl[0][1], p1h[R], accO[0][R]);
      if constexpr (!KDA) {
#pragma unroll
        for (int R = 2; R < 4; ++R) accO[0][R] = mfma32(nh[0][1], p1l[R], accO[0][R]);
      }
      emit(2);
      emit(3);
    } else {
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        const int r = 16 * R + ln;
        const float er = KDA ? 1.f : sc[C + r];
        // P: from the T/P buffer (key gate; PWS with its low part after it) or from the P buffer
        const uint4 *ph = KDA || Cfg::PWS ? cT + NFRAG * 64 : sPh;
        const uint4 *pl = Cfg::PWS ? cT + 2 * NFRAG * 64 : sPl;
        const half8 p0h = __builtin_bit_cast(half8, ph[frag_index(R, 0) * 64 + l]);
        const half8 p1h = R >= 2 ? __builtin_bit_cast(half8, ph[frag_index(R, 1) * 64 + l]) : half8{};
        half8 p0l = {}, p1l = {};
        if constexpr (!KDA) {
          p0l = __builtin_bit_cast(half8, pl[frag_index(R, 0) * 64 + l]);
          if (R >= 2) p1l = __builtin_bit_cast(half8, pl[frag_index(R, 1) * 64 + l]);
        }
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          float4v acc = accO[t][R];
          if constexpr (!KDA) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) acc[ii] *= er;
          }
          acc = mfma32(nh[t][0], p0h, acc);
          acc = mfma32(nl[t][0], p0h, acc);
          if constexpr (!KDA) acc = mfma32(nh[t][0], p0l, acc);
          if (R >= 2) {
            acc = mfma32(nh[t][1], p1h, acc);
            acc = mfma32(nl[t][1], p1h, acc);
            if constexpr (!KDA) acc = mfma32(nh[t][1], p1l, acc);
          }
          accO[t][R] = acc;
        }
        emit(R);
      }
    }
  };
  // the outputs of row block R of chunk c (issued as soon as they are made,
  // between the products of the next row blocks)
  auto store_o = [&](int c, int R) {
    const int t0 = c * C;
    const int r = 16 * R + ln;
    if (t0 + r < T)
#pragma unroll
      for (int t = 0; t < RT; ++t)
        *reinterpret_cast<float4 *>(ob + (size_t)(t0 + r) * v_rs + 16 * t) =
            make_float4(accO[t][R][0], accO[t][R][1], accO[t][R][2], accO[t][R][3]);
  };

  // the wave's partial row sums of squares of the chunk's outputs (over its
  // 32 value rows: the lane's 8 in order, then lane groups g4 ^ 1 and g4 ^ 2)
  auto gate_partials = [&](int c) {
    float *ss = reinterpret_cast<float *>(smem + Cfg::OFF_SS) + ((c - c_begin) & 1) * C * NW;
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      const float x[8] = {accO[0][R][0], accO[0][R][1], accO[0][R][2], accO[0][R][3],
                          accO[1][R][0], accO[1][R][1], accO[1][R][2], accO[1][R][3]};
      float p = gate_sumsq8(x);
      p = p + __shfl_xor(p, 16, 64);
      p = p + __shfl_xor(p, 32, 64);
      if (g4 == 0) ss[(16 * R + ln) * NW + w] = p;
    }
  };
  // after the chunk's last barrier: the row sums over the waves (in wave
  // order), then y of chunk c as 16-bit values in yp.  The z loads were
  // issued half a chunk earlier; one wait for all of them here (for the
  // compiler, a wait for a load issued after a store would also wait for
  // that store).
  auto gate_finish = [&](int c) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    // this lane's 4 rows of z per (tile, row block): keep one half of each
    // load, take the other from the partner lane
    uint2 zr[RT][4];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint4 vz = zl[t][p];
        const uint2 keep = godd ? make_uint2(vz.z, vz.w) : make_uint2(vz.x, vz.y);
        const uint2 send = godd ? make_uint2(vz.x, vz.y) : make_uint2(vz.z, vz.w);
        const uint2 recv = make_uint2(__shfl_xor(send.x, 16, 64), __shfl_xor(send.y, 16, 64));
        zr[t][2 * p] = godd ? recv : keep;
        zr[t][2 * p + 1] = godd ? keep : recv;
      }
    const float4 *ss = reinterpret_cast<const float4 *>(smem + Cfg::OFF_SS) + ((c - c_begin) & 1) * C;
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      const float4 pw = ss[16 * R + ln];
      const float inv = gate_inv_rms<DV>(((pw.x + pw.y) + pw.z) + pw.w, ga.eps);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const uint2 u = zr[t][R];
        const float zz[4] = {__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                             __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
        float yv[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) yv[ii] = gate_apply(accO[t][R][ii], inv, gw[t][ii], zz[ii]);
        yp[t][R] = ga.yt == DType::BF16 ? pack4_bf16(yv) : pack4_f16(yv);
      }
    }
  };
  // the stores of chunk c's y (issued in the middle of the next chunk's
  // arithmetic, away from the loading waves' burst of loads after the
  // barrier), then the z loads of chunk c + 1 (rows past the end of the
  // sequence re-read the last one)
  auto gate_emit = [&](int c) {
    const int t0 = c * C;
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint2 a = yp[t][2 * p], bq = yp[t][2 * p + 1];
        const uint2 send = godd ? a : bq;
        const uint2 recv = make_uint2(__shfl_xor(send.x, 16, 64), __shfl_xor(send.y, 16, 64));
        const uint4 out = godd ? make_uint4(recv.x, recv.y, bq.x, bq.y) : make_uint4(a.x, a.y, recv.x, recv.y);
        const int tok = t0 + 16 * (2 * p + godd) + ln;
        if (tok < T) *reinterpret_cast<uint4 *>((uint16_t *)ga.y + yoff + (size_t)tok * v_rs + 16 * t) = out;
      }
  };
  auto gate_load_z = [&](int c) {
    const int t0 = c * C;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const size_t tt = (size_t)min(t0 + 16 * (2 * p + godd) + ln, T - 1);
#pragma unroll
      for (int t = 0; t < RT; ++t) zl[t][p] = *reinterpret_cast<const uint4 *>(zb + tt * v_rs + 16 * t);
    }
  };

  // No loads after the entering state but the gate's z values (whose wait
  // comes a whole chunk after the previous output stores), so the output
  // stores never hold up a wait.  With the gate, the entering state and the
  // gain are waited for here: otherwise the compiler's wait for them inside
  // the loop (the loop merges the first iteration with the later ones) would
  // also wait for the previous chunk's output stores.
  if constexpr (GATE) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  lds_barrier();
  for (int c = c_begin; c < c_end; ++c) {
    compute_a(c, [&] {
      if constexpr (GATE) {
        __builtin_amdgcn_sched_barrier(0);
        if (c > c_begin) gate_emit(c - 1);
        gate_load_z(c);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
    lds_barrier();   // B1: every wave's P blocks of chunk c are in LDS; V of chunk c has been read
    compute_b(c, [&](int R) {
      if constexpr (!GATE) store_o(c, R);
    });
    if constexpr (GATE) gate_partials(c);
    lds_barrier();   // B2
    if constexpr (GATE) gate_finish(c);
  }
  if constexpr (GATE) gate_emit(c_end - 1);

  // final state
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int J = 0; J < 8; ++J)
      *reinterpret_cast<float4 *>(ST + ((size_t)bh * DV + iw0 + 16 * t + ln) * DK + 16 * J + 4 * g4) =
          make_float4(accS[t][J][0], accS[t][J][1], accS[t][J][2], accS[t][J][3]);
}

// Chunks per (sequence, value head) in the workspace: ceil(T / C); for packed
// sequences, chunk slots per value head.
inline int chunks_per_chain(const Shape &sh) {
  return sh.packed ? packed_slots(sh.T, sh.B, C) : (sh.T + C - 1) / C;
}
// Tokens of all the sequences of a call.
inline size_t tokens(const Shape &sh) { return sh.packed ? (size_t)sh.T : (size_t)sh.B * sh.T; }

// Packed sequences in order of decreasing chunk count (ties in any order),
// for the sequential pass: a counting sort in one workgroup, over bins of
// chunk counts (1023 chunks and more share the first bin).
constexpr int kOrderBins = 1024;
__global__ __launch_bounds__(kOrderBins) void seq_order_kernel(Seqs sq, int Tall, int *__restrict__ order) {
  __shared__ int bin[kOrderBins];
  __shared__ int wsum[kOrderBins / 64];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  auto key = [&](int s) {
    int start, len;
    seq_bounds(sq, s, Tall, start, len);
    return kOrderBins - 1 - min((len + C - 1) / C, kOrderBins - 1);   // bin 0: the longest
  };
  bin[t] = 0;
  __syncthreads();
  for (int s = t; s < sq.B; s += kOrderBins) atomicAdd(&bin[key(s)], 1);
  __syncthreads();
  const int n = bin[t];   // exclusive prefix sum over the bins: wave scans, then the waves' totals
  int x = n;
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  for (int i = 0; i < wv; ++i) x += wsum[i];
  bin[t] = x - n;
  __syncthreads();
  for (int s = t; s < sq.B; s += kOrderBins) order[atomicAdd(&bin[key(s)], 1)] = s;
}

// Bytes of the chunk matrices in the workspace; packed sequences keep their
// order after them (B ints, rounded up to 256 bytes).
// The head gate's prep stores P too when the sequential pass runs two
// compute waves per workgroup: at most 64 chains.
inline bool p_in_workspace(const Shape &sh) { return !sh.key_gate && (long)sh.B * sh.Hv <= 64; }
inline size_t chunk_matrix_bytes(const Shape &sh) {
  const size_t per_chunk =
      (size_t)(sh.key_gate ? KDA_CHUNK_U4 : p_in_workspace(sh) ? GDN_CHUNK_U4_P : GDN_CHUNK_U4) * 16;
  return (size_t)(sh.packed ? 1 : sh.B) * sh.Hv * chunks_per_chain(sh) * per_chunk;
}
inline size_t order_bytes(const Shape &sh) { return sh.packed ? ((size_t)sh.B * 4 + 255) / 256 * 256 : 0; }
inline int *seq_order(const Shape &sh, const void *ws) {
  return sh.packed ? (int *)((char *)ws + chunk_matrix_bytes(sh)) : nullptr;
}
hipError_t launch_order(const Shape &sh, void *ws, hipStream_t st) {
  if (!sh.packed) return hipSuccess;
  hipLaunchKernelGGL(seq_order_kernel, dim3(1), dim3(kOrderBins), 0, st, Seqs{sh.cu, sh.B}, sh.T,
                     seq_order(sh, ws));
  return hipGetLastError();
}

template <typename TQ, typename TG, int NW, int RT, bool KDA, bool CONV = false, bool GATE = false,
          bool ND = false>
hipError_t launch_seq(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                      const void *beta, const uint4 *TPws, const float *S0, float *o, float *ST,
                      int nchunks, int c_begin, int c_end, hipStream_t st, const ConvIn &cv = ConvIn{},
                      const GateArgs &ga = GateArgs{}) {
  using Cfg = SeqCfg<NW, RT, KDA, CONV>;
  constexpr int smem = GATE ? Cfg::SMEM_GATE : Cfg::SMEM;
  static_assert(smem <= 160 * 1024, "LDS");
  auto kern = chunk_seq_kernel<TQ, TG, NW, RT, KDA, CONV, GATE, ND>;
  hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return e;
  const int ntasks = sh.B * sh.Hv * Cfg::NS;
  // packed sequences: (sequence, key head) groups rounded up to a multiple of 8
  const int grid = sh.packed ? (sh.B * sh.Hk + 7) / 8 * 8 * (sh.Hv / sh.Hk) * Cfg::NS : ntasks;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(Cfg::THREADS), smem, st, (const TQ *)q, (const TQ *)k,
                     (const TQ *)v, (const TG *)g, (const TG *)beta, TPws, S0, o, ST, sh.T, sh.Hk, sh.Hv,
                     ntasks, nchunks, c_begin, c_end, cv, ga, Seqs{sh.cu, sh.B, seq_order(sh, TPws)});
  return hipGetLastError();
}

// At most 4 segments: the long prefill (1024 chunks) took 2.49 ms in 4, 2.5-2.64
// ms in 2, 3, 6, 8 or 16 (the first segment's prep runs alone, each further one
// adds a launch of the pass).
constexpr int kMaxSeg = 4;
// A side stream and events for one pipelined call, taken from a per-device
// pool and returned when the call has enqueued its work (the pool grows to
// the number of concurrent calls).  Streams have the default priority.
struct SideSlot {
  hipStream_t stream = nullptr;
  hipEvent_t ev[kMaxSeg + 1] = {};
};
class SidePool {
 public:
  static SidePool &get() {
    static SidePool p;
    return p;
  }
  SideSlot *acquire(int dev) {
    {
      std::lock_guard<std::mutex> g(mu_);
      auto &fl = free_[dev];
      if (!fl.empty()) {
        SideSlot *x = fl.back();
        fl.pop_back();
        return x;
      }
    }
    SideSlot *x = new SideSlot;
    bool ok = hipStreamCreateWithFlags(&x->stream, hipStreamNonBlocking) == hipSuccess;
    for (int i = 0; ok && i <= kMaxSeg; ++i)
      ok = hipEventCreateWithFlags(&x->ev[i], hipEventDisableTiming) == hipSuccess;
    if (!ok) {
      for (auto &e : x->ev)
        if (e) (void)hipEventDestroy(e);
      if (x->stream) (void)hipStreamDestroy(x->stream);
      delete x;
      return nullptr;
    }
    return x;
  }
  void release(int dev, SideSlot *x) {
    std::lock_guard<std::mutex> g(mu_);
    free_[dev].push_back(x);
  }

 private:
  std::mutex mu_;
  std::map<int, std::vector<SideSlot *>> free_;
};

// Enqueue the chunked forward, with `overlap` over up to kMaxSeg segments of
// consecutive chunks: the state-independent launch of segment s + 1 (prep)
// runs on a side stream while the sequential pass (seq) works through
// segment s on the caller's stream; segment s + 1 of the pass starts from
// the state segment s left in S_T.  prep(c_begin, c_end, stream) and
// seq(c_begin, c_end, S0, stream) enqueue one launch each.  Overlap pays when
// the pass leaves most compute units idle; when it fills the GPU the two
// launches only compete for it.
template <typename PrepFn, typename SeqFn>
hipError_t pipelined(int nchunks, bool overlap, const float *S0, float *ST, hipStream_t st, PrepFn prep,
                     SeqFn seq) {
  const int nseg = overlap ? std::min(kMaxSeg, nchunks / 16) : 1;
  int dev = 0;
  SideSlot *side = nullptr;
  if (nseg > 1 && hipGetDevice(&dev) == hipSuccess) side = SidePool::get().acquire(dev);
  hipError_t e;
  if (!side) {
    if ((e = prep(0, nchunks, st)) != hipSuccess) return e;
    return seq(0, nchunks, S0, st);
  }
  auto bound = [&](int i) { return (int)((long)nchunks * i / nseg); };
  // the side stream starts once segment 0 is prepared (and so after all the
  // caller enqueued before), when the pass takes the GPU
  e = prep(bound(0), bound(1), st);
  if (e == hipSuccess) e = hipEventRecord(side->ev[0], st);
  if (e == hipSuccess) e = hipStreamWaitEvent(side->stream, side->ev[0], 0);
  for (int i = 1; i < nseg && e == hipSuccess; ++i) {
    e = prep(bound(i), bound(i + 1), side->stream);
    if (e == hipSuccess) e = hipEventRecord(side->ev[i], side->stream);
  }
  for (int i = 0; i < nseg && e == hipSuccess; ++i) {
    if (i > 0) e = hipStreamWaitEvent(st, side->ev[i], 0);
    if (e == hipSuccess) e = seq(bound(i), bound(i + 1), i == 0 ? S0 : ST, st);
  }
  SidePool::get().release(dev, side);
  return e;
}

// Overlap the preparation of later segments with the sequential pass when
// the pass leaves room on the GPU: few sequences, each long (the pass then
// has at most 192 workgroups).
inline bool seq_overlap(long heads) { return heads <= 48; }

// CONV: the convolution prologue runs inside: the prep kernel makes q and k
// (into cv.q, cv.k, which the sequential pass then reads) and the
// sequential pass makes v; the q, k, v arguments are not read.
template <typename TQ, typename TG, bool CONV>
hipError_t launch_t(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                    const void *beta, const float *S0, float *o, float *ST, void *ws, hipStream_t st,
                    const ConvIn &cv, const GateArgs *gate = nullptr) {
  // chunks per (sequence, value head), or chunk slots per value head (packed sequences)
  const int nchunks = chunks_per_chain(sh);
  uint4 *TPws = (uint4 *)ws;
  const bool pw = p_in_workspace(sh);
  auto prep_k = pw ? chunk_prep_kernel<TQ, TG, CONV, true> : chunk_prep_kernel<TQ, TG, CONV, false>;
  const size_t smem = prep_smem(sh.Hv / sh.Hk, CONV, pw);
  if (smem > 160 * 1024) return hipErrorInvalidValue;
  hipError_t e =
      hipFuncSetAttribute((const void *)prep_k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  auto prep = [&](int cb, int ce, hipStream_t s) {
    const dim3 grid = sh.packed ? dim3(nchunks, sh.Hk) : dim3(ce - cb, sh.B * sh.Hk);
    hipLaunchKernelGGL(prep_k, grid, dim3(kThreads), smem, s, (const TQ *)q, (const TQ *)k, (const TG *)g,
                       (const TG *)beta, TPws, sh.T, sh.Hk, sh.Hv, nchunks, cb, cv, Seqs{sh.cu, sh.B});
    return hipGetLastError();
  };
  const void *qs = CONV ? cv.q : q, *ks = CONV ? cv.k : k;
  // Workgroups of the sequential pass: as few per head as keep every one of
  // them resident (one per compute unit).  128 value rows: four compute waves
  // holding two row tiles each (a K or Q fragment read from LDS then serves
  // two tiles); 64 and 32 rows: one row tile per compute wave.
  const long heads = (long)sh.B * sh.Hv;
  auto seq = [&](int cb, int ce, const float *s0, hipStream_t s) {
    if constexpr (CONV)
      if (gate)
        return launch_seq<TQ, TG, 4, 2, false, CONV, true>(sh, qs, ks, v, g, beta, TPws, s0, nullptr, ST,
                                                              nchunks, cb, ce, s, cv, *gate);
    if constexpr (!CONV)
      if (sh.no_delta) {
        if (heads > 128)
          return launch_seq<TQ, TG, 4, 2, false, false, false, true>(sh, qs, ks, v, g, beta, TPws, s0, o, ST,
                                                                        nchunks, cb, ce, s, cv);
        if (heads > 64)
          return launch_seq<TQ, TG, 4, 1, false, false, false, true>(sh, qs, ks, v, g, beta, TPws, s0, o, ST,
                                                                        nchunks, cb, ce, s, cv);
        return launch_seq<TQ, TG, 2, 1, false, false, false, true>(sh, qs, ks, v, g, beta, TPws, s0, o, ST,
                                                                      nchunks, cb, ce, s, cv);
      }
    if (heads > 128)
      return launch_seq<TQ, TG, 4, 2, false, CONV>(sh, qs, ks, v, g, beta, TPws, s0, o, ST, nchunks, cb,
                                                      ce, s, cv);
    if (heads > 64)
      return launch_seq<TQ, TG, 4, 1, false, CONV>(sh, qs, ks, v, g, beta, TPws, s0, o, ST, nchunks, cb,
                                                      ce, s, cv);
    return launch_seq<TQ, TG, 2, 1, false, CONV>(sh, qs, ks, v, g, beta, TPws, s0, o, ST, nchunks, cb,
                                                    ce, s, cv);
  };
  if ((e = launch_order(sh, ws, st)) != hipSuccess) return e;
  const bool overlap = !sh.packed && !sh.single_stream && seq_overlap(heads);
  return pipelined(nchunks, overlap, S0, ST, st, prep, seq);
}

// ============================================================================
// kda_prep: the state-independent work of the key-channel gate, per
// (batch, value head, chunk)
// ============================================================================
// The decay is a vector per token, so e^{gamma_r - gamma_s} sits inside the
// sum over key channels of A and P:
//     A[r][s] = beta_r sum_j k_rj k_sj e^{gamma_rj - gamma_sj}    (s < r)
//     P[r][s] =        sum_j q_rj k_sj e^{gamma_rj - gamma_sj}    (s <= r)
// Each block row of 16 rows is a product of decay-scaled K (or Q) and K about
// a reference token, on the matrix cores (details where A and P are formed).
constexpr int GST = DK + 4;                              // gamma row stride (fp32)
constexpr int KP_OFF_K = 0;                              // [C][KST] fp16
constexpr int KP_OFF_G = KP_OFF_K + C * KST * 2;         // [C][GST] fp32 (g, then gamma)
constexpr int KP_OFF_B = KP_OFF_G + C * GST * 4;         // beta [C] fp32
constexpr int KP_SMEM = KP_OFF_B + C * 4;
// once A and P are in registers, the matrices of the inverse reuse K and Q
constexpr int KP_OFF_T = 0;
constexpr int KP_OFF_P = KP_OFF_T + C * CST * 2;
constexpr int KP_OFF_AO = KP_OFF_P + C * CST * 2;
constexpr int KP_OFF_AD = KP_OFF_AO + C * CST * 2;
static_assert(KP_OFF_AD + 4 * 16 * DST * 4 <= KP_OFF_B, "inverse matrices overlap beta");
// three workgroups per compute unit
static_assert(3 * KP_SMEM <= 160 * 1024, "LDS");

// Eight consecutive channels of row `row` at kset(g4, kk) of a row-major fp32 matrix.
__device__ __forceinline__ void perm_row_f32(const float *M, int st, int row, int kk, int g4, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(M + row * st + 32 * kk + 4 * g4);
  const float4 b = *reinterpret_cast<const float4 *>(M + row * st + 32 * kk + 16 + 4 * g4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <typename TQ, typename TG>
__global__ __launch_bounds__(kThreads, 3) void kda_prep_kernel(
    const TQ *__restrict__ q, const TQ *__restrict__ k, const TG *__restrict__ g,
    const TG *__restrict__ beta, uint4 *__restrict__ ws, int Tall, int Hk, int Hv, int nchunks, int c0,
    Seqs sq) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  _Float16 *sK = reinterpret_cast<_Float16 *>(smem + KP_OFF_K);
  float *sG = reinterpret_cast<float *>(smem + KP_OFF_G);
  float *sB = reinterpret_cast<float *>(smem + KP_OFF_B);
  _Float16 *sT = reinterpret_cast<_Float16 *>(smem + KP_OFF_T);
  _Float16 *sP = reinterpret_cast<_Float16 *>(smem + KP_OFF_P);
  _Float16 *sAo = reinterpret_cast<_Float16 *>(smem + KP_OFF_AO);
  float *sAd = reinterpret_cast<float *>(smem + KP_OFF_AD);

  // block -> (chunk c of sequence b, value head h); packed sequences: blockIdx.x
  // is a chunk slot (nchunks = the slot count)
  const int h = blockIdx.y % Hv, kh = h / (Hv / Hk);
  int c, b, start, T;
  if (sq.cu) {
    b = seq_of_slot<C>(sq, Tall, blockIdx.x, c, start, T);
    if (b < 0) return;
  } else {
    c = c0 + blockIdx.x;
    b = blockIdx.y / Hv;
    seq_bounds(sq, b, Tall, start, T);
  }
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g4 = l >> 4, ln = l & 15;
  const int t0 = c * C, n = min(C, T - t0);
  const size_t bt0 = (size_t)start + t0;
  uint4 *wc = ws + (ws_chain(sq, b, h, Hv, nchunks, start) + c) * KDA_CHUNK_U4;

  // K, g and beta of the chunk into LDS; rows past the end are zero (so gamma
  // stays flat there).  Q stays in registers: qh holds the rows this thread
  // loaded (for Q o e^gamma), qd the rows of the wave's block row (for the
  // diagonal tile of P).
  half8 qh[4];
  uint2 qd[8];
  {
    constexpr int GW = sizeof(TG) == 4 ? 2 : 1;  // 16-byte pieces per 8 gate values
    uint4 uk[4], uq[4], ug[4][GW];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = min((tid >> 4) + 16 * it, n - 1);
      const size_t off = ((bt0 + row) * Hk + kh) * DK + (tid & 15) * 8;
      const size_t goff = ((bt0 + row) * Hv + h) * DK + (tid & 15) * 8;
      uk[it] = *reinterpret_cast<const uint4 *>(k + off);
      uq[it] = *reinterpret_cast<const uint4 *>(q + off);
#pragma unroll
      for (int u = 0; u < GW; ++u) ug[it][u] = *reinterpret_cast<const uint4 *>(g + goff + 4 * u);
    }
    const TG braw = beta[(bt0 + min(tid & 63, n - 1)) * Hv + h];
    // Q of the wave's block row, rows 16 w + ln at the channels kset(g4, kk)
    {
      const TQ *qp = q + ((bt0 + min(16 * w + ln, n - 1)) * Hk + kh) * DK + 4 * g4;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        qd[2 * kk] = *reinterpret_cast<const uint2 *>(qp + 32 * kk);
        qd[2 * kk + 1] = *reinterpret_cast<const uint2 *>(qp + 32 * kk + 16);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    const half8 hz = {};
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = (tid >> 4) + 16 * it;
      const bool ok = row < n;
      *reinterpret_cast<half8 *>(sK + row * KST + (tid & 15) * 8) = ok ? to_half8(uk[it], TQ{}) : hz;
      qh[it] = ok ? to_half8(uq[it], TQ{}) : hz;
      float gv[8];
      if constexpr (sizeof(TG) == 4) {
        const float4 a = __builtin_bit_cast(float4, ug[it][0]), bq = __builtin_bit_cast(float4, ug[it][1]);
        gv[0] = a.x; gv[1] = a.y; gv[2] = a.z; gv[3] = a.w;
        gv[4] = bq.x; gv[5] = bq.y; gv[6] = bq.z; gv[7] = bq.w;
      } else {
        const uint32_t wd[4] = {ug[it][0].x, ug[it][0].y, ug[it][0].z, ug[it][0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          gv[2 * i] = __uint_as_float(wd[i] << 16);
          gv[2 * i + 1] = __uint_as_float(wd[i] & 0xFFFF0000u);
        }
      }
      // in base 2: the decays below are all 2^x, one instruction each
#pragma unroll
      for (int j = 0; j < 8; ++j) gv[j] *= 1.44269504088896341f;   // log2(e)
      float *gp = sG + row * GST + (tid & 15) * 8;
      *reinterpret_cast<float4 *>(gp) = ok ? make_float4(gv[0], gv[1], gv[2], gv[3]) : make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4 *>(gp + 4) = ok ? make_float4(gv[4], gv[5], gv[6], gv[7]) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (tid < C) sB[tid] = tid < n ? to_f32(braw) : 0.f;
  }
  lds_barrier();

  // gamma: inclusive prefix over the rows, per channel (two halves of 32 rows);
  // held as gamma log2(e), so that every e^{...} below is one 2^x
  {
    const int ch = tid & 127, r0 = (tid >> 7) * 32;
    float x = 0.f;
#pragma unroll 8
    for (int r = r0; r < r0 + 32; ++r) {
      x += sG[r * GST + ch];
      sG[r * GST + ch] = x;
    }
  }
  lds_barrier();
  if (tid >= 128) {
    const int ch = tid & 127;
    const float base = sG[31 * GST + ch];
#pragma unroll 8
    for (int r = 32; r < 64; ++r) sG[r * GST + ch] += base;
  }
  lds_barrier();

  // operands of the sequential pass: K o e^gamma, Q o e^gamma, K o e^{gamma_n - gamma}
  // (gamma_n = gamma of the chunk's last token); beta; Gamma_n = e^{gamma_n}
  {
    const float *gl = sG + (n - 1) * GST;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int e = tid + kThreads * it;
      const int row = e >> 4, c8 = (e & 15) * 8;
      const half8 kv = *reinterpret_cast<const half8 *>(sK + row * KST + c8);
      const half8 qv = qh[it];
      half8 kg, qg, kd;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float gam = sG[row * GST + c8 + j];
        const float eg = __builtin_amdgcn_exp2f(gam), ed = __builtin_amdgcn_exp2f(gl[c8 + j] - gam);
        kg[j] = (_Float16)((float)kv[j] * eg);
        qg[j] = (_Float16)((float)qv[j] * eg);
        kd[j] = (_Float16)((float)kv[j] * ed);
      }
      wc[KDA_KG + e] = __builtin_bit_cast(uint4, kg);
      wc[KDA_QG + e] = __builtin_bit_cast(uint4, qg);
      wc[KDA_KD + e] = __builtin_bit_cast(uint4, kd);
    }
    float *wsc = reinterpret_cast<float *>(wc + KDA_SC);
    if (tid < C) wsc[tid] = sB[tid];
    if (tid < DK) wsc[C + tid] = __builtin_amdgcn_exp2f(gl[tid]);
  }

  // A and P for block row R = w (tiles S = 0..R), into registers.  Reference
  // token p = 16 R (the block row's first): e^{gamma_r - gamma_s} =
  // e^{gamma_r - gamma_p} e^{gamma_p - gamma_s}.
  //  * tiles S < R: s < p <= r, so both factors are <= 1; fp16 operands on the
  //    16x16x32 matrix cores (a factor that underflows belongs to a product
  //    that is itself that small);
  //  * tile S = R: e^{gamma_p - gamma_s} >= 1 for s > p, so fp32 operands on
  //    the 16x16x4 fp32 matrix cores; if a factor would overflow fp32 (a decay
  //    of e^-80 within 16 tokens), the wave computes that tile term by term.
  // The lane (g4, ln) holds row 16 R + ln at the channels kset(g4, kk), in
  // the same order for the fp16 and the fp32 products.
  const int R = w, p = 16 * R;
  float4v accA[4], accP[4];
  {
    half8 kl[4], ql[4];
    {
      float4v ad = {0.f, 0.f, 0.f, 0.f}, pd = {0.f, 0.f, 0.f, 0.f};
      bool ok = true;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        float gr[8], gp[8];
        perm_row_f32(sG, GST, 16 * R + ln, kk, g4, gr);
        perm_row_f32(sG, GST, p, kk, g4, gp);
        const half8 kv = perm_row(sK, KST, 16 * R + ln, kk, g4);
        const half4 qa = to_half4(qd[2 * kk], TQ{}), qb = to_half4(qd[2 * kk + 1], TQ{});
        const half8 qv = 16 * R + ln < n ? half8{qa[0], qa[1], qa[2], qa[3], qb[0], qb[1], qb[2], qb[3]}
                                         : half8{};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = __builtin_amdgcn_exp2f(gr[e] - gp[e]), fi = __builtin_amdgcn_exp2f(gp[e] - gr[e]);
          const float kf = (float)kv[e] * f, qf = (float)qv[e] * f, ki = (float)kv[e] * fi;
          ok = ok && fi <= 1.0e30f;
          kl[kk][e] = (_Float16)kf;
          ql[kk][e] = (_Float16)qf;
          ad = __builtin_amdgcn_mfma_f32_16x16x4f32(kf, ki, ad, 0, 0, 0);
          pd = __builtin_amdgcn_mfma_f32_16x16x4f32(qf, ki, pd, 0, 0, 0);
        }
      }
      if (__any(!ok)) {
        // exact diagonal tile: lane (g4, ln) holds r = 16 R + 4 g4 + ii, s = 16 R + ln
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * R + 4 * g4 + ii, s_ = 16 * R + ln;
          float a = 0.f, pp = 0.f;
          if (s_ <= r) {
            const TQ *qr = q + ((bt0 + min(r, n - 1)) * Hk + kh) * DK;
            for (int j = 0; j < DK; ++j) {
              const float e = __builtin_amdgcn_exp2f(sG[r * GST + j] - sG[s_ * GST + j]);
              const float ks = (float)sK[s_ * KST + j];
              const float qv = r < n ? (float)(_Float16)to_f32(qr[j]) : 0.f;
              a += (float)sK[r * KST + j] * ks * e;
              pp += qv * ks * e;
            }
          }
          ad[ii] = a;
          pd[ii] = pp;
        }
      }
#pragma unroll
      for (int S = 0; S < 4; ++S) {
        if (S == R) {
          accA[S] = ad;
          accP[S] = pd;
        }
      }
    }
#pragma unroll
    for (int S = 0; S < 3; ++S) {
      if (S < R) {
        float4v aa = {0.f, 0.f, 0.f, 0.f}, ap = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          float gs[8], gp[8];
          perm_row_f32(sG, GST, 16 * S + ln, kk, g4, gs);
          perm_row_f32(sG, GST, p, kk, g4, gp);
          const half8 kv = perm_row(sK, KST, 16 * S + ln, kk, g4);
          half8 ks;
#pragma unroll
          for (int e = 0; e < 8; ++e) ks[e] = (_Float16)((float)kv[e] * __builtin_amdgcn_exp2f(gp[e] - gs[e]));
          aa = mfma32(kl[kk], ks, aa);
          ap = mfma32(ql[kk], ks, ap);
        }
        accA[S] = aa;
        accP[S] = ap;
      }
    }
  }
  lds_barrier();  // K and gamma are no longer read: T, P, A take their place

  // A (diagonal blocks fp32 strictly lower, blocks below fp16) and P (lower incl. diagonal)
  {
    const int r0 = 16 * R + 4 * g4;
    float br[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) br[ii] = sB[r0 + ii];
#pragma unroll
    for (int S = 0; S < 4; ++S) {
      if (S > R) continue;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = r0 + ii, s_ = 16 * S + ln;
        if (S == R) {
          sAd[(R * 16 + 4 * g4 + ii) * DST + ln] = s_ < r ? br[ii] * accA[S][ii] : 0.f;
          sP[r * CST + s_] = (_Float16)(s_ <= r ? accP[S][ii] : 0.f);
        } else {
          sAo[r * CST + s_] = (_Float16)(br[ii] * accA[S][ii]);
          sP[r * CST + s_] = (_Float16)accP[S][ii];
        }
      }
    }
    const int rr = tid >> 4, cc = tid & 15;
    sT[rr * CST + 16 + cc] = (_Float16)0.f;
    sT[(32 + rr) * CST + 48 + cc] = (_Float16)0.f;
    sP[rr * CST + 16 + cc] = (_Float16)0.f;
    sP[(32 + rr) * CST + 48 + cc] = (_Float16)0.f;
  }
  invert_store<1>(sAd, sAo, sT, sP, nullptr, wc, w, l);
}

template <typename TQ, typename TG>
hipError_t launch_kda_t(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                        const void *beta, const float *S0, float *o, float *ST, void *ws,
                        hipStream_t st) {
  const int nchunks = chunks_per_chain(sh);
  uint4 *wsu = (uint4 *)ws;
  auto prep_k = kda_prep_kernel<TQ, TG>;
  hipError_t e =
      hipFuncSetAttribute((const void *)prep_k, hipFuncAttributeMaxDynamicSharedMemorySize, KP_SMEM);
  if (e != hipSuccess) return e;
  auto prep = [&](int cb, int ce, hipStream_t s) {
    const dim3 grid = sh.packed ? dim3(nchunks, sh.Hv) : dim3(ce - cb, sh.B * sh.Hv);
    hipLaunchKernelGGL(prep_k, grid, dim3(kThreads), KP_SMEM, s, (const TQ *)q, (const TQ *)k, (const TG *)g,
                       (const TG *)beta, wsu, sh.T, sh.Hk, sh.Hv, nchunks, cb, Seqs{sh.cu, sh.B});
    return hipGetLastError();
  };
  // The decayed K, Q and the state-update K all live in LDS here, so a
  // workgroup of the sequential pass holds at most 64 value rows.
  const long heads = (long)sh.B * sh.Hv;
  auto seq = [&](int cb, int ce, const float *s0, hipStream_t s) {
    if (sh.no_delta) {
      if (heads > 64)
        return launch_seq<TQ, TG, 4, 1, true, false, false, true>(sh, q, k, v, g, beta, wsu, s0, o, ST, nchunks,
                                                                     cb, ce, s);
      return launch_seq<TQ, TG, 2, 1, true, false, false, true>(sh, q, k, v, g, beta, wsu, s0, o, ST, nchunks,
                                                                   cb, ce, s);
    }
    if (heads > 64)
      return launch_seq<TQ, TG, 4, 1, true>(sh, q, k, v, g, beta, wsu, s0, o, ST, nchunks, cb, ce, s);
    return launch_seq<TQ, TG, 2, 1, true>(sh, q, k, v, g, beta, wsu, s0, o, ST, nchunks, cb, ce, s);
  };
  if ((e = launch_order(sh, ws, st)) != hipSuccess) return e;
  const bool overlap = !sh.packed && !sh.single_stream && seq_overlap(heads);
  return pipelined(nchunks, overlap, S0, ST, st, prep, seq);
}

}  // namespace

size_t chunk_mfma_workspace(const Shape &sh) { return chunk_matrix_bytes(sh) + order_bytes(sh); }

hipError_t launch_chunk_mfma(const Shape &sh, const void *q, const void *k, const void *v,
                             const void *g, const void *beta, const float *S0, float *o, float *ST,
                             void *ws, hipStream_t st) {
  if (sh.key_gate) {
    if (sh.qkv == DType::BF16)
      return sh.gate_t == DType::F32
                 ? launch_kda_t<bf16_t, float>(sh, q, k, v, g, beta, S0, o, ST, ws, st)
                 : launch_kda_t<bf16_t, bf16_t>(sh, q, k, v, g, beta, S0, o, ST, ws, st);
    return sh.gate_t == DType::F32 ? launch_kda_t<f16_t, float>(sh, q, k, v, g, beta, S0, o, ST, ws, st)
                                   : launch_kda_t<f16_t, bf16_t>(sh, q, k, v, g, beta, S0, o, ST, ws, st);
  }
  const ConvIn none{};
  if (sh.qkv == DType::BF16)
    return sh.gate_t == DType::F32
               ? launch_t<bf16_t, float, false>(sh, q, k, v, g, beta, S0, o, ST, ws, st, none)
               : launch_t<bf16_t, bf16_t, false>(sh, q, k, v, g, beta, S0, o, ST, ws, st, none);
  return sh.gate_t == DType::F32
             ? launch_t<f16_t, float, false>(sh, q, k, v, g, beta, S0, o, ST, ws, st, none)
             : launch_t<f16_t, bf16_t, false>(sh, q, k, v, g, beta, S0, o, ST, ws, st, none);
}

bool chunk_mfma_gate_inside(const Shape &sh) { return !sh.key_gate && (long)sh.B * sh.Hv > 128; }

hipError_t launch_chunk_mfma_conv(const Shape &sh, const void *xq, const void *xk, const void *xv,
                                  const float *conv_w, float eps, const void *g, const void *beta,
                                  const float *S0, float *o, float *ST, void *ws, hipStream_t st,
                                  const GateArgs *gate) {
  if (gate && (!chunk_mfma_gate_inside(sh) || gate->yt == DType::F32)) return hipErrorInvalidValue;
  // workspace: the chunk matrices, then q and k after the prologue
  const size_t nqk = tokens(sh) * sh.Hk * DK;
  char *base = (char *)ws;
  ConvIn cv;
  cv.xq = (const bf16_t *)xq;
  cv.xk = (const bf16_t *)xk;
  cv.xv = (const bf16_t *)xv;
  cv.wq = conv_w;
  cv.wk = conv_w + (size_t)sh.Hk * DK * 4;
  cv.wv = conv_w + (size_t)2 * sh.Hk * DK * 4;
  cv.q = base + chunk_mfma_workspace(sh);
  cv.k = (char *)cv.q + nqk * 2;
  cv.eps = eps;
  if (sh.qkv != DType::F16) return hipErrorInvalidValue;   // q, k after the prologue are fp16 here
  return sh.gate_t == DType::F32
             ? launch_t<f16_t, float, true>(sh, nullptr, nullptr, nullptr, g, beta, S0, o, ST, ws, st, cv, gate)
             : launch_t<f16_t, bf16_t, true>(sh, nullptr, nullptr, nullptr, g, beta, S0, o, ST, ws, st, cv, gate);
}

size_t chunk_mfma_conv_workspace(const Shape &sh) {
  return chunk_mfma_workspace(sh) + (size_t)2 * tokens(sh) * sh.Hk * DK * 2;
}

}  // namespace gdn
