// chunk_f32.hip -- chunked forward of the gated delta rule with fp32 arithmetic.
//
// The fp32-accurate path: every product is an fp32 multiply-add on the vector
// ALUs, every intermediate lives in LDS as fp32.  It handles both gates and
// small head dims, and is the path of the fp32 mode.
//
// Chunk algebra (derived from the recurrence of the "Source notes" page,
// "Linear attention", rows gdn/kda; the attention-sink study page, "SinkProbe",
// computes the same layer in exact chunkwise form).  For one chain and a chunk
// of n tokens with entering state S (dv x dk), in-chunk prefix
// gamma_r = g_1 + ... + g_r (a dk-vector for the key-channel gate):
//   A[r][s] = beta_r sum_j k_rj k_sj e^{gamma_rj - gamma_sj}   (s < r)
//   P[r][s] =        sum_j q_rj k_sj e^{gamma_rj - gamma_sj}   (s <= r)
//   X[r][i] = beta_r (v_ri - sum_j k_rj e^{gamma_rj} S_ij)
//   N       = (I + A)^{-1} X            (forward substitution, row by row)
//   o_r     = sum_j q_rj e^{gamma_rj} S_ij + sum_{s<=r} P[r][s] N[s][i]
//   S_ij   <- e^{gamma_nj} S_ij + sum_r N[r][i] k_rj e^{gamma_nj - gamma_rj}
// Every exponent is of a non-positive number, so nothing can overflow.
//
// One 256-thread block owns the rows [i0, i0 + DVS) of the state of one
// (batch, value head) and walks the chunks in order; the rows of the state
// evolve independently, so value-dim slices run as separate blocks.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;

template <int DK, int DVS, int C, bool KEYGATE>
struct F32Smem {
  static constexpr int KP = DK + 1;   // padded row strides
  static constexpr int VP = DVS + 1;
  static constexpr int CP = C + 1;
  static constexpr int nK = C * KP, nQ = C * KP;
  static constexpr int nGam = KEYGATE ? C * KP : C;
  static constexpr int nEg = KEYGATE ? C * KP : C;     // e^{gamma_r}
  static constexpr int nDec = KEYGATE ? C * KP : C;    // e^{gamma_n - gamma_r}
  static constexpr int nBeta = C;
  static constexpr int nV = C * VP, nX = C * VP, nO = C * VP;
  static constexpr int nS = DVS * KP;
  static constexpr int nA = C * CP, nP = C * CP;
  static constexpr int total =
      nK + nQ + nGam + nEg + nDec + nBeta + nV + nX + nO + nS + nA + nP;
  static constexpr size_t bytes = sizeof(float) * total;
};

template <typename TQ, typename TG, bool KEYGATE, int DK, int DVS, int C>
__global__ __launch_bounds__(kThreads) void chunk_f32_kernel(
    const TQ *__restrict__ q, const TQ *__restrict__ k, const TQ *__restrict__ v,
    const TG *__restrict__ g, const TG *__restrict__ beta, const float *__restrict__ S0,
    float *__restrict__ o, float *__restrict__ ST, int Tall, int Hk, int Hv, int dv, Seqs sq, int nodelta) {
  using L = F32Smem<DK, DVS, C, KEYGATE>;
  constexpr int KP = L::KP, VP = L::VP, CP = L::CP;
  extern __shared__ float smem[];
  float *sK = smem;
  float *sQ = sK + L::nK;
  float *sGam = sQ + L::nQ;
  float *sEg = sGam + L::nGam;
  float *sDec = sEg + L::nEg;
  float *sBeta = sDec + L::nDec;
  float *sV = sBeta + L::nBeta;
  float *sX = sV + L::nV;
  float *sO = sX + L::nX;
  float *sS = sO + L::nO;
  float *sA = sS + L::nS;
  float *sP = sA + L::nA;

  const int tid = threadIdx.x;
  const int b = blockIdx.z, h = blockIdx.y, i0 = blockIdx.x * DVS;
  const int kh = h / (Hv / Hk);
  const size_t bh = (size_t)b * Hv + h;
  int start, T;   // the sequence's first token and length
  seq_bounds(sq, b, Tall, start, T);

  for (int e = tid; e < DVS * DK; e += kThreads) {
    const int i = e / DK, j = e % DK;
    sS[i * KP + j] = S0 ? S0[(bh * dv + i0 + i) * DK + j] : 0.f;
  }

  for (int c0 = 0; c0 < T; c0 += C) {
    const int n = min(C, T - c0);
    __syncthreads();
    // ---- load the chunk (rows >= n are zero; zero g and beta there make the
    // padded rows inert) ----
    for (int e = tid; e < C * DK; e += kThreads) {
      const int r = e / DK, j = e % DK;
      const size_t t = (size_t)start + c0 + r;
      const bool ok = r < n;
      sK[r * KP + j] = ok ? to_f32(k[(t * Hk + kh) * DK + j]) : 0.f;
      sQ[r * KP + j] = ok ? to_f32(q[(t * Hk + kh) * DK + j]) : 0.f;
      if constexpr (KEYGATE) sGam[r * KP + j] = ok ? to_f32(g[(t * Hv + h) * DK + j]) : 0.f;
    }
    for (int e = tid; e < C * DVS; e += kThreads) {
      const int r = e / DVS, i = e % DVS;
      const size_t t = (size_t)start + c0 + r;
      sV[r * VP + i] = r < n ? to_f32(v[(t * Hv + h) * dv + i0 + i]) : 0.f;
    }
    for (int r = tid; r < C; r += kThreads) {
      const size_t t = (size_t)start + c0 + r;
      sBeta[r] = r < n ? to_f32(beta[t * Hv + h]) : 0.f;
      if constexpr (!KEYGATE) sGam[r] = r < n ? to_f32(g[t * Hv + h]) : 0.f;
    }
    __syncthreads();
    // ---- in-chunk prefix of the log decay, and its exponentials ----
    if constexpr (KEYGATE) {
      for (int j = tid; j < DK; j += kThreads) {
        float acc = 0.f;
        for (int r = 0; r < C; ++r) {
          acc += sGam[r * KP + j];
          sGam[r * KP + j] = acc;
        }
        for (int r = 0; r < C; ++r) {
          sEg[r * KP + j] = __expf(sGam[r * KP + j]);
          sDec[r * KP + j] = __expf(acc - sGam[r * KP + j]);
        }
      }
    } else {
      if (tid == 0) {
        float acc = 0.f;
        for (int r = 0; r < C; ++r) {
          acc += sGam[r];
          sGam[r] = acc;
        }
        for (int r = 0; r < C; ++r) {
          sEg[r] = __expf(sGam[r]);
          sDec[r] = __expf(acc - sGam[r]);
        }
      }
    }
    __syncthreads();
    // ---- A (strictly lower) and P (lower incl. diagonal) ----
    for (int e = tid; e < C * C; e += kThreads) {
      const int r = e / C, s = e % C;
      float a = 0.f, p = 0.f;
      if (s <= r) {
        if constexpr (KEYGATE) {
          for (int j = 0; j < DK; ++j) {
            const float d = __expf(sGam[r * KP + j] - sGam[s * KP + j]);
            const float ks = sK[s * KP + j] * d;
            a += sK[r * KP + j] * ks;
            p += sQ[r * KP + j] * ks;
          }
        } else {
          for (int j = 0; j < DK; ++j) {
            a += sK[r * KP + j] * sK[s * KP + j];
            p += sQ[r * KP + j] * sK[s * KP + j];
          }
          const float d = __expf(sGam[r] - sGam[s]);
          a *= d;
          p *= d;
        }
      }
      sA[r * CP + s] = s < r ? sBeta[r] * a : 0.f;
      sP[r * CP + s] = s <= r ? p : 0.f;
    }
    // ---- X = beta (V - (K o Gamma) S^T) and the inter-chunk read Q o Gamma S^T ----
    for (int e = tid; e < C * DVS; e += kThreads) {
      const int r = e / DVS, i = e % DVS;
      float kx = 0.f, qx = 0.f;
      for (int j = 0; j < DK; ++j) {
        const float eg = KEYGATE ? sEg[r * KP + j] : 1.f;
        const float sij = sS[i * KP + j];
        kx += sK[r * KP + j] * eg * sij;
        qx += sQ[r * KP + j] * eg * sij;
      }
      if constexpr (!KEYGATE) {
        kx *= sEg[r];
        qx *= sEg[r];
      }
      // without the delta correction the chunk's new values are beta V
      sX[r * VP + i] = sBeta[r] * (sV[r * VP + i] - (nodelta ? 0.f : kx));
      sO[r * VP + i] = qx;
    }
    __syncthreads();
    // ---- N = (I + A)^{-1} X by forward substitution, in place ----
    for (int i = tid; i < DVS && !nodelta; i += kThreads) {
      for (int r = 1; r < n; ++r) {
        float acc = sX[r * VP + i];
        for (int s = 0; s < r; ++s) acc -= sA[r * CP + s] * sX[s * VP + i];
        sX[r * VP + i] = acc;
      }
    }
    __syncthreads();
    // ---- outputs of the chunk ----
    for (int e = tid; e < C * DVS; e += kThreads) {
      const int r = e / DVS, i = e % DVS;
      if (r < n) {
        float acc = sO[r * VP + i];
        for (int s = 0; s <= r; ++s) acc += sP[r * CP + s] * sX[s * VP + i];
        o[(((size_t)start + c0 + r) * Hv + h) * dv + i0 + i] = acc;
      }
    }
    // ---- state update (reads only N, K and the decay tables) ----
    for (int e = tid; e < DVS * DK; e += kThreads) {
      const int i = e / DK, j = e % DK;
      const float gend = KEYGATE ? sEg[(C - 1) * KP + j] : sEg[C - 1];
      float acc = gend * sS[i * KP + j];
      for (int r = 0; r < n; ++r) {
        const float dec = KEYGATE ? sDec[r * KP + j] : sDec[r];
        acc += sX[r * VP + i] * sK[r * KP + j] * dec;
      }
      sS[i * KP + j] = acc;
    }
  }
  __syncthreads();
  for (int e = tid; e < DVS * DK; e += kThreads) {
    const int i = e / DK, j = e % DK;
    ST[(bh * dv + i0 + i) * DK + j] = sS[i * KP + j];
  }
}

template <typename TQ, typename TG, bool KEYGATE, int DK, int DVS, int C>
hipError_t launch_cfg(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                      const void *beta, const float *S0, float *o, float *ST, hipStream_t st) {
  constexpr size_t smem = F32Smem<DK, DVS, C, KEYGATE>::bytes;
  static_assert(smem <= 160 * 1024, "LDS budget");
  auto kern = chunk_f32_kernel<TQ, TG, KEYGATE, DK, DVS, C>;
  hipError_t e = hipFuncSetAttribute((const void *)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  dim3 grid(sh.dv / DVS, sh.Hv, sh.B);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, st, (const TQ *)q, (const TQ *)k,
                     (const TQ *)v, (const TG *)g, (const TG *)beta, S0, o, ST, sh.T, sh.Hk, sh.Hv,
                     sh.dv, Seqs{sh.cu, sh.B}, sh.no_delta ? 1 : 0);
  return hipGetLastError();
}

template <typename TQ, typename TG, bool KEYGATE, int DK, int DVS>
hipError_t launch_c(const Shape &sh, int C, const void *q, const void *k, const void *v,
                    const void *g, const void *beta, const float *S0, float *o, float *ST,
                    hipStream_t st) {
  if constexpr (DK <= 64) {
    switch (C) {
      case 16: return launch_cfg<TQ, TG, KEYGATE, DK, DVS, 16>(sh, q, k, v, g, beta, S0, o, ST, st);
      case 32: return launch_cfg<TQ, TG, KEYGATE, DK, DVS, 32>(sh, q, k, v, g, beta, S0, o, ST, st);
      case 64: return launch_cfg<TQ, TG, KEYGATE, DK, DVS, 64>(sh, q, k, v, g, beta, S0, o, ST, st);
    }
  } else {
    switch (C) {
      case 16: return launch_cfg<TQ, TG, KEYGATE, DK, DVS, 16>(sh, q, k, v, g, beta, S0, o, ST, st);
      case 32: return launch_cfg<TQ, TG, KEYGATE, DK, DVS, 32>(sh, q, k, v, g, beta, S0, o, ST, st);
    }
  }
  return hipErrorInvalidValue;
}

template <typename TQ, typename TG, bool KEYGATE>
hipError_t launch_k(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                    const void *beta, const float *S0, float *o, float *ST, hipStream_t st) {
  const int C = chunk_f32_internal(sh.chunk, sh.dk);
  // value-dim slice: min(dv, 32)
  if (sh.dv == 16) {
    switch (sh.dk) {
      case 16: return launch_c<TQ, TG, KEYGATE, 16, 16>(sh, C, q, k, v, g, beta, S0, o, ST, st);
      case 32: return launch_c<TQ, TG, KEYGATE, 32, 16>(sh, C, q, k, v, g, beta, S0, o, ST, st);
      case 64: return launch_c<TQ, TG, KEYGATE, 64, 16>(sh, C, q, k, v, g, beta, S0, o, ST, st);
      case 128: return launch_c<TQ, TG, KEYGATE, 128, 16>(sh, C, q, k, v, g, beta, S0, o, ST, st);
    }
  } else {
    switch (sh.dk) {
      case 16: return launch_c<TQ, TG, KEYGATE, 16, 32>(sh, C, q, k, v, g, beta, S0, o, ST, st);
      case 32: return launch_c<TQ, TG, KEYGATE, 32, 32>(sh, C, q, k, v, g, beta, S0, o, ST, st);
      case 64: return launch_c<TQ, TG, KEYGATE, 64, 32>(sh, C, q, k, v, g, beta, S0, o, ST, st);
      case 128: return launch_c<TQ, TG, KEYGATE, 128, 32>(sh, C, q, k, v, g, beta, S0, o, ST, st);
    }
  }
  return hipErrorInvalidValue;
}

template <typename TQ, typename TG>
hipError_t launch_tg(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                     const void *beta, const float *S0, float *o, float *ST, hipStream_t st) {
  return sh.key_gate ? launch_k<TQ, TG, true>(sh, q, k, v, g, beta, S0, o, ST, st)
                     : launch_k<TQ, TG, false>(sh, q, k, v, g, beta, S0, o, ST, st);
}

}  // namespace

int chunk_f32_internal(int chunk, int dk) {
  int c = chunk;
  while (c > 16 && c * dk > 4096) c /= 2;
  return c;
}

hipError_t launch_chunk_f32(const Shape &sh, const void *q, const void *k, const void *v,
                            const void *g, const void *beta, const float *S0, float *o, float *ST,
                            hipStream_t st) {
  if (sh.qkv == DType::F32)
    return sh.gate_t == DType::F32 ? launch_tg<float, float>(sh, q, k, v, g, beta, S0, o, ST, st)
                                   : launch_tg<float, bf16_t>(sh, q, k, v, g, beta, S0, o, ST, st);
  if (sh.qkv == DType::BF16)
    return sh.gate_t == DType::F32 ? launch_tg<bf16_t, float>(sh, q, k, v, g, beta, S0, o, ST, st)
                                   : launch_tg<bf16_t, bf16_t>(sh, q, k, v, g, beta, S0, o, ST, st);
  return sh.gate_t == DType::F32 ? launch_tg<f16_t, float>(sh, q, k, v, g, beta, S0, o, ST, st)
                                 : launch_tg<f16_t, bf16_t>(sh, q, k, v, g, beta, S0, o, ST, st);
}

}  // namespace gdn
