// gdn_launch.h -- host launchers of the gfx950 kernels.  Called by gdn_api.cpp
// after the arguments have been validated; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

enum class DType : int { F32 = 0, BF16 = 1, F16 = 2 };

// B sequences of T tokens each; or (packed) B sequences packed into T
// tokens, sequence s being tokens cu[s] .. cu[s+1]-1 (cu: device int32
// [B + 1]; null in a size query).
struct Shape {
  int B, T, Hk, Hv, dk, dv, chunk;
  DType qkv, gate_t;
  bool key_gate;
  bool packed = false;
  const int *cu = nullptr;
  bool no_delta = false;   // the update without the delta correction
  bool single_stream = false;   // all work on the caller's stream (no side stream)
};

// The gate's arguments for the chunked forward with the prologue inside,
// which applies it inside the sequential pass when chunk_mfma_gate_inside(sh)
// and y is 16-bit (z is bf16, like the raw inputs).
struct GateArgs {
  const void *z;
  const float *gain;
  float eps;
  void *y;
  DType yt;
};
bool chunk_mfma_gate_inside(const Shape &sh);

// Prologue: conv + SiLU over q, k, v (L2 over q and k rows); w holds the
// conv taps of q, then k, then v channels.  cu: packed sequences (see Shape).
hipError_t launch_prologue(const void *xq, const void *xk, const void *xv, DType xt, const float *w,
                           void *q, void *k, void *v, DType yt, int B, int T, int Hk, int Hv, int dk,
                           int dv, float eps, hipStream_t s, const int *cu = nullptr);

// One token per sequence from raw inputs xq, xk [B,Hk,dk], xv [B,Hv,dv] and
// the convolution history cs [B][3][2 Hk dk + Hv dv] (raw input type, moved
// on by one token in place): q, k, v of type yt, as the prologue makes them.
hipError_t launch_decode_prologue(const void *xq, const void *xk, const void *xv, DType xt, const float *w,
                                  void *cs, void *q, void *k, void *v, DType yt, int B, int Hk, int Hv,
                                  int dk, int dv, float eps, hipStream_t s);
// The convolution history after each sequence's last token (raw inputs of its
// last three tokens, zero before its first) into cs.
hipError_t launch_conv_state(const void *xq, const void *xk, const void *xv, DType xt, void *cs, int B,
                             int T, int Hk, int Hv, int dk, int dv, const int *cu, hipStream_t s);

// One decode step, state in place.
hipError_t launch_decode(const Shape &sh, const void *q, const void *k, const void *v,
                         const void *g, const void *beta, float *S, float *o, hipStream_t s);

// Chunked forward with fp32 arithmetic (any supported dtype in, fp32 math).
hipError_t launch_chunk_f32(const Shape &sh, const void *q, const void *k, const void *v,
                            const void *g, const void *beta, const float *S0, float *o,
                            float *ST, hipStream_t s);

// Chunked forward on the fp16 matrix cores (dk = dv = 128, chunk 64, either
// gate).  `ws` holds chunk_mfma_workspace(sh) bytes (16-byte aligned).
hipError_t launch_chunk_mfma(const Shape &sh, const void *q, const void *k, const void *v,
                             const void *g, const void *beta, const float *S0, float *o,
                             float *ST, void *ws, hipStream_t s);
size_t chunk_mfma_workspace(const Shape &sh);

// The same with the convolution prologue inside (bf16 raw inputs, head
// gate): equal to launch_prologue into q, k, v of sh.qkv followed by
// launch_chunk_mfma.  `ws` holds chunk_mfma_conv_workspace(sh) bytes.
// With `gate` (only where chunk_mfma_gate_inside(sh)), the gated output
// norm is applied in the sequential pass and y written instead of o.
hipError_t launch_chunk_mfma_conv(const Shape &sh, const void *xq, const void *xk, const void *xv,
                                  const float *conv_w, float eps, const void *g, const void *beta,
                                  const float *S0, float *o, float *ST, void *ws, hipStream_t s,
                                  const GateArgs *gate = nullptr);
size_t chunk_mfma_conv_workspace(const Shape &sh);

// The gated output norm over `rows` rows of dv channels: o fp32 -> y of yt,
// z of zt (same layout as o), gain fp32 [dv].  dv in {16, 32, 64, 128}.
hipError_t launch_output_gate(const float *o, const void *z, DType zt, const float *gain, float eps,
                              void *y, DType yt, long rows, int dv, hipStream_t s);

// Backward of the recurrence: dq, dk, dv, dg, dbeta, dS0 (fp32) from dO
// [B,T,Hv,dv] and dST (or null).  dk in {32, 64, 128}, dv a multiple of 32.
// Chunked, both gates: per chunk of 64 tokens, the state before it and the
// state gradient after it, U and E, T and P^T (the key-channel gate: also
// gamma [C][dk] and the decayed k and q) in the workspace, for the whole
// sequence or one segment of it at a time.  backward_workspace(sh, cap): the
// bytes of the fastest plan whose workspace fits in cap (the fewest segments;
// the smallest plan if none fits).  launch_backward runs the fastest plan
// that fits in ws_bytes.
size_t backward_workspace(const Shape &sh, size_t cap = ~(size_t)0);
hipError_t launch_backward(const Shape &sh, const void *q, const void *k, const void *v, const void *g,
                           const void *beta, const float *S0, const float *dO, const float *dST, float *dq,
                           float *dk, float *dv, float *dg, float *dbeta, float *dS0, void *ws, size_t ws_bytes,
                           hipStream_t st);

// Internal chunk length the fp32 kernels use for a requested chunk and dk.
int chunk_f32_internal(int chunk, int dk);

}  // namespace gdn
