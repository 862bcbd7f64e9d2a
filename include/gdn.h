/*
 * gdn.h -- C ABI of the Gated DeltaNet forward library for AMD Instinct MI355X
 * (gfx950).  Every operation runs as hand-written HIP kernels on the caller's
 * stream; the library never allocates or frees device memory.
 *
 * The method (the pages are cited by title and section):
 *   "Source notes" (NextTransformer methods), section "Linear attention",
 *   row gdn: per (batch, value head) a state S updated token by token with a
 *   scalar decay applied before the delta update; row kda: the same with a
 *   per-key-channel decay; row deltanet: causal conv + SiLU and L2-normalised
 *   q/k in front, read y = q^T S after the write.  Section "Backend and
 *   numerical limits": query scale 1; fp32 carry and accumulation.
 *   "Frontier model atlas", entries 03 and 08 (Gated DeltaNet): four-token
 *   causal convolution; 16 key heads shared by 48 value heads.
 *
 * Here the state of one (batch b, value head h) is S in R^{dv x dk} (the
 * transpose of the pages' K x V state), and for t = 1..T
 *
 *     S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T
 *         = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * with alpha_t = exp(g_t) (g is the natural-log decay), key/query head
 * h / (Hv / Hk) for value head h, and, for the per-key-channel gate,
 * alpha_t S_{t-1} replaced by S_{t-1} diag(exp(g_t)).
 *
 * Conventions shared by every entry point
 *  - Pointers marked "device" are device pointers, caller-owned, contiguous,
 *    16-byte aligned; they are read-only unless marked out / in-out.
 *  - Layouts are token-major: q, k [B,T,Hk,dk]; v [B,T,Hv,dv];
 *    g [B,T,Hv] (head gate) or [B,T,Hv,dk] (key-channel gate);
 *    beta [B,T,Hv]; o [B,T,Hv,dv]; states [B,Hv,dv,dk] fp32, dk contiguous.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous: they enqueue kernels and return; nothing synchronises.
 *  - Errors: arguments are validated first, on the host, before anything is
 *    enqueued; an invalid call returns a non-zero status and writes nothing.
 *    A failed launch returns GDN_E_HIP.  A fault inside a kernel surfaces at
 *    the caller's next synchronisation.  gdn_last_error() gives a message
 *    for the last failing call on the calling thread.
 *  - The library keeps no state between calls except that per-thread message
 *    and, per device, a pool of internal streams and events: a chunked call
 *    may run part of its work on one of them, ordered by events with the
 *    caller's stream (a fork and join, also under stream capture).  The pool
 *    holds one entry per concurrently running call and lives until the
 *    process ends.  Calls on different streams may run concurrently.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_E_ARG = 1,         /* null pointer, non-positive size, unknown enum value */
  GDN_E_SHAPE = 2,       /* inconsistent shapes, e.g. Hv not a multiple of Hk */
  GDN_E_UNSUPPORTED = 3, /* valid but not built: head dim, chunk, dtype combination */
  GDN_E_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  GDN_E_WORKSPACE = 5,   /* workspace smaller than gdn_fwd_workspace_bytes() */
  GDN_E_HIP = 6          /* a HIP launch failed */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1, GDN_F16 = 2 } gdn_dtype;

typedef enum {
  GDN_GATE_HEAD = 0,       /* g [B,T,Hv]: one decay per (token, value head) */
  GDN_GATE_KEY_CHANNEL = 1 /* g [B,T,Hv,dk]: one decay per key channel */
} gdn_gate;

typedef enum {
  GDN_RULE_DELTA = 0,   /* the gated delta rule above */
  GDN_RULE_NO_DELTA = 1 /* without the delta correction: S_t = alpha_t S_{t-1} + beta_t v_t k_t^T
                           (per-key-channel gate: S_{t-1} diag(alpha_t)); the "SinkProbe" page's
                           hybrid_nodelta layer, the "Source notes" gla row's update.  Supported by
                           the forward, decode and backward entry points, either gate. */
} gdn_rule;

/* Problem description shared by all entry points. */
typedef struct gdn_desc {
  int32_t B;          /* batch (independent sequences), >= 1 */
  int32_t T;          /* tokens per sequence, >= 1 (1 for gdn_decode_step) */
  int32_t Hk;         /* key/query heads, >= 1 */
  int32_t Hv;         /* value heads, a multiple of Hk */
  int32_t dk;         /* key head dim */
  int32_t dv;         /* value head dim */
  int32_t chunk;      /* tokens per chunk of gdn_fwd_chunked (a tuning choice; the
                         result does not depend on it beyond rounding) */
  int32_t qkv_dtype;  /* gdn_dtype of q, k, v (and of the prologue's outputs) */
  int32_t gate_dtype; /* gdn_dtype of g and beta */
  int32_t gate;       /* gdn_gate */
  int32_t rule;       /* gdn_rule (0, the gated delta rule, when zero-initialised) */
} gdn_desc;

/*
 * gdn_prologue -- 4-tap causal depthwise convolution, SiLU, and L2
 * normalisation of q and k ("Source notes", Linear attention, rows deltanet
 * and kda: causal conv + SiLU, L2-normalised Q/K; "Frontier model atlas"
 * entries 03/08: four-token causal convolution).
 *
 * For every channel c of the concatenation (q | k | v) and token t:
 *     y_t = sum_{j=0..3} conv_w[c][j] * x_{t-3+j}   (x_{t'} = 0 for t' < 0)
 *     z_t = y_t * sigmoid(y_t)
 * then each (token, head) row of q and of k is divided by
 * sqrt(sum z^2 + eps).  Tap 3 multiplies the current token.  There is no
 * bias and no carry between calls (every sequence starts from zeros).
 *
 *   xq, xk  device [B,T,Hk,dk]  x_dtype (GDN_BF16 or GDN_F32)
 *   xv      device [B,T,Hv,dv]  x_dtype
 *   conv_w  device fp32 [Hk*dk (q) + Hk*dk (k) + Hv*dv (v)][4]
 *   q, k    device out [B,T,Hk,dk]  d->qkv_dtype (GDN_F16, GDN_BF16 or GDN_F32)
 *   v       device out [B,T,Hv,dv]  d->qkv_dtype
 * Supported: dk, dv in {16, 32, 64, 128}.  d->chunk, gate and gate_dtype are
 * not used.  Outputs must not alias inputs.
 */
gdn_status gdn_prologue(const gdn_desc *d, int32_t x_dtype, const void *xq,
                        const void *xk, const void *xv, const float *conv_w,
                        float eps, void *q, void *k, void *v, void *stream);

/*
 * Device workspace bytes gdn_fwd_chunked needs for `d` (0 = none; then the
 * workspace pointer may be NULL).  The matrix-core path (16-bit q/k/v,
 * dk = dv = 128, chunk 64) keeps per (batch, value head, 64-token chunk):
 *   head gate: the triangular inverse (a 64 x 64 lower-triangular fp16
 *     matrix) and five fp32 values per token (cumulative log decay and the
 *     factors made from it): 7424 bytes; with at most 64 (batch, value
 *     head) pairs, also the decayed masked q.k products as high and low
 *     fp16 parts (two more 64 x 64 lower-triangular matrices): 19712 bytes;
 *   key-channel gate: the inverse, the decayed masked q.k products (another
 *     64 x 64 lower-triangular fp16 matrix), the decayed k, q and the
 *     state-update k (64 x 128 fp16 each), beta and the chunk's total decay:
 *     62208 bytes.
 * Returns 0 for an invalid description.  The caller owns the workspace; it
 * is scratch between calls and must not be shared by concurrent calls.
 */
size_t gdn_fwd_workspace_bytes(const gdn_desc *d);

/*
 * gdn_fwd_chunked -- the forward pass over T tokens from an entering state,
 * computed chunk by chunk (chunkwise-exact form; the attention-sink study page,
 * "SinkProbe", states that the chunkwise and token-by-token forms agree).
 *
 *   q, k   device [B,T,Hk,dk]  qkv_dtype      v device [B,T,Hv,dv] qkv_dtype
 *   g      device [B,T,Hv] or [B,T,Hv,dk] (per d->gate)  gate_dtype, natural log, < 0
 *   beta   device [B,T,Hv]  gate_dtype, in [0, 1]
 *   S0     device fp32 [B,Hv,dv,dk], or NULL for a zero entering state
 *   o      device out fp32 [B,T,Hv,dv]
 *   S_T    device out fp32 [B,Hv,dv,dk]: the state after token T; may be the
 *          same pointer as S0 (updated in place), must not overlap it otherwise
 *   workspace   device scratch of at least gdn_fwd_workspace_bytes(d) bytes,
 *               16-byte aligned, not overlapping any other argument
 *               (GDN_E_WORKSPACE if too small)
 *
 * Supported combinations:
 *  - fp32 mode (qkv_dtype = gate_dtype = GDN_F32): fp32 arithmetic throughout;
 *    dk, dv in {16, 32, 64, 128}; chunk in {16, 32, 64} with
 *    chunk * dk <= 4096; either gate.
 *  - matrix-core mode (qkv_dtype GDN_BF16 or GDN_F16; gate_dtype GDN_BF16 or
 *    GDN_F32): dk = dv = 128, chunk = 64, either gate.  Products run on the
 *    gfx950 fp16 matrix cores with fp32 accumulation; the state is carried in
 *    fp32.  Both the per-head and the per-key-channel gate run on the matrix
 *    cores at these sizes; the fp32 kernels serve only the other sizes (and
 *    16-bit inputs at them).  Operands are narrowed to fp16, so bf16 inputs
 *    must lie in fp16's range: a magnitude above 65504 becomes infinite and
 *    one below 2^-24 becomes zero (q and k are unit rows, and v and the state
 *    of the workloads here are far inside that range); the call does not
 *    check the values.
 * o must not alias any input.
 */
gdn_status gdn_fwd_chunked(const gdn_desc *d, const void *q, const void *k,
                           const void *v, const void *g, const void *beta,
                           const float *S0, float *o, float *S_T,
                           void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * gdn_fwd_chunked_noalloc -- gdn_fwd_chunked without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, hosts that forbid it).
 *
 * The chunk matrices live in a scratch array that the library's code object
 * holds on each device, GDN_NOALLOC_SCRATCH_BYTES bytes, made when the
 * library is loaded on that device and kept until the process ends.  The
 * call allocates nothing (no device memory, no streams or events: all work
 * runs on `stream`), and gives bit for bit the results of gdn_fwd_chunked
 * with the same arguments.
 *
 *   d, q, k, v, g, beta, S0, o, S_T, stream   as for gdn_fwd_chunked
 * Errors: as gdn_fwd_chunked; GDN_E_WORKSPACE when gdn_fwd_workspace_bytes(d)
 * exceeds GDN_NOALLOC_SCRATCH_BYTES (head gate: at most 18078 (batch, value
 * head, 64-token chunk) triples, e.g. B 4, Hv 48, T 4096, and at most 6808
 * with at most 64 (batch, value head) pairs, e.g. B 1, Hv 48, T 8192;
 * key-channel gate: at most 2157); GDN_E_HIP when the scratch address cannot be obtained on
 * the current device.  Nothing in the scratch needs to start at zero.
 * Every call on one device shares that device's scratch: calls that overlap
 * in time on one device (on different streams, or from several threads
 * without ordering) race and give wrong results.  Calls on one stream are
 * ordered and safe.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gdn_status gdn_fwd_chunked_noalloc(const gdn_desc *d, const void *q, const void *k,
                                   const void *v, const void *g, const void *beta,
                                   const float *S0, float *o, float *S_T, void *stream);

/*
 * gdn_fwd_chunked_conv -- the prologue and the chunked forward in one call:
 * what gdn_prologue(d, x_dtype, xq, xk, xv, conv_w, eps) into q, k, v of
 * d->qkv_dtype followed by gdn_fwd_chunked(d, q, k, v, g, beta, S0) computes,
 * without q, k, v as arguments.
 * For bf16 raw inputs, fp16 d->qkv_dtype, the per-head gate and the delta
 * rule on the matrix-core path the convolution runs inside the chunked
 * kernels: q and k are made once per (chunk, key head), rounded to fp16 and
 * kept in the workspace; v is made as the sequential pass loads it and stays
 * fp32 (it is not rounded to fp16 and never goes through memory), so this
 * form is slightly more accurate than the two calls and not bit-identical to
 * them.  Any other supported combination runs the prologue into the
 * workspace first and gives the two calls' results bit for bit.
 *
 *   x_dtype, xq, xk, xv, conv_w, eps   as for gdn_prologue
 *   g, beta, S0, o, S_T                as for gdn_fwd_chunked
 *   workspace   device scratch of at least gdn_fwd_conv_workspace_bytes(d,
 *               x_dtype) bytes, 16-byte aligned, not overlapping any other
 *               argument (GDN_E_WORKSPACE if too small)
 * Supported: what both gdn_prologue and gdn_fwd_chunked support for d.
 */
size_t gdn_fwd_conv_workspace_bytes(const gdn_desc *d, int32_t x_dtype);
gdn_status gdn_fwd_chunked_conv(const gdn_desc *d, int32_t x_dtype, const void *xq,
                                const void *xk, const void *xv, const float *conv_w,
                                float eps, const void *g, const void *beta,
                                const float *S0, float *o, float *S_T, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Packed sequences of different lengths ("_varlen" entry points): the same
 * operations over B sequences stored one after another along one token axis
 * of T tokens, sequence s being tokens cu_seqlens[s] .. cu_seqlens[s+1] - 1.
 * Each sequence is computed on its own, exactly as a call with that sequence
 * alone would compute it: its own entering state S0[s] (or zero), its own
 * chunks (a chunk never spans two sequences), convolution history zero before
 * its first token, its own S_T[s].
 *
 *   d->B        the number of sequences (<= 65535); d->T the total tokens
 *   cu_seqlens  device int32 [B + 1]: 0 = cu[0] <= cu[1] <= ... <= cu[B] = T;
 *               empty sequences are allowed (their S_T is their S0, or zero)
 *   token-major tensors (q, k, v, g, beta, o, raw inputs) have the layouts
 *               above with the batch dimension removed: q [T,Hk,dk], o [T,Hv,dv], ...
 *   S0, S_T     [B,Hv,dv,dk] as above, one state per sequence
 * The offsets are read on the device, so the host checks only that the
 * pointer is present and 4-byte aligned.  Each offset is clamped to [0, T]
 * and a sequence whose end precedes its start is read as empty: offsets that
 * break the rule above give unspecified results but no access outside the
 * arguments.  Supported: what the fixed-length entry point supports; the
 * workspace sizes are those of the _varlen queries (beside the chunk
 * matrices, the workspace holds the sequences' order by chunk count, the
 * longest first, which only decides the order in which the work is started).
 */
gdn_status gdn_prologue_varlen(const gdn_desc *d, const int32_t *cu_seqlens, int32_t x_dtype,
                               const void *xq, const void *xk, const void *xv,
                               const float *conv_w, float eps, void *q, void *k, void *v,
                               void *stream);
size_t gdn_fwd_varlen_workspace_bytes(const gdn_desc *d);
gdn_status gdn_fwd_chunked_varlen(const gdn_desc *d, const int32_t *cu_seqlens, const void *q,
                                  const void *k, const void *v, const void *g,
                                  const void *beta, const float *S0, float *o, float *S_T,
                                  void *workspace, size_t workspace_bytes, void *stream);
size_t gdn_fwd_conv_varlen_workspace_bytes(const gdn_desc *d, int32_t x_dtype);
gdn_status gdn_fwd_chunked_conv_varlen(const gdn_desc *d, const int32_t *cu_seqlens,
                                       int32_t x_dtype, const void *xq, const void *xk,
                                       const void *xv, const float *conv_w, float eps,
                                       const void *g, const void *beta, const float *S0,
                                       float *o, float *S_T, void *workspace,
                                       size_t workspace_bytes, void *stream);

/*
 * gdn_output_gate -- the gated output norm that follows the state read in a
 * Gated DeltaNet layer ("Source notes", Linear attention, row gdn: the
 * read-out is RMS-normalised, scaled by a learned gain and multiplied by a
 * SiLU gate; "Adopt vs. port", entry burn-rmsnorm, for the RMS norm: divide
 * by the square root of the mean of squares plus eps, multiply by the gain).
 * For every (batch, token, value head) row of dv channels:
 *     y_c = o_c / sqrt((1/dv) sum_c' o_c'^2 + eps) * gain_c * z_c sigmoid(z_c)
 *
 *   o      device fp32 [B,T,Hv,dv] (as gdn_fwd_chunked writes it)
 *   z      device [B,T,Hv,dv] z_dtype (GDN_F32, GDN_BF16 or GDN_F16): the gate
 *   gain   device fp32 [dv], the same for every value head
 *   eps    in [0, 1]
 *   y      device out [B,T,Hv,dv] y_dtype (GDN_F32, GDN_BF16 or GDN_F16),
 *          rounded to nearest even; must not overlap o, z or gain
 * d->Hk, dk, chunk, the dtypes and the gate kind must form a valid
 * description but are not used.  Supported: dv in {16, 32, 64, 128}.
 */
gdn_status gdn_output_gate(const gdn_desc *d, const float *o, int32_t z_dtype,
                           const void *z, const float *gain, float eps,
                           int32_t y_dtype, void *y, void *stream);

/*
 * gdn_fwd_chunked_conv_gated -- gdn_fwd_chunked_conv followed by
 * gdn_output_gate, without o as an argument: the same results (the same
 * arithmetic, roundings and order of the row sums) as
 *     gdn_fwd_chunked_conv(d, x_dtype, xq, xk, xv, conv_w, eps, g, beta, S0, o, S_T)
 *     gdn_output_gate(d, o, x_dtype, z, gain, norm_eps, y_dtype, y).
 * When the convolution runs inside the chunked kernels (bf16 raw inputs,
 * fp16 d->qkv_dtype, matrix-core path, per-head gate), B * Hv > 128 (a workgroup of the
 * sequential pass then holds a whole value head) and y is 16-bit, the gate
 * is applied there and o never goes through memory; otherwise o is kept in
 * the workspace and the gate runs after the forward.
 *
 *   x_dtype, xq, xk, xv, conv_w, eps   as for gdn_fwd_chunked_conv
 *   g, beta, S0, S_T                   as for gdn_fwd_chunked
 *   z      device [B,T,Hv,dv] x_dtype (the gate, like the raw projections)
 *   gain, norm_eps, y_dtype, y         as gain, eps, y_dtype, y of gdn_output_gate;
 *          y must not overlap any other argument
 *   workspace   device scratch of at least gdn_fwd_gated_workspace_bytes(d,
 *               x_dtype, y_dtype) bytes, 16-byte aligned, not overlapping any other
 *               argument (GDN_E_WORKSPACE if too small)
 * Supported: what gdn_fwd_chunked_conv and gdn_output_gate support for d.
 */
size_t gdn_fwd_gated_workspace_bytes(const gdn_desc *d, int32_t x_dtype, int32_t y_dtype);
gdn_status gdn_fwd_chunked_conv_gated(const gdn_desc *d, int32_t x_dtype, const void *xq,
                                      const void *xk, const void *xv, const float *conv_w,
                                      float eps, const void *g, const void *beta,
                                      const float *S0, const void *z, const float *gain,
                                      float norm_eps, int32_t y_dtype, void *y, float *S_T,
                                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_decode_step -- one token per sequence: the recurrence above with T = 1,
 * the state updated in place.  For state row i (old values S_i, decayed
 * row D_i = alpha S_i, or S_i o alpha for the key-channel gate):
 *     u_i = beta (v_i - D_i . k);   S_i <- D_i + u_i k;   o_i = D_i . q + u_i (k . q)
 *
 *   d->T must be 1; d->chunk is not used.
 *   q, k   device [B,Hk,dk] qkv_dtype (GDN_F32, GDN_BF16 or GDN_F16)
 *   v      device [B,Hv,dv] qkv_dtype
 *   g      device [B,Hv] or [B,Hv,dk]  gate_dtype (GDN_F32 or GDN_BF16)
 *   beta   device [B,Hv] gate_dtype
 *   S      device in-out fp32 [B,Hv,dv,dk]
 *   o      device out fp32 [B,Hv,dv]
 * Supported: dk in {16, 32, 64, 128}; dv a multiple of 16, <= 1024.
 */
gdn_status gdn_decode_step(const gdn_desc *d, const void *q, const void *k,
                           const void *v, const void *g, const void *beta,
                           float *S, float *o, void *stream);

/*
 * The convolution history, so that decode continues a prefill with the
 * convolution prologue ("Source notes", Linear attention, rows deltanet and
 * kda: causal conv in front of the state update; "Frontier model atlas"
 * entries 03/08: a four-token causal convolution, so three tokens of
 * history).  conv_state holds, per sequence, the raw inputs of its last three
 * tokens, oldest first, for every channel of q | k | v:
 *     conv_state [B][3][2 Hk dk + Hv dv]  x_dtype, channels in the order of conv_w
 *
 * gdn_conv_state -- the history after the last token of each sequence (zero
 * before a sequence's first token).  With cu_seqlens NULL the raw inputs are
 * [B,T,...]; otherwise packed sequences as for the _varlen entry points.
 *   conv_state  device out; must not overlap the inputs
 * Supported: dk, dv in {16, 32, 64, 128}; x_dtype GDN_BF16 or GDN_F32.
 */
gdn_status gdn_conv_state(const gdn_desc *d, const int32_t *cu_seqlens, int32_t x_dtype,
                          const void *xq, const void *xk, const void *xv, void *conv_state,
                          void *stream);

/*
 * gdn_decode_step_conv -- one decode step from raw inputs: q, k, v of the new
 * token are made exactly as gdn_prologue makes them (the same arithmetic and
 * rounding to d->qkv_dtype) from conv_state and the token, conv_state moves
 * on by one token in place, then gdn_decode_step runs on them.
 *   d->T must be 1.
 *   xq, xk      device [B,Hk,dk]  x_dtype;  xv device [B,Hv,dv] x_dtype
 *   conv_w, eps as for gdn_prologue
 *   conv_state  device in-out [B][3][2 Hk dk + Hv dv] x_dtype
 *   g, beta, S, o as for gdn_decode_step
 *   workspace   device scratch of gdn_decode_conv_workspace_bytes(d) bytes
 *               (q, k, v of the token), 16-byte aligned
 * Supported: what gdn_prologue and gdn_decode_step support for d.
 */
size_t gdn_decode_conv_workspace_bytes(const gdn_desc *d);
gdn_status gdn_decode_step_conv(const gdn_desc *d, int32_t x_dtype, const void *xq,
                                const void *xk, const void *xv, const float *conv_w, float eps,
                                void *conv_state, const void *g, const void *beta, float *S,
                                float *o, void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_bwd -- the backward of the recurrence: the gradients of
 * L = sum_t <dO_t, o_t> + <dS_T, S_T> with respect to q, k, v, g, beta and S0
 * (the first-order backward of "Source notes", Linear attention, row kda).
 * In chunks of 64 tokens (the exact chunkwise form of the "SinkProbe" page),
 * both gates.  A forward pass keeps the state before every chunk and the
 * chunk's U = (I + A)^-1 X; a backward pass runs the state gradient over the
 * chunks in reverse, keeping it after every chunk with E = (I + A)^-T dU; the
 * other gradients are then products of these per chunk, on the fp32 matrix
 * cores.  The chunked form assumes decays (g <= 0): factors e^(gamma_i -
 * gamma_j) with i >= j stay <= 1.  With the per-key-channel gate every decay
 * acts channel by channel; the masked products over a chunk's tokens are
 * taken in 16-token blocks, through a reference token between the two off
 * the diagonal and term by term on it, so no factor exceeds 1 however strong
 * the decay.  All arithmetic is fp32.
 *   q, k, v, g, beta, S0   the forward's inputs, as for gdn_fwd_chunked (S0 NULL: zeros)
 *   dO     device fp32 [B,T,Hv,dv]: the gradient of o
 *   dS_T   device fp32 [B,Hv,dv,dk] or NULL (zeros): the gradient of S_T
 *   dq, dk device out fp32 [B,T,Hk,dk] (summed over the value heads of a key head)
 *   dv     device out fp32 [B,T,Hv,dv]
 *   dg     device out fp32, g's shape ([B,T,Hv] or [B,T,Hv,dk]), the gradient of g = ln alpha
 *   dbeta  device out fp32 [B,T,Hv]
 *   dS0    device out fp32 [B,Hv,dv,dk]
 *   workspace   device scratch, 16-byte aligned, of workspace_bytes bytes.
 *     The call runs the fastest plan whose workspace fits in workspace_bytes.
 *     gdn_bwd_workspace_bytes(d) is the fastest plan's (one segment): per
 *     (batch, value head, chunk of 64) 2 (64 64 + 64 + dv dk + 64 dv) fp32
 *     with the per-head gate; the per-key-channel gate keeps gamma as
 *     [64][dk] in place of [64], and K o e^gamma, Q o e^gamma and
 *     K o e^(gamma_C - gamma), [64][dk] each, too.  With less, the sequence
 *     runs in segments of consecutive chunks, last segment first: T, gamma
 *     and beta (and the decayed k and q) are kept for every chunk (64 64 +
 *     2 64 fp32 per (batch, value head, chunk) with the per-head gate), the
 *     other arrays (64 64 + 2 dv dk + 2 64 dv fp32) for one segment's chunks,
 *     and the state at each segment start (B Hv dv dk fp32 per segment).  A
 *     forward pass over the chunks before the last segment keeps those
 *     states, and each segment runs its own forward pass again, so fewer
 *     bytes cost time (at B 4, T 4096, 48 value heads, d 128: 4.4 ms with
 *     2.82 GB, 5.2 ms with 0.91 GB in four segments).
 *     gdn_bwd_workspace_bytes_within(d, cap) is the workspace of the fewest
 *     segments that fit in cap, or the smallest plan's if none does; the call
 *     fails with GDN_E_WORKSPACE below that smallest size.
 * Outputs and workspace must not overlap each other or the inputs.
 * Supported: dk in {32, 64, 128}; dv a multiple of 32, <= 1024; q, k, v fp32,
 * bf16 or fp16; g and beta fp32 or bf16; either gate; d->chunk is not used;
 * d->rule either rule (without the delta correction A = 0, so T = I and
 * X = beta V).
 */
size_t gdn_bwd_workspace_bytes(const gdn_desc *d);
size_t gdn_bwd_workspace_bytes_within(const gdn_desc *d, size_t cap);
gdn_status gdn_bwd(const gdn_desc *d, const void *q, const void *k, const void *v, const void *g,
                   const void *beta, const float *S0, const float *dO, const float *dS_T, float *dq,
                   float *dk, float *dv, float *dg, float *dbeta, float *dS0, void *workspace,
                   size_t workspace_bytes, void *stream);

/* Static text for a status code. */
const char *gdn_status_str(gdn_status s);

/* Message for the last failing call on this thread ("" if none). */
const char *gdn_last_error(void);

/* Library version string. */
const char *gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
