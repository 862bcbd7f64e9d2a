// gdn_api.cpp -- the C ABI declared in include/gdn.h: argument validation on
// the host (before anything is enqueued) and dispatch to the kernel launchers.
#include "gdn.h"

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <atomic>
#include <string>

#include "gdn_launch.h"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

gdn_status ok() {
  g_last_error.clear();
  return GDN_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool is_dtype(int32_t t) { return t == GDN_F32 || t == GDN_BF16 || t == GDN_F16; }

size_t dsize(int32_t t) { return t == GDN_F32 ? 4 : 2; }

bool pow2_16_128(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

struct Range {
  uintptr_t lo, hi;
};
Range range(const void *p, size_t bytes) {
  return Range{(uintptr_t)p, (uintptr_t)p + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Tokens of all the sequences: B x T, or T for packed sequences.
size_t ntok(const gdn_desc *d, bool packed) { return packed ? (size_t)d->T : (size_t)d->B * d->T; }

// Checks common to every entry point; fills the launcher's shape.  packed: B
// sequences packed into T tokens.
gdn_status check_desc(const gdn_desc *d, gdn::Shape *sh, bool packed = false) {
  if (!d) return fail(GDN_E_ARG, "desc is NULL");
  if (d->B < 1 || d->T < 1 || d->Hk < 1 || d->Hv < 1 || d->dk < 1 || d->dv < 1)
    return fail(GDN_E_ARG, "B, T, Hk, Hv, dk, dv must be >= 1 (got %d %d %d %d %d %d)", d->B,
                d->T, d->Hk, d->Hv, d->dk, d->dv);
  if (!is_dtype(d->qkv_dtype) || !is_dtype(d->gate_dtype))
    return fail(GDN_E_ARG, "unknown dtype (qkv %d, gate %d)", d->qkv_dtype, d->gate_dtype);
  if (d->gate != GDN_GATE_HEAD && d->gate != GDN_GATE_KEY_CHANNEL)
    return fail(GDN_E_ARG, "unknown gate kind %d", d->gate);
  if (d->rule != GDN_RULE_DELTA && d->rule != GDN_RULE_NO_DELTA)
    return fail(GDN_E_ARG, "unknown update rule %d", d->rule);
  if (d->Hv % d->Hk != 0)
    return fail(GDN_E_SHAPE, "Hv (%d) must be a multiple of Hk (%d)", d->Hv, d->Hk);
  if (d->B > 65535 || d->Hv > 65535)
    return fail(GDN_E_UNSUPPORTED, "B and Hv must be <= 65535");
  // element counts must stay far from 64-bit overflow and kernel index limits
  const double n_big = (double)d->B * d->T * (double)(d->Hv > d->Hk ? d->Hv : d->Hk) *
                       (d->dv > d->dk ? d->dv : d->dk);
  if (n_big > 1e13) return fail(GDN_E_UNSUPPORTED, "problem too large");
  if (!packed && (double)d->B * d->T > 2147483647.0)
    return fail(GDN_E_UNSUPPORTED, "B * T too large");
  sh->B = d->B;
  sh->T = d->T;
  sh->Hk = d->Hk;
  sh->Hv = d->Hv;
  sh->dk = d->dk;
  sh->dv = d->dv;
  sh->chunk = d->chunk;
  sh->qkv = (gdn::DType)d->qkv_dtype;
  sh->gate_t = (gdn::DType)d->gate_dtype;
  sh->key_gate = d->gate == GDN_GATE_KEY_CHANNEL;
  sh->packed = packed;
  sh->no_delta = d->rule == GDN_RULE_NO_DELTA;
  return GDN_OK;
}

// The offsets of packed sequences: present and 4-byte aligned (their values
// are read on the device only).
gdn_status check_offsets(const int32_t *cu) {
  if (!cu) return fail(GDN_E_ARG, "cu_seqlens is NULL");
  if (((uintptr_t)cu & 3u) != 0) return fail(GDN_E_ALIGN, "cu_seqlens is not 4-byte aligned");
  return GDN_OK;
}

gdn_status check_ptrs(const char *const *names, const void *const *ptrs, int n) {
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i]) return fail(GDN_E_ARG, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(GDN_E_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  return GDN_OK;
}

// The matrix-core path: 16-bit q/k/v, either gate, dk = dv = 128, chunk 64.
bool uses_matrix_cores(const gdn_desc *d) {
  const bool mc_mode = (d->qkv_dtype == GDN_BF16 || d->qkv_dtype == GDN_F16) &&
                       (d->gate_dtype == GDN_BF16 || d->gate_dtype == GDN_F32);
  return mc_mode && d->dk == 128 && d->dv == 128 && d->chunk == 64;
}

gdn_status check_prologue_args(const gdn_desc *d, int32_t x_dtype, float eps);

gdn_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(GDN_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char *gdn_version(void) { return "gdn-gfx950 0.1.0"; }

const char *gdn_status_str(gdn_status s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_E_ARG: return "invalid argument";
    case GDN_E_SHAPE: return "inconsistent shapes";
    case GDN_E_UNSUPPORTED: return "unsupported configuration";
    case GDN_E_ALIGN: return "misaligned pointer";
    case GDN_E_WORKSPACE: return "workspace too small";
    case GDN_E_HIP: return "HIP error";
  }
  return "unknown status";
}

const char *gdn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {

gdn_status prologue_impl(const gdn_desc *d, const int32_t *cu, int32_t x_dtype, const void *xq,
                         const void *xk, const void *xv, const float *conv_w, float eps, void *q,
                         void *k, void *v, void *stream) {
  const bool packed = cu != nullptr;
  gdn::Shape sh;
  gdn_status st = check_desc(d, &sh, packed);
  if (st != GDN_OK) return st;
  if ((st = check_prologue_args(d, x_dtype, eps)) != GDN_OK) return st;
  const char *names[] = {"xq", "xk", "xv", "conv_w", "q", "k", "v"};
  const void *ptrs[] = {xq, xk, xv, conv_w, q, k, v};
  if ((st = check_ptrs(names, ptrs, 7)) != GDN_OK) return st;
  const size_t nqk = ntok(d, packed) * d->Hk * d->dk, nv = ntok(d, packed) * d->Hv * d->dv;
  const size_t xs = dsize(x_dtype), ys = dsize(d->qkv_dtype);
  const Range outs[] = {range(q, nqk * ys), range(k, nqk * ys), range(v, nv * ys)};
  if (packed)
    for (const Range &a : outs)
      if (overlap(a, range(cu, ((size_t)d->B + 1) * 4)))
        return fail(GDN_E_ARG, "prologue outputs must not overlap cu_seqlens");
  const Range ins[] = {range(xq, nqk * xs), range(xk, nqk * xs), range(xv, nv * xs),
                       range(conv_w, (2 * (size_t)d->Hk * d->dk + (size_t)d->Hv * d->dv) * 16)};
  for (const Range &a : outs)
    for (const Range &b : ins)
      if (overlap(a, b)) return fail(GDN_E_ARG, "prologue outputs must not overlap its inputs");
  if (overlap(outs[0], outs[1]) || overlap(outs[0], outs[2]) || overlap(outs[1], outs[2]))
    return fail(GDN_E_ARG, "prologue outputs must not overlap each other");

  hipError_t e = gdn::launch_prologue(xq, xk, xv, (gdn::DType)x_dtype, conv_w, q, k, v, sh.qkv, d->B,
                                      d->T, d->Hk, d->Hv, d->dk, d->dv, eps, (hipStream_t)stream, cu);
  return launched(e, "prologue launch");
}

}  // namespace

extern "C" {

gdn_status gdn_prologue(const gdn_desc *d, int32_t x_dtype, const void *xq, const void *xk,
                        const void *xv, const float *conv_w, float eps, void *q, void *k, void *v,
                        void *stream) {
  return prologue_impl(d, nullptr, x_dtype, xq, xk, xv, conv_w, eps, q, k, v, stream);
}

gdn_status gdn_prologue_varlen(const gdn_desc *d, const int32_t *cu_seqlens, int32_t x_dtype,
                               const void *xq, const void *xk, const void *xv, const float *conv_w,
                               float eps, void *q, void *k, void *v, void *stream) {
  const gdn_status st = check_offsets(cu_seqlens);
  if (st != GDN_OK) return st;
  return prologue_impl(d, cu_seqlens, x_dtype, xq, xk, xv, conv_w, eps, q, k, v, stream);
}

size_t gdn_fwd_workspace_bytes(const gdn_desc *d) {
  gdn::Shape sh;
  const std::string saved = g_last_error;  // a query does not change the last error
  const gdn_status st = check_desc(d, &sh);
  g_last_error = saved;
  if (st != GDN_OK) return 0;
  return uses_matrix_cores(d) ? gdn::chunk_mfma_workspace(sh) : 0;
}

size_t gdn_fwd_varlen_workspace_bytes(const gdn_desc *d) {
  gdn::Shape sh;
  const std::string saved = g_last_error;
  const gdn_status st = check_desc(d, &sh, true);
  g_last_error = saved;
  if (st != GDN_OK) return 0;
  return uses_matrix_cores(d) ? gdn::chunk_mfma_workspace(sh) : 0;
}

}  // extern "C"

namespace {

// Everything gdn_fwd_chunked checks, without launching.  `ws_need` is the
// workspace the chosen kernels need (the caller checks the one it passes).
gdn_status check_chunked(const gdn_desc *d, gdn::Shape *sh, bool *use_mfma_out, bool packed = false) {
  gdn_status st = check_desc(d, sh, packed);
  if (st != GDN_OK) return st;
  const bool fp32_mode = d->qkv_dtype == GDN_F32 && d->gate_dtype == GDN_F32;
  const bool mc_mode = (d->qkv_dtype == GDN_BF16 || d->qkv_dtype == GDN_F16) &&
                       (d->gate_dtype == GDN_BF16 || d->gate_dtype == GDN_F32);
  if (!fp32_mode && !mc_mode)
    return fail(GDN_E_UNSUPPORTED,
                "dtype combination not built (qkv %d, gate %d): use fp32/fp32, or bf16|fp16 with "
                "bf16|fp32 gates",
                d->qkv_dtype, d->gate_dtype);
  // 16-bit inputs run on the matrix cores at dk = dv = 128, chunk 64; the
  // key-channel gate at other sizes runs on the fp32 vector path.
  const bool use_mfma = uses_matrix_cores(d);
  if (mc_mode && !use_mfma && !sh->key_gate)
    return fail(GDN_E_UNSUPPORTED,
                "matrix-core mode supports dk = dv = 128 and chunk = 64 (got %d, %d, %d)", d->dk,
                d->dv, d->chunk);
  if (!use_mfma) {
    if (!pow2_16_128(d->dk) || !pow2_16_128(d->dv))
      return fail(GDN_E_UNSUPPORTED, "dk, dv must be in {16,32,64,128} (got %d, %d)", d->dk, d->dv);
    if (d->chunk != 16 && d->chunk != 32 && d->chunk != 64)
      return fail(GDN_E_UNSUPPORTED, "chunk must be 16, 32 or 64 (got %d)", d->chunk);
    if (fp32_mode && d->chunk * d->dk > 4096)
      return fail(GDN_E_UNSUPPORTED, "fp32 mode needs chunk * dk <= 4096 (got %d * %d)", d->chunk,
                  d->dk);
  }
  *use_mfma_out = use_mfma;
  return GDN_OK;
}

// Pointer checks of the chunked forward: ins are the ranges of q, k, v (or
// the raw inputs and taps of the convolution), g and beta.
gdn_status check_chunked_ptrs(const gdn_desc *d, const gdn::Shape &sh, const Range *ins, int nins,
                              const void *g, const void *beta, const float *S0, const void *o,
                              float *S_T, size_t o_bytes = 0) {
  const bool packed = sh.packed;
  const char *names[] = {"g", "beta", "o", "S_T"};
  const void *ptrs[] = {g, beta, o, S_T};
  gdn_status st = check_ptrs(names, ptrs, 4);
  if (st != GDN_OK) return st;
  if (S0 && !aligned16(S0)) return fail(GDN_E_ALIGN, "S0 is not 16-byte aligned");
  const size_t bt = ntok(d, packed);
  const size_t gs = dsize(d->gate_dtype);
  const size_t state_bytes = (size_t)d->B * d->Hv * d->dv * d->dk * 4;
  const Range ro = range(o, o_bytes ? o_bytes : bt * d->Hv * d->dv * 4);
  const Range rst = range(S_T, state_bytes);
  const Range rg = range(g, bt * d->Hv * (sh.key_gate ? d->dk : 1) * gs), rb = range(beta, bt * d->Hv * gs);
  for (int i = 0; i < nins + 2; ++i) {
    const Range &r = i < nins ? ins[i] : (i == nins ? rg : rb);
    if (overlap(ro, r)) return fail(GDN_E_ARG, "o must not overlap an input");
    if (overlap(rst, r)) return fail(GDN_E_ARG, "S_T must not overlap an input other than S0");
  }
  if (overlap(ro, rst)) return fail(GDN_E_ARG, "o must not overlap S_T");
  if (S0) {
    const Range rs0 = range(S0, state_bytes);
    if (overlap(ro, rs0)) return fail(GDN_E_ARG, "o must not overlap S0");
    if ((const void *)S0 != (const void *)S_T && overlap(rst, rs0))
      return fail(GDN_E_ARG, "S_T must be S0 itself or not overlap it");
  }
  return GDN_OK;
}

// The caller's workspace: large enough, aligned, and apart from every other
// argument.
gdn_status check_workspace(const gdn_desc *d, void *workspace, size_t workspace_bytes, size_t need,
                           const Range *ins, int nins, const void *g, const void *beta,
                           const float *S0, const void *o, float *S_T, bool key_gate,
                           size_t o_bytes = 0, bool packed = false) {
  if (workspace_bytes < need)
    return fail(GDN_E_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (need == 0) return GDN_OK;
  if (!workspace) return fail(GDN_E_ARG, "workspace is NULL");
  if (!aligned16(workspace)) return fail(GDN_E_ALIGN, "workspace is not 16-byte aligned");
  const size_t bt = ntok(d, packed), gs = dsize(d->gate_dtype);
  const size_t state_bytes = (size_t)d->B * d->Hv * d->dv * d->dk * 4;
  const Range rw = range(workspace, need);
  for (int i = 0; i < nins; ++i)
    if (overlap(rw, ins[i])) return fail(GDN_E_ARG, "workspace must not overlap an input");
  if (overlap(rw, range(g, bt * d->Hv * (key_gate ? d->dk : 1) * gs)) ||
      overlap(rw, range(beta, bt * d->Hv * gs)))
    return fail(GDN_E_ARG, "workspace must not overlap an input");
  if (overlap(rw, range(o, o_bytes ? o_bytes : bt * d->Hv * d->dv * 4)) ||
      overlap(rw, range(S_T, state_bytes)) ||
      (S0 && overlap(rw, range(S0, state_bytes))))
    return fail(GDN_E_ARG, "workspace must not overlap o, S0 or S_T");
  return GDN_OK;
}

// Everything gdn_prologue checks about its dtypes, sizes and eps.
gdn_status check_prologue_args(const gdn_desc *d, int32_t x_dtype, float eps) {
  if (x_dtype != GDN_BF16 && x_dtype != GDN_F32)
    return fail(x_dtype == GDN_F16 ? GDN_E_UNSUPPORTED : GDN_E_ARG,
                "prologue inputs must be bf16 or fp32 (got dtype %d)", x_dtype);
  if (!pow2_16_128(d->dk) || !pow2_16_128(d->dv))
    return fail(GDN_E_UNSUPPORTED, "prologue supports dk, dv in {16,32,64,128} (got %d, %d)",
                d->dk, d->dv);
  if (!(eps >= 0.f) || eps > 1.f) return fail(GDN_E_ARG, "eps must be in [0, 1]");
  return GDN_OK;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// The convolution runs inside the chunked kernels for bf16 raw inputs and
// fp16 q, k (the prologue's output type) on the matrix-core path with the
// per-head gate and the delta rule; otherwise the prologue writes q, k, v
// into the workspace first.
bool conv_fused(const gdn_desc *d, const gdn::Shape &sh, bool use_mfma, int32_t x_dtype) {
  return use_mfma && !sh.key_gate && !sh.no_delta && x_dtype == GDN_BF16 && d->qkv_dtype == GDN_F16;
}

size_t conv_workspace(const gdn_desc *d, const gdn::Shape &sh, bool use_mfma, int32_t x_dtype) {
  if (conv_fused(d, sh, use_mfma, x_dtype)) return gdn::chunk_mfma_conv_workspace(sh);
  const size_t ys = dsize(d->qkv_dtype);
  const size_t nqk = ntok(d, sh.packed) * d->Hk * d->dk, nv = ntok(d, sh.packed) * d->Hv * d->dv;
  return 2 * round256(nqk * ys) + round256(nv * ys) + (use_mfma ? gdn::chunk_mfma_workspace(sh) : 0);
}

// The prologue and the chunked forward after validation (the workspace holds
// conv_workspace(d, sh, use_mfma, x_dtype) bytes).
gdn_status run_chunked_conv(const gdn_desc *d, const gdn::Shape &sh, bool use_mfma, int32_t x_dtype,
                            const void *xq, const void *xk, const void *xv, const float *conv_w,
                            float eps, const void *g, const void *beta, const float *S0, float *o,
                            float *S_T, void *workspace, hipStream_t s) {
  if (conv_fused(d, sh, use_mfma, x_dtype))
    return launched(gdn::launch_chunk_mfma_conv(sh, xq, xk, xv, conv_w, eps, g, beta, S0, o, S_T,
                                                workspace, s),
                    "chunked forward with convolution launch");
  // the prologue into the workspace, then the chunked forward
  const size_t nqk = ntok(d, sh.packed) * d->Hk * d->dk, nv = ntok(d, sh.packed) * d->Hv * d->dv;
  const size_t ys = dsize(d->qkv_dtype);
  char *q = (char *)workspace, *k = q + round256(nqk * ys), *v = k + round256(nqk * ys);
  char *rest = v + round256(nv * ys);
  hipError_t e = gdn::launch_prologue(xq, xk, xv, (gdn::DType)x_dtype, conv_w, q, k, v, sh.qkv, d->B,
                                      d->T, d->Hk, d->Hv, d->dk, d->dv, eps, s, sh.cu);
  if (e != hipSuccess) return launched(e, "prologue launch");
  e = use_mfma ? gdn::launch_chunk_mfma(sh, q, k, v, g, beta, S0, o, S_T, rest, s)
               : gdn::launch_chunk_f32(sh, q, k, v, g, beta, S0, o, S_T, s);
  return launched(e, "chunked forward launch");
}

// The gated output norm inside the sequential pass: the prologue runs inside
// the chunked kernels, a workgroup holds a whole value head and y is 16-bit.
bool gate_inside(const gdn_desc *d, const gdn::Shape &sh, bool use_mfma, int32_t x_dtype,
                 int32_t y_dtype) {
  return conv_fused(d, sh, use_mfma, x_dtype) && gdn::chunk_mfma_gate_inside(sh) && y_dtype != GDN_F32;
}

size_t gated_workspace(const gdn_desc *d, const gdn::Shape &sh, bool use_mfma, int32_t x_dtype,
                       int32_t y_dtype) {
  if (gate_inside(d, sh, use_mfma, x_dtype, y_dtype)) return gdn::chunk_mfma_conv_workspace(sh);
  return round256(conv_workspace(d, sh, use_mfma, x_dtype)) +
         (size_t)d->B * d->T * d->Hv * d->dv * 4;   // then o
}

// Everything the gate checks about its sizes, dtypes and eps.
gdn_status check_gate_args(const gdn_desc *d, int32_t z_dtype, int32_t y_dtype, float eps) {
  if (!is_dtype(z_dtype) || !is_dtype(y_dtype))
    return fail(GDN_E_ARG, "unknown dtype (z %d, y %d)", z_dtype, y_dtype);
  if (!pow2_16_128(d->dv))
    return fail(GDN_E_UNSUPPORTED, "the output gate supports dv in {16,32,64,128} (got %d)", d->dv);
  if (!(eps >= 0.f) || eps > 1.f) return fail(GDN_E_ARG, "norm eps must be in [0, 1]");
  return GDN_OK;
}

}  // namespace

namespace {

// The workspace of gdn_fwd_chunked_noalloc: one copy per device, held by the
// code object from the time it is loaded on that device.  In host code
// `scratch` names a host-side stand-in, not device memory: its device address
// comes from hipGetSymbolAddress, looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The scratch's device address on the current device.  Two threads that
// race the first lookup on a device store the same address.
gdn_status scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GDN_E_HIP, "no current device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GDN_E_UNSUPPORTED, "device %d: the scratch is kept for devices 0..%d", dev, kMaxDevices - 1);
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(GDN_E_HIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return GDN_OK;
}

// gdn_fwd_chunked and its packed-sequence form (cu: device offsets, or null).
// noalloc: the workspace is the library's scratch (the workspace arguments
// are ignored) and every launch goes on the caller's stream.
gdn_status chunked_impl(const gdn_desc *d, const int32_t *cu, const void *q, const void *k, const void *v,
                        const void *g, const void *beta, const float *S0, float *o, float *S_T,
                        void *workspace, size_t workspace_bytes, void *stream, bool noalloc = false) {
  const bool packed = cu != nullptr;
  gdn::Shape sh;
  bool use_mfma = false;
  gdn_status st = check_chunked(d, &sh, &use_mfma, packed);
  if (st != GDN_OK) return st;
  const char *names[] = {"q", "k", "v"};
  const void *ptrs[] = {q, k, v};
  if ((st = check_ptrs(names, ptrs, 3)) != GDN_OK) return st;
  const size_t bt = ntok(d, packed), qs = dsize(d->qkv_dtype);
  const Range ins[] = {range(q, bt * d->Hk * d->dk * qs), range(k, bt * d->Hk * d->dk * qs),
                       range(v, bt * d->Hv * d->dv * qs), range(cu, ((size_t)d->B + 1) * 4)};
  const int nins = packed ? 4 : 3;
  if ((st = check_chunked_ptrs(d, sh, ins, nins, g, beta, S0, o, S_T)) != GDN_OK) return st;
  const size_t need = use_mfma ? gdn::chunk_mfma_workspace(sh) : 0;
  if (noalloc) {
    if (need > GDN_NOALLOC_SCRATCH_BYTES)
      return fail(GDN_E_WORKSPACE, "the problem needs %zu bytes of workspace; the no-allocation form "
                  "holds %zu", need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      if ((st = scratch_address(&workspace)) != GDN_OK) return st;
      workspace_bytes = GDN_NOALLOC_SCRATCH_BYTES;
    }
    sh.single_stream = true;
  }
  if ((st = check_workspace(d, workspace, workspace_bytes, need, ins, nins, g, beta, S0, o, S_T,
                            sh.key_gate, 0, packed)) != GDN_OK)
    return st;

  sh.cu = cu;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = use_mfma ? gdn::launch_chunk_mfma(sh, q, k, v, g, beta, S0, o, S_T, workspace, s)
                          : gdn::launch_chunk_f32(sh, q, k, v, g, beta, S0, o, S_T, s);
  return launched(e, "chunked forward launch");
}

// gdn_fwd_chunked_conv and its packed-sequence form.
gdn_status chunked_conv_impl(const gdn_desc *d, const int32_t *cu, int32_t x_dtype, const void *xq,
                             const void *xk, const void *xv, const float *conv_w, float eps,
                             const void *g, const void *beta, const float *S0, float *o, float *S_T,
                             void *workspace, size_t workspace_bytes, void *stream) {
  const bool packed = cu != nullptr;
  gdn::Shape sh;
  bool use_mfma = false;
  gdn_status st = check_chunked(d, &sh, &use_mfma, packed);
  if (st != GDN_OK) return st;
  if ((st = check_prologue_args(d, x_dtype, eps)) != GDN_OK) return st;
  const char *names[] = {"xq", "xk", "xv", "conv_w"};
  const void *ptrs[] = {xq, xk, xv, conv_w};
  if ((st = check_ptrs(names, ptrs, 4)) != GDN_OK) return st;
  const size_t nqk = ntok(d, packed) * d->Hk * d->dk, nv = ntok(d, packed) * d->Hv * d->dv;
  const size_t xs = dsize(x_dtype);
  const Range ins[] = {range(xq, nqk * xs), range(xk, nqk * xs), range(xv, nv * xs),
                       range(conv_w, (2 * (size_t)d->Hk * d->dk + (size_t)d->Hv * d->dv) * 16),
                       range(cu, ((size_t)d->B + 1) * 4)};
  const int nins = packed ? 5 : 4;
  if ((st = check_chunked_ptrs(d, sh, ins, nins, g, beta, S0, o, S_T)) != GDN_OK) return st;
  const size_t need = conv_workspace(d, sh, use_mfma, x_dtype);
  if ((st = check_workspace(d, workspace, workspace_bytes, need, ins, nins, g, beta, S0, o, S_T,
                            sh.key_gate, 0, packed)) != GDN_OK)
    return st;

  sh.cu = cu;
  return run_chunked_conv(d, sh, use_mfma, x_dtype, xq, xk, xv, conv_w, eps, g, beta, S0, o, S_T,
                          workspace, (hipStream_t)stream);
}

}  // namespace

extern "C" {

gdn_status gdn_fwd_chunked(const gdn_desc *d, const void *q, const void *k, const void *v,
                           const void *g, const void *beta, const float *S0, float *o, float *S_T,
                           void *workspace, size_t workspace_bytes, void *stream) {
  return chunked_impl(d, nullptr, q, k, v, g, beta, S0, o, S_T, workspace, workspace_bytes, stream);
}

gdn_status gdn_fwd_chunked_noalloc(const gdn_desc *d, const void *q, const void *k, const void *v,
                                   const void *g, const void *beta, const float *S0, float *o,
                                   float *S_T, void *stream) {
  return chunked_impl(d, nullptr, q, k, v, g, beta, S0, o, S_T, nullptr, 0, stream, true);
}

gdn_status gdn_fwd_chunked_varlen(const gdn_desc *d, const int32_t *cu_seqlens, const void *q,
                                  const void *k, const void *v, const void *g, const void *beta,
                                  const float *S0, float *o, float *S_T, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  const gdn_status st = check_offsets(cu_seqlens);
  if (st != GDN_OK) return st;
  return chunked_impl(d, cu_seqlens, q, k, v, g, beta, S0, o, S_T, workspace, workspace_bytes, stream);
}

size_t gdn_fwd_conv_workspace_bytes(const gdn_desc *d, int32_t x_dtype) {
  gdn::Shape sh;
  bool use_mfma = false;
  const std::string saved = g_last_error;  // a query does not change the last error
  gdn_status st = check_chunked(d, &sh, &use_mfma);
  if (st == GDN_OK) st = check_prologue_args(d, x_dtype, 0.f);
  g_last_error = saved;
  if (st != GDN_OK) return 0;
  return conv_workspace(d, sh, use_mfma, x_dtype);
}

size_t gdn_fwd_conv_varlen_workspace_bytes(const gdn_desc *d, int32_t x_dtype) {
  gdn::Shape sh;
  bool use_mfma = false;
  const std::string saved = g_last_error;
  gdn_status st = check_chunked(d, &sh, &use_mfma, true);
  if (st == GDN_OK) st = check_prologue_args(d, x_dtype, 0.f);
  g_last_error = saved;
  if (st != GDN_OK) return 0;
  return conv_workspace(d, sh, use_mfma, x_dtype);
}

gdn_status gdn_fwd_chunked_conv(const gdn_desc *d, int32_t x_dtype, const void *xq, const void *xk,
                                const void *xv, const float *conv_w, float eps, const void *g,
                                const void *beta, const float *S0, float *o, float *S_T,
                                void *workspace, size_t workspace_bytes, void *stream) {
  return chunked_conv_impl(d, nullptr, x_dtype, xq, xk, xv, conv_w, eps, g, beta, S0, o, S_T, workspace,
                           workspace_bytes, stream);
}

gdn_status gdn_fwd_chunked_conv_varlen(const gdn_desc *d, const int32_t *cu_seqlens, int32_t x_dtype,
                                       const void *xq, const void *xk, const void *xv,
                                       const float *conv_w, float eps, const void *g, const void *beta,
                                       const float *S0, float *o, float *S_T, void *workspace,
                                       size_t workspace_bytes, void *stream) {
  const gdn_status st = check_offsets(cu_seqlens);
  if (st != GDN_OK) return st;
  return chunked_conv_impl(d, cu_seqlens, x_dtype, xq, xk, xv, conv_w, eps, g, beta, S0, o, S_T,
                           workspace, workspace_bytes, stream);
}

gdn_status gdn_output_gate(const gdn_desc *d, const float *o, int32_t z_dtype, const void *z,
                           const float *gain, float eps, int32_t y_dtype, void *y, void *stream) {
  gdn::Shape sh;
  gdn_status st = check_desc(d, &sh);
  if (st != GDN_OK) return st;
  if ((st = check_gate_args(d, z_dtype, y_dtype, eps)) != GDN_OK) return st;
  const char *names[] = {"o", "z", "gain", "y"};
  const void *ptrs[] = {o, z, gain, y};
  if ((st = check_ptrs(names, ptrs, 4)) != GDN_OK) return st;
  const size_t n = (size_t)d->B * d->T * d->Hv * d->dv;
  const Range ry = range(y, n * dsize(y_dtype));
  if (overlap(ry, range(o, n * 4)) || overlap(ry, range(z, n * dsize(z_dtype))) ||
      overlap(ry, range(gain, (size_t)d->dv * 4)))
    return fail(GDN_E_ARG, "y must not overlap o, z or gain");
  return launched(gdn::launch_output_gate(o, z, (gdn::DType)z_dtype, gain, eps, y, (gdn::DType)y_dtype,
                                          (long)d->B * d->T * d->Hv, d->dv, (hipStream_t)stream),
                  "output gate launch");
}

size_t gdn_fwd_gated_workspace_bytes(const gdn_desc *d, int32_t x_dtype, int32_t y_dtype) {
  gdn::Shape sh;
  bool use_mfma = false;
  const std::string saved = g_last_error;  // a query does not change the last error
  gdn_status st = check_chunked(d, &sh, &use_mfma);
  if (st == GDN_OK) st = check_prologue_args(d, x_dtype, 0.f);
  if (st == GDN_OK) st = check_gate_args(d, x_dtype, y_dtype, 0.f);
  g_last_error = saved;
  if (st != GDN_OK) return 0;
  return gated_workspace(d, sh, use_mfma, x_dtype, y_dtype);
}

gdn_status gdn_fwd_chunked_conv_gated(const gdn_desc *d, int32_t x_dtype, const void *xq,
                                      const void *xk, const void *xv, const float *conv_w, float eps,
                                      const void *g, const void *beta, const float *S0,
                                      const void *z, const float *gain, float norm_eps,
                                      int32_t y_dtype, void *y, float *S_T, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  gdn::Shape sh;
  bool use_mfma = false;
  gdn_status st = check_chunked(d, &sh, &use_mfma);
  if (st != GDN_OK) return st;
  if ((st = check_prologue_args(d, x_dtype, eps)) != GDN_OK) return st;
  if ((st = check_gate_args(d, x_dtype, y_dtype, norm_eps)) != GDN_OK) return st;
  const char *names[] = {"xq", "xk", "xv", "conv_w", "z", "gain"};
  const void *ptrs[] = {xq, xk, xv, conv_w, z, gain};
  if ((st = check_ptrs(names, ptrs, 6)) != GDN_OK) return st;
  const size_t nqk = (size_t)d->B * d->T * d->Hk * d->dk, nv = (size_t)d->B * d->T * d->Hv * d->dv;
  const size_t xs = dsize(x_dtype);
  const Range ins[] = {range(xq, nqk * xs), range(xk, nqk * xs), range(xv, nv * xs),
                       range(conv_w, (2 * (size_t)d->Hk * d->dk + (size_t)d->Hv * d->dv) * 16),
                       range(z, nv * xs), range(gain, (size_t)d->dv * 4)};
  const size_t y_bytes = nv * dsize(y_dtype);
  if ((st = check_chunked_ptrs(d, sh, ins, 6, g, beta, S0, y, S_T, y_bytes)) != GDN_OK) return st;
  const size_t need = gated_workspace(d, sh, use_mfma, x_dtype, y_dtype);
  if ((st = check_workspace(d, workspace, workspace_bytes, need, ins, 6, g, beta, S0, y, S_T,
                            sh.key_gate, y_bytes)) != GDN_OK)
    return st;

  hipStream_t s = (hipStream_t)stream;
  if (gate_inside(d, sh, use_mfma, x_dtype, y_dtype)) {
    const gdn::GateArgs ga{z, gain, norm_eps, y, (gdn::DType)y_dtype};
    return launched(gdn::launch_chunk_mfma_conv(sh, xq, xk, xv, conv_w, eps, g, beta, S0, nullptr, S_T,
                                                workspace, s, &ga),
                    "gated chunked forward launch");
  }
  // o into the workspace after what the forward uses, then the gate
  float *o = (float *)((char *)workspace + round256(conv_workspace(d, sh, use_mfma, x_dtype)));
  if ((st = run_chunked_conv(d, sh, use_mfma, x_dtype, xq, xk, xv, conv_w, eps, g, beta, S0, o, S_T,
                             workspace, s)) != GDN_OK)
    return st;
  return launched(gdn::launch_output_gate(o, z, (gdn::DType)x_dtype, gain, norm_eps, y,
                                          (gdn::DType)y_dtype, (long)d->B * d->T * d->Hv, d->dv, s),
                  "output gate launch");
}

namespace {
// What the backward checks about the sizes and dtypes of d.
gdn_status check_bwd(const gdn_desc *d, gdn::Shape *sh) {
  gdn_status st = check_desc(d, sh);
  if (st != GDN_OK) return st;
  if (d->dk != 32 && d->dk != 64 && d->dk != 128)
    return fail(GDN_E_UNSUPPORTED, "the backward supports dk in {32,64,128} (got %d)", d->dk);
  if (d->dv % 32 != 0 || d->dv > 1024)
    return fail(GDN_E_UNSUPPORTED, "the backward supports dv a multiple of 32, <= 1024 (got %d)", d->dv);
  if (d->gate_dtype == GDN_F16) return fail(GDN_E_UNSUPPORTED, "the backward's gates must be fp32 or bf16");
  return GDN_OK;
}
}  // namespace

size_t gdn_bwd_workspace_bytes(const gdn_desc *d) {
  gdn::Shape sh;
  const std::string saved = g_last_error;
  const gdn_status st = check_bwd(d, &sh);
  g_last_error = saved;
  return st == GDN_OK ? gdn::backward_workspace(sh) : 0;
}

size_t gdn_bwd_workspace_bytes_within(const gdn_desc *d, size_t cap) {
  gdn::Shape sh;
  const std::string saved = g_last_error;
  const gdn_status st = check_bwd(d, &sh);
  g_last_error = saved;
  return st == GDN_OK ? gdn::backward_workspace(sh, cap) : 0;
}

gdn_status gdn_bwd(const gdn_desc *d, const void *q, const void *k, const void *v, const void *g,
                   const void *beta, const float *S0, const float *dO, const float *dS_T, float *dq,
                   float *dk, float *dv, float *dg, float *dbeta, float *dS0, void *workspace,
                   size_t workspace_bytes, void *stream) {
  gdn::Shape sh;
  gdn_status st = check_bwd(d, &sh);
  if (st != GDN_OK) return st;
  const char *names[] = {"q", "k", "v", "g", "beta", "dO", "dq", "dk", "dv", "dg", "dbeta", "dS0", "workspace"};
  const void *ptrs[] = {q, k, v, g, beta, dO, dq, dk, dv, dg, dbeta, dS0, workspace};
  if ((st = check_ptrs(names, ptrs, 13)) != GDN_OK) return st;
  if ((S0 && !aligned16(S0)) || (dS_T && !aligned16(dS_T)))
    return fail(GDN_E_ALIGN, "S0 and dS_T must be 16-byte aligned");
  // the fastest plan that fits in the workspace given; below the smallest plan it is too small
  const size_t need = gdn::backward_workspace(sh, workspace_bytes);
  if (workspace_bytes < need)
    return fail(GDN_E_WORKSPACE, "workspace needs at least %zu bytes, got %zu", need, workspace_bytes);
  const size_t bt = (size_t)d->B * d->T, qs = dsize(d->qkv_dtype), gs = dsize(d->gate_dtype);
  const size_t gdim = sh.key_gate ? d->dk : 1, sb = (size_t)d->B * d->Hv * d->dv * d->dk * 4;
  const Range ins[] = {range(q, bt * d->Hk * d->dk * qs), range(k, bt * d->Hk * d->dk * qs),
                       range(v, bt * d->Hv * d->dv * qs), range(g, bt * d->Hv * gdim * gs),
                       range(beta, bt * d->Hv * gs), range(S0, S0 ? sb : 0), range(dO, bt * d->Hv * d->dv * 4),
                       range(dS_T, dS_T ? sb : 0)};
  const Range outs[] = {range(dq, bt * d->Hk * d->dk * 4), range(dk, bt * d->Hk * d->dk * 4),
                        range(dv, bt * d->Hv * d->dv * 4), range(dg, bt * d->Hv * gdim * 4),
                        range(dbeta, bt * d->Hv * 4), range(dS0, sb), range(workspace, need)};
  for (int i = 0; i < 7; ++i) {
    for (const Range &r : ins)
      if (overlap(outs[i], r)) return fail(GDN_E_ARG, "outputs and workspace must not overlap the inputs");
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i], outs[j])) return fail(GDN_E_ARG, "outputs and workspace must not overlap each other");
  }
  return launched(gdn::launch_backward(sh, q, k, v, g, beta, S0, dO, dS_T, dq, dk, dv, dg, dbeta, dS0, workspace,
                                       workspace_bytes, (hipStream_t)stream),
                  "backward launch");
}

size_t gdn_decode_conv_workspace_bytes(const gdn_desc *d) {
  gdn::Shape sh;
  const std::string saved = g_last_error;
  const gdn_status st = check_desc(d, &sh);
  g_last_error = saved;
  if (st != GDN_OK) return 0;
  const size_t qs = dsize(d->qkv_dtype);
  return 2 * round256((size_t)d->B * d->Hk * d->dk * qs) + round256((size_t)d->B * d->Hv * d->dv * qs);
}

gdn_status gdn_decode_step_conv(const gdn_desc *d, int32_t x_dtype, const void *xq, const void *xk,
                                const void *xv, const float *conv_w, float eps, void *conv_state,
                                const void *g, const void *beta, float *S, float *o, void *workspace,
                                size_t workspace_bytes, void *stream) {
  gdn::Shape sh;
  gdn_status st = check_desc(d, &sh);
  if (st != GDN_OK) return st;
  if (d->T != 1) return fail(GDN_E_SHAPE, "decode step needs T == 1 (got %d)", d->T);
  if ((st = check_prologue_args(d, x_dtype, eps)) != GDN_OK) return st;
  const char *names[] = {"xq", "xk", "xv", "conv_w", "conv_state", "workspace"};
  const void *ptrs[] = {xq, xk, xv, conv_w, conv_state, workspace};
  if ((st = check_ptrs(names, ptrs, 6)) != GDN_OK) return st;
  const size_t need = gdn_decode_conv_workspace_bytes(d);
  if (workspace_bytes < need)
    return fail(GDN_E_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  const size_t xs = dsize(x_dtype), nch = 2 * (size_t)d->Hk * d->dk + (size_t)d->Hv * d->dv;
  const Range rcs = range(conv_state, (size_t)d->B * 3 * nch * xs), rw = range(workspace, need);
  const Range ins[] = {range(xq, (size_t)d->B * d->Hk * d->dk * xs), range(xk, (size_t)d->B * d->Hk * d->dk * xs),
                       range(xv, (size_t)d->B * d->Hv * d->dv * xs), range(conv_w, nch * 16),
                       range(g, (size_t)d->B * d->Hv * (sh.key_gate ? d->dk : 1) * dsize(d->gate_dtype)),
                       range(beta, (size_t)d->B * d->Hv * dsize(d->gate_dtype)),
                       range(S, (size_t)d->B * d->Hv * d->dv * d->dk * 4), range(o, (size_t)d->B * d->Hv * d->dv * 4)};
  for (const Range &r : ins)
    if (overlap(rcs, r) || overlap(rw, r))
      return fail(GDN_E_ARG, "conv_state and the workspace must not overlap another argument");
  if (overlap(rcs, rw)) return fail(GDN_E_ARG, "conv_state must not overlap the workspace");
  // q, k, v of the token into the workspace, then the decode step on them
  const size_t qs = dsize(d->qkv_dtype);
  char *q = (char *)workspace, *k = q + round256((size_t)d->B * d->Hk * d->dk * qs);
  char *v = k + round256((size_t)d->B * d->Hk * d->dk * qs);
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = gdn::launch_decode_prologue(xq, xk, xv, (gdn::DType)x_dtype, conv_w, conv_state, q, k, v,
                                                   sh.qkv, d->B, d->Hk, d->Hv, d->dk, d->dv, eps, s);
  if (e != hipSuccess) return launched(e, "decode prologue launch");
  return gdn_decode_step(d, q, k, v, g, beta, S, o, stream);
}

gdn_status gdn_conv_state(const gdn_desc *d, const int32_t *cu_seqlens, int32_t x_dtype, const void *xq,
                          const void *xk, const void *xv, void *conv_state, void *stream) {
  const bool packed = cu_seqlens != nullptr;
  gdn::Shape sh;
  gdn_status st = check_desc(d, &sh, packed);
  if (st != GDN_OK) return st;
  if ((st = check_prologue_args(d, x_dtype, 0.f)) != GDN_OK) return st;
  const char *names[] = {"xq", "xk", "xv", "conv_state"};
  const void *ptrs[] = {xq, xk, xv, conv_state};
  if ((st = check_ptrs(names, ptrs, 4)) != GDN_OK) return st;
  if (packed && ((uintptr_t)cu_seqlens & 3u) != 0) return fail(GDN_E_ALIGN, "cu_seqlens is not 4-byte aligned");
  const size_t xs = dsize(x_dtype), nt = ntok(d, packed);
  const Range rcs = range(conv_state, (size_t)d->B * 3 * (2 * (size_t)d->Hk * d->dk + (size_t)d->Hv * d->dv) * xs);
  if (overlap(rcs, range(xq, nt * d->Hk * d->dk * xs)) || overlap(rcs, range(xk, nt * d->Hk * d->dk * xs)) ||
      overlap(rcs, range(xv, nt * d->Hv * d->dv * xs)) ||
      (packed && overlap(rcs, range(cu_seqlens, ((size_t)d->B + 1) * 4))))
    return fail(GDN_E_ARG, "conv_state must not overlap an input");
  return launched(gdn::launch_conv_state(xq, xk, xv, (gdn::DType)x_dtype, conv_state, d->B, d->T, d->Hk, d->Hv,
                                         d->dk, d->dv, cu_seqlens, (hipStream_t)stream),
                  "conv state launch");
}

gdn_status gdn_decode_step(const gdn_desc *d, const void *q, const void *k, const void *v,
                           const void *g, const void *beta, float *S, float *o, void *stream) {
  gdn::Shape sh;
  gdn_status st = check_desc(d, &sh);
  if (st != GDN_OK) return st;
  if (d->T != 1) return fail(GDN_E_SHAPE, "decode step needs T == 1 (got %d)", d->T);
  if (!pow2_16_128(d->dk))
    return fail(GDN_E_UNSUPPORTED, "decode supports dk in {16,32,64,128} (got %d)", d->dk);
  if (d->dv % 16 != 0 || d->dv > 1024)
    return fail(GDN_E_UNSUPPORTED, "decode supports dv a multiple of 16, <= 1024 (got %d)", d->dv);
  if (d->gate_dtype == GDN_F16)
    return fail(GDN_E_UNSUPPORTED, "decode gates must be fp32 or bf16");
  const char *names[] = {"q", "k", "v", "g", "beta", "S", "o"};
  const void *ptrs[] = {q, k, v, g, beta, S, o};
  if ((st = check_ptrs(names, ptrs, 7)) != GDN_OK) return st;
  const size_t qs = dsize(d->qkv_dtype), gs = dsize(d->gate_dtype);
  const Range rS = range(S, (size_t)d->B * d->Hv * d->dv * d->dk * 4);
  const Range ro = range(o, (size_t)d->B * d->Hv * d->dv * 4);
  const Range ins[] = {range(q, (size_t)d->B * d->Hk * d->dk * qs),
                       range(k, (size_t)d->B * d->Hk * d->dk * qs),
                       range(v, (size_t)d->B * d->Hv * d->dv * qs),
                       range(g, (size_t)d->B * d->Hv * (sh.key_gate ? d->dk : 1) * gs),
                       range(beta, (size_t)d->B * d->Hv * gs)};
  for (const Range &r : ins)
    if (overlap(rS, r) || overlap(ro, r)) return fail(GDN_E_ARG, "S and o must not overlap inputs");
  if (overlap(rS, ro)) return fail(GDN_E_ARG, "S and o must not overlap");
  return launched(gdn::launch_decode(sh, q, k, v, g, beta, S, o, (hipStream_t)stream),
                  "decode launch");
}

}  // extern "C"
