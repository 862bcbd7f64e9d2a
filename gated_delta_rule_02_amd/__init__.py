"""Gated DeltaNet forward pass on AMD Instinct MI355X (gfx950).

Python binding of ``libgdn.so`` (the C ABI of ``include/gdn.h``).  This module
only marshals arguments: it checks that tensors are contiguous device tensors
of the expected shapes, passes their device pointers and the current HIP
stream to the library, and turns a non-zero status into ``GdnError``.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback of any kind.  PyTorch provides device memory and streams.

Entry points (same names as the C functions):
  prologue(xq, xk, xv, conv_w, out_dtype, eps) -> (q, k, v)
  fwd_chunked(q, k, v, g, beta, S0, chunk) -> (o, S_T)
  fwd_chunked_conv(xq, xk, xv, conv_w, g, beta, S0, qkv_dtype, eps, chunk) -> (o, S_T)
  decode_step(q, k, v, g, beta, S) -> o          (S updated in place)
  output_gate(o, z, gain, eps, out_dtype) -> y
  prologue_varlen, fwd_chunked_varlen, fwd_chunked_conv_varlen: packed sequences
      of different lengths (token tensors [1,T,...], cu_seqlens int32 [N+1])
  conv_state(xq, xk, xv, cu_seqlens=None) -> conv_state [B,3,channels]
  decode_step_conv(xq, xk, xv, conv_w, conv_state, g, beta, S) -> o   (conv_state, S in place)
  bwd(q, k, v, g, beta, S0, dO, dS_T) -> dict of dq, dk, dv, dg, dbeta, dS0 (fp32)
  fwd_chunked_conv_gated(xq, xk, xv, conv_w, g, beta, z, gain, S0, ...) -> (y, S_T)
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_LIBRARY names another build of the same library (the sanitizer tests load
# one built with host AddressSanitizer and UBSan)
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(HERE, "libgdn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "gdn.h")
NOALLOC_SCRATCH_BYTES = 128 << 20   # GDN_NOALLOC_SCRATCH_BYTES

F32, BF16, F16 = 0, 1, 2
GATE_HEAD, GATE_KEY_CHANNEL = 0, 1
STATUS = {0: "GDN_OK", 1: "GDN_E_ARG", 2: "GDN_E_SHAPE", 3: "GDN_E_UNSUPPORTED",
          4: "GDN_E_ALIGN", 5: "GDN_E_WORKSPACE", 6: "GDN_E_HIP"}

_DTYPE_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


class GdnDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "T", "Hk", "Hv", "dk", "dv", "chunk", "qkv_dtype", "gate_dtype", "gate", "rule")]


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgdn.so is not built: run __graft_entry__.build() "
                               "(or python gated_delta_rule_02_amd/_build.py)")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        D = ctypes.POINTER(GdnDesc)
        L.gdn_prologue.argtypes = [D, I, P, P, P, P, ctypes.c_float, P, P, P, P]
        L.gdn_prologue.restype = I
        L.gdn_fwd_workspace_bytes.argtypes = [D]
        L.gdn_fwd_workspace_bytes.restype = S
        L.gdn_fwd_chunked.argtypes = [D, P, P, P, P, P, P, P, P, P, S, P]
        L.gdn_fwd_chunked.restype = I
        L.gdn_fwd_chunked_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P]
        L.gdn_fwd_chunked_noalloc.restype = I
        L.gdn_fwd_conv_workspace_bytes.argtypes = [D, I]
        L.gdn_fwd_conv_workspace_bytes.restype = S
        L.gdn_fwd_chunked_conv.argtypes = [D, I, P, P, P, P, ctypes.c_float, P, P, P, P, P, P, S, P]
        L.gdn_fwd_chunked_conv.restype = I
        L.gdn_prologue_varlen.argtypes = [D, P, I, P, P, P, P, ctypes.c_float, P, P, P, P]
        L.gdn_prologue_varlen.restype = I
        L.gdn_fwd_varlen_workspace_bytes.argtypes = [D]
        L.gdn_fwd_varlen_workspace_bytes.restype = S
        L.gdn_fwd_chunked_varlen.argtypes = [D, P, P, P, P, P, P, P, P, P, P, S, P]
        L.gdn_fwd_chunked_varlen.restype = I
        L.gdn_fwd_conv_varlen_workspace_bytes.argtypes = [D, I]
        L.gdn_fwd_conv_varlen_workspace_bytes.restype = S
        L.gdn_fwd_chunked_conv_varlen.argtypes = [D, P, I, P, P, P, P, ctypes.c_float, P, P, P, P, P, P, S, P]
        L.gdn_fwd_chunked_conv_varlen.restype = I
        L.gdn_conv_state.argtypes = [D, P, I, P, P, P, P, P]
        L.gdn_conv_state.restype = I
        L.gdn_decode_conv_workspace_bytes.argtypes = [D]
        L.gdn_decode_conv_workspace_bytes.restype = S
        L.gdn_decode_step_conv.argtypes = [D, I, P, P, P, P, ctypes.c_float, P, P, P, P, P, P, S, P]
        L.gdn_decode_step_conv.restype = I
        L.gdn_bwd_workspace_bytes.argtypes = [D]
        L.gdn_bwd_workspace_bytes.restype = S
        L.gdn_bwd_workspace_bytes_within.argtypes = [D, S]
        L.gdn_bwd_workspace_bytes_within.restype = S
        L.gdn_bwd.argtypes = [D] + [P] * 15 + [S, P]
        L.gdn_bwd.restype = I
        L.gdn_output_gate.argtypes = [D, P, I, P, P, ctypes.c_float, I, P, P]
        L.gdn_output_gate.restype = I
        L.gdn_fwd_gated_workspace_bytes.argtypes = [D, I, I]
        L.gdn_fwd_gated_workspace_bytes.restype = S
        L.gdn_fwd_chunked_conv_gated.argtypes = [D, I, P, P, P, P, ctypes.c_float, P, P, P, P, P,
                                                 ctypes.c_float, I, P, P, P, S, P]
        L.gdn_fwd_chunked_conv_gated.restype = I
        L.gdn_decode_step.argtypes = [D, P, P, P, P, P, P, P, P]
        L.gdn_decode_step.restype = I
        L.gdn_status_str.argtypes = [I]
        L.gdn_status_str.restype = ctypes.c_char_p
        L.gdn_last_error.argtypes = []
        L.gdn_last_error.restype = ctypes.c_char_p
        L.gdn_version.argtypes = []
        L.gdn_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/gdn.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(gdn_[a-z_]+)\s*\(", text, flags=re.M)


def check(status: int) -> None:
    if status != 0:
        raise GdnError(status, lib().gdn_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(name, t, shape=None, dtypes=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError("%s has dtype %s" % (name, t.dtype))
    return t


RULE_DELTA, RULE_NO_DELTA = 0, 1

_poison = False


def poison_workspace(on: bool = True) -> None:
    """Fill every workspace this module allocates with 0xFF bytes before the
    call (NaN as fp16 and fp32, -1 as int32), so that a kernel that reads
    workspace memory it has not written first produces NaN instead of stale
    values.  A testing aid; off by default."""
    global _poison
    _poison = bool(on)


def _workspace(nbytes, device):
    if not nbytes:
        return None
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if _poison:
        ws.fill_(0xFF)
    return ws


def make_desc(B, T, Hk, Hv, dk, dv, chunk, qkv_dtype, gate_dtype, gate, rule=RULE_DELTA) -> GdnDesc:
    return GdnDesc(B, T, Hk, Hv, dk, dv, chunk, qkv_dtype, gate_dtype, gate, rule)


def prologue(xq, xk, xv, conv_w, out_dtype=torch.float16, eps=1e-6, stream=None):
    """4-tap causal conv + SiLU over q|k|v, then L2 normalisation of q and k rows.

    xq, xk [B,T,Hk,dk], xv [B,T,Hv,dv] (bf16 or fp32); conv_w fp32
    [2*Hk*dk + Hv*dv, 4].  Returns new tensors q, k, v in out_dtype.
    """
    B, T, Hk, dk = xq.shape
    Hv, dv = xv.shape[2], xv.shape[3]
    _dev("xq", xq, (B, T, Hk, dk))
    _dev("xk", xk, (B, T, Hk, dk), (xq.dtype,))
    _dev("xv", xv, (B, T, Hv, dv), (xq.dtype,))
    _dev("conv_w", conv_w, (2 * Hk * dk + Hv * dv, 4), (torch.float32,))
    q = torch.empty((B, T, Hk, dk), dtype=out_dtype, device=xq.device)
    k = torch.empty_like(q)
    v = torch.empty((B, T, Hv, dv), dtype=out_dtype, device=xq.device)
    d = make_desc(B, T, Hk, Hv, dk, dv, 64, _DTYPE_CODE[out_dtype], F32, GATE_HEAD)
    check(lib().gdn_prologue(ctypes.byref(d), _DTYPE_CODE[xq.dtype], _ptr(xq), _ptr(xk), _ptr(xv),
                             _ptr(conv_w), float(eps), _ptr(q), _ptr(k), _ptr(v), _stream(stream)))
    return q, k, v


def _gate_kind(g, B, T, Hv, dk):
    if tuple(g.shape) == (B, T, Hv):
        return GATE_HEAD
    if tuple(g.shape) == (B, T, Hv, dk):
        return GATE_KEY_CHANNEL
    raise ValueError("g must be [B,T,Hv] or [B,T,Hv,dk], got %s" % (tuple(g.shape),))


def fwd_chunked(q, k, v, g, beta, S0=None, chunk=64, o=None, S_T=None, stream=None, delta=True):
    """Chunked forward over T tokens.  q, k [B,T,Hk,dk]; v [B,T,Hv,dv];
    g [B,T,Hv] or [B,T,Hv,dk]; beta [B,T,Hv]; S0 fp32 [B,Hv,dv,dk] or None.
    Returns (o fp32 [B,T,Hv,dv], S_T fp32 [B,Hv,dv,dk]); S_T may be S0.
    delta=False: the update without the delta correction."""
    d, o, S_T = _chunked_args(q, k, v, g, beta, S0, chunk, o, S_T, delta)
    L = lib()
    ws_bytes = L.gdn_fwd_workspace_bytes(ctypes.byref(d))
    ws = _workspace(ws_bytes, q.device)
    check(L.gdn_fwd_chunked(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                            _ptr(S0), _ptr(o), _ptr(S_T), _ptr(ws), ws_bytes, _stream(stream)))
    return o, S_T


def fwd_chunked_noalloc(q, k, v, g, beta, S0=None, chunk=64, o=None, S_T=None, stream=None, delta=True):
    """fwd_chunked through gdn_fwd_chunked_noalloc: no workspace argument (the
    library's per-device scratch, GDN_NOALLOC_SCRATCH_BYTES, holds the chunk
    matrices).  With o and S_T given, nothing is allocated."""
    d, o, S_T = _chunked_args(q, k, v, g, beta, S0, chunk, o, S_T, delta)
    check(lib().gdn_fwd_chunked_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                        _ptr(S0), _ptr(o), _ptr(S_T), _stream(stream)))
    return o, S_T


def _chunked_args(q, k, v, g, beta, S0, chunk, o, S_T, delta):
    """Checks of the chunked forward's tensors; the description and the outputs."""
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    _dev("q", q)
    _dev("k", k, q.shape, (q.dtype,))
    _dev("v", v, (B, T, Hv, dv), (q.dtype,))
    gate = _gate_kind(_dev("g", g), B, T, Hv, dk)
    _dev("beta", beta, (B, T, Hv), (g.dtype,))
    if S0 is not None:
        _dev("S0", S0, (B, Hv, dv, dk), (torch.float32,))
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=torch.float32, device=q.device)
    if S_T is None:
        S_T = torch.empty((B, Hv, dv, dk), dtype=torch.float32, device=q.device)
    _dev("o", o, (B, T, Hv, dv), (torch.float32,))
    _dev("S_T", S_T, (B, Hv, dv, dk), (torch.float32,))
    d = make_desc(B, T, Hk, Hv, dk, dv, chunk, _DTYPE_CODE[q.dtype], _DTYPE_CODE[g.dtype], gate,
                  RULE_DELTA if delta else RULE_NO_DELTA)
    return d, o, S_T


def fwd_chunked_conv(xq, xk, xv, conv_w, g, beta, S0=None, qkv_dtype=torch.float16, eps=1e-6,
                     chunk=64, o=None, S_T=None, stream=None, delta=True):
    """prologue(xq, xk, xv, conv_w, qkv_dtype, eps) then fwd_chunked, in one call
    (q, k, v are not returned).  Returns (o, S_T)."""
    B, T, Hk, dk = xq.shape
    Hv, dv = xv.shape[2], xv.shape[3]
    _dev("xq", xq, (B, T, Hk, dk))
    _dev("xk", xk, (B, T, Hk, dk), (xq.dtype,))
    _dev("xv", xv, (B, T, Hv, dv), (xq.dtype,))
    _dev("conv_w", conv_w, (2 * Hk * dk + Hv * dv, 4), (torch.float32,))
    gate = _gate_kind(_dev("g", g), B, T, Hv, dk)
    _dev("beta", beta, (B, T, Hv), (g.dtype,))
    if S0 is not None:
        _dev("S0", S0, (B, Hv, dv, dk), (torch.float32,))
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=torch.float32, device=xq.device)
    if S_T is None:
        S_T = torch.empty((B, Hv, dv, dk), dtype=torch.float32, device=xq.device)
    _dev("o", o, (B, T, Hv, dv), (torch.float32,))
    _dev("S_T", S_T, (B, Hv, dv, dk), (torch.float32,))
    d = make_desc(B, T, Hk, Hv, dk, dv, chunk, _DTYPE_CODE[qkv_dtype], _DTYPE_CODE[g.dtype], gate,
                  RULE_DELTA if delta else RULE_NO_DELTA)
    L = lib()
    xt = _DTYPE_CODE[xq.dtype]
    ws_bytes = L.gdn_fwd_conv_workspace_bytes(ctypes.byref(d), xt)
    ws = _workspace(ws_bytes, xq.device)
    check(L.gdn_fwd_chunked_conv(ctypes.byref(d), xt, _ptr(xq), _ptr(xk), _ptr(xv), _ptr(conv_w),
                                 float(eps), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T),
                                 _ptr(ws), ws_bytes, _stream(stream)))
    return o, S_T


def output_gate(o, z, gain, eps=1e-5, out_dtype=torch.bfloat16, y=None, stream=None):
    """Gated output norm of every (token, value head) row of o (fp32 [B,T,Hv,dv]):
    y = o / sqrt(mean(o^2) + eps) * gain * silu(z).  z [B,T,Hv,dv] (fp32, bf16
    or fp16), gain fp32 [dv].  Returns y in out_dtype."""
    B, T, Hv, dv = o.shape
    _dev("o", o, None, (torch.float32,))
    _dev("z", z, o.shape, tuple(_DTYPE_CODE))
    _dev("gain", gain, (dv,), (torch.float32,))
    if y is None:
        y = torch.empty(o.shape, dtype=out_dtype, device=o.device)
    _dev("y", y, o.shape, tuple(_DTYPE_CODE))
    d = make_desc(B, T, 1, Hv, 16, dv, 64, F32, F32, GATE_HEAD)
    check(lib().gdn_output_gate(ctypes.byref(d), _ptr(o), _DTYPE_CODE[z.dtype], _ptr(z), _ptr(gain),
                                float(eps), _DTYPE_CODE[y.dtype], _ptr(y), _stream(stream)))
    return y


def fwd_chunked_conv_gated(xq, xk, xv, conv_w, g, beta, z, gain, S0=None, qkv_dtype=torch.float16,
                           eps=1e-6, norm_eps=1e-5, out_dtype=torch.bfloat16, chunk=64, y=None,
                           S_T=None, stream=None):
    """fwd_chunked_conv followed by output_gate(o, z, gain, norm_eps) in one call
    (o is not returned).  z [B,T,Hv,dv] in the raw inputs' dtype.  Returns (y, S_T)."""
    B, T, Hk, dk = xq.shape
    Hv, dv = xv.shape[2], xv.shape[3]
    _dev("xq", xq, (B, T, Hk, dk))
    _dev("xk", xk, (B, T, Hk, dk), (xq.dtype,))
    _dev("xv", xv, (B, T, Hv, dv), (xq.dtype,))
    _dev("conv_w", conv_w, (2 * Hk * dk + Hv * dv, 4), (torch.float32,))
    gate = _gate_kind(_dev("g", g), B, T, Hv, dk)
    _dev("beta", beta, (B, T, Hv), (g.dtype,))
    _dev("z", z, (B, T, Hv, dv), (xq.dtype,))
    _dev("gain", gain, (dv,), (torch.float32,))
    if S0 is not None:
        _dev("S0", S0, (B, Hv, dv, dk), (torch.float32,))
    if y is None:
        y = torch.empty((B, T, Hv, dv), dtype=out_dtype, device=xq.device)
    if S_T is None:
        S_T = torch.empty((B, Hv, dv, dk), dtype=torch.float32, device=xq.device)
    _dev("y", y, (B, T, Hv, dv), tuple(_DTYPE_CODE))
    _dev("S_T", S_T, (B, Hv, dv, dk), (torch.float32,))
    d = make_desc(B, T, Hk, Hv, dk, dv, chunk, _DTYPE_CODE[qkv_dtype], _DTYPE_CODE[g.dtype], gate)
    L = lib()
    xt = _DTYPE_CODE[xq.dtype]
    ws_bytes = L.gdn_fwd_gated_workspace_bytes(ctypes.byref(d), xt, _DTYPE_CODE[y.dtype])
    ws = _workspace(ws_bytes, xq.device)
    check(L.gdn_fwd_chunked_conv_gated(ctypes.byref(d), xt, _ptr(xq), _ptr(xk), _ptr(xv), _ptr(conv_w),
                                       float(eps), _ptr(g), _ptr(beta), _ptr(S0), _ptr(z), _ptr(gain),
                                       float(norm_eps), _DTYPE_CODE[y.dtype], _ptr(y), _ptr(S_T),
                                       _ptr(ws), ws_bytes, _stream(stream)))
    return y, S_T


def _offsets(cu_seqlens, T):
    _dev("cu_seqlens", cu_seqlens, None, (torch.int32,))
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be int32 [N+1] with N >= 1")
    return cu_seqlens.numel() - 1


def prologue_varlen(xq, xk, xv, conv_w, cu_seqlens, out_dtype=torch.float16, eps=1e-6, stream=None):
    """prologue over packed sequences: xq, xk [1,T,Hk,dk], xv [1,T,Hv,dv];
    the convolution history is zero before each sequence's first token."""
    _, T, Hk, dk = xq.shape
    Hv, dv = xv.shape[2], xv.shape[3]
    N = _offsets(cu_seqlens, T)
    _dev("xq", xq, (1, T, Hk, dk))
    _dev("xk", xk, (1, T, Hk, dk), (xq.dtype,))
    _dev("xv", xv, (1, T, Hv, dv), (xq.dtype,))
    _dev("conv_w", conv_w, (2 * Hk * dk + Hv * dv, 4), (torch.float32,))
    q = torch.empty((1, T, Hk, dk), dtype=out_dtype, device=xq.device)
    k = torch.empty_like(q)
    v = torch.empty((1, T, Hv, dv), dtype=out_dtype, device=xq.device)
    d = make_desc(N, T, Hk, Hv, dk, dv, 64, _DTYPE_CODE[out_dtype], F32, GATE_HEAD)
    check(lib().gdn_prologue_varlen(ctypes.byref(d), _ptr(cu_seqlens), _DTYPE_CODE[xq.dtype], _ptr(xq),
                                    _ptr(xk), _ptr(xv), _ptr(conv_w), float(eps), _ptr(q), _ptr(k), _ptr(v),
                                    _stream(stream)))
    return q, k, v


def fwd_chunked_varlen(q, k, v, g, beta, cu_seqlens, S0=None, chunk=64, o=None, S_T=None, stream=None,
                       delta=True):
    """fwd_chunked over packed sequences: q, k [1,T,Hk,dk]; v [1,T,Hv,dv];
    g [1,T,Hv] or [1,T,Hv,dk]; beta [1,T,Hv]; cu_seqlens int32 [N+1];
    S0 fp32 [N,Hv,dv,dk] or None.  Returns (o [1,T,Hv,dv], S_T [N,Hv,dv,dk])."""
    _, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    N = _offsets(cu_seqlens, T)
    _dev("q", q, (1, T, Hk, dk))
    _dev("k", k, q.shape, (q.dtype,))
    _dev("v", v, (1, T, Hv, dv), (q.dtype,))
    gate = _gate_kind(_dev("g", g), 1, T, Hv, dk)
    _dev("beta", beta, (1, T, Hv), (g.dtype,))
    if S0 is not None:
        _dev("S0", S0, (N, Hv, dv, dk), (torch.float32,))
    if o is None:
        o = torch.empty((1, T, Hv, dv), dtype=torch.float32, device=q.device)
    if S_T is None:
        S_T = torch.empty((N, Hv, dv, dk), dtype=torch.float32, device=q.device)
    _dev("o", o, (1, T, Hv, dv), (torch.float32,))
    _dev("S_T", S_T, (N, Hv, dv, dk), (torch.float32,))
    d = make_desc(N, T, Hk, Hv, dk, dv, chunk, _DTYPE_CODE[q.dtype], _DTYPE_CODE[g.dtype], gate,
                  RULE_DELTA if delta else RULE_NO_DELTA)
    L = lib()
    ws_bytes = L.gdn_fwd_varlen_workspace_bytes(ctypes.byref(d))
    ws = _workspace(ws_bytes, q.device)
    check(L.gdn_fwd_chunked_varlen(ctypes.byref(d), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T), _ptr(ws), ws_bytes,
                                   _stream(stream)))
    return o, S_T


def fwd_chunked_conv_varlen(xq, xk, xv, conv_w, g, beta, cu_seqlens, S0=None, qkv_dtype=torch.float16,
                            eps=1e-6, chunk=64, o=None, S_T=None, stream=None):
    """prologue_varlen then fwd_chunked_varlen in one call.  Returns (o, S_T)."""
    _, T, Hk, dk = xq.shape
    Hv, dv = xv.shape[2], xv.shape[3]
    N = _offsets(cu_seqlens, T)
    _dev("xq", xq, (1, T, Hk, dk))
    _dev("xk", xk, (1, T, Hk, dk), (xq.dtype,))
    _dev("xv", xv, (1, T, Hv, dv), (xq.dtype,))
    _dev("conv_w", conv_w, (2 * Hk * dk + Hv * dv, 4), (torch.float32,))
    gate = _gate_kind(_dev("g", g), 1, T, Hv, dk)
    _dev("beta", beta, (1, T, Hv), (g.dtype,))
    if S0 is not None:
        _dev("S0", S0, (N, Hv, dv, dk), (torch.float32,))
    if o is None:
        o = torch.empty((1, T, Hv, dv), dtype=torch.float32, device=xq.device)
    if S_T is None:
        S_T = torch.empty((N, Hv, dv, dk), dtype=torch.float32, device=xq.device)
    _dev("o", o, (1, T, Hv, dv), (torch.float32,))
    _dev("S_T", S_T, (N, Hv, dv, dk), (torch.float32,))
    d = make_desc(N, T, Hk, Hv, dk, dv, chunk, _DTYPE_CODE[qkv_dtype], _DTYPE_CODE[g.dtype], gate)
    L = lib()
    xt = _DTYPE_CODE[xq.dtype]
    ws_bytes = L.gdn_fwd_conv_varlen_workspace_bytes(ctypes.byref(d), xt)
    ws = _workspace(ws_bytes, xq.device)
    check(L.gdn_fwd_chunked_conv_varlen(ctypes.byref(d), _ptr(cu_seqlens), xt, _ptr(xq), _ptr(xk), _ptr(xv),
                                        _ptr(conv_w), float(eps), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o),
                                        _ptr(S_T), _ptr(ws), ws_bytes, _stream(stream)))
    return o, S_T


def conv_state(xq, xk, xv, cu_seqlens=None, stream=None):
    """The convolution history after each sequence's last token: the raw inputs
    of its last three tokens (zero before its first), [B,3,2*Hk*dk+Hv*dv] in the
    raw dtype.  xq, xk [B,T,Hk,dk], xv [B,T,Hv,dv]; or packed sequences
    ([1,T,...] with cu_seqlens int32 [B+1])."""
    Bx, T, Hk, dk = xq.shape
    Hv, dv = xv.shape[2], xv.shape[3]
    _dev("xq", xq)
    _dev("xk", xk, xq.shape, (xq.dtype,))
    _dev("xv", xv, (Bx, T, Hv, dv), (xq.dtype,))
    B = Bx if cu_seqlens is None else _offsets(cu_seqlens, T)
    cs = torch.empty((B, 3, 2 * Hk * dk + Hv * dv), dtype=xq.dtype, device=xq.device)
    d = make_desc(B, T, Hk, Hv, dk, dv, 64, F16, F32, GATE_HEAD)
    check(lib().gdn_conv_state(ctypes.byref(d), _ptr(cu_seqlens), _DTYPE_CODE[xq.dtype], _ptr(xq), _ptr(xk),
                               _ptr(xv), _ptr(cs), _stream(stream)))
    return cs


def decode_step_conv(xq, xk, xv, conv_w, conv_st, g, beta, S, qkv_dtype=torch.float16, eps=1e-6, o=None,
                     stream=None, delta=True):
    """One decode step from raw inputs xq, xk [B,Hk,dk], xv [B,Hv,dv] and the
    convolution history conv_st [B,3,channels] (moved on by one token in place);
    S updated in place.  Returns o fp32 [B,Hv,dv].  delta=False: the update
    without the delta correction."""
    B, Hk, dk = xq.shape
    Hv, dv = xv.shape[1], xv.shape[2]
    _dev("xq", xq)
    _dev("xk", xk, xq.shape, (xq.dtype,))
    _dev("xv", xv, (B, Hv, dv), (xq.dtype,))
    _dev("conv_w", conv_w, (2 * Hk * dk + Hv * dv, 4), (torch.float32,))
    _dev("conv_state", conv_st, (B, 3, 2 * Hk * dk + Hv * dv), (xq.dtype,))
    _dev("g", g)
    gate = GATE_HEAD if tuple(g.shape) == (B, Hv) else GATE_KEY_CHANNEL
    _dev("beta", beta, (B, Hv), (g.dtype,))
    _dev("S", S, (B, Hv, dv, dk), (torch.float32,))
    if o is None:
        o = torch.empty((B, Hv, dv), dtype=torch.float32, device=xq.device)
    _dev("o", o, (B, Hv, dv), (torch.float32,))
    d = make_desc(B, 1, Hk, Hv, dk, dv, 64, _DTYPE_CODE[qkv_dtype], _DTYPE_CODE[g.dtype], gate,
                  RULE_DELTA if delta else RULE_NO_DELTA)
    L = lib()
    ws_bytes = L.gdn_decode_conv_workspace_bytes(ctypes.byref(d))
    ws = _workspace(ws_bytes, xq.device)
    check(L.gdn_decode_step_conv(ctypes.byref(d), _DTYPE_CODE[xq.dtype], _ptr(xq), _ptr(xk), _ptr(xv),
                                 _ptr(conv_w), float(eps), _ptr(conv_st), _ptr(g), _ptr(beta), _ptr(S), _ptr(o),
                                 _ptr(ws), ws_bytes, _stream(stream)))
    return o


def bwd(q, k, v, g, beta, S0, dO, dS_T=None, stream=None, workspace_cap=None, delta=True):
    """Gradients of sum <dO, o> + <dS_T, S_T> with respect to q, k, v, g, beta,
    S0 (fp32).  Shapes as for fwd_chunked; dO fp32 [B,T,Hv,dv].  With
    workspace_cap (bytes), the workspace of the fastest plan within it;
    delta=False: the update without the delta correction (per-head gate)."""
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    _dev("q", q)
    _dev("k", k, q.shape, (q.dtype,))
    _dev("v", v, (B, T, Hv, dv), (q.dtype,))
    gate = _gate_kind(_dev("g", g), B, T, Hv, dk)
    _dev("beta", beta, (B, T, Hv), (g.dtype,))
    _dev("dO", dO, (B, T, Hv, dv), (torch.float32,))
    for n, x in (("S0", S0), ("dS_T", dS_T)):
        if x is not None:
            _dev(n, x, (B, Hv, dv, dk), (torch.float32,))
    f = lambda shape: torch.empty(shape, dtype=torch.float32, device=q.device)
    out = {"dq": f(q.shape), "dk": f(q.shape), "dv": f(v.shape), "dg": f(g.shape), "dbeta": f(beta.shape),
           "dS0": f((B, Hv, dv, dk))}
    d = make_desc(B, T, Hk, Hv, dk, dv, 64, _DTYPE_CODE[q.dtype], _DTYPE_CODE[g.dtype], gate,
                  RULE_DELTA if delta else RULE_NO_DELTA)
    L = lib()
    ws_bytes = L.gdn_bwd_workspace_bytes(ctypes.byref(d)) if workspace_cap is None else \
        L.gdn_bwd_workspace_bytes_within(ctypes.byref(d), int(workspace_cap))
    ws = _workspace(ws_bytes, q.device)
    check(L.gdn_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(dO),
                    _ptr(dS_T), *(_ptr(out[n]) for n in ("dq", "dk", "dv", "dg", "dbeta", "dS0")), _ptr(ws),
                    ws_bytes, _stream(stream)))
    return out


def decode_step(q, k, v, g, beta, S, o=None, stream=None, delta=True):
    """One token per sequence.  q, k [B,Hk,dk]; v [B,Hv,dv]; g [B,Hv] or
    [B,Hv,dk]; beta [B,Hv]; S fp32 [B,Hv,dv,dk] updated in place.
    Returns o fp32 [B,Hv,dv]."""
    B, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    _dev("q", q)
    _dev("k", k, q.shape, (q.dtype,))
    _dev("v", v, (B, Hv, dv), (q.dtype,))
    _dev("g", g)
    if tuple(g.shape) == (B, Hv):
        gate = GATE_HEAD
    elif tuple(g.shape) == (B, Hv, dk):
        gate = GATE_KEY_CHANNEL
    else:
        raise ValueError("g must be [B,Hv] or [B,Hv,dk]")
    _dev("beta", beta, (B, Hv), (g.dtype,))
    _dev("S", S, (B, Hv, dv, dk), (torch.float32,))
    if o is None:
        o = torch.empty((B, Hv, dv), dtype=torch.float32, device=q.device)
    _dev("o", o, (B, Hv, dv), (torch.float32,))
    d = make_desc(B, 1, Hk, Hv, dk, dv, 64, _DTYPE_CODE[q.dtype], _DTYPE_CODE[g.dtype], gate,
                  RULE_DELTA if delta else RULE_NO_DELTA)
    check(lib().gdn_decode_step(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(S), _ptr(o), _stream(stream)))
    return o
