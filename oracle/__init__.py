"""fp64 CPU oracle for the Gated DeltaNet forward pass.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` are the only callers.  The GPU library never
imports, links or runs anything here, and nothing here imports the GPU
library.

``gdnref.c`` holds the token-by-token recurrence and its backward (reverse
mode over the stored state history), the conv/SiLU/L2 prologue and the gated
output norm that follows the state read, compiled with gcc into ``libgdnref.so`` and called through ctypes.
``chunked.py`` holds a second, chunk-parallel formulation in NumPy that is used
only to pin the recurrence (the two must agree to 1e-10).

Every function is pinned by ``tests/test_oracle_pins.py``; no function here is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdnref.c")
_LIB = os.path.join(_HERE, "libgdnref.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gdnref.c with gcc into libgdnref.so (next to the source)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-D_POSIX_C_SOURCE=200112L",
             "-Wall", "-Werror", "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(path: str) -> str:
    """Compile gdnref.c with AddressSanitizer and UBSan (gcc; every finding
    aborts) into `path`.  Loaded in place of the plain build when the
    environment names it in GDNREF_LIBRARY, with gcc's libasan preloaded."""
    subprocess.run(
        ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-std=c99", "-fPIC", "-shared", "-pthread", "-D_POSIX_C_SOURCE=200112L",
         "-Wall", "-Werror", "-o", path, _SRC, "-lm"],
        check=True,
    )
    return path


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("GDNREF_LIBRARY")
        if not path:
            build(force=False)
            path = _LIB
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.gdnref_recurrent.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, I, I, P, P, P, P, I]
        lib.gdnref_recurrent.restype = I
        lib.gdnref_conv_silu.argtypes = [I, I, I, I, P, P, I, ctypes.c_double, P]
        lib.gdnref_conv_silu.restype = I
        lib.gdnref_output_gate.argtypes = [ctypes.c_long, I, P, P, P, ctypes.c_double, P]
        lib.gdnref_output_gate.restype = I
        lib.gdnref_backward.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.gdnref_backward.restype = I
        _lib = lib
    return _lib


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def recurrent(q, k, v, g, beta, S0=None, chains=None, nthreads=None, delta=True):
    """Token-by-token fp64 recurrence.

    q, k: [B,T,Hk,dk]; v: [B,T,Hv,dv]; g: [B,T,Hv] (per-head decay) or
    [B,T,Hv,dk] (per-key-channel decay), natural log of alpha; beta: [B,T,Hv];
    S0: [B,Hv,dv,dk] or None (float64 S0 is used as is, anything else is
    converted to float32).  All values are taken exactly as given (float32
    arrays holding bf16/fp16/fp32 values).

    chains: list of (b, h) pairs to run (default: all, in b-major order).
    delta=False: the update without the delta correction, S <- decay(S) + beta v k^T.
    Returns (o [n,T,dv] float64, S_T [n,dv,dk] float64) for the chains in order.
    """
    lib = _load()
    q, k, v, g, beta = (_f32(a) for a in (q, k, v, g, beta))
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or beta.shape != (B, T, Hv):
        raise ValueError("shape mismatch")
    if g.shape == (B, T, Hv):
        per_channel = 0
    elif g.shape == (B, T, Hv, dk):
        per_channel = 1
    else:
        raise ValueError("g must be [B,T,Hv] or [B,T,Hv,dk]")
    s0_double = 0
    if S0 is not None:
        if np.asarray(S0).dtype == np.float64:
            S0 = np.ascontiguousarray(S0)
            s0_double = 1
        else:
            S0 = _f32(S0)
        if S0.shape != (B, Hv, dv, dk):
            raise ValueError("S0 must be [B,Hv,dv,dk]")
    if chains is None:
        chains = [(b, h) for b in range(B) for h in range(Hv)]
    sb = np.ascontiguousarray([c[0] for c in chains], dtype=np.int32)
    sh = np.ascontiguousarray([c[1] for c in chains], dtype=np.int32)
    n = len(chains)
    o = np.empty((n, T, dv), dtype=np.float64)
    ST = np.empty((n, dv, dk), dtype=np.float64)
    if nthreads is None:
        # one GPU's share of the host: OMP_NUM_THREADS when set, at most 16
        nthreads = min(int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1), 16)
    rc = lib.gdnref_recurrent(B, T, Hk, Hv, dk, dv, per_channel | (0 if delta else 2), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                              _ptr(beta), _ptr(S0), s0_double, n, _ptr(sb), _ptr(sh), _ptr(o), _ptr(ST),
                              int(nthreads))
    if rc != 0:
        raise ValueError("gdnref_recurrent rejected its arguments")
    return o, ST


def recurrent_full(q, k, v, g, beta, S0=None, nthreads=None, delta=True):
    """All chains; returns o [B,T,Hv,dv] and S_T [B,Hv,dv,dk] (float64)."""
    B, T = q.shape[:2]
    Hv, dv = v.shape[2], v.shape[3]
    dk = q.shape[3]
    o, ST = recurrent(q, k, v, g, beta, S0, None, nthreads, delta)
    return (o.reshape(B, Hv, T, dv).transpose(0, 2, 1, 3).copy(), ST.reshape(B, Hv, dv, dk))


def conv_silu(x, w, l2norm, eps=1e-6):
    """4-tap causal depthwise conv + SiLU (+ per-head L2 normalisation).

    x: [B,T,H,d]; w: [H*d, 4] (tap 3 multiplies the current token).
    Returns float64 [B,T,H,d].
    """
    lib = _load()
    x = _f32(x)
    w = _f32(w)
    B, T, H, d = x.shape
    if w.shape != (H * d, 4):
        raise ValueError("w must be [H*d, 4]")
    y = np.empty((B, T, H, d), dtype=np.float64)
    rc = lib.gdnref_conv_silu(B, T, H, d, _ptr(x), _ptr(w), 1 if l2norm else 0, float(eps), _ptr(y))
    if rc != 0:
        raise ValueError("gdnref_conv_silu rejected its arguments")
    return y


def prologue(xq, xk, xv, w, eps=1e-6):
    """The whole prologue: w is [Hk*dk (q) + Hk*dk (k) + Hv*dv (v), 4].

    Returns (q, k, v) float64: q and k L2-normalised per (token, head), v not.
    """
    Hk, dk = xq.shape[2], xq.shape[3]
    Hv, dv = xv.shape[2], xv.shape[3]
    w = _f32(w)
    nq = Hk * dk
    q = conv_silu(xq, w[:nq], True, eps)
    k = conv_silu(xk, w[nq:2 * nq], True, eps)
    v = conv_silu(xv, w[2 * nq:2 * nq + Hv * dv], False, eps)
    return q, k, v


def output_gate(o, z, gain, eps):
    """Gated output norm: every row of o over its last axis (d channels),
    y = o / sqrt(mean(o^2) + eps) * gain * z * sigmoid(z).

    o: [..., d] (taken as float64), z: same shape (float32 values as stored),
    gain: [d].  Returns float64 of o's shape.
    """
    lib = _load()
    o = np.ascontiguousarray(np.asarray(o, dtype=np.float64))
    z = _f32(z)
    gain = _f32(gain)
    d = o.shape[-1]
    if z.shape != o.shape or gain.shape != (d,):
        raise ValueError("z must match o and gain must be [d]")
    y = np.empty(o.shape, dtype=np.float64)
    rc = lib.gdnref_output_gate(int(o.size // d), d, _ptr(o), _ptr(z), _ptr(gain), float(eps), _ptr(y))
    if rc != 0:
        raise ValueError("gdnref_output_gate rejected its arguments")
    return y


def backward(q, k, v, g, beta, S0, dO, dST=None, delta=True):
    """Gradients of L = sum <dO, o> + <dST, S_T> with respect to q, k, v, g,
    beta and S0 (fp64, reverse mode over the stored state history).

    Shapes as for recurrent(); dO [B,T,Hv,dv]; dST [B,Hv,dv,dk] or None; S0
    [B,Hv,dv,dk] or None; delta=False: the update without the delta
    correction, as for recurrent().  Returns a dict dq, dk, dv, dg, dbeta, dS0
    (float64).
    """
    lib = _load()
    q, k, v, g, beta = (_f32(a) for a in (q, k, v, g, beta))
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    per_channel = 1 if g.ndim == 4 else 0
    d64 = lambda a: None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    S0, dO, dST = d64(S0), d64(dO), d64(dST)
    if dO.shape != (B, T, Hv, dv):
        raise ValueError("dO must be [B,T,Hv,dv]")
    out = {"dq": np.empty(q.shape), "dk": np.empty(k.shape), "dv": np.empty(v.shape),
           "dg": np.empty(g.shape), "dbeta": np.empty(beta.shape), "dS0": np.empty((B, Hv, dv, dk))}
    rc = lib.gdnref_backward(B, T, Hk, Hv, dk, dv, per_channel | (0 if delta else 2), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(g), _ptr(beta),
                             _ptr(S0), _ptr(dO), _ptr(dST), *(_ptr(out[n]) for n in
                                                             ("dq", "dk", "dv", "dg", "dbeta", "dS0")))
    if rc != 0:
        raise ValueError("gdnref_backward rejected its arguments")
    return out
