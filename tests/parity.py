"""Parity measures and bars (GPU result vs the fp64 oracle).

fp32 mode: max|x - x_ref| / max|x_ref| <= 1e-4 for o and S_T.
bf16-input / fp32-state mode: max|o - o_ref| / rms(o_ref) <= 2e-2 (rms over the
whole compared tensor) and max|S - S_ref| / max|S_ref| <= 1e-2.
"""
from __future__ import annotations

import sys

import numpy as np

TOL_F32 = 1e-4
TOL_O_BF16 = 2e-2
TOL_S_BF16 = 1e-2


def rel_inf(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / den) if den > 0 else float(np.max(np.abs(x)))


def rms_inf(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(x - ref)) / np.sqrt(np.mean(ref * ref)))


def check(mode: str, o, o_ref, S=None, S_ref=None, label=""):
    """Assert the bar of `mode` ("f32" or "bf16"); returns the measured errors."""
    assert np.all(np.isfinite(o)), "non-finite output"
    if mode == "f32":
        eo = rel_inf(o, o_ref)
        es = rel_inf(S, S_ref) if S is not None else 0.0
        bar_o, bar_s = TOL_F32, TOL_F32
    else:
        eo = rms_inf(o, o_ref)
        es = rel_inf(S, S_ref) if S is not None else 0.0
        bar_o, bar_s = TOL_O_BF16, TOL_S_BF16
    print("[parity] %s mode=%s err_o=%.3e (bar %.0e) err_S=%.3e (bar %.0e)" %
          (label, mode, eo, bar_o, es, bar_s), file=sys.stderr, flush=True)
    assert eo <= bar_o, "%s: o error %.3e > %.0e" % (label, eo, bar_o)
    assert es <= bar_s, "%s: S error %.3e > %.0e" % (label, es, bar_s)
    return eo, es
