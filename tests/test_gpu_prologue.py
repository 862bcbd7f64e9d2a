"""Prologue (conv + SiLU + L2) on the GPU vs the fp64 oracle, element by element."""
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_02_amd as gdn
import oracle
from gdn_inputs import PREFILL_CONV, make_prefill, to_torch

pytestmark = pytest.mark.gpu

# fp16 output: rounding is 2^-11 relative; fp32 arithmetic adds ~1e-6
TOL = {torch.float16: (1.0e-3, 2e-6), torch.bfloat16: (8.0e-3, 2e-6), torch.float32: (2e-5, 2e-6)}


def say(msg):
    print("[case] " + msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gdn.lib()


def compare(y, ref, dt, label):
    rtol, atol = TOL[dt]
    y = y.float().cpu().numpy().astype(np.float64)
    err = np.max(np.abs(y - ref) / (np.abs(ref) * rtol + atol))
    print("[parity] %s worst |d|/(rtol|ref|+atol) = %.3f" % (label, err), file=sys.stderr, flush=True)
    assert err <= 1.0, label


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d,T", [(128, 150), (16, 70), (64, 1), (32, 3)])
def test_prologue_small(out_dtype, d, T):
    wl = PREFILL_CONV.with_(B=2, T=T, Hk=2, Hv=6, dk=d, dv=d)
    say("prologue B=2 T=%d d=%d out=%s" % (T, d, out_dtype))
    inp = make_prefill(wl)
    xq, xk, xv = (to_torch(inp[n]) for n in ("xq", "xk", "xv"))
    w = to_torch(inp["conv_w"])
    q, k, v = gdn.prologue(xq, xk, xv, w, out_dtype=out_dtype)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.prologue(inp["xq"].f32(), inp["xk"].f32(), inp["xv"].f32(), inp["conv_w"])
    compare(q, rq, out_dtype, "q")
    compare(k, rk, out_dtype, "k")
    compare(v, rv, out_dtype, "v")


def test_prologue_fp32_inputs():
    wl = PREFILL_CONV.with_(B=1, T=90, Hk=2, Hv=4, dtype="f32")
    say("prologue fp32 inputs")
    inp = make_prefill(wl)
    q, k, v = gdn.prologue(*(to_torch(inp[n]) for n in ("xq", "xk", "xv")), to_torch(inp["conv_w"]),
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.prologue(inp["xq"].f32(), inp["xk"].f32(), inp["xv"].f32(), inp["conv_w"])
    for y, r, n in ((q, rq, "q"), (k, rk, "k"), (v, rv, "v")):
        compare(y, r, torch.float32, n)


def test_prologue_full_size_sampled():
    """The conv-prologue workload at full size (B 4, T 4096, 16/48 heads, d 128); the oracle
    recomputes sampled heads of every batch over all tokens."""
    wl = PREFILL_CONV
    say("prologue full size B=4 T=4096")
    inp = make_prefill(wl)
    xq, xk, xv = (to_torch(inp[n]) for n in ("xq", "xk", "xv"))
    w = inp["conv_w"]
    q, k, v = gdn.prologue(xq, xk, xv, to_torch(w), out_dtype=torch.float16)
    torch.cuda.synchronize()
    d = wl.dk
    nq = wl.Hk * d
    for name, y, x, woff, H, l2 in (("q", q, inp["xq"], 0, wl.Hk, True), ("k", k, inp["xk"], nq, wl.Hk, True),
                                    ("v", v, inp["xv"], 2 * nq, wl.Hv, False)):
        for h in (0, H // 2, H - 1):
            xs = np.ascontiguousarray(x.f32()[:, :, h:h + 1])
            ws = np.ascontiguousarray(w[woff + h * d: woff + (h + 1) * d])
            ref = oracle.conv_silu(xs, ws, l2)
            compare(y[:, :, h:h + 1], ref, torch.float16, "%s head %d" % (name, h))
