"""The backward (gdn_bwd) on the GPU against the fp64 oracle backward, whose
own pins are central finite differences of the forward oracle.

Bar: the fp32-mode bar of the forward, max|x - x_ref| / max|x_ref| <= 1e-4 for
every gradient: the backward computes in fp32 from the stored input values,
as the forward's fp32 mode does.
"""
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_02_amd as gdn
import oracle
from gdn_inputs import KDA_PREFILL, PREFILL_CONV, TINY_F32, make_prefill, to_torch
from parity import rel_inf

pytestmark = pytest.mark.gpu


def say(msg):
    print("[case] " + msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gdn.lib()


def run_case(wl, label, s0=True, dst=True, seed=0):
    inp = make_prefill(wl.with_(s0_std=0.0))
    say("%s: B=%d T=%d Hk=%d Hv=%d d=%d/%d %s gate=%s" % (label, wl.B, wl.T, wl.Hk, wl.Hv, wl.dk, wl.dv,
                                                          wl.dtype, wl.gate))
    r = np.random.default_rng(500 + seed)
    S0 = np.ascontiguousarray(r.normal(0, 0.05, (wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32) if s0 else None
    dO = np.ascontiguousarray(r.standard_normal((wl.B, wl.T, wl.Hv, wl.dv)), dtype=np.float32)
    dST = np.ascontiguousarray(r.standard_normal((wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32) if dst else None
    args = [to_torch(inp[n]) for n in ("q", "k", "v", "g", "beta")]
    got = gdn.bwd(*args, None if S0 is None else to_torch(S0), to_torch(dO),
                  None if dST is None else to_torch(dST))
    torch.cuda.synchronize()
    ref = oracle.backward(*(inp[n].f32() for n in ("q", "k", "v", "g", "beta")),
                          None if S0 is None else S0.astype(np.float64), dO, dST)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
        x = got[n].cpu().numpy()
        assert np.all(np.isfinite(x)), "%s: non-finite %s" % (label, n)
        e = rel_inf(x, ref[n])
        print("[parity] %s %s rel %.3e (bar 1e-4)" % (label, n, e), file=sys.stderr, flush=True)
        assert e <= 1e-4, "%s: %s error %.3e" % (label, n, e)


@pytest.mark.parametrize("gate", ["head", "key"])
def test_bwd_fp32_small(gate):
    wl = TINY_F32.with_(B=2, T=70, Hk=1, Hv=2, dk=32, dv=64, gate=gate)
    run_case(wl, "bwd fp32 %s" % gate)


@pytest.mark.parametrize("dk,dv", [(64, 32), (128, 96)])
def test_bwd_shapes(dk, dv):
    run_case(TINY_F32.with_(B=1, T=40, Hk=2, Hv=4, dk=dk, dv=dv), "bwd d %d/%d" % (dk, dv), seed=dk)


def test_bwd_without_state_gradients():
    run_case(TINY_F32.with_(B=1, T=33, Hk=1, Hv=1, dk=32, dv=32), "bwd no S0, no dS_T", s0=False, dst=False)


def test_bwd_bf16_grouped():
    run_case(PREFILL_CONV.with_(B=1, T=130, Hk=2, Hv=6, conv=False), "bwd bf16 16/48-style groups")


def test_bwd_bf16_key_gate():
    run_case(KDA_PREFILL.with_(B=1, T=100, Hk=2, Hv=2), "bwd bf16 key gate")
