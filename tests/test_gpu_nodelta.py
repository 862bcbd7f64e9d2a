"""The update without the delta correction (rule GDN_RULE_NO_DELTA: the
"SinkProbe" page's hybrid_nodelta layer) on the GPU against the fp64 oracle
run with delta=False, on every path: matrix cores with either gate, fp32
mode, decode, and the composite entry points (convolution, packed sequences)."""
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_02_amd as gdn
import oracle
from gdn_inputs import KDA_PREFILL, PREFILL_CONV, TINY_F32, make_decode_token, make_prefill, to_torch
from parity import check

pytestmark = pytest.mark.gpu


def say(msg):
    print("[case] " + msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gdn.lib()


def run_case(wl, mode, label):
    inp = make_prefill(wl)
    say("%s: B=%d T=%d Hk=%d Hv=%d d=%d C=%d %s gate=%s" % (label, wl.B, wl.T, wl.Hk, wl.Hv, wl.dk, wl.chunk,
                                                            wl.dtype, wl.gate))
    args = [to_torch(inp[n]) for n in ("q", "k", "v", "g", "beta")]
    S0 = None if inp["S0"] is None else to_torch(inp["S0"])
    o, ST = gdn.fwd_chunked(*args, S0=S0, chunk=wl.chunk, delta=False)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.recurrent_full(*(inp[n].f32() for n in ("q", "k", "v", "g", "beta")), inp["S0"],
                                         delta=False)
    check(mode, o.cpu().numpy(), o_ref, ST.cpu().numpy(), S_ref, label)
    return inp, ST


@pytest.mark.parametrize("B,Hk,Hv", [(2, 2, 6), (2, 8, 64), (3, 16, 48)])
def test_no_delta_head_gate(B, Hk, Hv):
    # 32-, 64- and 128-row workgroups of the sequential pass
    run_case(PREFILL_CONV.with_(B=B, T=130, Hk=Hk, Hv=Hv, conv=False, s0_std=0.02), "bf16", "no delta %d heads" % Hv)


def test_no_delta_key_gate():
    run_case(KDA_PREFILL.with_(B=1, T=130, Hk=2, Hv=2), "bf16", "no delta key gate")


@pytest.mark.parametrize("gate", ["head", "key"])
def test_no_delta_fp32(gate):
    run_case(TINY_F32.with_(gate=gate, s0_std=0.5), "f32", "no delta fp32 %s" % gate)


def test_no_delta_prefill_then_decode():
    wl = PREFILL_CONV.with_(B=2, T=70, Hk=2, Hv=6, conv=False)
    inp, ST = run_case(wl, "bf16", "no delta prefill")
    tok = make_decode_token(wl, 0)
    d = [to_torch(tok[n]) for n in ("q", "k", "v", "g", "beta")]
    o = gdn.decode_step(*d, ST, delta=False)
    torch.cuda.synchronize()
    cat = lambda n: np.concatenate([inp[n].f32(), tok[n].f32()[:, None]], axis=1)
    o_ref, S_ref = oracle.recurrent_full(cat("q"), cat("k"), cat("v"), cat("g"), cat("beta"), delta=False)
    check("bf16", o.cpu().numpy(), o_ref[:, -1], ST.cpu().numpy(), S_ref, "no delta decode")


def test_no_delta_composites():
    # convolution inside (the prologue into the workspace, then the forward)
    wl = PREFILL_CONV.with_(B=2, T=100, Hk=2, Hv=6)
    inp = make_prefill(wl)
    say("no delta with the convolution, and packed")
    xs = [to_torch(inp[n]) for n in ("xq", "xk", "xv")]
    w, g, beta = to_torch(inp["conv_w"]), to_torch(inp["g"]), to_torch(inp["beta"])
    o1, S1 = gdn.fwd_chunked_conv(*xs, w, g, beta, delta=False)
    q, k, v = gdn.prologue(*xs, w)
    o2, S2 = gdn.fwd_chunked(q, k, v, g, beta, delta=False)
    # packed sequences of equal lengths give the fixed-length bits
    cu = torch.tensor([0, 100, 200], dtype=torch.int32, device="cuda")
    pack = lambda t: t.reshape((1, 200) + tuple(t.shape[2:])).contiguous()
    o3, S3 = gdn.fwd_chunked_varlen(pack(q), pack(k), pack(v), pack(g), pack(beta), cu, delta=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    assert torch.equal(pack(o2), o3) and torch.equal(S2, S3)
    rq, rk, rv = oracle.prologue(inp["xq"].f32(), inp["xk"].f32(), inp["xv"].f32(), inp["conv_w"])
    o_ref, S_ref = oracle.recurrent_full(rq, rk, rv, inp["g"].f32(), inp["beta"].f32(), delta=False)
    check("bf16", o1.cpu().numpy(), o_ref, S1.cpu().numpy(), S_ref, "no delta conv")
