"""The prologue inside the chunked forward (gdn_fwd_chunked_conv) on the GPU.

Where its fused kernels run (bf16 raw inputs, fp16 q and k, per-head gate,
d 128, chunk 64) the convolution, SiLU and L2 normalisation of q and k use
the prologue's arithmetic and roundings, and v keeps its fp32 value (as fp16
high and low parts) instead of being rounded to fp16 as gdn_prologue stores
it; so the call is checked against the fp64 oracle (oracle prologue, then the
token-by-token recurrence), and the two calls it replaces (gdn_prologue, then
gdn_fwd_chunked) against the same oracle and against it.  Everywhere else the
call runs those two steps itself and must give exactly their results."""
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_02_amd as gdn
import oracle
from gdn_inputs import KDA_PREFILL, PREFILL_CONV, TINY_F32, make_prefill, to_torch
from parity import check

pytestmark = pytest.mark.gpu


def say(msg):
    print("[case] " + msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gdn.lib()


def raw(inp):
    return [to_torch(inp[n]) for n in ("xq", "xk", "xv")], to_torch(inp["conv_w"])


def fused_kernels(wl, qkv):
    return qkv == torch.float16 and wl.gate == "head" and wl.dk == 128 and wl.dv == 128 and wl.chunk == 64


def fused_vs_two_calls(wl, label, qkv=torch.float16, gates_f32=False, S0=None):
    inp = make_prefill(wl)
    say("%s: B=%d T=%d Hk=%d Hv=%d gate=%s qkv=%s" % (label, wl.B, wl.T, wl.Hk, wl.Hv, wl.gate, qkv))
    xs, w = raw(inp)
    g, beta = to_torch(inp["g"]), to_torch(inp["beta"])
    if gates_f32:
        g, beta = g.float(), beta.float()
    q, k, v = gdn.prologue(*xs, w, out_dtype=qkv)
    o2, S2 = gdn.fwd_chunked(q, k, v, g, beta, S0=S0, chunk=wl.chunk)
    o1 = torch.full_like(o2, float("nan"))
    S1 = torch.full_like(S2, float("nan"))
    gdn.fwd_chunked_conv(*xs, w, g, beta, S0=S0, qkv_dtype=qkv, chunk=wl.chunk, o=o1, S_T=S1)
    torch.cuda.synchronize()
    if not fused_kernels(wl, qkv):
        assert torch.equal(o1, o2), "%s: o differs from prologue + chunked (max %g)" % (
            label, (o1 - o2).abs().nan_to_num(float("inf")).max().item())
        assert torch.equal(S1, S2), "%s: S_T differs from prologue + chunked" % label
        return
    rq, rk, rv = oracle.prologue(inp["xq"].f32(), inp["xk"].f32(), inp["xv"].f32(), inp["conv_w"])
    S0n = None if S0 is None else S0.cpu().numpy()
    o_ref, S_ref = oracle.recurrent_full(rq, rk, rv, inp["g"].f32(), inp["beta"].f32(), S0n)
    a, b = o1.cpu().numpy(), o2.cpu().numpy()
    check("bf16", a, o_ref, S1.cpu().numpy(), S_ref, "%s, prologue inside" % label)
    check("bf16", b, o_ref, S2.cpu().numpy(), S_ref, "%s, two calls" % label)
    check("bf16", a, b, S1.cpu().numpy(), S2.cpu().numpy(), "%s, prologue inside vs two calls" % label)


SMALL = PREFILL_CONV.with_(B=2, T=130, Hk=2, Hv=6)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 63, 64, 65, 130])
def test_fused_and_two_calls_T(T):
    fused_vs_two_calls(SMALL.with_(T=T), "conv T=%d" % T)


@pytest.mark.parametrize("B,Hk,Hv", [(2, 8, 32), (3, 8, 40), (3, 16, 48)])
def test_fused_and_two_calls_shapes(B, Hk, Hv):
    # 32, 64 and 128 value rows per workgroup of the sequential pass
    fused_vs_two_calls(SMALL.with_(B=B, Hk=Hk, Hv=Hv, T=100), "conv %d x %d heads" % (B, Hv))


def test_fused_and_two_calls_variants():
    fused_vs_two_calls(SMALL, "conv bf16 q/k/v", qkv=torch.bfloat16)
    fused_vs_two_calls(SMALL, "conv fp32 gates", gates_f32=True)
    S0 = torch.randn(SMALL.B, SMALL.Hv, 128, 128, device="cuda") * 0.02
    fused_vs_two_calls(SMALL, "conv S0", S0=S0)
    fused_vs_two_calls(SMALL.with_(B=1, Hk=1, Hv=8, T=150), "conv group of 8")


def test_composite_paths_equal_two_calls():
    # no fused kernels here: the prologue runs into the workspace first
    fused_vs_two_calls(KDA_PREFILL.with_(B=1, T=130, Hk=2, Hv=2, conv=True), "conv key gate")
    fused_vs_two_calls(TINY_F32.with_(T=50, conv=True), "conv fp32 mode", qkv=torch.float32)


def test_fused_vs_oracle():
    wl = PREFILL_CONV.with_(B=1, T=300, Hk=2, Hv=6)
    inp = make_prefill(wl)
    say("conv fused vs oracle")
    xs, w = raw(inp)
    o, ST = gdn.fwd_chunked_conv(*xs, w, to_torch(inp["g"]), to_torch(inp["beta"]), chunk=wl.chunk)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.prologue(inp["xq"].f32(), inp["xk"].f32(), inp["xv"].f32(), inp["conv_w"])
    o_ref, S_ref = oracle.recurrent_full(rq, rk, rv, inp["g"].f32(), inp["beta"].f32())
    check("bf16", o.cpu().numpy(), o_ref, ST.cpu().numpy(), S_ref, "conv fused small")


def test_fused_full_size_and_two_calls():
    fused_vs_two_calls(PREFILL_CONV, "prefill with conv, full size")


def test_fused_graph_capture_segmented():
    """The fused call in a configuration that runs as two overlapped segments
    (side stream), captured into a graph and replayed with eager work between
    the replays: every replay equals the eager call."""
    wl = PREFILL_CONV.with_(B=1, T=64 * 33 + 17, Hk=2, Hv=6)
    inp = make_prefill(wl)
    say("conv graph capture: B=1 T=%d Hk=2 Hv=6 (two segments)" % wl.T)
    xs, w = raw(inp)
    g, beta = to_torch(inp["g"]), to_torch(inp["beta"])
    o_e, S_e = gdn.fwd_chunked_conv(*xs, w, g, beta, chunk=64)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.prologue(inp["xq"].f32(), inp["xk"].f32(), inp["xv"].f32(), inp["conv_w"])
    o_ref, S_ref = oracle.recurrent_full(rq, rk, rv, inp["g"].f32(), inp["beta"].f32())
    check("bf16", o_e.cpu().numpy(), o_ref, S_e.cpu().numpy(), S_ref, "conv graph capture eager")
    o = torch.full_like(o_e, float("nan"))
    ST = torch.full_like(S_e, float("nan"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):           # warm the allocator outside the capture
        gdn.fwd_chunked_conv(*xs, w, g, beta, chunk=64, o=o, S_T=ST)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.fwd_chunked_conv(*xs, w, g, beta, chunk=64, o=o, S_T=ST)
    for rep in range(3):
        o.fill_(float("nan"))
        ST.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(o, o_e) and torch.equal(ST, S_e), "replay %d differs from the eager call" % rep
