"""The gated output norm on the GPU: the standalone kernel (gdn_output_gate)
and the forward with the gate (gdn_fwd_chunked_conv_gated), against the fp64
oracle, and the fused form against the two calls it replaces.

Bars for y, derived from the arithmetic, each plus the rounding of y to its
stored type, u |y_ref| with u = 2^-8 (bf16) or 2^-11 (fp16) (half an ulp,
with margin):
 - the gate alone on given o: |y - y_ref| <= 1e-5 rms(y_ref) (fp32 rounding
   and the hardware reciprocal, square root and exponential);
 - the whole path: the forward's bar on o, max|do| <= 2e-2 rms(o), carried
   through the row normalisation.  With rho the row's root mean square (eps
   included), o^ = o / rho and w = gain silu(z):  d(o^) = do / rho - o^ d(rho) / rho
   and |d(rho)| <= max|do|, so |dy| <= 2e-2 rms(o) (1 + |o^|) |w| / rho.  A row
   whose own rms is far below the tensor's takes a proportionally larger
   error, as any normalisation of it would.
"""
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_02_amd as gdn
import oracle
from gdn_inputs import PREFILL_CONV, make_gate_inputs, make_prefill, to_torch

pytestmark = pytest.mark.gpu

ROUND = {torch.float32: 0.0, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


def say(msg):
    print("[case] " + msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gdn.lib()


def check_y(y, y_ref, ydt, bar, label):
    y = y.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(y)), "%s: non-finite y" % label
    rms = np.sqrt(np.mean(y_ref * y_ref))
    err = np.abs(y - y_ref)
    excess = np.max(err - ROUND[ydt] * np.abs(y_ref)) / rms
    print("[parity] %s y: max|dy|/rms %.3e, beyond rounding %.3e (bar %.0e)" %
          (label, np.max(err) / rms, excess, bar), file=sys.stderr, flush=True)
    assert excess <= bar, "%s: y error %.3e rms beyond rounding > %.0e" % (label, excess, bar)


# ---------------------------------------------------------------- the gate alone
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16, torch.float16])
def test_output_gate_vs_oracle(dv, ydt):
    B, T, Hv = 2, 37, 3            # 222 rows: a ragged last block
    say("output gate: B=%d T=%d Hv=%d dv=%d y=%s" % (B, T, Hv, dv, ydt))
    gen = torch.Generator().manual_seed(100 + dv)
    o = torch.randn((B, T, Hv, dv), generator=gen) * 3.0
    o[0, 0, 0] = 0.0                # a zero row: y = 0 (eps > 0)
    o[1, 5, 2] *= 1e-4              # a small row: normalised like any other
    for zdt in (torch.bfloat16, torch.float16, torch.float32):
        z = (torch.randn((B, T, Hv, dv), generator=gen) * 2.0).to(zdt)
        gain = 1.0 + 0.1 * torch.randn((dv,), generator=gen)
        y = gdn.output_gate(o.cuda(), z.cuda(), gain.cuda(), eps=1e-5, out_dtype=ydt)
        torch.cuda.synchronize()
        y_ref = oracle.output_gate(o.numpy(), z.float().numpy(), gain.numpy(), 1e-5)
        check_y(y, y_ref, ydt, 1e-5, "gate dv=%d z=%s y=%s" % (dv, zdt, ydt))
        assert torch.all(y[0, 0, 0] == 0)


def test_output_gate_one_row_per_block_tail():
    # rows = 1 and a count just past a block (16 rows of 128 per block)
    for T in (1, 17):
        o = torch.randn((1, T, 1, 128), device="cuda")
        z = torch.randn((1, T, 1, 128), device="cuda").bfloat16()
        gain = torch.ones(128, device="cuda")
        y = gdn.output_gate(o, z, gain, eps=1e-5, out_dtype=torch.float32)
        torch.cuda.synchronize()
        y_ref = oracle.output_gate(o.cpu().numpy(), z.float().cpu().numpy(), gain.cpu().numpy(), 1e-5)
        check_y(y, y_ref, torch.float32, 1e-5, "gate T=%d" % T)


# ---------------------------------------------------------------- the forward with the gate
def gated_inputs(wl):
    inp = make_prefill(wl)
    gi = make_gate_inputs(wl)
    xs = [to_torch(inp[n]) for n in ("xq", "xk", "xv")]
    return inp, gi, xs, to_torch(inp["conv_w"]), to_torch(inp["g"]), to_torch(inp["beta"])


def fused_vs_two_calls(wl, label, ydt=torch.bfloat16, qkv=torch.float16, gates_f32=False, S0=None):
    inp, gi, xs, w, g, beta = gated_inputs(wl)
    say("%s: B=%d T=%d Hk=%d Hv=%d y=%s qkv=%s" % (label, wl.B, wl.T, wl.Hk, wl.Hv, ydt, qkv))
    if gates_f32:
        g, beta = g.float(), beta.float()
    z, gain = to_torch(gi["z"]), to_torch(gi["gain"])
    o, S2 = gdn.fwd_chunked_conv(*xs, w, g, beta, S0=S0, qkv_dtype=qkv, chunk=wl.chunk)
    y2 = gdn.output_gate(o, z, gain, eps=gi["norm_eps"], out_dtype=ydt)
    y1 = torch.full_like(y2, float("nan"))
    S1 = torch.full_like(S2, float("nan"))
    gdn.fwd_chunked_conv_gated(*xs, w, g, beta, z, gain, S0=S0, qkv_dtype=qkv, norm_eps=gi["norm_eps"],
                               chunk=wl.chunk, y=y1, S_T=S1)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), "%s: y differs from forward + gate (max %g)" % (
        label, (y1.float() - y2.float()).abs().nan_to_num(float("inf")).max().item())
    assert torch.equal(S1, S2), "%s: S_T differs from forward + gate" % label


# B * Hv > 128: the gate runs inside the sequential pass
FUSED = PREFILL_CONV.with_(B=3, T=130, Hk=16, Hv=48)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
def test_gated_equals_two_calls_T(T):
    fused_vs_two_calls(FUSED.with_(T=T), "gated T=%d" % T)


@pytest.mark.parametrize("ydt", [torch.float32, torch.float16])
def test_gated_equals_two_calls_ydtype(ydt):
    fused_vs_two_calls(FUSED.with_(T=100), "gated y=%s" % ydt, ydt=ydt)


def test_gated_equals_two_calls_variants():
    fused_vs_two_calls(FUSED.with_(T=100), "gated bf16 q/k", qkv=torch.bfloat16)
    fused_vs_two_calls(FUSED.with_(T=100), "gated fp32 gates", gates_f32=True)
    S0 = torch.randn(FUSED.B, FUSED.Hv, 128, 128, device="cuda") * 0.02
    fused_vs_two_calls(FUSED, "gated S0", S0=S0)
    fused_vs_two_calls(FUSED.with_(B=1, Hk=4, Hv=132, T=70), "gated group of 33")


@pytest.mark.parametrize("B,Hk,Hv", [(2, 2, 6), (2, 8, 64)])
def test_gated_after_forward_equals_two_calls(B, Hk, Hv):
    # B * Hv <= 128: o through the workspace, then the gate
    fused_vs_two_calls(FUSED.with_(B=B, Hk=Hk, Hv=Hv, T=100), "gated %d x %d heads" % (B, Hv))


def check_y_path(y, o_ref, z, gain, eps, ydt, label):
    """The whole path's bar: the error beyond rounding, in units of
    rms(o) (1 + |o^|) |w| / rho, at most 2e-2."""
    y = y.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(y)), "%s: non-finite y" % label
    y_ref = oracle.output_gate(o_ref, z, gain, eps)
    rho = np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True) + eps)
    zz = z.astype(np.float64)
    w = gain.astype(np.float64) * zz / (1 + np.exp(-zz))
    scale = np.sqrt(np.mean(o_ref * o_ref)) * (1 + np.abs(o_ref) / rho) * np.abs(w) / rho
    excess = np.maximum(np.abs(y - y_ref) - ROUND[ydt] * np.abs(y_ref), 0.0)
    err = float(np.max(excess / np.maximum(scale, 1e-300)))
    rms_y = np.sqrt(np.mean(y_ref * y_ref))
    print("[parity] %s y: max|dy|/rms(y) %.3e; beyond rounding, in units of the carried o bar %.3e "
          "(bar 2e-2)" % (label, np.max(np.abs(y - y_ref)) / rms_y, err), file=sys.stderr, flush=True)
    assert err <= 2e-2, "%s: y error %.3e > 2e-2" % (label, err)


def gated_vs_oracle(wl, label, ydt=torch.bfloat16):
    inp, gi, xs, w, g, beta = gated_inputs(wl)
    say("%s vs oracle: B=%d T=%d Hk=%d Hv=%d" % (label, wl.B, wl.T, wl.Hk, wl.Hv))
    y, ST = gdn.fwd_chunked_conv_gated(*xs, w, g, beta, to_torch(gi["z"]), to_torch(gi["gain"]),
                                       norm_eps=gi["norm_eps"], out_dtype=ydt, chunk=wl.chunk)
    torch.cuda.synchronize()
    del xs
    rq, rk, rv = oracle.prologue(inp["xq"].f32(), inp["xk"].f32(), inp["xv"].f32(), inp["conv_w"])
    o_ref, S_ref = oracle.recurrent_full(rq, rk, rv, inp["g"].f32(), inp["beta"].f32())
    del rq, rk, rv
    check_y_path(y, o_ref, gi["z"].f32(), gi["gain"], gi["norm_eps"], ydt, label)
    ST = ST.cpu().numpy()
    es = np.max(np.abs(ST - S_ref)) / np.max(np.abs(S_ref))
    print("[parity] %s S_T rel %.3e (bar 1e-2)" % (label, es), file=sys.stderr, flush=True)
    assert es <= 1e-2


def test_gated_fused_vs_oracle():
    gated_vs_oracle(FUSED.with_(T=100), "gated fused small")


def test_gated_after_forward_vs_oracle():
    gated_vs_oracle(FUSED.with_(B=1, Hk=2, Hv=6, T=200), "gated unfused small", ydt=torch.float32)


def test_gated_full_size_vs_oracle_and_two_calls():
    fused_vs_two_calls(PREFILL_CONV, "gated full size")
    gated_vs_oracle(PREFILL_CONV, "gated full size, whole tensor")


def test_gated_graph_capture():
    """The gated call with the gate inside the pass, captured into a graph and
    replayed with eager work between the replays: every replay equals the
    eager call."""
    wl = FUSED.with_(T=100)
    inp, gi, xs, w, g, beta = gated_inputs(wl)
    say("gated graph capture: B=%d T=%d Hv=%d" % (wl.B, wl.T, wl.Hv))
    z, gain = to_torch(gi["z"]), to_torch(gi["gain"])
    y_e, S_e = gdn.fwd_chunked_conv_gated(*xs, w, g, beta, z, gain, norm_eps=gi["norm_eps"])
    y = torch.full_like(y_e, float("nan"))
    ST = torch.full_like(S_e, float("nan"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):           # warm the allocator outside the capture
        gdn.fwd_chunked_conv_gated(*xs, w, g, beta, z, gain, norm_eps=gi["norm_eps"], y=y, S_T=ST)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.fwd_chunked_conv_gated(*xs, w, g, beta, z, gain, norm_eps=gi["norm_eps"], y=y, S_T=ST)
    for rep in range(3):
        y.fill_(float("nan"))
        ST.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(y, y_e) and torch.equal(ST, S_e), "replay %d differs from the eager call" % rep
