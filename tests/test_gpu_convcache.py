"""Decode continuing a prefill through the convolution history (conv_state,
decode_step_conv) on the GPU.

A decode step from raw inputs must make the token's q, k, v exactly as the
prologue over the longer sequence makes them, so it is checked bit for bit
against gdn_prologue over T + n tokens followed by gdn_decode_step on the last
n tokens; the whole prefill-then-decode chain is also checked against the fp64
oracle (prologue and recurrence over T + n tokens)."""
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_02_amd as gdn
import oracle
from gdn_inputs import PREFILL_CONV, make_prefill, to_torch
from parity import check

pytestmark = pytest.mark.gpu


def say(msg):
    print("[case] " + msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gdn.lib()


def channels_history(xs, T):
    """The expected history after token T - 1: raw q | k | v of tokens T-3..T-1
    (zero before 0), [B,3,channels], built by slicing."""
    B = xs[0].shape[0]
    parts = []
    for j in range(3):
        t = T - 3 + j
        if t < 0:
            parts.append(torch.zeros((B, sum(x.shape[2] * x.shape[3] for x in xs)), dtype=xs[0].dtype,
                                     device=xs[0].device))
        else:
            parts.append(torch.cat([x[:, t].reshape(B, -1) for x in xs], dim=1))
    return torch.stack(parts, dim=1).contiguous()


@pytest.mark.parametrize("T,steps", [(100, 1), (64, 3), (1, 2), (2, 1)])
def test_decode_continues_prefill(T, steps):
    wl = PREFILL_CONV.with_(B=2, T=T + steps, Hk=2, Hv=6)
    inp = make_prefill(wl)
    say("prefill %d tokens, then %d decode steps from raw inputs" % (T, steps))
    xs = [to_torch(inp[n]) for n in ("xq", "xk", "xv")]
    w, g, beta = to_torch(inp["conv_w"]), to_torch(inp["g"]), to_torch(inp["beta"])
    pre = [x[:, :T].contiguous() for x in xs]
    o_pre, S = gdn.fwd_chunked_conv(*pre, w, g[:, :T].contiguous(), beta[:, :T].contiguous())
    cs = gdn.conv_state(*pre)
    torch.cuda.synchronize()
    assert torch.equal(cs, channels_history(xs, T)), "conv_state is not the last three raw tokens"
    # the same steps from the prologue over all T + steps tokens
    q, k, v = gdn.prologue(*xs, w)
    S2 = S.clone()
    outs, outs2 = [], []
    for t in range(T, T + steps):
        outs.append(gdn.decode_step_conv(*(x[:, t].contiguous() for x in xs), w, cs, g[:, t].contiguous(),
                                         beta[:, t].contiguous(), S))
        outs2.append(gdn.decode_step(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
                                     g[:, t].contiguous(), beta[:, t].contiguous(), S2))
    torch.cuda.synchronize()
    for a, b in zip(outs, outs2):
        assert torch.equal(a, b), "decode from raw inputs differs from prologue + decode"
    assert torch.equal(S, S2), "state differs from prologue + decode"
    assert torch.equal(cs, channels_history(xs, T + steps)), "conv_state did not move on"
    # the oracle over all T + steps tokens
    rq, rk, rv = oracle.prologue(inp["xq"].f32(), inp["xk"].f32(), inp["xv"].f32(), inp["conv_w"])
    o_ref, S_ref = oracle.recurrent_full(rq, rk, rv, inp["g"].f32(), inp["beta"].f32())
    o_all = torch.cat([o_pre] + [x[:, None] for x in outs], dim=1)
    check("bf16", o_all.cpu().numpy(), o_ref, S.cpu().numpy(), S_ref, "prefill %d + %d decode" % (T, steps))


def test_decode_conv_fp32_inputs():
    wl = PREFILL_CONV.with_(B=3, T=9, Hk=2, Hv=4, dtype="f32")
    inp = make_prefill(wl)
    say("fp32 raw inputs, prefill 8 then decode 1")
    xs = [to_torch(inp[n]) for n in ("xq", "xk", "xv")]
    w, g, beta = to_torch(inp["conv_w"]), to_torch(inp["g"]), to_torch(inp["beta"])
    cs = gdn.conv_state(*(x[:, :8].contiguous() for x in xs))
    S = torch.randn(3, 4, 128, 128, device="cuda") * 0.02
    S2 = S.clone()
    o1 = gdn.decode_step_conv(*(x[:, 8].contiguous() for x in xs), w, cs, g[:, 8].contiguous(),
                              beta[:, 8].contiguous(), S, qkv_dtype=torch.float32)
    q, k, v = gdn.prologue(*xs, w, out_dtype=torch.float32)
    o2 = gdn.decode_step(q[:, 8].contiguous(), k[:, 8].contiguous(), v[:, 8].contiguous(), g[:, 8].contiguous(),
                         beta[:, 8].contiguous(), S2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S, S2)


@pytest.mark.parametrize("d,gate,qkv,delta", [
    (64, "head", torch.float16, True),      # other head dims: q, k, v through the workspace
    (32, "key", torch.bfloat16, True),
    (128, "key", torch.float16, True),      # dk 128: one kernel
    (128, "head", torch.bfloat16, True),
    (128, "head", torch.float16, False),    # without the delta correction
])
def test_decode_conv_forms(d, gate, qkv, delta):
    """decode_step_conv against the prologue over the whole sequence followed
    by decode_step, bit for bit, for each form of the step."""
    wl = PREFILL_CONV.with_(B=3, T=9, Hk=2, Hv=6, dk=d, dv=d, gate=gate)
    inp = make_prefill(wl)
    say("decode from raw inputs: d %d, %s gate, %s, delta %s" % (d, gate, qkv, delta))
    xs = [to_torch(inp[n]) for n in ("xq", "xk", "xv")]
    w, g, beta = to_torch(inp["conv_w"]), to_torch(inp["g"]), to_torch(inp["beta"])
    cs = gdn.conv_state(*(x[:, :8].contiguous() for x in xs))
    S = torch.randn(3, 6, d, d, device="cuda") * 0.05
    S2 = S.clone()
    o1 = gdn.decode_step_conv(*(x[:, 8].contiguous() for x in xs), w, cs, g[:, 8].contiguous(),
                              beta[:, 8].contiguous(), S, qkv_dtype=qkv, delta=delta)
    q, k, v = gdn.prologue(*xs, w, out_dtype=qkv)
    o2 = gdn.decode_step(q[:, 8].contiguous(), k[:, 8].contiguous(), v[:, 8].contiguous(), g[:, 8].contiguous(),
                         beta[:, 8].contiguous(), S2, delta=delta)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "o differs from prologue + decode"
    assert torch.equal(S, S2), "state differs from prologue + decode"
    assert torch.equal(cs, channels_history(xs, 9)), "conv_state did not move on"


def test_conv_state_packed():
    lens = [1, 5, 0, 70, 2]
    T = sum(lens)
    wl = PREFILL_CONV.with_(B=1, T=T, Hk=2, Hv=4)
    inp = make_prefill(wl)
    say("conv_state of packed sequences %s" % lens)
    xs = [to_torch(inp[n]) for n in ("xq", "xk", "xv")]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cs = gdn.conv_state(*xs, cu_seqlens=torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    for s in range(len(lens)):
        a, e = int(cu[s]), int(cu[s + 1])
        alone = channels_history([x[:, a:e] for x in xs], e - a)
        assert torch.equal(cs[s:s + 1], alone), "sequence %d" % s
