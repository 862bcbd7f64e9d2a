"""Decode step on the GPU vs the fp64 oracle (the recurrence with T = 1, state carried)."""
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_02_amd as gdn
import oracle
from gdn_inputs import (BATCHED_DECODE, TINY_F32, decode_tokens_device, make_decode_token,
                        make_prefill, make_state, to_torch)
from parity import check

pytestmark = pytest.mark.gpu


def say(msg):
    print("[case] " + msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gdn.lib()


def stack_steps(tokens):
    """List of per-step dicts of Tensor [B,...] -> float32 arrays [B,steps,...] for the oracle."""
    out = {}
    for n in ("q", "k", "v", "g", "beta"):
        out[n] = np.stack([t[n].f32() for t in tokens], axis=1)
    return out


def run_gpu_steps(tokens, S):
    os_ = []
    for t in tokens:
        o = gdn.decode_step(*(to_torch(t[n]) for n in ("q", "k", "v", "g", "beta")), S)
        os_.append(o)
    torch.cuda.synchronize()
    return torch.stack(os_, dim=1).cpu().numpy()


@pytest.mark.parametrize("gate", ["head", "key"])
def test_decode_tiny_fp32(gate):
    """One fp32 decode step from the state a 64-token prefill left (the tiny workload)."""
    wl = TINY_F32.with_(gate=gate)
    say("decode tiny fp32 gate=%s" % gate)
    inp = make_prefill(wl)
    _, ST = oracle.recurrent_full(inp["q"].f32(), inp["k"].f32(), inp["v"].f32(), inp["g"].f32(),
                                  inp["beta"].f32(), None)
    S_in = ST.astype(np.float32)                       # an input: the oracle's state, rounded to fp32
    tok = make_decode_token(wl, 0)
    S = to_torch(S_in)
    o = run_gpu_steps([tok], S)
    r = stack_steps([tok])
    o_ref, S_ref = oracle.recurrent_full(r["q"], r["k"], r["v"], r["g"], r["beta"], S_in)
    check("f32", o, o_ref, S.cpu().numpy(), S_ref, "decode tiny fp32 %s" % gate)


@pytest.mark.parametrize("gate,qdt", [("head", "bf16"), ("key", "bf16"), ("head", "f32")])
def test_decode_steps_small(gate, qdt):
    """20 consecutive steps, B = 4, 16 key / 48 value heads, state carried on the GPU."""
    wl = BATCHED_DECODE.with_(B=4, gate=gate, dtype=qdt)
    say("decode small 20 steps gate=%s dtype=%s" % (gate, qdt))
    S0 = make_state(wl)
    toks = [make_decode_token(wl, s) for s in range(20)]
    S = to_torch(S0)
    o = run_gpu_steps(toks, S)
    r = stack_steps(toks)
    o_ref, S_ref = oracle.recurrent_full(r["q"], r["k"], r["v"], r["g"], r["beta"], S0)
    mode = "f32" if qdt == "f32" else "bf16"
    check(mode, o, o_ref, S.cpu().numpy(), S_ref, "decode small %s %s" % (gate, qdt))
    if qdt == "bf16":                                   # fp32 state arithmetic: far inside the bar
        check("f32", o, o_ref, S.cpu().numpy(), S_ref, "decode small %s %s (fp32 bar)" % (gate, qdt))


def test_decode_full_batch_sampled():
    """The batched-decode workload at its full size and length: B = 256, 16/48
    heads, d 128, 1000 consecutive steps on the GPU with the state carried in
    place.  The oracle replays 48 sampled chains over all 1000 steps; o is
    compared at steps 1, 10, 100, 200, ..., 1000 and S after step 1000, and
    the error is logged at every checkpoint to show how it grows."""
    wl = BATCHED_DECODE
    steps = wl.decode_steps
    assert steps == 1000
    say("decode full batch B=256 steps=%d" % steps)
    S0 = make_state(wl)
    toks = decode_tokens_device(wl, steps)
    S = to_torch(S0)
    idx = [0, 9] + list(range(99, steps, 100))
    grp = wl.Hv // wl.Hk
    r = np.random.default_rng(1000)
    chains = [(0, 0), (255, 47), (17, 5), (101, 31), (200, 46), (128, 24)] + \
        [(int(b), int(h)) for b, h in zip(r.integers(0, wl.B, 42), r.integers(0, wl.Hv, 42))]
    bi = torch.tensor([c[0] for c in chains], device="cuda")
    hi = torch.tensor([c[1] for c in chains], device="cuda")
    o_steps = []
    for s in range(steps):
        o = gdn.decode_step(toks["q"][s], toks["k"][s], toks["v"][s], toks["g"][s], toks["beta"][s], S)
        if s in idx:
            o_steps.append(o[bi, hi])
    torch.cuda.synchronize()
    o_gpu = torch.stack(o_steps, 1).cpu().numpy()                 # [chains, checkpoints, dv]
    S_gpu = S[bi, hi].cpu().numpy()
    f = lambda x: x.float().cpu().numpy()
    kh = hi // grp
    q = f(toks["q"][:, bi, kh]).transpose(1, 0, 2)[:, :, None]     # [chains, steps, 1, dk]
    k = f(toks["k"][:, bi, kh]).transpose(1, 0, 2)[:, :, None]
    v = f(toks["v"][:, bi, hi]).transpose(1, 0, 2)[:, :, None]
    g = f(toks["g"][:, bi, hi]).T[:, :, None]
    beta = f(toks["beta"][:, bi, hi]).T[:, :, None]
    S0c = np.stack([S0[b, h] for b, h in chains])[:, None]
    o_ref, S_ref = oracle.recurrent(q, k, v, g, beta, S0c)           # every chain as its own sequence
    o_ref = o_ref[:, idx]
    for j, s in enumerate(idx):
        check("f32", o_gpu[:, j], o_ref[:, j], None, None, "decode 48 chains, step %d" % (s + 1))
    check("bf16", o_gpu, o_ref, S_gpu, S_ref, "decode 48 chains, steps 1..1000")
    check("f32", o_gpu, o_ref, S_gpu, S_ref, "decode 48 chains, steps 1..1000 (fp32 bar)")


def test_decode_deterministic_and_in_place():
    wl = BATCHED_DECODE.with_(B=8)
    say("decode determinism")
    S0 = make_state(wl)
    tok = make_decode_token(wl, 3)
    args = [to_torch(tok[n]) for n in ("q", "k", "v", "g", "beta")]
    S1, S2 = to_torch(S0), to_torch(S0)
    o1 = gdn.decode_step(*args, S1)
    o2 = gdn.decode_step(*args, S2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    assert not torch.equal(S1, to_torch(S0))


def test_decode_loop_graph_capture():
    """A loop of decode steps captured into one graph (the state carried in
    place from step to step) and replayed several times from a reset state,
    with eager work between replays: every replay equals the eager loop."""
    wl = BATCHED_DECODE.with_(B=16)
    steps = 12
    say("decode loop graph capture: B=%d, %d steps" % (wl.B, steps))
    S_init = to_torch(make_state(wl))
    toks = [make_decode_token(wl, s) for s in range(steps)]
    args = [[to_torch(t[n]) for n in ("q", "k", "v", "g", "beta")] for t in toks]
    S = S_init.clone()
    o = torch.empty((wl.B, wl.Hv, wl.dv), device="cuda")
    outs = torch.empty((steps, wl.B, wl.Hv, wl.dv), device="cuda")

    def loop():
        for s in range(steps):
            gdn.decode_step(*args[s], S, o=o)
            outs[s].copy_(o)

    loop()
    torch.cuda.synchronize()
    S_e, outs_e = S.clone(), outs.clone()
    graph = torch.cuda.CUDAGraph()
    S.copy_(S_init)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):        # warm-up on a side stream before capture
        loop()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        loop()
    for rep in range(3):
        S.copy_(S_init)
        outs.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(S, S_e) and torch.equal(outs, outs_e), "replay %d differs" % rep
