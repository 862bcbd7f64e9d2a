"""The backward (gdn_bwd) on the GPU against the fp64 oracle backward, whose
own pins are central finite differences of the forward oracle.

Bar: the fp32-mode bar of the forward, max|x - x_ref| / max|x_ref| <= 1e-4 for
every gradient: the backward computes in fp32 from the stored input values,
as the forward's fp32 mode does.
"""
import ctypes
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


def run_case(wl, label, s0=True, dst=True, seed=0, delta=True, workspace_cap=None):
    inp = make_prefill(wl.with_(s0_std=0.0))
    say("%s: B=%d T=%d Hk=%d Hv=%d d=%d/%d %s gate=%s" % (label, wl.B, wl.T, wl.Hk, wl.Hv, wl.dk, wl.dv,
                                                          wl.dtype, wl.gate))
    r = np.random.default_rng(500 + seed)
    S0 = np.ascontiguousarray(r.normal(0, 0.05, (wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32) if s0 else None
    dO = np.ascontiguousarray(r.standard_normal((wl.B, wl.T, wl.Hv, wl.dv)), dtype=np.float32)
    dST = np.ascontiguousarray(r.standard_normal((wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32) if dst else None
    args = [to_torch(inp[n]) for n in ("q", "k", "v", "g", "beta")]
    got = gdn.bwd(*args, None if S0 is None else to_torch(S0), to_torch(dO),
                  None if dST is None else to_torch(dST), delta=delta, workspace_cap=workspace_cap)
    torch.cuda.synchronize()
    ref = oracle.backward(*(inp[n].f32() for n in ("q", "k", "v", "g", "beta")),
                          None if S0 is None else S0.astype(np.float64), dO, dST, delta=delta)
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


@pytest.mark.parametrize("dk,dv,grp", [(32, 64, 2), (64, 32, 1), (128, 96, 3)])
def test_bwd_key_gate_shapes(dk, dv, grp):
    """Per-key-channel gate, fp32, each head dim, with one to three value
    heads per key head, over several chunks and a ragged last one."""
    run_case(TINY_F32.with_(B=2, T=150, Hk=2, Hv=2 * grp, dk=dk, dv=dv, gate="key"),
             "bwd key gate d %d/%d groups of %d" % (dk, dv, grp), seed=dk + grp)


def test_bwd_key_gate_strong_decay():
    """Per-key-channel gate with g = logsigmoid(N(-4, 1)), about -4 per token
    and channel: the decay between two tokens of one 16-token block reaches
    e^-60 and more, far past fp32's range, so every decay factor must be
    formed between tokens in order (each at most 1)."""
    run_case(KDA_PREFILL.with_(B=1, T=200, Hk=2, Hv=2, g_mu=-4.0), "bwd key gate strong decay", seed=11)


@pytest.mark.parametrize("T", [1, 64, 65])
def test_bwd_key_gate_chunk_edges(T):
    """Per-key-channel gate: one token, exactly one chunk, one chunk and a token."""
    run_case(KDA_PREFILL.with_(B=2, T=T, Hk=1, Hv=1), "bwd key gate T=%d" % T, seed=T)


def test_bwd_key_gate_segments():
    """Per-key-channel gate with workspaces too small for one segment: the
    segments give the one-segment result bit for bit, and the oracle's."""
    wl = KDA_PREFILL.with_(B=2, T=700, Hk=2, Hv=4)
    inp = make_prefill(wl)
    r = np.random.default_rng(919)
    S0 = np.ascontiguousarray(r.normal(0, 0.05, (wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32)
    dO = np.ascontiguousarray(r.standard_normal((wl.B, wl.T, wl.Hv, wl.dv)), dtype=np.float32)
    dST = np.ascontiguousarray(r.standard_normal((wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32)
    args = [to_torch(inp[n]) for n in ("q", "k", "v", "g", "beta")] + [to_torch(S0), to_torch(dO), to_torch(dST)]
    one = gdn.bwd(*args)
    full = gdn.lib().gdn_bwd_workspace_bytes(ctypes.byref(gdn.make_desc(
        wl.B, wl.T, wl.Hk, wl.Hv, wl.dk, wl.dv, 64, gdn.BF16, gdn.BF16, gdn.GATE_KEY_CHANNEL)))
    for cap in (full // 2, 0):
        say("bwd key gate segments: workspace cap %d of %d bytes" % (cap, full))
        seg = gdn.bwd(*args, workspace_cap=cap)
        torch.cuda.synchronize()
        for n in one:
            assert torch.equal(one[n], seg[n]), "cap %d: %s differs from one segment" % (cap, n)
    ref = oracle.backward(*(inp[n].f32() for n in ("q", "k", "v", "g", "beta")), S0.astype(np.float64), dO, dST)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
        e = rel_inf(seg[n].cpu().numpy(), ref[n])
        print("[parity] bwd key gate segments %s rel %.3e (bar 1e-4)" % (n, e), file=sys.stderr, flush=True)
        assert e <= 1e-4, "%s error %.3e" % (n, e)


def test_bwd_key_gate_full_size_sampled():
    """Per-key-channel gate at its prefill workload's full size (B 2, T 8192,
    32 heads, d 128, bf16 inputs), every chain on the GPU; the oracle
    recomputes two sampled (batch, head) chains over the whole sequence."""
    wl = KDA_PREFILL
    inp = make_prefill(wl)
    say("bwd key gate full size: B=%d T=%d H=%d d=128 bf16" % (wl.B, wl.T, wl.Hv))
    r = np.random.default_rng(4343)
    S0 = np.ascontiguousarray(r.normal(0, 0.05, (wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32)
    dO = np.ascontiguousarray(r.standard_normal((wl.B, wl.T, wl.Hv, wl.dv)), dtype=np.float32)
    dST = np.ascontiguousarray(r.standard_normal((wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32)
    args = [to_torch(inp[n]) for n in ("q", "k", "v", "g", "beta")]
    got = gdn.bwd(*args, to_torch(S0), to_torch(dO), to_torch(dST))
    torch.cuda.synchronize()
    got = {n: x.cpu().numpy() for n, x in got.items()}
    del args
    x = {n: inp[n].f32() for n in ("q", "k", "v", "g", "beta")}
    for b, h in ((0, 0), (1, 31)):
        bs, hs = slice(b, b + 1), slice(h, h + 1)
        ref = oracle.backward(x["q"][bs, :, hs], x["k"][bs, :, hs], x["v"][bs, :, hs], x["g"][bs, :, hs],
                              x["beta"][bs, :, hs], S0[bs, hs].astype(np.float64), dO[bs, :, hs], dST[bs, hs])
        for n in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
            mine = got[n][bs, hs] if n == "dS0" else got[n][bs, :, hs]
            assert np.all(np.isfinite(mine)), "non-finite %s" % n
            e = rel_inf(mine, ref[n])
            print("[parity] bwd key gate 2x8192 batch %d head %d %s rel %.3e (bar 1e-4)" % (b, h, n, e),
                  file=sys.stderr, flush=True)
            assert e <= 1e-4, "batch %d head %d: %s error %.3e" % (b, h, n, e)


def test_bwd_full_heads_long():
    """The backward at the prefill workload's head shape (16 key / 48 value
    heads, d 128, bf16 inputs) over T = 1024 tokens, on the GPU for every
    head; the oracle recomputes the gradients of two sampled key heads (each
    with its three value heads: a key head's dq and dk depend on no other)."""
    wl = PREFILL_CONV.with_(B=1, T=1024, conv=False)
    inp = make_prefill(wl)
    say("bwd full heads: B=1 T=%d Hk=%d Hv=%d d=128 bf16" % (wl.T, wl.Hk, wl.Hv))
    r = np.random.default_rng(777)
    S0 = np.ascontiguousarray(r.normal(0, 0.05, (wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32)
    dO = np.ascontiguousarray(r.standard_normal((wl.B, wl.T, wl.Hv, wl.dv)), dtype=np.float32)
    dST = np.ascontiguousarray(r.standard_normal((wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32)
    args = [to_torch(inp[n]) for n in ("q", "k", "v", "g", "beta")]
    got = gdn.bwd(*args, to_torch(S0), to_torch(dO), to_torch(dST))
    torch.cuda.synchronize()
    got = {n: x.cpu().numpy() for n, x in got.items()}
    del args
    grp = wl.Hv // wl.Hk
    for kh in (0, 11):
        hs = slice(kh * grp, (kh + 1) * grp)
        x = {n: inp[n].f32() for n in ("q", "k", "v", "g", "beta")}
        ref = oracle.backward(x["q"][:, :, kh:kh + 1], x["k"][:, :, kh:kh + 1], x["v"][:, :, hs], x["g"][:, :, hs],
                              x["beta"][:, :, hs], S0[:, hs].astype(np.float64), dO[:, :, hs], dST[:, hs])
        mine = {"dq": got["dq"][:, :, kh:kh + 1], "dk": got["dk"][:, :, kh:kh + 1], "dv": got["dv"][:, :, hs],
                "dg": got["dg"][:, :, hs], "dbeta": got["dbeta"][:, :, hs], "dS0": got["dS0"][:, hs]}
        for n in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
            assert np.all(np.isfinite(mine[n])), "non-finite %s" % n
            e = rel_inf(mine[n], ref[n])
            print("[parity] bwd 16/48 T=1024 key head %d %s rel %.3e (bar 1e-4)" % (kh, n, e),
                  file=sys.stderr, flush=True)
            assert e <= 1e-4, "key head %d: %s error %.3e" % (kh, n, e)


def test_bwd_segments_ragged():
    """Per-head gate with a workspace too small for one segment: the sequence
    runs in segments (here 1000 tokens, a ragged last chunk), which must give
    the one-segment result bit for bit, and the oracle's gradients."""
    wl = PREFILL_CONV.with_(B=2, T=1000, Hk=2, Hv=6, conv=False)
    inp = make_prefill(wl)
    r = np.random.default_rng(909)
    S0 = np.ascontiguousarray(r.normal(0, 0.05, (wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32)
    dO = np.ascontiguousarray(r.standard_normal((wl.B, wl.T, wl.Hv, wl.dv)), dtype=np.float32)
    dST = np.ascontiguousarray(r.standard_normal((wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32)
    args = [to_torch(inp[n]) for n in ("q", "k", "v", "g", "beta")] + [to_torch(S0), to_torch(dO), to_torch(dST)]
    one = gdn.bwd(*args)
    full = gdn.lib().gdn_bwd_workspace_bytes(ctypes.byref(gdn.make_desc(
        wl.B, wl.T, wl.Hk, wl.Hv, wl.dk, wl.dv, 64, gdn.BF16, gdn.BF16, gdn.GATE_HEAD)))
    for cap in (full // 2, full // 5, 0):
        say("bwd segments: workspace cap %d of %d bytes" % (cap, full))
        seg = gdn.bwd(*args, workspace_cap=cap)
        torch.cuda.synchronize()
        for n in one:
            assert torch.equal(one[n], seg[n]), "cap %d: %s differs from one segment" % (cap, n)
    ref = oracle.backward(*(inp[n].f32() for n in ("q", "k", "v", "g", "beta")), S0.astype(np.float64), dO, dST)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
        e = rel_inf(seg[n].cpu().numpy(), ref[n])
        print("[parity] bwd segments %s rel %.3e (bar 1e-4)" % (n, e), file=sys.stderr, flush=True)
        assert e <= 1e-4, "%s error %.3e" % (n, e)


def test_bwd_prefill_full_size_sampled():
    """The backward at the prefill workload's full size (B 4, T 4096, 16 key /
    48 value heads, d 128, bf16 inputs), every chain on the GPU, in one segment
    and within a 1 GB workspace (four segments): the two agree bit for bit,
    and the oracle recomputes two sampled (batch, key head) groups over the
    whole sequence, each with its three value heads."""
    wl = PREFILL_CONV.with_(conv=False)
    inp = make_prefill(wl)
    say("bwd full size: B=%d T=%d Hk=%d Hv=%d d=128 bf16" % (wl.B, wl.T, wl.Hk, wl.Hv))
    r = np.random.default_rng(4242)
    S0 = np.ascontiguousarray(r.normal(0, 0.05, (wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32)
    dO = np.ascontiguousarray(r.standard_normal((wl.B, wl.T, wl.Hv, wl.dv)), dtype=np.float32)
    dST = np.ascontiguousarray(r.standard_normal((wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32)
    args = [to_torch(inp[n]) for n in ("q", "k", "v", "g", "beta")]
    got = gdn.bwd(*args, to_torch(S0), to_torch(dO), to_torch(dST))
    capped = gdn.bwd(*args, to_torch(S0), to_torch(dO), to_torch(dST), workspace_cap=10 ** 9)
    torch.cuda.synchronize()
    for n in got:
        assert torch.equal(got[n], capped[n]), "%s: the 1 GB workspace differs from one segment" % n
    del capped
    got = {n: x.cpu().numpy() for n, x in got.items()}
    del args
    grp = wl.Hv // wl.Hk
    x = {n: inp[n].f32() for n in ("q", "k", "v", "g", "beta")}
    for b, kh in ((0, 0), (3, 15)):
        hs = slice(kh * grp, (kh + 1) * grp)
        bs = slice(b, b + 1)
        ref = oracle.backward(x["q"][bs, :, kh:kh + 1], x["k"][bs, :, kh:kh + 1], x["v"][bs, :, hs],
                              x["g"][bs, :, hs], x["beta"][bs, :, hs], S0[bs, hs].astype(np.float64), dO[bs, :, hs],
                              dST[bs, hs])
        mine = {"dq": got["dq"][bs, :, kh:kh + 1], "dk": got["dk"][bs, :, kh:kh + 1], "dv": got["dv"][bs, :, hs],
                "dg": got["dg"][bs, :, hs], "dbeta": got["dbeta"][bs, :, hs], "dS0": got["dS0"][bs, hs]}
        for n in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
            assert np.all(np.isfinite(mine[n])), "non-finite %s" % n
            e = rel_inf(mine[n], ref[n])
            print("[parity] bwd 4x4096 batch %d key head %d %s rel %.3e (bar 1e-4)" % (b, kh, n, e),
                  file=sys.stderr, flush=True)
            assert e <= 1e-4, "batch %d key head %d: %s error %.3e" % (b, kh, n, e)


@pytest.mark.parametrize("T", [1, 64, 65])
def test_bwd_chunk_edges(T):
    """One token, exactly one chunk, one chunk and a token: the chunked
    backward's padding and its single-chunk case, one key and one value head."""
    run_case(PREFILL_CONV.with_(B=2, T=T, Hk=1, Hv=1, conv=False), "bwd T=%d" % T, seed=T)


def test_bwd_without_delta_correction():
    """The update without the delta correction (per-head gate): fp32 at small
    head dims, and bf16 grouped heads over several chunks, one segment and
    several (the smallest workspace)."""
    run_case(TINY_F32.with_(B=2, T=70, Hk=1, Hv=2, dk=32, dv=64), "bwd no-delta fp32", delta=False)
    wl = PREFILL_CONV.with_(B=1, T=300, Hk=2, Hv=6, conv=False)
    run_case(wl, "bwd no-delta bf16", delta=False, seed=3)
    run_case(wl, "bwd no-delta bf16 segments", delta=False, seed=3, workspace_cap=0)


def test_bwd_key_gate_without_delta_correction():
    """The update without the delta correction with the per-key-channel gate:
    fp32 at small head dims with grouped heads, and bf16 at d 128 over several
    chunks, one segment and several (the smallest workspace)."""
    run_case(TINY_F32.with_(B=2, T=150, Hk=1, Hv=2, dk=64, dv=32, gate="key"), "bwd key gate no-delta fp32",
             delta=False, seed=5)
    wl = KDA_PREFILL.with_(B=1, T=300, Hk=2, Hv=4)
    run_case(wl, "bwd key gate no-delta bf16", delta=False, seed=6)
    run_case(wl, "bwd key gate no-delta bf16 segments", delta=False, seed=6, workspace_cap=0)


@pytest.mark.parametrize("cap", [None, 0])
def test_bwd_graph_capture(cap):
    """The backward captured into a graph (one segment, and the smallest
    workspace's several) and replayed three times with eager work between the
    replays: every replay equals the eager call bit for bit."""
    wl = PREFILL_CONV.with_(B=1, T=300, Hk=2, Hv=6, conv=False)
    inp = make_prefill(wl)
    say("bwd graph capture, workspace cap %s" % cap)
    r = np.random.default_rng(77)
    S0 = to_torch(np.ascontiguousarray(r.normal(0, 0.05, (wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32))
    dO = to_torch(np.ascontiguousarray(r.standard_normal((wl.B, wl.T, wl.Hv, wl.dv)), dtype=np.float32))
    dST = to_torch(np.ascontiguousarray(r.standard_normal((wl.B, wl.Hv, wl.dv, wl.dk)), dtype=np.float32))
    args = [to_torch(inp[n]) for n in ("q", "k", "v", "g", "beta")] + [S0, dO, dST]
    eager = gdn.bwd(*args, workspace_cap=cap)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):           # warm the allocator outside the capture
        gdn.bwd(*args, workspace_cap=cap)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        got = gdn.bwd(*args, workspace_cap=cap)
    for rep in range(3):
        for x in got.values():
            x.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for n in eager:
            assert torch.equal(got[n], eager[n]), "replay %d: %s differs from the eager call" % (rep, n)
