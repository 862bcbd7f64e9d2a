"""Packed sequences of different lengths (the _varlen entry points) on the GPU.

Each sequence must come out as if computed alone: checked against the fp64
oracle run on each sequence separately (its own entering state, its own
convolution history starting from zero), and, bit for bit, against the
fixed-length entry points when every sequence has the same length (the
kernels then do the same arithmetic in the same order).
"""
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


def offsets(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def states(n, Hv, dv, dk, seed):
    r = np.random.default_rng(seed)
    return np.ascontiguousarray(r.normal(0, 0.05, (n, Hv, dv, dk)), dtype=np.float32)


def packed_case(wl, lens, seed=0, conv=False):
    """Inputs of one packed call: a workload drawn at B = 1, T = sum(lens)."""
    T = int(np.sum(lens))
    inp = make_prefill(wl.with_(B=1, T=T, s0_std=0.0, conv=conv))
    cu = offsets(lens)
    S0 = states(len(lens), wl.Hv, wl.dv, wl.dk, 1000 + seed)
    return inp, cu, S0


def oracle_per_sequence(inp, cu, S0, conv):
    """o [1,T,Hv,dv] and S_T [N,Hv,dv,dk] from the oracle, one sequence at a time."""
    if not conv:
        q, k, v = (inp[n].f32() for n in ("q", "k", "v"))
    g, beta = inp["g"].f32(), inp["beta"].f32()
    T = g.shape[1]
    Hv, dv = S0.shape[1], S0.shape[2]
    o = np.zeros((1, T, Hv, dv), dtype=np.float64)
    ST = np.zeros(S0.shape, dtype=np.float64)
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        if conv:
            # the prologue of this sequence alone: zero history before its first token
            qs, ks, vs = oracle.prologue(inp["xq"].f32()[:, a:e], inp["xk"].f32()[:, a:e],
                                         inp["xv"].f32()[:, a:e], inp["conv_w"]) if e > a else (None,) * 3
        else:
            qs, ks, vs = q[:, a:e], k[:, a:e], v[:, a:e]
        if e == a:
            ST[s] = S0[s]
            continue
        os_, Ss = oracle.recurrent_full(qs, ks, vs, g[:, a:e], beta[:, a:e], S0[s:s + 1].astype(np.float64))
        o[:, a:e] = os_
        ST[s] = Ss[0]
    return o, ST


LENS = [130, 0, 1, 63, 64, 65, 7, 200]


@pytest.mark.parametrize("Hk,Hv", [(2, 6), (16, 48)])
def test_varlen_vs_oracle(Hk, Hv):
    # 8 sequences x Hv value heads: 48 and 384 chains (32- and 128-row workgroups)
    wl = PREFILL_CONV.with_(Hk=Hk, Hv=Hv, conv=False)
    inp, cu, S0 = packed_case(wl, LENS, seed=Hv)
    say("varlen: lens %s, Hk=%d Hv=%d" % (LENS, Hk, Hv))
    args = [to_torch(inp[n]) for n in ("q", "k", "v", "g", "beta")]
    o, ST = gdn.fwd_chunked_varlen(*args, torch.from_numpy(cu).cuda(), S0=to_torch(S0))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_per_sequence(inp, cu, S0, conv=False)
    check("bf16", o.cpu().numpy(), o_ref, ST.cpu().numpy(), S_ref, "varlen Hv=%d" % Hv)


def test_varlen_conv_vs_oracle_and_two_calls():
    wl = PREFILL_CONV.with_(Hk=2, Hv=6)
    lens = [3, 130, 0, 64, 2, 97]
    inp, cu, S0 = packed_case(wl, lens, seed=7, conv=True)
    say("varlen conv: lens %s" % lens)
    xs = [to_torch(inp[n]) for n in ("xq", "xk", "xv")]
    w, g, beta = to_torch(inp["conv_w"]), to_torch(inp["g"]), to_torch(inp["beta"])
    cut = torch.from_numpy(cu).cuda()
    o1, S1 = gdn.fwd_chunked_conv_varlen(*xs, w, g, beta, cut, S0=to_torch(S0))
    q, k, v = gdn.prologue_varlen(*xs, w, cut)
    o2, S2 = gdn.fwd_chunked_varlen(q, k, v, g, beta, cut, S0=to_torch(S0))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_per_sequence(inp, cu, S0, conv=True)
    # the fused kernels keep v at fp32 where the prologue stores fp16: the
    # two forms are each checked against the oracle and against each other
    check("bf16", o1.cpu().numpy(), o_ref, S1.cpu().numpy(), S_ref, "varlen conv inside")
    check("bf16", o2.cpu().numpy(), o_ref, S2.cpu().numpy(), S_ref, "varlen conv two calls")
    check("bf16", o1.cpu().numpy(), o2.cpu().numpy(), S1.cpu().numpy(), S2.cpu().numpy(),
          "varlen conv inside vs two calls")


def test_prologue_varlen_resets_history():
    # fp32 raw inputs and outputs: the packed prologue against the oracle's,
    # run on each sequence alone
    wl = PREFILL_CONV.with_(Hk=2, Hv=4, dtype="f32")
    lens = [1, 2, 3, 17, 16, 0, 40]
    inp, cu, _ = packed_case(wl, lens, conv=True)
    say("prologue varlen: lens %s" % lens)
    xs = [to_torch(inp[n]) for n in ("xq", "xk", "xv")]
    q, k, v = gdn.prologue_varlen(*xs, to_torch(inp["conv_w"]), torch.from_numpy(cu).cuda(),
                                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    for s in range(len(lens)):
        a, e = int(cu[s]), int(cu[s + 1])
        if e == a:
            continue
        rq, rk, rv = oracle.prologue(*(inp[n].f32()[:, a:e] for n in ("xq", "xk", "xv")), inp["conv_w"])
        for got, ref in ((q, rq), (k, rk), (v, rv)):
            err = np.max(np.abs(got[:, a:e].cpu().numpy() - ref)) / np.max(np.abs(ref))
            assert err < 1e-5, "sequence %d: prologue error %.3e" % (s, err)


@pytest.mark.parametrize("kind", ["head", "key", "f32", "conv"])
def test_equal_lengths_equal_fixed_length(kind):
    """Equal lengths: the packed call gives the fixed-length call's bits."""
    if kind == "head":
        wl = PREFILL_CONV.with_(B=3, T=130, Hk=2, Hv=6, conv=False)
    elif kind == "key":
        wl = KDA_PREFILL.with_(B=3, T=130, Hk=2, Hv=2)
    elif kind == "f32":
        wl = TINY_F32.with_(B=3, T=50)
    else:
        wl = PREFILL_CONV.with_(B=3, T=130, Hk=2, Hv=6)
    inp = make_prefill(wl)
    say("equal lengths (%s): B=%d T=%d" % (kind, wl.B, wl.T))
    S0 = to_torch(states(wl.B, wl.Hv, wl.dv, wl.dk, 5))
    cu = torch.from_numpy(offsets([wl.T] * wl.B)).cuda()
    pack = lambda t: t.reshape((1, wl.B * wl.T) + tuple(t.shape[2:])).contiguous()
    g, beta = to_torch(inp["g"]), to_torch(inp["beta"])
    if kind == "conv":
        xs = [to_torch(inp[n]) for n in ("xq", "xk", "xv")]
        w = to_torch(inp["conv_w"])
        o1, S1 = gdn.fwd_chunked_conv(*xs, w, g, beta, S0=S0)
        o2, S2 = gdn.fwd_chunked_conv_varlen(*(pack(x) for x in xs), w, pack(g), pack(beta), cu, S0=S0)
    else:
        args = [to_torch(inp[n]) for n in ("q", "k", "v")]
        o1, S1 = gdn.fwd_chunked(*args, g, beta, S0=S0, chunk=wl.chunk)
        o2, S2 = gdn.fwd_chunked_varlen(*(pack(a) for a in args), pack(g), pack(beta), cu, S0=S0,
                                        chunk=wl.chunk)
    torch.cuda.synchronize()
    assert torch.equal(pack(o1), o2), "%s: packed o differs from the fixed-length call" % kind
    assert torch.equal(S1, S2), "%s: packed S_T differs from the fixed-length call" % kind


@pytest.mark.parametrize("kind", ["key", "f32"])
def test_varlen_other_paths_vs_oracle(kind):
    if kind == "key":
        wl = KDA_PREFILL.with_(Hk=2, Hv=2)
        lens, mode = [70, 0, 1, 129], "bf16"
    else:
        wl = TINY_F32
        lens, mode = [17, 0, 16, 1, 40], "f32"
    inp, cu, S0 = packed_case(wl, lens, seed=3)
    say("varlen %s: lens %s" % (kind, lens))
    args = [to_torch(inp[n]) for n in ("q", "k", "v", "g", "beta")]
    o, ST = gdn.fwd_chunked_varlen(*args, torch.from_numpy(cu).cuda(), S0=to_torch(S0), chunk=wl.chunk)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_per_sequence(inp, cu, S0, conv=False)
    check(mode, o.cpu().numpy(), o_ref, ST.cpu().numpy(), S_ref, "varlen %s" % kind)


def test_varlen_many_sequences():
    """More sequences than the workgroup that orders them (1024 threads), most
    of them 0 to 3 tokens long (ties everywhere), a few long ones among them,
    and a group count that is not a multiple of 8."""
    wl = PREFILL_CONV.with_(Hk=1, Hv=1, conv=False)
    r = np.random.default_rng(21)
    lens = r.integers(0, 4, 1101)
    lens[[3, 700, 1100]] = [300, 129, 64]
    inp, cu, S0 = packed_case(wl, lens, seed=21)
    say("varlen: %d sequences, %d tokens" % (len(lens), int(cu[-1])))
    args = [to_torch(inp[n]) for n in ("q", "k", "v", "g", "beta")]
    o, ST = gdn.fwd_chunked_varlen(*args, torch.from_numpy(cu).cuda(), S0=to_torch(S0))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_per_sequence(inp, cu, S0, conv=False)
    check("bf16", o.cpu().numpy(), o_ref, ST.cpu().numpy(), S_ref, "varlen 1101 sequences")


def test_varlen_long_mix_vs_oracle_sampled():
    """A long mix (total 20 000 tokens, 24 sequences) on 128-row workgroups,
    checked on sampled sequences."""
    wl = PREFILL_CONV.with_(Hk=16, Hv=48, conv=False)
    r = np.random.default_rng(11)
    lens = r.integers(0, 1700, 24)
    lens[-1] = 20000 - int(np.sum(lens[:-1])) if np.sum(lens[:-1]) < 20000 else 5
    inp, cu, S0 = packed_case(wl, lens, seed=11)
    say("varlen long mix: %d tokens, %d sequences" % (int(cu[-1]), len(lens)))
    args = [to_torch(inp[n]) for n in ("q", "k", "v", "g", "beta")]
    o, ST = gdn.fwd_chunked_varlen(*args, torch.from_numpy(cu).cuda(), S0=to_torch(S0))
    torch.cuda.synchronize()
    o, ST = o.cpu().numpy(), ST.cpu().numpy()
    q, k, v = (inp[n].f32() for n in ("q", "k", "v"))
    g, beta = inp["g"].f32(), inp["beta"].f32()
    for s in (0, 5, len(lens) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        if e == a:
            continue
        for h in (0, 47):
            os_, Ss = oracle.recurrent(q[:, a:e], k[:, a:e], v[:, a:e], g[:, a:e], beta[:, a:e],
                                       S0[s:s + 1].astype(np.float64), chains=[(0, h)])
            check("bf16", o[0, a:e, h], os_[0], ST[s, h], Ss[0], "long mix seq %d head %d" % (s, h))


def test_varlen_graph_capture():
    """Packed sequences with the prologue inside, captured into a graph and
    replayed with eager work between the replays."""
    wl = PREFILL_CONV.with_(Hk=2, Hv=6)
    lens = [70, 0, 130, 1]
    inp, cu, S0 = packed_case(wl, lens, seed=9, conv=True)
    say("varlen graph capture: lens %s" % lens)
    xs = [to_torch(inp[n]) for n in ("xq", "xk", "xv")]
    w, g, beta = to_torch(inp["conv_w"]), to_torch(inp["g"]), to_torch(inp["beta"])
    cut, S0t = torch.from_numpy(cu).cuda(), to_torch(S0)
    o_e, S_e = gdn.fwd_chunked_conv_varlen(*xs, w, g, beta, cut, S0=S0t)
    o = torch.full_like(o_e, float("nan"))
    ST = torch.full_like(S_e, float("nan"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gdn.fwd_chunked_conv_varlen(*xs, w, g, beta, cut, S0=S0t, o=o, S_T=ST)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.fwd_chunked_conv_varlen(*xs, w, g, beta, cut, S0=S0t, o=o, S_T=ST)
    for rep in range(3):
        o.fill_(float("nan"))
        ST.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(o, o_e) and torch.equal(ST, S_e), "replay %d differs from the eager call" % rep
