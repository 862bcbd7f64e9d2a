"""Properties of the GPU path that hold bit for bit, whatever the rounding:
causality, resuming from a returned state, and grouped heads against
explicitly repeated ones.

- Causality (the "SinkProbe" page lists delta-rule causality among its
  tests): changing the inputs of token t' leaves every output before t'
  unchanged.  In the chunked kernels the later tokens of a chunk enter the
  earlier rows' results only through entries that the triangular masks set
  to zero, so the earlier outputs keep their bits; with the prologue inside,
  token t' reaches outputs t' .. t' + 3 only.
- Resume (the state is the carry between calls, "Source notes", "Linear
  attention"): a prefill of T1 tokens, a multiple of the chunk size, then a
  prefill of T2 tokens from the returned state equals one prefill of
  T1 + T2 tokens: the chunks and their arithmetic are the same.
- Grouped heads (key head of value head h is h / (Hv / Hk)): the call with
  grouped key heads equals the call with every key head repeated for its
  value heads.
"""
import sys

import pytest
import torch

import gated_delta_rule_02_amd as gdn
from gdn_inputs import KDA_PREFILL, LONG_PREFILL, PREFILL_CONV, TINY_F32, make_prefill, to_torch

pytestmark = pytest.mark.gpu


def say(msg):
    print("[case] " + msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gdn.lib()


def inputs(wl):
    inp = make_prefill(wl)
    args = [to_torch(inp[n]) for n in ("q", "k", "v", "g", "beta")]
    S0 = None if inp["S0"] is None else to_torch(inp["S0"])
    return args, S0


def perturb_token(args, tp):
    """New q, k, v, g, beta with token tp of every sequence and head changed
    (q and k stay unit rows, g and beta stay in range)."""
    q, k, v, g, beta = (a.clone() for a in args)
    q[:, tp] = torch.roll(q[:, tp], 1, dims=-1)
    k[:, tp] = -k[:, tp]
    v[:, tp] = v[:, tp] * 0.5 + 0.25
    g[:, tp] = g[:, tp] * 0.5
    beta[:, tp] = 1.0 - beta[:, tp]
    return [q, k, v, g, beta]


CAUSAL = {
    # 12 chains: 32-row workgroups, P from the workspace
    "head gate, 32-row workgroups": LONG_PREFILL.with_(B=2, T=200, Hk=2, Hv=6),
    # 144 chains: 128-row workgroups, P formed in the pass
    "head gate, 128-row workgroups": LONG_PREFILL.with_(B=3, T=150, Hk=16, Hv=48, s0_std=0.0),
    "key gate": KDA_PREFILL.with_(B=2, T=150, Hk=1, Hv=3, s0_std=0.05),
    "fp32 mode": TINY_F32.with_(T=50),
}


@pytest.mark.parametrize("name", list(CAUSAL))
def test_causality_bitwise(name):
    wl = CAUSAL[name]
    tp = wl.T * 2 // 3
    say("causality %s: B=%d T=%d Hk=%d Hv=%d C=%d, token %d changed" % (name, wl.B, wl.T, wl.Hk, wl.Hv,
                                                                          wl.chunk, tp))
    args, S0 = inputs(wl)
    o1, S1 = gdn.fwd_chunked(*args, S0=S0, chunk=wl.chunk)
    o2, S2 = gdn.fwd_chunked(*perturb_token(args, tp), S0=S0, chunk=wl.chunk)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :tp], o2[:, :tp]), "an output before the changed token differs"
    assert not torch.equal(o1[:, tp], o2[:, tp]), "the changed token's output did not change"
    assert not torch.equal(S1, S2)


def test_causality_bitwise_prologue_inside():
    """Raw inputs of token t' changed: with the convolution inside the chunked
    kernels, every output before t' keeps its bits."""
    wl = PREFILL_CONV.with_(B=2, T=200, Hk=2, Hv=6)
    tp = 133
    say("causality, prologue inside: B=%d T=%d Hk=%d Hv=%d, raw token %d changed" % (wl.B, wl.T, wl.Hk,
                                                                                      wl.Hv, tp))
    inp = make_prefill(wl)
    raw = [to_torch(inp[n]) for n in ("xq", "xk", "xv")]
    rest = [to_torch(inp["conv_w"]), to_torch(inp["g"]), to_torch(inp["beta"])]
    o1, _ = gdn.fwd_chunked_conv(*raw, *rest, chunk=wl.chunk)
    raw2 = [x.clone() for x in raw]
    for x in raw2:
        x[:, tp] = x[:, tp] * -0.5 + 0.125
    o2, _ = gdn.fwd_chunked_conv(*raw2, *rest, chunk=wl.chunk)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :tp], o2[:, :tp]), "an output before the changed token differs"
    assert not torch.equal(o1[:, tp], o2[:, tp])


RESUME = {
    "head gate bf16": (LONG_PREFILL.with_(B=2, T=200, Hk=2, Hv=6), 128),
    "head gate bf16, 128-row workgroups": (LONG_PREFILL.with_(B=3, T=150, Hk=16, Hv=48), 64),
    "key gate bf16": (KDA_PREFILL.with_(B=2, T=150, Hk=1, Hv=3, s0_std=0.05), 64),
    "fp32 mode": (TINY_F32.with_(T=50), 32),
}


@pytest.mark.parametrize("name", list(RESUME))
def test_resume_bitwise(name):
    wl, T1 = RESUME[name]
    say("resume %s: B=%d T=%d split at %d, C=%d" % (name, wl.B, wl.T, T1, wl.chunk))
    args, S0 = inputs(wl)
    o, ST = gdn.fwd_chunked(*args, S0=S0, chunk=wl.chunk)
    first = [a[:, :T1].contiguous() for a in args]
    second = [a[:, T1:].contiguous() for a in args]
    oa, Sa = gdn.fwd_chunked(*first, S0=S0, chunk=wl.chunk)
    ob, Sb = gdn.fwd_chunked(*second, S0=Sa, chunk=wl.chunk)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([oa, ob], dim=1), o), "outputs differ"
    assert torch.equal(Sb, ST), "final states differ"


@pytest.mark.parametrize("gate", ["head", "key"])
def test_grouped_heads_equal_repeated_bitwise(gate):
    """Hk = 2 key heads for Hv = 6 value heads against Hk = 6 with each key
    head's q and k repeated for its three value heads."""
    wl = (LONG_PREFILL.with_(B=2, T=150, Hk=2, Hv=6) if gate == "head"
          else KDA_PREFILL.with_(B=2, T=150, Hk=2, Hv=6, s0_std=0.05))
    say("grouped vs repeated heads, %s gate: B=%d T=%d Hk=%d Hv=%d" % (gate, wl.B, wl.T, wl.Hk, wl.Hv))
    args, S0 = inputs(wl)
    grp = wl.Hv // wl.Hk
    rep = [args[0].repeat_interleave(grp, dim=2).contiguous(), args[1].repeat_interleave(grp, dim=2).contiguous()]
    o1, S1 = gdn.fwd_chunked(*args, S0=S0, chunk=wl.chunk)
    o2, S2 = gdn.fwd_chunked(*rep, *args[2:], S0=S0, chunk=wl.chunk)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
