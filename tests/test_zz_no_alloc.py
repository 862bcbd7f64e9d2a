"""gdn_fwd_chunked_noalloc, the chunked forward whose chunk matrices live in
the library's own per-device scratch, called through the C ABI: two calls in
a row (the second smaller, so it runs over what the first left in the
scratch) must give gdn_fwd_chunked's results bit for bit, and both must meet
the oracle's bar."""
import ctypes
import sys

import pytest
import torch

import gated_delta_rule_02_amd as gdn
import oracle
from gdn_inputs import KDA_PREFILL, LONG_PREFILL, PREFILL_CONV, TINY_F32, make_prefill, to_torch
from parity import check

pytestmark = pytest.mark.gpu


def say(msg):
    print("[case] " + msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gdn.lib()


def nan_outputs(wl):
    o = torch.full((wl.B, wl.T, wl.Hv, wl.dv), float("nan"), device="cuda")
    ST = torch.full((wl.B, wl.Hv, wl.dv, wl.dk), float("nan"), device="cuda")
    return o, ST


def both(wl, label, chains=None):
    """One problem through the no-allocation form and through gdn_fwd_chunked
    with its own workspace; the two must agree bit for bit and meet the
    oracle's bar on `chains` (all when None)."""
    say("%s: B=%d T=%d Hk=%d Hv=%d C=%d %s gate=%s" % (label, wl.B, wl.T, wl.Hk, wl.Hv, wl.chunk,
                                                       wl.dtype, wl.gate))
    inp = make_prefill(wl)
    args = [to_torch(inp[n]) for n in ("q", "k", "v", "g", "beta")]
    S0 = None if inp["S0"] is None else to_torch(inp["S0"])
    o_n, S_n = nan_outputs(wl)
    L = gdn.lib()
    d = gdn.make_desc(wl.B, wl.T, wl.Hk, wl.Hv, wl.dk, wl.dv, wl.chunk, gdn._DTYPE_CODE[args[0].dtype],
                      gdn._DTYPE_CODE[args[3].dtype],
                      gdn.GATE_HEAD if args[3].dim() == 3 else gdn.GATE_KEY_CHANNEL)
    assert L.gdn_fwd_workspace_bytes(ctypes.byref(d)) <= gdn.NOALLOC_SCRATCH_BYTES
    P = lambda t: ctypes.c_void_p(None if t is None else t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    gdn.check(L.gdn_fwd_chunked_noalloc(ctypes.byref(d), *(P(a) for a in args), P(S0), P(o_n), P(S_n),
                                        stream))
    o_w, S_w = nan_outputs(wl)
    gdn.fwd_chunked(*args, S0=S0, chunk=wl.chunk, o=o_w, S_T=S_w)
    torch.cuda.synchronize()
    assert torch.equal(o_n, o_w), label + ": o differs from gdn_fwd_chunked"
    assert torch.equal(S_n, S_w), label + ": S_T differs from gdn_fwd_chunked"
    sel = list(range(wl.B * wl.Hv)) if chains is None else chains
    pairs = [(c // wl.Hv, c % wl.Hv) for c in sel]
    o_ref, S_ref = oracle.recurrent(*(inp[n].f32() for n in ("q", "k", "v", "g", "beta")), inp["S0"],
                                    chains=pairs)
    o_g = o_n.permute(0, 2, 1, 3).reshape(wl.B * wl.Hv, wl.T, wl.dv)[sel].cpu().numpy()
    S_g = S_n.reshape(wl.B * wl.Hv, wl.dv, wl.dk)[sel].cpu().numpy()
    check("f32" if wl.dtype == "f32" else "bf16", o_g, o_ref, S_g, S_ref, label)


SMALL = LONG_PREFILL.with_(B=3, T=300, Hk=2, Hv=6)


def test_head_gate_two_calls():
    both(SMALL, "head gate, first call")
    both(SMALL.with_(B=1, T=130), "head gate, second call, smaller")


def test_key_gate_two_calls():
    kda = KDA_PREFILL.with_(B=2, T=150, Hk=1, Hv=3, s0_std=0.05)
    both(kda, "key gate, first call")
    both(kda.with_(B=1, T=65), "key gate, second call, smaller")


def test_fp32_mode_two_calls():
    # fp32 mode keeps nothing in a workspace: the scratch is not touched
    both(TINY_F32.with_(T=100), "fp32, first call")
    both(TINY_F32.with_(T=17), "fp32, second call, smaller")


def test_largest_then_smaller():
    # the headline prefill (12288 (sequence, value head, chunk) triples, 87 MiB
    # of chunk matrices) fills most of the scratch; then one long sequence,
    # which gdn_fwd_chunked splits over a side stream and this form does not
    wl = PREFILL_CONV.with_(conv=False)
    both(wl, "B4 T4096 Hv48, first call", chains=[0, 47, 100, 191])
    both(LONG_PREFILL.with_(T=4096), "B1 T4096 Hv48, second call, smaller", chains=[0, 13, 47])


def test_too_large_is_rejected_and_leaves_later_calls_intact():
    wl = LONG_PREFILL.with_(T=48 * 1024)   # 768 chunks x 48 heads: 261 MiB
    d = gdn.make_desc(wl.B, wl.T, wl.Hk, wl.Hv, 128, 128, 64, gdn.BF16, gdn.BF16, gdn.GATE_HEAD)
    L = gdn.lib()
    assert L.gdn_fwd_workspace_bytes(ctypes.byref(d)) > gdn.NOALLOC_SCRATCH_BYTES
    # distinct aligned addresses that are never dereferenced: the size is
    # checked on the host before anything is enqueued
    p = [ctypes.c_void_p((1 << 20) + i * (1 << 36)) for i in range(7)]
    st = L.gdn_fwd_chunked_noalloc(ctypes.byref(d), *p[:5], None, p[5], p[6], None)
    assert st == 5 and b"no-allocation" in L.gdn_last_error()
    both(SMALL.with_(T=70), "after a rejected call")
