"""Throughput benchmark of the Gated DeltaNet forward hot path on one MI355X.

One step = the whole hot path over one batch of the conv-prologue prefill
workload (B 4, T 4096, 16 key / 48 value heads, d 128, chunk 64, bf16
inputs): 4-tap conv + SiLU + L2 prologue -> chunked prefill (fp16 matrix
cores, fp32 state) -> one decode step from the final state on a fresh token.
The prologue runs inside the chunked kernels (gdn_fwd_chunked_conv, the same
results as gdn_prologue followed by gdn_fwd_chunked); the two separate calls
are timed too and reported under "workloads".
`value` is prefill tokens/s of that step (B*T / step time).  Inputs are
seeded synthetic data resident in HBM before the timed region.

Also reported on the same line (each timed with HIP events on the stream the
kernels run on):
  roofline      the dominant kernel (the chunked forward with the prologue
                inside: prep + sequential launches) against the dense fp16
                matrix-core peak;
  kernels       prologue and decode against the HBM peak;
  decode        steps/s of the batched-decode workload (B 256, 1000 steps);
  workloads     the chunked forward on the long-prefill workload (B 1, T 65536,
                S0 given, slow decay) and on the per-key-channel-gate workload
                (B 2, 32 heads, T 8192), tokens/s and fractions of both roofs;
                and the step's prefill followed by the gated output norm (RMS
                norm x gain x SiLU gate, bf16 out): inside the sequential pass
                (gdn_fwd_chunked_conv_gated) against the forward followed by
                gdn_output_gate; the step's 16 384 tokens as 16 packed
                sequences of mixed lengths (gdn_fwd_chunked_conv_varlen); and
                the backward of the step's prefill (gdn_bwd: chunked, fp32
                matrix cores); the same forward without the delta correction;
  cpu_baseline  the fp64 oracle on the host cores on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --calibrate-copy   (a plain 1 GiB device copy, five times: the
                                          reference for scaling rocprofv3 HBM byte counters)
       python bench.py --profile-steps N  (N steps only, no JSON line: the program that
                                          hardware-counter passes profile)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, GB/s
PEAK_F16_TFLOPS = 2500.0         # MI355X dense fp16/bf16 matrix cores, TFLOP/s
PEAK_F32_TFLOPS = 157.3          # MI355X fp32 (matrix and vector), TFLOP/s
FLOPS_PER_TOKEN_HEAD = 180224    # algorithmic prefill flops per (token, value head) at C 64, d 128
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "chunk_fwd_prefill_conv_B4_T4096_pmc.txt")
# the sources the chunked kernels are compiled from
KERNEL_SOURCES = [os.path.join(ROOT, "gated_delta_rule_02_amd", "csrc", f) for f in ("chunk_mfma.hip", "gdn_device.h")]


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def source_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the chunked forward from the committed rocprofv3
    summary, or None when the kernel source changed since it was taken."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    fields = dict(line.split("=", 1) for line in text.splitlines() if "=" in line and not line.startswith("#"))
    if fields.get("kernel_source_sha256_16", "").strip() != source_hash(KERNEL_SOURCES):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_cpu():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def warm_up(fn, seconds=0.03):
    """Call fn until `seconds` of wall time have passed (at least twice), so
    that the GPU's clocks have come up before a timed region."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < 2 or time.perf_counter() - t0 < seconds:
        fn()
        torch.cuda.synchronize()
        n += 1


def time_events(fn, reps, stream, repeats=3, warm=0.05):
    """Seconds per call of fn: `reps` calls between two HIP events recorded on
    `stream` (the stream the kernels are launched on), after a time-based
    warm-up; the median over `repeats` such timings."""
    import torch
    warm_up(fn, warm)
    times = []
    for _ in range(repeats):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / reps / 1e3)
    return sorted(times)[len(times) // 2]


def git_sha():
    """The commit of the working tree; where there is no git history, the
    commit the library was built from (recorded by the build next to it), or
    None."""
    import subprocess
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        if r.returncode == 0 and r.stdout.strip():
            return r.stdout.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open(os.path.join(ROOT, "gated_delta_rule_02_amd", "build_info.json")) as f:
            info = json.load(f)
        sha = info.get("git_sha")
        if sha and info.get("sources_modified_since_commit"):
            sha += "+modified"
        return sha
    except (OSError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU's clocks take some milliseconds of load to come up from idle: the
    # default warm-up runs about 20 ms of steps, the timed region about 70 ms
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=0)
    ap.add_argument("--profile-workload", choices=["step", "long", "key"], default="step",
                    help="with --profile-steps: the bench step, the long prefill or the key-gate prefill")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the forward pass here runs on a single MI355X "
              "(no multi-GPU path is built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_rule_02_amd as gdn
    from gdn_inputs import BATCHED_DECODE, KDA_PREFILL, LONG_PREFILL, PREFILL_CONV, decode_tokens_device, \
        make_decode_token, make_gate_inputs, make_prefill, make_state, packed_lengths, prefill_device, to_torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)      # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_each_way": src.numel() * 4, "copies": 5}), flush=True)
        return
    stream = torch.cuda.current_stream()
    gdn.lib()

    # ------------------------------------------------------------------ inputs
    wl = PREFILL_CONV
    B, T, Hk, Hv, dk, dv, C = wl.B, wl.T, wl.Hk, wl.Hv, wl.dk, wl.dv, wl.chunk
    log("generating inputs: %s" % wl.name)
    inp = make_prefill(wl)
    xq, xk, xv = (to_torch(inp[n], dev) for n in ("xq", "xk", "xv"))
    w = to_torch(inp["conv_w"], dev)
    g, beta = to_torch(inp["g"], dev), to_torch(inp["beta"], dev)
    tok = make_decode_token(wl, 0)
    dq, dk_, dv_, dg, db = (to_torch(tok[n], dev) for n in ("q", "k", "v", "g", "beta"))
    q = torch.empty((B, T, Hk, dk), dtype=torch.float16, device=dev)
    k = torch.empty_like(q)
    v = torch.empty((B, T, Hv, dv), dtype=torch.float16, device=dev)
    o = torch.empty((B, T, Hv, dv), dtype=torch.float32, device=dev)
    ST = torch.empty((B, Hv, dv, dk), dtype=torch.float32, device=dev)
    od = torch.empty((B, Hv, dv), dtype=torch.float32, device=dev)
    L = gdn.lib()
    desc = gdn.make_desc(B, T, Hk, Hv, dk, dv, C, gdn.F16, gdn.BF16, gdn.GATE_HEAD)
    ws = torch.empty(L.gdn_fwd_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    cws = torch.empty(L.gdn_fwd_conv_workspace_bytes(desc, gdn.BF16), dtype=torch.uint8, device=dev)
    import ctypes
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    pdesc = gdn.make_desc(B, T, Hk, Hv, dk, dv, C, gdn.F16, gdn.F32, gdn.GATE_HEAD)
    ddesc = gdn.make_desc(B, 1, Hk, Hv, dk, dv, C, gdn.BF16, gdn.BF16, gdn.GATE_HEAD)
    s_ptr = ctypes.c_void_p(stream.cuda_stream)

    def prologue():
        gdn.check(L.gdn_prologue(ctypes.byref(pdesc), gdn.BF16, P(xq), P(xk), P(xv), P(w), 1e-6,
                                 P(q), P(k), P(v), s_ptr))

    def chunked():
        gdn.check(L.gdn_fwd_chunked(ctypes.byref(desc), P(q), P(k), P(v), P(g), P(beta), None,
                                    P(o), P(ST), P(ws), ws.numel(), s_ptr))

    def fused():
        gdn.check(L.gdn_fwd_chunked_conv(ctypes.byref(desc), gdn.BF16, P(xq), P(xk), P(xv), P(w), 1e-6,
                                         P(g), P(beta), None, P(o), P(ST), P(cws), cws.numel(), s_ptr))

    def decode():
        gdn.check(L.gdn_decode_step(ctypes.byref(ddesc), P(dq), P(dk_), P(dv_), P(dg), P(db), P(ST),
                                    P(od), s_ptr))

    def step():
        fused()
        decode()

    def chunked_call(xwl):
        """One gdn_fwd_chunked call of workload xwl on device-drawn inputs."""
        xi = prefill_device(xwl, dev)
        xo = torch.empty((xwl.B, xwl.T, xwl.Hv, xwl.dv), dtype=torch.float32, device=dev)
        xst = torch.empty((xwl.B, xwl.Hv, xwl.dv, xwl.dk), dtype=torch.float32, device=dev)
        gate = gdn.GATE_HEAD if xwl.gate == "head" else gdn.GATE_KEY_CHANNEL
        xd = gdn.make_desc(xwl.B, xwl.T, xwl.Hk, xwl.Hv, xwl.dk, xwl.dv, xwl.chunk, gdn.BF16, gdn.BF16, gate)
        xws = torch.empty(L.gdn_fwd_workspace_bytes(xd), dtype=torch.uint8, device=dev)

        def xrun():
            gdn.check(L.gdn_fwd_chunked(ctypes.byref(xd), P(xi["q"]), P(xi["k"]), P(xi["v"]), P(xi["g"]),
                                        P(xi["beta"]), None if xi["S0"] is None else P(xi["S0"]),
                                        P(xo), P(xst), P(xws), xws.numel(), s_ptr))
        return xrun, xi, xo, xst, xd, xws

    if args.profile_steps > 0:
        fn = step if args.profile_workload == "step" else \
            chunked_call(LONG_PREFILL if args.profile_workload == "long" else KDA_PREFILL)[0]
        for _ in range(args.profile_steps):
            fn()
        torch.cuda.synchronize()
        log("%d profile steps done (%s)" % (args.profile_steps, args.profile_workload))
        return

    # ------------------------------------------------------------------ timed steps
    log("warmup %d, timed %d steps, 3 times" % (args.warmup, args.steps))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the GPU's clocks need some milliseconds of load to come up from idle,
    # whatever --warmup asks for
    warm_up(step, 0.1)
    step_reps = []
    for _ in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        step_reps.append((time.perf_counter() - t0) / args.steps)
    t_step = sorted(step_reps)[1]
    tokens_per_s = B * T / t_step
    log("step %.1f us (median of %s) -> %.3e tokens/s" %
        (t_step * 1e6, ", ".join("%.1f" % (x * 1e6) for x in step_reps), tokens_per_s))
    # the step's outputs, kept for the parity check against the oracle below
    fused()
    torch.cuda.synchronize()
    o_step, ST_step = o.cpu().numpy(), ST.cpu().numpy()
    decode()
    torch.cuda.synchronize()
    od_step = od.cpu().numpy()

    # ------------------------------------------------------------------ per-kernel (HIP events)
    reps = max(5, args.steps)
    t_fus = time_events(fused, reps, stream)
    t_pro = time_events(prologue, reps, stream)
    t_chk = time_events(chunked, reps, stream)
    ndesc = gdn.make_desc(B, T, Hk, Hv, dk, dv, C, gdn.F16, gdn.BF16, gdn.GATE_HEAD, gdn.RULE_NO_DELTA)

    def chunked_nd():
        gdn.check(L.gdn_fwd_chunked(ctypes.byref(ndesc), P(q), P(k), P(v), P(g), P(beta), None,
                                    P(o), P(ST), P(ws), ws.numel(), s_ptr))

    t_nd = time_events(chunked_nd, reps, stream)
    bytes_pro = (2 * B * T * Hk * dk + B * T * Hv * dv) * (2 + 2) + w.numel() * 4
    # the same bytes whether q, k, v or the raw inputs are read (both 2 bytes each)
    bytes_chk = (2 * B * T * Hk * dk + B * T * Hv * dv) * 2 + 2 * B * T * Hv * 2 \
        + B * T * Hv * dv * 4 + B * Hv * dv * dk * 4
    bytes_fus = bytes_chk + w.numel() * 4
    flops_chk = FLOPS_PER_TOKEN_HEAD * B * T * Hv
    achieved = flops_chk / t_fus / 1e12
    traffic = read_traffic()
    log("chunked with prologue inside %.1f us (%.1f TFLOP/s, %.0f GB/s algorithmic); separately: "
        "prologue %.1f us (%.0f GB/s) + chunked %.1f us" %
        (t_fus * 1e6, achieved, bytes_fus / t_fus / 1e9, t_pro * 1e6, bytes_pro / t_pro / 1e9, t_chk * 1e6))

    # ------------------------------------------------------------------ batched decode workload
    dwl = BATCHED_DECODE
    nsteps = args.decode_steps
    log("decode workload: %s, %d steps" % (dwl.name, nsteps))
    S_init = to_torch(make_state(dwl), dev)
    S = S_init.clone()
    toks = decode_tokens_device(dwl, nsteps, dev)
    od2 = torch.empty((dwl.B, dwl.Hv, dwl.dv), dtype=torch.float32, device=dev)
    d3 = gdn.make_desc(dwl.B, 1, dwl.Hk, dwl.Hv, dwl.dk, dwl.dv, 64, gdn.BF16, gdn.BF16, gdn.GATE_HEAD)
    tq, tk, tv, tg, tb = (toks[n] for n in ("q", "k", "v", "g", "beta"))

    def decode_run():
        for s in range(nsteps):
            gdn.check(L.gdn_decode_step(ctypes.byref(d3), P(tq[s]), P(tk[s]), P(tv[s]), P(tg[s]),
                                        P(tb[s]), P(S), P(od2), s_ptr))

    decode_run()                                   # warm-up pass
    torch.cuda.synchronize()
    t_dec = time_events(decode_run, 1, stream, warm=0) / nsteps
    S.copy_(S_init)
    decode_run()                                   # the eager result the graph must reproduce
    torch.cuda.synchronize()
    bytes_dec = 2 * S.numel() * 4 + od2.numel() * 4 + (2 * dwl.B * dwl.Hk * dwl.dk + dwl.B * dwl.Hv * dwl.dv) * 2 \
        + 2 * dwl.B * dwl.Hv * 2
    log("decode %.1f us/step, %.0f steps/s, %.0f GB/s" % (t_dec * 1e6, 1 / t_dec, bytes_dec / t_dec / 1e9))
    # the same loop captured into one HIP graph (1000 kernel nodes); its final
    # state and last output must equal the eager loop's
    S_eager, o_eager = S.clone(), od2.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for st in range(nsteps):
            gdn.check(L.gdn_decode_step(ctypes.byref(d3), P(tq[st]), P(tk[st]), P(tv[st]), P(tg[st]),
                                        P(tb[st]), P(S), P(od2), cap))
    S.copy_(S_init)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    graph_equal = bool(torch.equal(S, S_eager) and torch.equal(od2, o_eager))
    t_dec_graph = time_events(graph.replay, 1, stream, warm=0) / nsteps
    log("decode as one graph %.1f us/step (final state %s the eager loop's)" %
        (t_dec_graph * 1e6, "equals" if graph_equal else "DIFFERS FROM"))
    # the same steps from raw inputs through the convolution history
    # (gdn_decode_step_conv: the decode prologue, then the decode step); the
    # step's tokens serve as the raw inputs
    cst = torch.zeros((dwl.B, 3, 2 * dwl.Hk * dwl.dk + dwl.Hv * dwl.dv), dtype=torch.bfloat16, device=dev)
    cws = torch.empty(L.gdn_decode_conv_workspace_bytes(d3), dtype=torch.uint8, device=dev)
    w_dec = to_torch(np.ascontiguousarray(np.random.default_rng(3).normal(
        0, 0.5, (2 * dwl.Hk * dwl.dk + dwl.Hv * dwl.dv, 4)), dtype=np.float32), dev)

    def decode_conv_run():
        for s in range(nsteps):
            gdn.check(L.gdn_decode_step_conv(ctypes.byref(d3), gdn.BF16, P(tq[s]), P(tk[s]), P(tv[s]), P(w_dec),
                                             1e-6, P(cst), P(tg[s]), P(tb[s]), P(S), P(od2), P(cws), cws.numel(),
                                             s_ptr))

    decode_conv_run()
    torch.cuda.synchronize()
    t_dec_conv = time_events(decode_conv_run, 1, stream, warm=0) / nsteps
    log("decode from raw inputs (conv history) %.1f us/step" % (t_dec_conv * 1e6))
    # a sample of the decode workload's chains for the oracle's decode rate:
    # 384 (sequence, value head) chains over the first 100 steps
    dsel = np.random.default_rng(31).choice(dwl.B * dwl.Hv, 384, replace=False)
    dsb = torch.from_numpy(dsel // dwl.Hv).to(dev)
    dsh = torch.from_numpy(dsel % dwl.Hv).to(dev)
    dsk = dsh // (dwl.Hv // dwl.Hk)
    ftok = lambda x: x.float().cpu().numpy()
    dec_sample = {"q": ftok(tq[:100, dsb, dsk]), "k": ftok(tk[:100, dsb, dsk]), "v": ftok(tv[:100, dsb, dsh]),
                  "g": ftok(tg[:100, dsb, dsh]), "beta": ftok(tb[:100, dsb, dsh]),
                  "S0": S_init[dsb, dsh].cpu().numpy()}
    del toks, tq, tk, tv, tg, tb, S, S_init, S_eager, graph, cst, cws

    # ------------------------------------------------------------------ other prefill workloads
    extra = {"prefill_no_delta": {
        "workload": wl.name + ", fp16 q/k/v after the prologue, the update without the delta correction",
        "us_per_call": t_nd * 1e6, "tokens_per_s": B * T / t_nd, "delta_rule_us": t_chk * 1e6},
        "decode_from_raw_inputs": {
        "workload": dwl.name + ", tokens as raw inputs through the 3-token convolution history",
        "us_per_step": t_dec_conv * 1e6, "steps_per_s": 1 / t_dec_conv,
        "hbm_frac_algorithmic": bytes_dec / t_dec_conv / 1e9 / PEAK_HBM_GBS},
        "prefill_conv_two_calls": {
        "workload": wl.name + ", gdn_prologue then gdn_fwd_chunked",
        "us_per_call": (t_pro + t_chk) * 1e6, "tokens_per_s": B * T / (t_pro + t_chk),
        "prologue_us": t_pro * 1e6, "chunked_us": t_chk * 1e6,
        "chunked_mfma_frac": flops_chk / t_chk / 1e12 / PEAK_F16_TFLOPS}}
    # the gated output norm after the step's prefill: inside the sequential
    # pass, and as the forward followed by the standalone gate
    log("workload: %s, then the gated output norm" % wl.name)
    gi = make_gate_inputs(wl)
    z, gain = to_torch(gi["z"], dev), to_torch(gi["gain"], dev)
    y = torch.empty((B, T, Hv, dv), dtype=torch.bfloat16, device=dev)
    gws = torch.empty(L.gdn_fwd_gated_workspace_bytes(desc, gdn.BF16, gdn.BF16), dtype=torch.uint8, device=dev)
    neps = gi["norm_eps"]

    def gated():
        gdn.check(L.gdn_fwd_chunked_conv_gated(ctypes.byref(desc), gdn.BF16, P(xq), P(xk), P(xv), P(w), 1e-6,
                                               P(g), P(beta), None, P(z), P(gain), neps, gdn.BF16, P(y),
                                               P(ST), P(gws), gws.numel(), s_ptr))

    def gate_alone():
        gdn.check(L.gdn_output_gate(ctypes.byref(desc), P(o), gdn.BF16, P(z), P(gain), neps, gdn.BF16, P(y),
                                    s_ptr))

    t_gated = time_events(gated, 20, stream)
    t_gate = time_events(gate_alone, 20, stream)
    bytes_gate = B * T * Hv * dv * (4 + 2 + 2) + dv * 4
    # the forward's algorithmic bytes with y (bf16) read as z and written in place of o (fp32)
    bytes_gated = bytes_fus - B * T * Hv * dv * 4 + B * T * Hv * dv * (2 + 2) + dv * 4
    extra["prefill_conv_gated"] = {
        "workload": wl.name + ", then y = RMSNorm(o) * gain * SiLU(z), bf16 y",
        "us_per_call": t_gated * 1e6, "tokens_per_s": B * T / t_gated,
        "mfma_frac": flops_chk / t_gated / 1e12 / PEAK_F16_TFLOPS,
        "hbm_frac_algorithmic": bytes_gated / t_gated / 1e9 / PEAK_HBM_GBS,
        "two_calls_us": (t_fus + t_gate) * 1e6, "gate_alone_us": t_gate * 1e6,
        "gate_alone_hbm_gbs": bytes_gate / t_gate / 1e9,
        "gate_alone_hbm_frac": bytes_gate / t_gate / 1e9 / PEAK_HBM_GBS}
    log("gated: %.1f us inside the pass; forward + gate %.1f + %.1f us (gate %.0f GB/s)" %
        (t_gated * 1e6, t_fus * 1e6, t_gate * 1e6, bytes_gate / t_gate / 1e9))
    del z, gain, y, gws

    # the step's tokens as packed sequences of mixed lengths (the same inputs,
    # read as one token axis)
    lens = packed_lengths(B * T, 16, wl.seed)
    N = len(lens)
    log("workload: %d tokens as %d packed sequences, lengths %s" % (B * T, N, lens.tolist()))
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
    vdesc = gdn.make_desc(N, B * T, Hk, Hv, dk, dv, C, gdn.F16, gdn.BF16, gdn.GATE_HEAD)
    vws = torch.empty(L.gdn_fwd_conv_varlen_workspace_bytes(vdesc, gdn.BF16), dtype=torch.uint8, device=dev)
    vST = torch.empty((N, Hv, dv, dk), dtype=torch.float32, device=dev)

    def varlen():
        gdn.check(L.gdn_fwd_chunked_conv_varlen(ctypes.byref(vdesc), P(cu), gdn.BF16, P(xq), P(xk), P(xv), P(w),
                                                1e-6, P(g), P(beta), None, P(o), P(vST), P(vws), vws.numel(),
                                                s_ptr))

    t_var = time_events(varlen, 20, stream)
    extra["prefill_conv_varlen"] = {
        "workload": "%d tokens (16 key / 48 value heads, d 128, C 64, bf16, conv prologue) packed as %d "
                    "sequences of mixed lengths" % (B * T, N),
        "lengths": lens.tolist(), "us_per_call": t_var * 1e6, "tokens_per_s": B * T / t_var,
        "mfma_frac": flops_chk / t_var / 1e12 / PEAK_F16_TFLOPS}
    log("packed sequences: %.1f us, %.3e tokens/s (longest %d tokens)" % (t_var * 1e6, B * T / t_var, lens.max()))
    del vws, vST

    # the backward of the step's prefill: q, k, v as the prologue makes them,
    # a random dO; per chunk and value head the workspace holds T, P^T, the
    # state before the chunk, the state gradient after it, U and E (fp32)
    prologue()
    dO = torch.randn((B, T, Hv, dv), device=dev)
    pdesc_bwd = gdn.make_desc(B, T, Hk, Hv, dk, dv, C, gdn.F16, gdn.BF16, gdn.GATE_HEAD)
    bws = torch.empty(L.gdn_bwd_workspace_bytes(pdesc_bwd), dtype=torch.uint8, device=dev)
    log("workload: backward of the prefill (workspace %.2f GB)" % (bws.numel() / 1e9))
    grads = [torch.empty_like(x, dtype=torch.float32) for x in (q, k, v, g, beta)] + [torch.empty_like(ST)]

    def backward():
        gdn.check(L.gdn_bwd(ctypes.byref(pdesc_bwd), P(q), P(k), P(v), P(g), P(beta), None, P(dO), None,
                            *(P(x) for x in grads), P(bws), bws.numel(), s_ptr))

    t_bwd = time_events(backward, 2, stream, warm=0)
    # matrix products per (chunk, value head), multiply-adds: the two passes
    # 5 C dv dk + 3 C^2 dv, the gradients 3 C dv dk + 2 C^2 dv + 4 C^2 dk, the
    # prep C^2 dk (the lower halves of Q K^T and K K^T) + C^3 / 6 (T)
    units = B * Hv * ((T + C - 1) // C)
    bwd_flops = 2 * units * (8 * C * dv * dk + 5 * C * C * dv + 5 * C * C * dk + C ** 3 // 6)
    # the same within a workspace of at most 1 GB (the sequence in segments, a
    # forward pass more for the segment starts)
    del bws
    cap_bytes = L.gdn_bwd_workspace_bytes_within(ctypes.byref(pdesc_bwd), 10 ** 9)
    bws = torch.empty(cap_bytes, dtype=torch.uint8, device=dev)
    t_cap = time_events(backward, 2, stream, warm=0)
    extra["backward"] = {
        "workload": wl.name + ", backward (dq, dk, dv, dg, dbeta, dS0 fp32) from a random dO",
        "us_per_call": t_bwd * 1e6, "tokens_per_s": B * T / t_bwd,
        "tflops": bwd_flops / t_bwd / 1e12, "mfma_f32_frac": bwd_flops / t_bwd / 1e12 / PEAK_F32_TFLOPS,
        "workspace_bytes": int(L.gdn_bwd_workspace_bytes(ctypes.byref(pdesc_bwd))),
        "within_1gb": {"us_per_call": t_cap * 1e6, "workspace_bytes": int(cap_bytes)}}
    log("backward: %.2f ms, %.3e tokens/s, %.1f TFLOP/s = %.1f%% of the fp32 matrix cores; "
        "%.2f ms within a %.2f GB workspace" %
        (t_bwd * 1e3, B * T / t_bwd, bwd_flops / t_bwd / 1e12, 100 * bwd_flops / t_bwd / 1e12 / PEAK_F32_TFLOPS,
         t_cap * 1e3, cap_bytes / 1e9))
    del bws, grads, dO

    for key, xwl in (("long_prefill", LONG_PREFILL), ("key_gate_prefill", KDA_PREFILL)):
        log("workload: %s" % xwl.name)
        xrun, xi, xo, xst, xd, xws = chunked_call(xwl)
        tx = time_events(xrun, 10, stream)
        ntok = xwl.B * xwl.T
        gdim = xwl.dk if xwl.gate == "key" else 1
        xbytes = (2 * ntok * xwl.Hk * xwl.dk + ntok * xwl.Hv * xwl.dv + ntok * xwl.Hv * (gdim + 1)) * 2 \
            + ntok * xwl.Hv * xwl.dv * 4 + (2 if xi["S0"] is not None else 1) * xwl.B * xwl.Hv * xwl.dv * xwl.dk * 4
        xfl = FLOPS_PER_TOKEN_HEAD * ntok * xwl.Hv
        extra[key] = {"workload": xwl.name, "us_per_call": tx * 1e6, "tokens_per_s": ntok / tx,
                      "mfma_tflops": xfl / tx / 1e12, "mfma_frac": xfl / tx / 1e12 / PEAK_F16_TFLOPS,
                      "hbm_gbs_algorithmic": xbytes / tx / 1e9,
                      "hbm_frac_algorithmic": xbytes / tx / 1e9 / PEAK_HBM_GBS}
        log("%s: %.1f us, %.3e tokens/s, %.1f TFLOP/s" % (key, tx * 1e6, ntok / tx, xfl / tx / 1e12))
        if xwl.gate == "key":
            # the backward of the key-gate prefill (chunked, one segment)
            xdO = torch.randn((xwl.B, xwl.T, xwl.Hv, xwl.dv), device=dev)
            xgr = [torch.empty(x.shape, dtype=torch.float32, device=dev) for x in
                   (xi["q"], xi["k"], xi["v"], xi["g"], xi["beta"])] + [torch.empty_like(xst)]
            del xws
            xws = torch.empty(L.gdn_bwd_workspace_bytes(ctypes.byref(xd)), dtype=torch.uint8, device=dev)

            def xback(xi=xi, xd=xd, xws=xws, xgr=xgr, xdO=xdO):
                gdn.check(L.gdn_bwd(ctypes.byref(xd), P(xi["q"]), P(xi["k"]), P(xi["v"]), P(xi["g"]),
                                    P(xi["beta"]), None if xi["S0"] is None else P(xi["S0"]), P(xdO), None,
                                    *(P(x) for x in xgr), P(xws), xws.numel(), s_ptr))

            tb = time_events(xback, 3, stream)
            extra[key]["backward_us_per_call"] = tb * 1e6
            extra[key]["backward_workspace_bytes"] = int(xws.numel())
            log("%s backward: %.2f ms (chunked, workspace %.2f GB)" % (key, tb * 1e3, xws.numel() / 1e9))
            del xdO, xgr
        del xi, xo, xst, xws

    # ------------------------------------------------------------------ CPU baseline (oracle)
    import oracle
    nthreads = min(os.cpu_count() or 1, 16)
    log("cpu baseline: fp64 oracle, prologue + recurrence over the whole prefill workload (%d chains), "
        "%d threads" % (B * Hv, nthreads))
    t0 = time.perf_counter()
    rq, rk, rv = oracle.prologue(inp["xq"].f32(), inp["xk"].f32(), inp["xv"].f32(), inp["conv_w"])
    o_ref, S_ref = oracle.recurrent_full(rq, rk, rv, inp["g"].f32(), inp["beta"].f32(), nthreads=nthreads)
    t_cpu = time.perf_counter() - t0
    cpu_tokens_per_s = B * T / t_cpu
    log("cpu baseline %.1f s -> %.3e tokens/s" % (t_cpu, cpu_tokens_per_s))
    # the same recurrence on one thread, two chains: the rate of one core
    t0 = time.perf_counter()
    oracle.recurrent(rq, rk, rv, inp["g"].f32(), inp["beta"].f32(), None, [(0, 0), (0, 1)], nthreads=1)
    t_one = time.perf_counter() - t0
    one_thread_tokens_per_s = B * T / (t_one * (B * Hv) / 2)
    # the decode workload's sampled chains, 100 steps each, scaled to all 12 288 chains
    ds = dec_sample
    t0 = time.perf_counter()
    oracle.recurrent(ds["q"].transpose(1, 0, 2)[:, :, None], ds["k"].transpose(1, 0, 2)[:, :, None],
                     ds["v"].transpose(1, 0, 2)[:, :, None], ds["g"].T[:, :, None], ds["beta"].T[:, :, None],
                     ds["S0"][:, None], nthreads=nthreads)
    t_dcpu = time.perf_counter() - t0
    cpu_decode_steps_per_s = 100 / (t_dcpu * dwl.B * dwl.Hv / len(ds["S0"]))
    log("cpu baseline: one thread %.3e tokens/s; decode %.2f steps/s" %
        (one_thread_tokens_per_s, cpu_decode_steps_per_s))
    # the timed step's results against the oracle: the prefill's o and S_T,
    # then the decode step from the oracle's S_T
    rms_inf = lambda x, r: float(np.max(np.abs(x - r)) / np.sqrt(np.mean(r * r)))
    rel_inf = lambda x, r: float(np.max(np.abs(x - r)) / np.max(np.abs(r)))
    od_ref, _ = oracle.recurrent(tok["q"].f32()[:, None], tok["k"].f32()[:, None], tok["v"].f32()[:, None],
                                 tok["g"].f32()[:, None], tok["beta"].f32()[:, None], S_ref, nthreads=nthreads)
    step_parity = {"o_max_err_over_rms": rms_inf(o_step, o_ref), "S_T_rel_err": rel_inf(ST_step, S_ref),
                   "decode_o_max_err_over_rms": rms_inf(od_step, od_ref.reshape(od_step.shape)),
                   "bars": {"o": 2e-2, "S_T": 1e-2},
                   "against": "fp64 oracle (prologue + token recurrence) on the step's own inputs"}
    log("step parity: %s" % step_parity)

    line = {
        "metric": "GDN fwd prefill tokens/s + decode steps/s on 1 GPU; % of MFMA/HBM roofline",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "precision": "bf16 inputs; fp16 matrix-core operands; fp32 accumulation, state and output",
        "data": "synthetic",
        "config": {"workload": "prefill with conv prologue, then one decode step", "B": B, "T": T,
                   "Hk": Hk, "Hv": Hv, "dk": dk, "dv": dv, "chunk": C, "gate": "per value head",
                   "step": "chunked prefill with the conv prologue inside (gdn_fwd_chunked_conv) "
                           "+ 1 decode step"},
        "roofline": {"kernel": "chunked forward with the prologue inside (chunk_prep + chunk_seq launches)",
                     "bound": "mfma", "achieved": achieved, "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_F16_TFLOPS, "traffic": traffic,
                     "algorithmic_bytes": bytes_fus, "us_per_launch": t_fus * 1e6,
                     "hbm_frac_algorithmic": bytes_fus / t_fus / 1e9 / PEAK_HBM_GBS,
                     # the bytes the kernels actually move (rocprofv3 counters), per second, against the HBM peak
                     "hbm_frac_traffic": None if traffic is None else traffic / t_fus / 1e9 / PEAK_HBM_GBS},
        "kernels": {
            "prologue": {"bound": "hbm", "achieved": bytes_pro / t_pro / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": bytes_pro / t_pro / 1e9 / PEAK_HBM_GBS,
                         "us_per_launch": t_pro * 1e6},
            "decode": {"bound": "hbm", "achieved": bytes_dec / t_dec / 1e9, "peak": PEAK_HBM_GBS,
                       "unit": "GB/s", "frac": bytes_dec / t_dec / 1e9 / PEAK_HBM_GBS,
                       "us_per_launch": t_dec * 1e6},
        },
        "decode": {"workload": "batched decode: B 256, 16/48 heads, d 128, fp32 state, %d steps" % nsteps,
                   "steps_per_s": 1.0 / t_dec, "tokens_per_s": dwl.B / t_dec,
                   "graph_steps_per_s": 1.0 / t_dec_graph, "graph_equals_eager": graph_equal},
        "workloads": extra,
        "step_parity": step_parity,
        "cpu_baseline": {"value": cpu_tokens_per_s, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
                         "sample": "fp64 prologue + token recurrence over the whole prefill workload "
                                   "(4 x 4096 tokens, all 192 chains); the decode step is not included",
                         "seconds": t_cpu, "host_cpu": host_cpu(), "host_logical_cpus": os.cpu_count(),
                         "one_thread_tokens_per_s": one_thread_tokens_per_s,
                         "one_thread_sample": "2 of the 192 chains, whole length, scaled to all chains",
                         "decode_steps_per_s": cpu_decode_steps_per_s,
                         "decode_sample": "384 of the 12 288 (sequence, value head) chains of the batched "
                                          "decode workload over its first 100 steps, %d threads, scaled to "
                                          "all chains" % nthreads},
        "step_repetitions_ms": [x * 1e3 for x in step_reps],
        "git_sha": git_sha(),
        "source_sha16": source_hash(sorted(os.path.join(ROOT, "gated_delta_rule_02_amd", "csrc", f) for f in
                                           os.listdir(os.path.join(ROOT, "gated_delta_rule_02_amd", "csrc")))
                                    + [os.path.join(ROOT, "bench.py")]),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
