"""Seeded synthetic inputs for the Gated DeltaNet forward pass.

Shared by the oracle tests, the GPU parity tests and the benchmark.  This
module holds none of the method's arithmetic: it draws random numbers, applies
the distribution transforms that the workloads name (L2-normalised normal
vectors, sigmoid, log-sigmoid), and rounds to the stored dtype
(round-to-nearest-even).  The same stored bits go to the GPU and, widened
exactly to float32, to the oracle.

Seeds: every tensor has its own stream,
``numpy.random.Generator(PCG64(SeedSequence([workload_seed, *extra, stream])))``
with streams q=0, k=1, v=2, beta=3, g=4, conv_w=5, S0=6, in that order, and
z=7, gain=8 for the output gate that follows the forward pass.
Normals are drawn in float64 for small tensors and in float32 for tensors of
10**7 elements or more (then widened for the transforms).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

STREAM = {"q": 0, "k": 1, "v": 2, "beta": 3, "g": 4, "conv_w": 5, "S0": 6, "z": 7, "gain": 8}
BIG = 10 ** 7


@dataclass(frozen=True)
class Workload:
    """One synthetic workload of the forward pass (sizes, dtypes, distributions)."""
    name: str
    B: int
    T: int
    Hk: int
    Hv: int
    dk: int
    dv: int
    chunk: int
    dtype: str = "bf16"      # stored dtype of q, k, v, g, beta: "f32" or "bf16"
    gate: str = "head"       # "head": g [B,T,Hv]; "key": g [B,T,Hv,dk]
    g_mu: float = 2.0        # g = logsigmoid(N(g_mu, 1))
    s0_std: float = 0.0      # S0 ~ N(0, s0_std) per entry; 0 means S0 = 0 (absent)
    conv: bool = False       # raw q/k/v go through the conv + SiLU + L2 prologue
    seed: int = 0            # first word of every seed sequence
    decode_steps: int = 0    # > 0: a decode workload (T = 1 per step)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the forward pass.  Reduced copies for quick tests are
# made with Workload.with_().
TINY_F32 = Workload("tiny fp32: B1 H2/2 T64 d16 C16", B=1, T=64, Hk=2, Hv=2, dk=16, dv=16, chunk=16,
                    dtype="f32", g_mu=2.0, seed=0)
PREFILL_CONV = Workload("prefill with conv prologue: B4 Hk16 Hv48 d128 T4096 C64 bf16", B=4, T=4096,
                        Hk=16, Hv=48, dk=128, dv=128, chunk=64, conv=True, g_mu=2.0, seed=1)
LONG_PREFILL = Workload("long prefill: B1 Hk16 Hv48 d128 T65536 C64 bf16, slow decay, S0~N(0,0.02)",
                        B=1, T=65536, Hk=16, Hv=48, dk=128, dv=128, chunk=64, g_mu=4.0, s0_std=0.02,
                        seed=2)
BATCHED_DECODE = Workload("batched decode: B256 Hk16 Hv48 d128, 1000 steps, fp32 state", B=256, T=1,
                          Hk=16, Hv=48, dk=128, dv=128, chunk=64, g_mu=2.0, s0_std=0.02, seed=3,
                          decode_steps=1000)
KDA_PREFILL = Workload("per-key-channel gate: B2 H32/32 d128 T8192 C64 bf16", B=2, T=8192, Hk=32,
                       Hv=32, dk=128, dv=128, chunk=64, gate="key", g_mu=3.0, seed=4)
WORKLOADS = [TINY_F32, PREFILL_CONV, LONG_PREFILL, BATCHED_DECODE, KDA_PREFILL]


def rng(seed: int, stream: str, extra: tuple = ()) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *extra, STREAM[stream]])))


def normal(r: np.random.Generator, shape, mean=0.0, std=1.0) -> np.ndarray:
    n = int(np.prod(shape))
    if n >= BIG:
        x = r.standard_normal(shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        if mean != 0.0:
            x += np.float32(mean)
        return x
    return r.normal(mean, std, size=shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (nearest even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def unit_rows(x: np.ndarray) -> np.ndarray:
    """Scale every last-axis vector to unit Euclidean length (input recipe 'L2-normalised')."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def logsigmoid(x):
    """log(sigmoid(x)) without overflow: -log1p(exp(-x)) for x >= 0, x - log1p(exp(x)) otherwise."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x >= 0, -np.log1p(np.exp(-np.abs(x))), x - np.log1p(np.exp(-np.abs(x))))


class Tensor:
    """A stored tensor: its dtype ("f32" or "bf16") and the raw array
    (float32 values, or uint16 bf16 bit patterns)."""
    __slots__ = ("dtype", "data")

    def __init__(self, dtype: str, data: np.ndarray):
        self.dtype = dtype
        self.data = data

    @property
    def shape(self):
        return self.data.shape

    def f32(self) -> np.ndarray:
        """The exact stored values as float32."""
        return bf16_to_f32(self.data) if self.dtype == "bf16" else self.data


def store(x: np.ndarray, dtype: str) -> Tensor:
    if dtype == "bf16":
        return Tensor("bf16", bf16_bits(x))
    if dtype == "f32":
        return Tensor("f32", np.ascontiguousarray(x, dtype=np.float32))
    raise ValueError(dtype)


def make_gates(wl: Workload, shape_bt, extra: tuple = ()):
    """beta = sigmoid(N(0,1)) [.., Hv]; g = logsigmoid(N(g_mu,1)) [.., Hv] or [.., Hv, dk]."""
    beta = sigmoid(normal(rng(wl.seed, "beta", extra), (*shape_bt, wl.Hv)))
    gshape = (*shape_bt, wl.Hv) if wl.gate == "head" else (*shape_bt, wl.Hv, wl.dk)
    g = logsigmoid(normal(rng(wl.seed, "g", extra), gshape, mean=wl.g_mu))
    return store(beta, wl.dtype), store(g, wl.dtype)


def make_prefill(wl: Workload) -> dict:
    """Inputs of one forward call.

    Without conv: q, k = unit_rows(N(0,1)) [B,T,Hk,dk]; v ~ N(0,1) [B,T,Hv,dv].
    With conv: raw xq, xk [B,T,Hk,dk] and xv [B,T,Hv,dv] ~ N(0,1) and conv_w
    [Hk*dk*2 + Hv*dv, 4] ~ N(0, 0.5) (float32); q, k, v are then the prologue's
    outputs and are not part of the returned dict.
    beta, g as in make_gates; S0 ~ N(0, s0_std) [B,Hv,dv,dk] float32, or None.
    """
    B, T = wl.B, wl.T
    out = {}
    if wl.conv:
        out["xq"] = store(normal(rng(wl.seed, "q"), (B, T, wl.Hk, wl.dk)), wl.dtype)
        out["xk"] = store(normal(rng(wl.seed, "k"), (B, T, wl.Hk, wl.dk)), wl.dtype)
        out["xv"] = store(normal(rng(wl.seed, "v"), (B, T, wl.Hv, wl.dv)), wl.dtype)
    else:
        out["q"] = store(unit_rows(normal(rng(wl.seed, "q"), (B, T, wl.Hk, wl.dk))), wl.dtype)
        out["k"] = store(unit_rows(normal(rng(wl.seed, "k"), (B, T, wl.Hk, wl.dk))), wl.dtype)
        out["v"] = store(normal(rng(wl.seed, "v"), (B, T, wl.Hv, wl.dv)), wl.dtype)
    out["beta"], out["g"] = make_gates(wl, (B, T))
    if wl.conv:
        nch = 2 * wl.Hk * wl.dk + wl.Hv * wl.dv
        out["conv_w"] = np.ascontiguousarray(normal(rng(wl.seed, "conv_w"), (nch, 4), std=0.5),
                                             dtype=np.float32)
    out["S0"] = make_state(wl)
    return out


def make_state(wl: Workload) -> Optional[np.ndarray]:
    """S0 ~ N(0, s0_std) [B,Hv,dv,dk] float32, or None when s0_std == 0."""
    if wl.s0_std == 0.0:
        return None
    return np.ascontiguousarray(normal(rng(wl.seed, "S0"), (wl.B, wl.Hv, wl.dv, wl.dk), std=wl.s0_std),
                                dtype=np.float32)


def make_gate_inputs(wl: Workload) -> dict:
    """Inputs of the gated output norm after the forward pass: the gate
    z ~ N(0,1) [B,T,Hv,dv] in the workload dtype (like the raw projections),
    and one gain vector 1 + N(0, 0.1) [dv] float32 (a learned gain near its
    initial value of one), plus the norm's eps = 1e-5."""
    z = store(normal(rng(wl.seed, "z"), (wl.B, wl.T, wl.Hv, wl.dv)), wl.dtype)
    gain = np.ascontiguousarray(1.0 + normal(rng(wl.seed, "gain"), (wl.dv,), std=0.1), dtype=np.float32)
    return {"z": z, "gain": gain, "norm_eps": 1e-5}


def packed_lengths(total: int, n: int, seed: int) -> np.ndarray:
    """Lengths of n packed sequences summing to total: a seeded mix of short
    and long prompts, log-uniform between a quarter and four times the mean
    length, rescaled to the total, every length at least 1.  int32 [n]."""
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    mean = total / n
    raw = np.exp(r.uniform(np.log(mean / 4), np.log(mean * 4), n))
    lens = np.maximum(1, np.floor(raw / raw.sum() * total)).astype(np.int64)
    lens[np.argmax(lens)] += total - int(lens.sum())
    return lens.astype(np.int32)


def make_decode_token(wl: Workload, step: int) -> dict:
    """Fresh tokens of decode step `step` (0-based): q, k [B,Hk,dk] unit rows, v [B,Hv,dv] ~ N(0,1),
    beta, g [B,Hv] (or g [B,Hv,dk]).  Seeds [seed, 1 + step, stream]."""
    extra = (1 + step,)
    B = wl.B
    out = {
        "q": store(unit_rows(normal(rng(wl.seed, "q", extra), (B, wl.Hk, wl.dk))), wl.dtype),
        "k": store(unit_rows(normal(rng(wl.seed, "k", extra), (B, wl.Hk, wl.dk))), wl.dtype),
        "v": store(normal(rng(wl.seed, "v", extra), (B, wl.Hv, wl.dv)), wl.dtype),
    }
    out["beta"], out["g"] = make_gates(wl, (B,), extra)
    return out


def to_torch(t, device="cuda"):
    """Upload a stored tensor (Tensor, or a float32 ndarray) as a contiguous torch tensor
    with the same bits (bfloat16 or float32)."""
    import torch
    if isinstance(t, Tensor):
        if t.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(t.data)).to(device)
    return torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).to(device)


def decode_tokens_device(wl: Workload, steps: int, device="cuda", first_step: int = 0):
    """Fresh tokens for `steps` decode steps drawn on the device (fast path for the
    1000-step workload): q, k [steps,B,Hk,dk] unit rows, v [steps,B,Hv,dv] ~ N(0,1),
    beta = sigmoid(N(0,1)), g = logsigmoid(N(g_mu,1)), all rounded to bf16 (or kept fp32).
    Step s uses torch.Generator seeded with (seed, 1 + s) mixed into one 64-bit word;
    the same seeds give the same tokens on the same device type."""
    import torch
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    B = wl.B
    outs = {n: [] for n in ("q", "k", "v", "beta", "g")}
    gen = torch.Generator(device=device)
    for s in range(first_step, first_step + steps):
        gen.manual_seed((wl.seed * 1_000_003 + 1 + s) & 0x7FFFFFFFFFFFFFFF)
        q = torch.randn((B, wl.Hk, wl.dk), generator=gen, device=device, dtype=torch.float32)
        k = torch.randn((B, wl.Hk, wl.dk), generator=gen, device=device, dtype=torch.float32)
        v = torch.randn((B, wl.Hv, wl.dv), generator=gen, device=device, dtype=torch.float32)
        bx = torch.randn((B, wl.Hv), generator=gen, device=device, dtype=torch.float32)
        gshape = (B, wl.Hv) if wl.gate == "head" else (B, wl.Hv, wl.dk)
        gx = torch.randn(gshape, generator=gen, device=device, dtype=torch.float32) + wl.g_mu
        outs["q"].append((q / q.norm(dim=-1, keepdim=True)).to(dt))
        outs["k"].append((k / k.norm(dim=-1, keepdim=True)).to(dt))
        outs["v"].append(v.to(dt))
        outs["beta"].append(torch.sigmoid(bx).to(dt))
        outs["g"].append(torch.nn.functional.logsigmoid(gx).to(dt))
    return {n: torch.stack(x).contiguous() for n, x in outs.items()}


def prefill_device(wl: Workload, device="cuda"):
    """Inputs of one forward call drawn on the device (fast path for timing the
    large workloads; the parity tests use make_prefill): q, k [B,T,Hk,dk] unit
    rows, v [B,T,Hv,dv] ~ N(0,1), beta = sigmoid(N(0,1)), g = logsigmoid(N(g_mu,1))
    ([B,T,Hv] or [B,T,Hv,dk]), rounded to the workload dtype; S0 ~ N(0, s0_std)
    fp32 or None.  Seeded with the workload seed on torch's device generator.
    Workloads with the conv prologue are not covered (their raw inputs differ)."""
    import torch
    assert not wl.conv
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed((wl.seed * 1_000_003) & 0x7FFFFFFFFFFFFFFF)
    B, T = wl.B, wl.T

    def unit(shape):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return (x / x.norm(dim=-1, keepdim=True)).to(dt)

    out = {"q": unit((B, T, wl.Hk, wl.dk)), "k": unit((B, T, wl.Hk, wl.dk))}
    out["v"] = torch.randn((B, T, wl.Hv, wl.dv), generator=gen, device=device, dtype=torch.float32).to(dt)
    out["beta"] = torch.sigmoid(torch.randn((B, T, wl.Hv), generator=gen, device=device)).to(dt)
    gshape = (B, T, wl.Hv) if wl.gate == "head" else (B, T, wl.Hv, wl.dk)
    out["g"] = torch.nn.functional.logsigmoid(
        torch.randn(gshape, generator=gen, device=device) + wl.g_mu).to(dt)
    out["S0"] = None if wl.s0_std == 0.0 else \
        torch.randn((B, wl.Hv, wl.dv, wl.dk), generator=gen, device=device) * wl.s0_std
    return out
