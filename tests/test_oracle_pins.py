"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: a worked
example done by hand, closed forms, the page's own DeltaNet rule in its own
(K x V) orientation, a product-of-matrices history expansion, a second
(chunkwise) formulation, invariances (causality, resume, grouped heads,
channel permutation) and a textbook convolution.  A plausible slip in the
oracle (a dropped decay, the read before the write, a wrong sign, a wrong
head grouping, the conv taps reversed) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.chunked import chunked
from gdn_inputs import logsigmoid, sigmoid, unit_rows

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_problem(seed, B=1, T=12, Hk=1, Hv=1, dk=6, dv=5, gate="head", s0=True, g_mu=1.0):
    r = np.random.default_rng(seed)
    q = unit_rows(r.standard_normal((B, T, Hk, dk)))
    k = unit_rows(r.standard_normal((B, T, Hk, dk)))
    v = r.standard_normal((B, T, Hv, dv))
    beta = sigmoid(r.standard_normal((B, T, Hv)))
    gshape = (B, T, Hv) if gate == "head" else (B, T, Hv, dk)
    g = logsigmoid(r.normal(g_mu, 1.0, gshape))
    S0 = r.normal(0, 0.5, (B, Hv, dv, dk)) if s0 else None
    # the oracle reads float32 values: hand it values that float32 holds exactly
    f = lambda a: None if a is None else a.astype(np.float32).astype(np.float64)
    return f(q), f(k), f(v), f(g), f(beta), f(S0)


def run(q, k, v, g, beta, S0=None):
    return oracle.recurrent_full(q, k, v, g, beta, S0)


# --------------------------------------------------------------------------
# Worked example done by hand (tests/golden/hand_worked.json)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", json.load(open(os.path.join(HERE, "golden", "hand_worked.json")))["cases"],
                         ids=lambda c: c["name"])
def test_hand_worked_example(case):
    k = np.array(case["k"])[None, :, None, :]
    q = np.array(case["q"])[None, :, None, :]
    v = np.array(case["v"])[None, :, None, :]
    beta = np.array(case["beta"])[None, :, None]
    g = np.log(np.array(case["alpha"]))[None, :, None]
    o, ST = run(q, k, v, g, beta)
    # g = ln(alpha) rounded to float32 moves alpha by < 1e-7 relative
    np.testing.assert_allclose(o[0, :, 0], np.array(case["o"]), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(ST[0, 0], np.array(case["S_T"]), rtol=1e-6, atol=1e-7)


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("gate", ["head", "key"])
def test_beta_zero_is_pure_decay(gate):
    """beta = 0: S_T is S0 decayed by the product of the alphas (per key channel
    for the key-channel gate) and o_t = (decayed S0) q_t."""
    q, k, v, g, beta, S0 = rand_problem(1, T=9, gate=gate)
    beta = np.zeros_like(beta)
    g = g.astype(np.float32).astype(np.float64)
    o, ST = run(q, k, v, g, beta, S0)
    cum = np.cumsum(g[0, :, 0], axis=0)                 # [T] or [T, dk]
    for t in range(q.shape[1]):
        St = S0[0, 0] * np.exp(cum[t])                   # broadcasts over key columns for "key"
        np.testing.assert_allclose(o[0, t, 0], St @ q[0, t, 0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ST[0, 0], S0[0, 0] * np.exp(cum[-1]), rtol=1e-12, atol=1e-14)


def test_orthonormal_keys_store_and_recall():
    """alpha = 1, beta = 1, orthonormal keys, S0 = 0: writing v_i under k_i and
    reading with q = k_j returns v_j exactly; writing a new value under a used
    key replaces the old value."""
    dk, dv, n = 8, 5, 6
    r = np.random.default_rng(2)
    H4 = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]]) / 2.0
    K = np.zeros((dk, dk))
    K[:4, :4], K[4:, 4:] = H4, H4                       # exactly orthonormal, entries 0 and +-1/2
    keys = K[r.permutation(dk)[:n]]                     # n orthonormal rows
    vals = r.standard_normal((n, dv)).astype(np.float32).astype(np.float64)
    new_val = r.standard_normal(dv).astype(np.float32).astype(np.float64)
    # tokens 0..n-1 write (k_i, v_i) and read key (i*5) % (i+1); token n rewrites key 2, reads it
    kk = np.vstack([keys, keys[2]])
    vv = np.vstack([vals, new_val])
    reads = [(i * 5) % (i + 1) for i in range(n)] + [2]
    qq = np.vstack([keys[j] for j in reads])
    T = n + 1
    o, ST = run(qq[None, :, None], kk[None, :, None], vv[None, :, None],
                np.zeros((1, T, 1)), np.ones((1, T, 1)))
    for t in range(n):
        np.testing.assert_allclose(o[0, t, 0], vals[reads[t]], atol=1e-13)
    np.testing.assert_allclose(o[0, n, 0], new_val, atol=1e-13)
    # the state is exactly sum_i v_i k_i^T with v_2 replaced
    vals2 = vals.copy()
    vals2[2] = new_val
    np.testing.assert_allclose(ST[0, 0], vals2.T @ keys, atol=1e-13)


def test_alpha_one_is_the_deltanet_rule():
    """alpha = 1 reduces to the DeltaNet row of the 'Source notes' page, written
    here in the page's own K x V orientation: S <- S + k [beta (v - k^T S)]^T,
    y = q^T S."""
    q, k, v, g, beta, S0 = rand_problem(3, T=10)
    g = np.zeros_like(g)
    o, ST = run(q, k, v, g, beta, S0)
    S = S0[0, 0].T.copy()                               # K x V
    for t in range(q.shape[1]):
        kt, vt, qt, bt = k[0, t, 0], v[0, t, 0], q[0, t, 0], beta[0, t, 0]
        S = S + np.outer(kt, bt * (vt - kt @ S))
        np.testing.assert_allclose(o[0, t, 0], qt @ S, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ST[0, 0], S.T, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# Brute force on tiny inputs: history expansion with explicit dk x dk matrices
# --------------------------------------------------------------------------
@pytest.mark.parametrize("gate", ["head", "key"])
@pytest.mark.parametrize("T", [1, 3, 8])
def test_history_expansion(gate, T):
    """S_t = S0 M_1 ... M_t + sum_s beta_s v_s k_s^T M_{s+1} ... M_t with
    M_t = D_t (I - beta_t k_t k_t^T), D_t = alpha_t I (scalar gate) or
    diag(alpha_t) (key-channel gate): the 'history expansion' form named in the
    'Source notes' page (Linear attention)."""
    dk, dv = 4, 3
    q, k, v, g, beta, S0 = rand_problem(10 + T, T=T, dk=dk, dv=dv, gate=gate)
    g = g.astype(np.float32).astype(np.float64)
    o, ST = run(q, k, v, g, beta, S0)
    I = np.eye(dk)
    M = []
    for t in range(T):
        D = np.exp(g[0, t, 0]) * I if gate == "head" else np.diag(np.exp(g[0, t, 0]))
        kt = k[0, t, 0][:, None]
        M.append(D @ (I - beta[0, t, 0] * kt @ kt.T))

    def prod(a, b):                                     # M_a ... M_b (identity if empty)
        P = I
        for t in range(a, b + 1):
            P = P @ M[t]
        return P

    for t in range(T):
        St = S0[0, 0] @ prod(0, t)
        for s in range(t + 1):
            St = St + beta[0, s, 0] * np.outer(v[0, s, 0], k[0, s, 0]) @ prod(s + 1, t)
        np.testing.assert_allclose(o[0, t, 0], St @ q[0, t, 0], rtol=1e-11, atol=1e-12)
        if t == T - 1:
            np.testing.assert_allclose(ST[0, 0], St, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# Second formulation: exact chunkwise form at chunk sizes 1, 8, 16, 64 (<= 1e-10)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("gate", ["head", "key"])
@pytest.mark.parametrize("chunk", [1, 8, 16, 64])
def test_chunkwise_form_agrees(gate, chunk):
    q, k, v, g, beta, S0 = rand_problem(20 + chunk, B=2, T=75, Hk=2, Hv=4, dk=16, dv=12, gate=gate,
                                        g_mu=2.0)
    g = g.astype(np.float32).astype(np.float64)
    o, ST = run(q, k, v, g, beta, S0)
    oc, STc = chunked(q, k, v, g, beta, S0, chunk=chunk)
    assert np.max(np.abs(o - oc)) <= 1e-10 * max(1.0, np.max(np.abs(o)))
    assert np.max(np.abs(ST - STc)) <= 1e-10 * max(1.0, np.max(np.abs(ST)))


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------
def test_key_channel_gate_with_equal_channels_is_scalar_gate():
    """GDN is the per-key-channel (KDA) form with the scalar log decay
    broadcast across key channels ('Source notes', Backend and numerical limits)."""
    q, k, v, g, beta, S0 = rand_problem(4, B=2, T=20, Hk=1, Hv=2)
    g = g.astype(np.float32).astype(np.float64)
    gk = np.repeat(g[..., None], q.shape[3], axis=-1)
    o1, S1 = run(q, k, v, g, beta, S0)
    o2, S2 = run(q, k, v, gk, beta, S0)
    np.testing.assert_allclose(o1, o2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(S1, S2, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("gate", ["head", "key"])
def test_causality(gate):
    q, k, v, g, beta, S0 = rand_problem(5, T=16, gate=gate)
    o, _ = run(q, k, v, g, beta, S0)
    tp = 9
    q2, k2, v2, g2, b2 = (a.copy() for a in (q, k, v, g, beta))
    q2[:, tp:] = -q2[:, tp:]
    k2[:, tp:] = unit_rows(k2[:, tp:] + 0.3)
    v2[:, tp:] += 1.0
    g2[:, tp:] -= 0.5
    b2[:, tp:] *= 0.5
    o2, _ = run(q2, k2, v2, g2, b2, S0)
    assert np.array_equal(o[:, :tp], o2[:, :tp])
    assert not np.allclose(o[:, tp], o2[:, tp])


@pytest.mark.parametrize("gate", ["head", "key"])
def test_resume_from_final_state(gate):
    """prefill(T1) then prefill(T2) from its final state equals prefill(T1 + T2);
    a decode step (T = 1) from the final state equals the next prefill token."""
    q, k, v, g, beta, S0 = rand_problem(6, B=2, T=13, Hk=1, Hv=2, gate=gate)
    o, ST = run(q, k, v, g, beta, S0)
    T1 = 8
    oa, Sa = run(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], S0)
    ob, Sb = run(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], Sa)
    assert np.array_equal(np.concatenate([oa, ob], axis=1), o)
    assert np.array_equal(Sb, ST)
    od, Sd = run(q[:, 12:13], k[:, 12:13], v[:, 12:13], g[:, 12:13], beta[:, 12:13],
                 run(q[:, :12], k[:, :12], v[:, :12], g[:, :12], beta[:, :12], S0)[1])
    assert np.array_equal(od[:, 0], o[:, 12])
    assert np.array_equal(Sd, ST)


def test_grouped_heads_equal_repeated_heads():
    """Value head h reads key/query head h // (Hv // Hk): the same as giving every
    value head its own copy of that key/query head."""
    q, k, v, g, beta, S0 = rand_problem(7, B=2, T=11, Hk=2, Hv=6)
    o, ST = run(q, k, v, g, beta, S0)
    rep = lambda a: np.repeat(a, 3, axis=2)
    o2, ST2 = run(rep(q), rep(k), v, g, beta, S0)
    assert np.array_equal(o, o2) and np.array_equal(ST, ST2)
    # and not the interleaved grouping h % Hk
    o3, _ = run(np.tile(q, (1, 1, 3, 1)), np.tile(k, (1, 1, 3, 1)), v, g, beta, S0)
    assert not np.allclose(o, o3)


def test_value_channels_are_independent():
    """Each state row evolves with its own value channel only: permuting the
    value channels permutes state rows and output channels."""
    q, k, v, g, beta, S0 = rand_problem(8, T=10, dv=7)
    perm = np.random.default_rng(0).permutation(7)
    o, ST = run(q, k, v, g, beta, S0)
    o2, ST2 = run(q, k, v[..., perm], g, beta, S0[:, :, perm])
    np.testing.assert_allclose(o2, o[..., perm], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(ST2, ST[:, :, perm], rtol=1e-14, atol=1e-15)


def test_contraction_without_writes():
    """v = 0: S_T = S0 M_1 ... M_T with ||M_t||_2 = alpha_t for unit keys and
    beta in (0, 1], so ||S_T||_2 <= (prod alpha) ||S0||_2."""
    q, k, v, g, beta, S0 = rand_problem(9, T=30, dk=8, dv=8)
    v = np.zeros_like(v)
    _, ST = run(q, k, v, g, beta, S0)
    bound = np.exp(np.sum(g.astype(np.float32).astype(np.float64))) * np.linalg.norm(S0[0, 0], 2)
    assert np.linalg.norm(ST[0, 0], 2) <= bound * (1 + 1e-12)


# --------------------------------------------------------------------------
# Prologue: textbook convolution, SiLU, unit rows
# --------------------------------------------------------------------------
def test_prologue_matches_numpy_convolve():
    r = np.random.default_rng(11)
    B, T, Hk, Hv, d = 2, 9, 2, 3, 8
    xq = r.standard_normal((B, T, Hk, d)).astype(np.float32)
    xk = r.standard_normal((B, T, Hk, d)).astype(np.float32)
    xv = r.standard_normal((B, T, Hv, d)).astype(np.float32)
    w = r.normal(0, 0.5, (2 * Hk * d + Hv * d, 4)).astype(np.float32)
    q, k, v = oracle.prologue(xq, xk, xv, w)

    def ref(x, ww, l2):
        Bx, Tx, H, dd = x.shape
        y = np.zeros((Bx, Tx, H, dd))
        for b in range(Bx):
            for h in range(H):
                for c in range(dd):
                    # y_t = sum_j w[j] x_{t-3+j}: a full convolution with the taps reversed
                    z = np.convolve(x[b, :, h, c].astype(np.float64), ww[h * dd + c, ::-1].astype(np.float64))[:Tx]
                    y[b, :, h, c] = z * (1.0 / (1.0 + np.exp(-z)))
        if l2:
            y = y / np.sqrt(np.sum(y * y, axis=-1, keepdims=True) + 1e-6)
        return y

    nq = Hk * d
    np.testing.assert_allclose(q, ref(xq, w[:nq], True), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(k, ref(xk, w[nq:2 * nq], True), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(v, ref(xv, w[2 * nq:], False), rtol=1e-13, atol=1e-14)
    norms = np.linalg.norm(q, axis=-1)                  # sqrt(s / (s + eps)): just below 1
    assert np.all(norms <= 1 + 1e-15) and np.all(norms > 0.99)
    # the first output sees only the current token (zero history, tap 3)
    z0 = xv[:, 0].astype(np.float64) * w[2 * nq:, 3].reshape(Hv, d)
    np.testing.assert_allclose(v[:, 0], z0 / (1 + np.exp(-z0)), rtol=1e-13)


def test_oracle_rejects_bad_shapes():
    q, k, v, g, beta, S0 = rand_problem(12, Hk=2, Hv=3)
    with pytest.raises(ValueError):
        oracle.recurrent(q, k, v, g, beta, S0)


# --------------------------------------------------------------------------
# Gated output norm: library routines, unit RMS rows, per-row scale, eps
# --------------------------------------------------------------------------
def _gate_problem(seed, shape=(2, 5, 3, 8)):
    r = np.random.default_rng(seed)
    o = r.standard_normal(shape)
    z = r.standard_normal(shape).astype(np.float32)
    gain = (1.0 + 0.3 * r.standard_normal(shape[-1])).astype(np.float32)
    return o, z, gain


def test_output_gate_matches_torch_rms_norm_and_silu():
    # the whole operation is two library routines: torch's RMS norm (mean of
    # squares over the last axis, eps inside the root, then the weight) and SiLU
    import torch
    import torch.nn.functional as F
    o, z, gain = _gate_problem(21)
    for eps in (0.0, 1e-5, 0.7):
        y = oracle.output_gate(o, z, gain, eps)
        ot = torch.from_numpy(o)
        ref = F.rms_norm(ot, (o.shape[-1],), torch.from_numpy(gain.astype(np.float64)), eps) * \
            F.silu(torch.from_numpy(z.astype(np.float64)))
        np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=1e-15)


def test_output_gate_rows_have_unit_rms():
    # with eps = 0 every row divided by its gate and gain has mean square 1
    o, z, gain = _gate_problem(22)
    z = np.where(np.abs(z) < 0.1, np.float32(0.5), z)          # keep the gate away from 0
    y = oracle.output_gate(o, z, gain, 0.0)
    zz = z.astype(np.float64)
    ohat = y / (gain.astype(np.float64) * zz / (1 + np.exp(-zz)))
    np.testing.assert_allclose(np.mean(ohat * ohat, axis=-1), 1.0, rtol=1e-12)
    # and points the way o does
    assert np.all(np.sign(ohat) == np.sign(o))


def test_output_gate_scale_per_row():
    # eps = 0: each (batch, token, head) row is normalised on its own, so a
    # positive factor per row changes nothing and a negative one flips the sign
    o, z, gain = _gate_problem(23)
    r = np.random.default_rng(24)
    f = r.uniform(0.01, 100.0, o.shape[:-1] + (1,)) * r.choice([-1.0, 1.0], o.shape[:-1] + (1,))
    y = oracle.output_gate(o, z, gain, 0.0)
    y2 = oracle.output_gate(o * f, z, gain, 0.0)
    np.testing.assert_allclose(y2, y * np.sign(f), rtol=1e-12, atol=1e-15)


def test_output_gate_constant_rows_closed_form():
    # a row of d equal values a: o / rms = a / sqrt(a^2 + eps); with z large
    # the gate is z itself (sigmoid(40) = 1 in double), with z = 0 it is 0
    d = 16
    a = np.array([0.01, -0.02, 3.0])
    o = np.repeat(a[:, None], d, axis=1)
    gain = np.linspace(0.5, 2.0, d).astype(np.float32)
    eps = 1e-4
    z = np.full(o.shape, 40.0, np.float32)
    y = oracle.output_gate(o, z, gain, eps)
    expect = (a / np.sqrt(a * a + eps))[:, None] * gain.astype(np.float64)[None, :] * 40.0
    np.testing.assert_allclose(y, expect, rtol=1e-14)
    assert np.all(oracle.output_gate(o, np.zeros(o.shape, np.float32), gain, eps) == 0.0)


def test_output_gate_gain_is_per_channel():
    # a one-hot gain keeps exactly its channel in every row
    o, z, gain = _gate_problem(25)
    j = 5
    e = np.zeros(o.shape[-1], np.float32)
    e[j] = 1.0
    y = oracle.output_gate(o, z, e, 1e-5)
    assert np.all(np.delete(y, j, axis=-1) == 0.0)
    full = oracle.output_gate(o, z, np.ones_like(e), 1e-5)
    np.testing.assert_array_equal(y[..., j], full[..., j])


def test_output_gate_rejects_bad_shapes():
    o, z, gain = _gate_problem(26)
    with pytest.raises(ValueError):
        oracle.output_gate(o, z[..., :-1], gain, 1e-5)
    with pytest.raises(ValueError):
        oracle.output_gate(o, z, gain[:-1], 1e-5)


# --------------------------------------------------------------------------
# Backward: central finite differences of the forward oracle, every input
# --------------------------------------------------------------------------
def _loss(q, k, v, g, beta, S0, dO, dST, delta=True):
    o, ST = oracle.recurrent_full(q, k, v, g, beta, S0, delta=delta)
    return float(np.sum(o * dO) + np.sum(ST * dST))


@pytest.mark.parametrize("gate,delta", [("head", True), ("key", True), ("head", False), ("key", False)])
def test_backward_matches_finite_differences(gate, delta):
    # grouped heads (2 value heads per key head), S0 given, dS_T given; with and
    # without the delta correction (the forward oracle of each is pinned above)
    q, k, v, g, beta, S0 = rand_problem(31, B=1, T=5, Hk=1, Hv=2, dk=3, dv=2, gate=gate)
    r = np.random.default_rng(32)
    dO = r.standard_normal(v.shape)
    dST = r.standard_normal(S0.shape)
    grads = oracle.backward(q, k, v, g, beta, S0, dO, dST, delta=delta)
    inputs = {"q": q, "k": k, "v": v, "g": g, "beta": beta, "S0": S0}
    for name, x in inputs.items():
        fd = np.zeros(x.shape)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            if name == "S0":        # the oracle takes S0 in double
                xp[idx] += 1e-4
                xm[idx] -= 1e-4
            else:                   # the others in float32: use the stored values' actual step
                xp[idx] = np.float32(x[idx] + 1e-3)
                xm[idx] = np.float32(x[idx] - 1e-3)
            args = dict(inputs)
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], args["g"], args["beta"], args["S0"], dO, dST, delta)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], args["g"], args["beta"], args["S0"], dO, dST, delta)
            fd[idx] = (lp - lm) / (xp[idx] - xm[idx])
        np.testing.assert_allclose(grads["d" + name], fd, rtol=2e-5, atol=2e-6, err_msg=name)


def test_backward_without_state_gradients():
    # S0 absent and dS_T absent: the same as zeros
    q, k, v, g, beta, S0 = rand_problem(33, B=2, T=4, Hk=1, Hv=1, dk=4, dv=3, s0=False)
    dO = np.random.default_rng(34).standard_normal(v.shape)
    a = oracle.backward(q, k, v, g, beta, None, dO, None)
    b = oracle.backward(q, k, v, g, beta, np.zeros((2, 1, 3, 4)), dO, np.zeros((2, 1, 3, 4)))
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])


# --------------------------------------------------------------------------
# Without the delta correction: a plain decayed sum of outer products
# --------------------------------------------------------------------------
@pytest.mark.parametrize("gate", ["head", "key"])
def test_no_delta_is_decayed_sum(gate):
    q, k, v, g, beta, S0 = rand_problem(41, B=2, T=9, Hk=1, Hv=2, dk=4, dv=3, gate=gate)
    o, ST = oracle.recurrent_full(q, k, v, g, beta, S0, delta=False)
    B, T, Hv, dv = v.shape
    dk = q.shape[3]
    for b in range(B):
        for h in range(Hv):
            for t in range(T):
                # S_t = S0 decayed by every alpha up to t, plus each write decayed by the alphas after it
                dec = lambda a, z: np.exp(np.sum(g[b, a:z, h], axis=0))   # scalar or [dk]
                S = S0[b, h] * dec(0, t + 1)
                for s in range(t + 1):
                    S = S + beta[b, s, h] * np.outer(v[b, s, h], k[b, s, 0] * dec(s + 1, t + 1))
                np.testing.assert_allclose(o[b, t, h], S @ q[b, t, 0], rtol=1e-12, atol=1e-13)
                if t == T - 1:
                    np.testing.assert_allclose(ST[b, h], S, rtol=1e-12, atol=1e-13)


def test_no_delta_accumulates_where_delta_overwrites():
    # alpha = 1, beta = 1, one key written twice: the delta rule keeps the
    # second value, the rule without the correction keeps the sum
    k = np.zeros((1, 2, 1, 4))
    k[0, :, 0, 1] = 1.0
    q = k.copy()
    v = np.array([[[[1.0, 2.0]], [[10.0, -3.0]]]])
    g = np.zeros((1, 2, 1))
    beta = np.ones((1, 2, 1))
    o_d, _ = oracle.recurrent_full(q, k, v, g, beta)
    o_n, _ = oracle.recurrent_full(q, k, v, g, beta, delta=False)
    np.testing.assert_array_equal(o_d[0, 1, 0], [10.0, -3.0])
    np.testing.assert_array_equal(o_n[0, 1, 0], [11.0, -1.0])
