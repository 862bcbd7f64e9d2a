"""Second CPU formulation of the gated delta rule: exact chunkwise form, fp64, NumPy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Its one job is to pin
the token-by-token oracle: the attention-sink study page ("SinkProbe" README,
test description next to the layer notes) checks its chunkwise delta-rule layer
against the token-by-token recurrence in 64-bit arithmetic at chunk sizes 1,
8, 16 and 64 to within 1e-10; ``tests/test_oracle_pins.py`` makes the same
check here.

The chunk algebra is derived (the pages do not print it).  For one chain and
one chunk of n tokens, with entering state S0 (dv x dk), in-chunk prefix
gamma_r = g_1 + ... + g_r and Gamma_r = exp(gamma_r), unrolling the recurrence
gives, for the new values nu_r = beta_r (v_r - alpha_r S_{r-1} k_r):

    (I + A) N = diag(beta) V - diag(beta Gamma) K S0^T,
        A[r, s] = beta_r exp(gamma_r - gamma_s) (k_r . k_s)   for s < r, else 0
    O   = diag(Gamma) Q S0^T + (L o Q K^T) N,
        L[r, s] = exp(gamma_r - gamma_s)                         for s <= r, else 0
    S_n = Gamma_n S0 + N^T diag(exp(gamma_n - gamma)) K

and with a per-key-channel decay (gamma_r a vector over key channels):

    A[r, s] = beta_r sum_c k_rc k_sc exp(gamma_rc - gamma_sc)           (s < r)
    rhs     = diag(beta) V - diag(beta) (K o Gamma) S0^T
    O       = (Q o Gamma) S0^T + M N,  M[r, s] = sum_c q_rc k_sc exp(gamma_rc - gamma_sc)  (s <= r)
    S_n     = S0 diag(Gamma_n) + N^T (K o exp(gamma_n - gamma))

The triangular system is solved with numpy.linalg.solve (a library primitive).
"""
from __future__ import annotations

import numpy as np


def chunked_chain(q, k, v, g, beta, S0, chunk):
    """One chain.  q, k: [T,dk]; v: [T,dv]; g: [T] or [T,dk]; beta: [T];
    S0: [dv,dk] or None.  Returns (o [T,dv], S_T [dv,dk]) in float64."""
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    per_channel = g.ndim == 2
    o = np.zeros((T, dv))
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(T, c0 + chunk))
        Q, K, V, G, bt = q[sl], k[sl], v[sl], g[sl], beta[sl]
        n = Q.shape[0]
        gam = np.cumsum(G, axis=0)
        tri_strict = np.tril(np.ones((n, n)), -1)
        tri_incl = np.tril(np.ones((n, n)), 0)
        if not per_channel:
            diff = gam[:, None] - gam[None, :]
            decay = np.exp(np.where(tri_incl > 0, diff, -np.inf))
            A = bt[:, None] * decay * (K @ K.T) * tri_strict
            rhs = bt[:, None] * V - (bt * np.exp(gam))[:, None] * (K @ S.T)
            N = np.linalg.solve(np.eye(n) + A, rhs)
            O = np.exp(gam)[:, None] * (Q @ S.T) + (decay * (Q @ K.T)) @ N
            S = np.exp(gam[-1]) * S + N.T @ (np.exp(gam[-1] - gam)[:, None] * K)
        else:
            # pairwise per-channel decay, exponent <= 0 wherever it is used
            diff = gam[:, None, :] - gam[None, :, :]                  # [r, s, c]
            ok = tri_incl[:, :, None] > 0
            dec = np.exp(np.where(ok, diff, -np.inf))
            A = bt[:, None] * np.einsum("rc,sc,rsc->rs", K, K, dec) * tri_strict
            rhs = bt[:, None] * V - bt[:, None] * ((K * np.exp(gam)) @ S.T)
            N = np.linalg.solve(np.eye(n) + A, rhs)
            M = np.einsum("rc,sc,rsc->rs", Q, K, dec)
            O = (Q * np.exp(gam)) @ S.T + M @ N
            S = S * np.exp(gam[-1])[None, :] + N.T @ (K * np.exp(gam[-1][None, :] - gam))
        o[sl] = O
    return o, S


def chunked(q, k, v, g, beta, S0=None, chunk=64):
    """All chains.  Shapes as in ``oracle.recurrent``; returns
    (o [B,T,Hv,dv], S_T [B,Hv,dv,dk]) float64."""
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    grp = Hv // Hk
    o = np.zeros((B, T, Hv, dv))
    ST = np.zeros((B, Hv, dv, dk))
    for b in range(B):
        for h in range(Hv):
            kh = h // grp
            oc, sc = chunked_chain(q[b, :, kh], k[b, :, kh], v[b, :, h], g[b, :, h], beta[b, :, h],
                                   None if S0 is None else S0[b, h], chunk)
            o[b, :, h] = oc
            ST[b, h] = sc
    return o, ST
