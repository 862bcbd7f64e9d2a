"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects invalid calls with the documented status before touching
the device.  No call here reaches a kernel launch."""
import ctypes

import pytest

import gated_delta_rule_02_amd as gdn

FAKE = 1 << 20          # a 16-byte aligned non-null address; never dereferenced by these calls


@pytest.fixture(scope="module")
def L():
    return gdn.lib()


def test_exports_every_header_function(L):
    names = gdn.header_functions()
    assert set(names) >= {"gdn_prologue", "gdn_fwd_chunked", "gdn_decode_step",
                          "gdn_fwd_workspace_bytes", "gdn_status_str", "gdn_last_error", "gdn_version"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in range(7):
        assert L.gdn_status_str(code)
    assert L.gdn_version().startswith(b"gdn-gfx950")


def desc(**kw):
    base = dict(B=2, T=100, Hk=2, Hv=6, dk=128, dv=128, chunk=64, qkv_dtype=gdn.BF16,
                gate_dtype=gdn.BF16, gate=gdn.GATE_HEAD)
    base.update(kw)
    return gdn.GdnDesc(**base)


def fwd(L, d, ptrs=None, S0=None):
    p = [FAKE + i * (1 << 32) for i in range(7)] if ptrs is None else ptrs
    P = ctypes.c_void_p
    return L.gdn_fwd_chunked(ctypes.byref(d), *[P(x) for x in p[:5]], P(S0), P(p[5]), P(p[6]),
                             None, 0, None)


def dec(L, d, ptrs=None):
    p = [FAKE + i * (1 << 32) for i in range(7)] if ptrs is None else ptrs
    return L.gdn_decode_step(ctypes.byref(d), *[ctypes.c_void_p(x) for x in p], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 1), (dict(T=0), 1), (dict(Hk=0), 1), (dict(dk=-1), 1),
    (dict(qkv_dtype=7), 1), (dict(gate=3), 1),
    (dict(Hv=5), 2),                                     # Hv % Hk != 0
    (dict(dk=64), 3), (dict(chunk=32), 3),               # matrix-core mode: d 128, chunk 64 only
    (dict(qkv_dtype=gdn.F32, gate_dtype=gdn.BF16), 3),    # unbuilt dtype mix
    (dict(qkv_dtype=gdn.F32, gate_dtype=gdn.F32, dk=100, dv=100), 3),
    (dict(qkv_dtype=gdn.F32, gate_dtype=gdn.F32, chunk=64), 3),   # fp32 mode: chunk * dk <= 4096
    (dict(qkv_dtype=gdn.F32, gate_dtype=gdn.F32, chunk=48, dk=16, dv=16), 3),
])
def test_fwd_rejects(L, kw, status):
    assert fwd(L, desc(**kw)) == status
    assert L.gdn_last_error()


def test_fwd_rejects_null_and_misaligned(L):
    p = [FAKE + i * (1 << 32) for i in range(7)]
    for i in range(7):
        bad = list(p)
        bad[i] = 0
        assert fwd(L, desc(), bad) == 1
        bad[i] = p[i] + 8
        assert fwd(L, desc(), bad) == 4
    assert fwd(L, desc(), p, S0=FAKE + 7 * (1 << 32) + 4) == 4


def noalloc(L, d, ptrs=None):
    p = [FAKE + i * (1 << 32) for i in range(7)] if ptrs is None else ptrs
    P = ctypes.c_void_p
    return L.gdn_fwd_chunked_noalloc(ctypes.byref(d), *[P(x) for x in p[:5]], None, P(p[5]), P(p[6]), None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 1), (dict(gate=3), 1), (dict(Hv=5), 2), (dict(dk=64), 3),
    (dict(B=8, T=4096, Hk=16, Hv=48), 5),                 # 174 MiB of chunk matrices > 128 MiB
    (dict(B=2, T=4096, Hk=32, Hv=32, gate=gdn.GATE_KEY_CHANNEL), 5),   # 4096 x 62208 B
])
def test_noalloc_rejects(L, kw, status):
    d = desc(**kw)
    assert noalloc(L, d) == status
    assert L.gdn_last_error()
    if status == 5:
        assert b"no-allocation" in L.gdn_last_error()
        assert L.gdn_fwd_workspace_bytes(ctypes.byref(d)) > gdn.NOALLOC_SCRATCH_BYTES


def test_noalloc_scratch_size_matches_header(L):
    text = open(gdn.HEADER).read()
    assert "#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)" in text
    assert gdn.NOALLOC_SCRATCH_BYTES == 128 << 20
    # the largest problems the scratch holds: B4 Hv48 T4096 (head gate), B1 H32 T4096 (key gate)
    for d in (desc(B=4, T=4096, Hk=16, Hv=48), desc(B=1, T=4096, Hk=32, Hv=32, gate=gdn.GATE_KEY_CHANNEL)):
        assert 0 < L.gdn_fwd_workspace_bytes(ctypes.byref(d)) <= gdn.NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_null_and_misaligned(L):
    p = [FAKE + i * (1 << 32) for i in range(7)]
    for i in range(7):
        bad = list(p)
        bad[i] = 0
        assert noalloc(L, desc(), bad) == 1
        bad[i] = p[i] + 8
        assert noalloc(L, desc(), bad) == 4


def test_fwd_rejects_overlaps(L):
    p = [FAKE + i * (1 << 32) for i in range(7)]
    o_on_v = list(p)
    o_on_v[5] = p[2] + 1024                              # o inside v
    assert fwd(L, desc(), o_on_v) == 1
    st_partial = list(p)
    assert fwd(L, desc(), st_partial, S0=p[6] + 4096) == 1   # S_T partly overlapping S0


def test_decode_rejects(L):
    assert dec(L, desc(T=2)) == 2
    assert dec(L, desc(T=1, dk=48)) == 3
    assert dec(L, desc(T=1, dv=40)) == 3
    assert dec(L, desc(T=1, gate_dtype=gdn.F16)) == 3
    p = [FAKE + i * (1 << 32) for i in range(7)]
    p[5] = 0
    assert dec(L, desc(T=1), p) == 1


def test_prologue_rejects(L):
    d = desc()
    P = ctypes.c_void_p
    ptrs = [P(FAKE + i * (1 << 32)) for i in range(7)]
    assert L.gdn_prologue(ctypes.byref(d), gdn.F16, *ptrs[:4], 1e-6, *ptrs[4:], None) == 3
    assert L.gdn_prologue(ctypes.byref(d), 9, *ptrs[:4], 1e-6, *ptrs[4:], None) == 1
    assert L.gdn_prologue(ctypes.byref(desc(dk=96)), gdn.BF16, *ptrs[:4], 1e-6, *ptrs[4:], None) == 3
    assert L.gdn_prologue(ctypes.byref(d), gdn.BF16, *ptrs[:4], -1.0, *ptrs[4:], None) == 1
    out_on_in = list(ptrs)
    out_on_in[4] = ptrs[0]                               # q written over xq
    assert L.gdn_prologue(ctypes.byref(d), gdn.BF16, *out_on_in[:4], 1e-6, *out_on_in[4:], None) == 1


def test_workspace_query(L):
    # matrix-core path: 7424 bytes per (batch, value head, 64-token chunk)
    # above 64 (batch, value head) pairs, 19712 (P's two parts too) up to 64,
    # 62208 with the key-channel gate
    assert L.gdn_fwd_workspace_bytes(ctypes.byref(desc(Hk=16, Hv=48))) == 2 * 48 * 2 * 7424
    assert L.gdn_fwd_workspace_bytes(ctypes.byref(desc(B=1, Hk=16, Hv=64))) == 1 * 64 * 2 * 19712
    assert L.gdn_fwd_workspace_bytes(ctypes.byref(desc(B=5, Hk=13, Hv=13))) == 5 * 13 * 2 * 7424
    assert L.gdn_fwd_workspace_bytes(ctypes.byref(desc())) == 2 * 6 * 2 * 19712
    assert L.gdn_fwd_workspace_bytes(ctypes.byref(desc(T=1))) == 2 * 6 * 1 * 19712
    assert L.gdn_fwd_workspace_bytes(ctypes.byref(desc(gate=gdn.GATE_KEY_CHANNEL))) == 2 * 6 * 2 * 62208
    assert L.gdn_fwd_workspace_bytes(ctypes.byref(desc(gate=gdn.GATE_KEY_CHANNEL, dk=64, dv=64))) == 0
    assert L.gdn_fwd_workspace_bytes(ctypes.byref(desc(qkv_dtype=gdn.F32, gate_dtype=gdn.F32, chunk=32))) == 0
    assert L.gdn_fwd_workspace_bytes(ctypes.byref(desc(Hv=5))) == 0       # invalid description
    assert L.gdn_fwd_workspace_bytes(None) == 0


def test_workspace_checked_before_launch(L):
    d = desc()
    need = L.gdn_fwd_workspace_bytes(ctypes.byref(d))
    P = ctypes.c_void_p
    p = [FAKE + i * (1 << 32) for i in range(8)]
    args = [P(x) for x in p[:5]] + [None, P(p[5]), P(p[6])]
    assert L.gdn_fwd_chunked(ctypes.byref(d), *args, None, 0, None) == 5
    assert L.gdn_fwd_chunked(ctypes.byref(d), *args, P(p[7]), need - 16, None) == 5
    assert L.gdn_fwd_chunked(ctypes.byref(d), *args, None, need, None) == 1
    assert L.gdn_fwd_chunked(ctypes.byref(d), *args, P(p[7] + 8), need, None) == 4
    assert L.gdn_fwd_chunked(ctypes.byref(d), *args, P(p[2]), need, None) == 1   # on top of v


def test_null_desc(L):
    assert L.gdn_fwd_chunked(None, *([None] * 9), 0, None) == 1


def test_conv_workspace_query(L):
    d = desc(qkv_dtype=gdn.F16)      # B 2, 6 value heads, 2 chunks, matrix-core path
    ws = L.gdn_fwd_workspace_bytes(ctypes.byref(d))
    B, T, Hk, Hv = d.B, d.T, d.Hk, d.Hv
    # fused (bf16 raw inputs, fp16 q and k): the chunk matrices, then q and k after the prologue
    assert L.gdn_fwd_conv_workspace_bytes(ctypes.byref(d), gdn.BF16) == ws + 2 * B * T * Hk * 128 * 2
    # fp32 raw inputs, or bf16 q, k, v: q, k, v buffers (256-byte rounded) and the chunk matrices
    r = lambda x: (x + 255) // 256 * 256
    nqk, nv = B * T * Hk * 128 * 2, B * T * Hv * 128 * 2
    assert L.gdn_fwd_conv_workspace_bytes(ctypes.byref(d), gdn.F32) == 2 * r(nqk) + r(nv) + ws
    assert L.gdn_fwd_conv_workspace_bytes(ctypes.byref(desc()), gdn.BF16) == 2 * r(nqk) + r(nv) + ws
    assert L.gdn_fwd_conv_workspace_bytes(ctypes.byref(d), gdn.F16) == 0    # raw fp16 is not supported
    assert L.gdn_fwd_conv_workspace_bytes(ctypes.byref(desc(Hv=5)), gdn.BF16) == 0


def test_conv_rejects_before_launch(L):
    d = desc()
    need = L.gdn_fwd_conv_workspace_bytes(ctypes.byref(d), gdn.BF16)
    P = ctypes.c_void_p
    p = [P(FAKE + i * (1 << 32)) for i in range(10)]
    # xq, xk, xv, conv_w | g, beta | S0 | o, S_T | workspace
    call = lambda dd, xt, ptrs, eps=1e-6, ws=p[9], nbytes=need: L.gdn_fwd_chunked_conv(
        ctypes.byref(dd), xt, *ptrs[:4], eps, *ptrs[4:6], None, *ptrs[6:8], ws, nbytes, None)
    assert call(d, gdn.F16, p) == 3                      # raw fp16
    assert call(d, gdn.BF16, p, eps=-1.0) == 1
    assert call(d, gdn.BF16, p, nbytes=need - 16) == 5
    assert call(d, gdn.BF16, p, ws=None) == 1
    bad = list(p)
    bad[6] = p[2]                                        # o written over xv
    assert call(d, gdn.BF16, bad) == 1
    bad = list(p)
    bad[0] = P(FAKE + 8)
    assert call(d, gdn.BF16, bad) == 4                   # misaligned xq
    assert call(desc(Hv=5), gdn.BF16, p) == 2


def test_gated_workspace_query(L):
    r = lambda x: (x + 255) // 256 * 256
    # B * Hv = 12 <= 128: the gate runs after the forward, o kept in the workspace
    d = desc()
    conv = L.gdn_fwd_conv_workspace_bytes(ctypes.byref(d), gdn.BF16)
    o_bytes = d.B * d.T * d.Hv * 128 * 4
    assert L.gdn_fwd_gated_workspace_bytes(ctypes.byref(d), gdn.BF16, gdn.BF16) == r(conv) + o_bytes
    # B * Hv = 192 > 128 with bf16 raw inputs, fp16 q and k and 16-bit y:
    # the gate runs inside the sequential pass
    d = desc(B=4, Hk=16, Hv=48, qkv_dtype=gdn.F16)
    inside = L.gdn_fwd_conv_workspace_bytes(ctypes.byref(d), gdn.BF16)
    assert L.gdn_fwd_gated_workspace_bytes(ctypes.byref(d), gdn.BF16, gdn.BF16) == inside
    assert L.gdn_fwd_gated_workspace_bytes(ctypes.byref(d), gdn.BF16, gdn.F16) == inside
    o_bytes = d.B * d.T * d.Hv * 128 * 4
    assert L.gdn_fwd_gated_workspace_bytes(ctypes.byref(d), gdn.BF16, gdn.F32) == r(inside) + o_bytes
    # fp32 raw inputs never take the fused form
    conv = L.gdn_fwd_conv_workspace_bytes(ctypes.byref(d), gdn.F32)
    assert L.gdn_fwd_gated_workspace_bytes(ctypes.byref(d), gdn.F32, gdn.BF16) == r(conv) + o_bytes
    assert L.gdn_fwd_gated_workspace_bytes(ctypes.byref(desc(Hv=5)), gdn.BF16, gdn.BF16) == 0
    assert L.gdn_fwd_gated_workspace_bytes(ctypes.byref(d), gdn.BF16, 9) == 0
    assert L.gdn_fwd_gated_workspace_bytes(ctypes.byref(desc(gate=gdn.GATE_KEY_CHANNEL, dk=64, dv=48,
                                                             qkv_dtype=gdn.F32, gate_dtype=gdn.F32,
                                                             chunk=16)), gdn.F32, gdn.F32) == 0   # dv 48


def test_output_gate_rejects(L):
    P = ctypes.c_void_p
    p = [P(FAKE + i * (1 << 32)) for i in range(4)]      # o, z, gain, y
    call = lambda dd, ptrs, zt=gdn.BF16, yt=gdn.BF16, eps=1e-5: L.gdn_output_gate(
        ctypes.byref(dd), ptrs[0], zt, ptrs[1], ptrs[2], eps, yt, ptrs[3], None)
    assert call(desc(dv=48), p) == 3                     # dv not in {16, 32, 64, 128}
    assert call(desc(), p, zt=5) == 1
    assert call(desc(), p, yt=-1) == 1
    assert call(desc(), p, eps=-1.0) == 1
    assert call(desc(), p, eps=float("nan")) == 1
    assert call(desc(Hv=5), p) == 2
    for i in range(4):
        bad = list(p)
        bad[i] = None
        assert call(desc(), bad) == 1
        bad[i] = P(p[i].value + 8)
        assert call(desc(), bad) == 4
    bad = list(p)
    bad[3] = P(p[0].value + 4096)                        # y written over o
    assert call(desc(), bad) == 1
    assert L.gdn_last_error()


def test_gated_rejects_before_launch(L):
    d = desc(B=4, Hk=16, Hv=48)
    need = L.gdn_fwd_gated_workspace_bytes(ctypes.byref(d), gdn.BF16, gdn.BF16)
    P = ctypes.c_void_p
    p = [P(FAKE + i * (1 << 36)) for i in range(11)]
    # xq, xk, xv, conv_w | g, beta | z, gain | y, S_T | workspace
    call = lambda dd, ptrs, xt=gdn.BF16, yt=gdn.BF16, neps=1e-5, ws=p[10], nbytes=need: \
        L.gdn_fwd_chunked_conv_gated(ctypes.byref(dd), xt, *ptrs[:4], 1e-6, *ptrs[4:6], None,
                                     *ptrs[6:8], neps, yt, *ptrs[8:10], ws, nbytes, None)
    assert call(d, p, xt=gdn.F16) == 3                   # raw fp16
    assert call(d, p, yt=4) == 1
    assert call(d, p, neps=2.0) == 1
    assert call(d, p, nbytes=need - 16) == 5
    assert call(d, p, ws=None) == 1
    for i, code in ((6, 1), (7, 1)):                     # z, gain missing
        bad = list(p)
        bad[i] = None
        assert call(d, bad) == code
    bad = list(p)
    bad[8] = P(p[6].value + 256)                         # y written over z
    assert call(d, bad) == 1
    assert call(d, p, ws=P(p[8].value + 256)) == 1      # workspace over y
    assert call(desc(B=4, Hk=16, Hv=48, dv=64), p) == 3  # matrix-core mode needs dv 128


def test_varlen_checks(L):
    P = ctypes.c_void_p
    d = desc(B=5, T=1000)                                # 5 packed sequences, 1000 tokens in all
    p = [P(FAKE + i * (1 << 36)) for i in range(12)]
    cu = P(FAKE + 11 * (1 << 36))
    need = L.gdn_fwd_varlen_workspace_bytes(ctypes.byref(d))
    # matrix-core path: chunk slots per value head = T / 64 + B = 20, 19712
    # bytes each (30 (sequence, value head) pairs: P's two parts too)
    assert need == 6 * (1000 // 64 + 5) * 19712 + 256   # and the sequence order (5 ints, in 256 bytes)
    assert L.gdn_fwd_varlen_workspace_bytes(ctypes.byref(desc(B=5, T=1000, Hv=5))) == 0
    call = lambda dd, cu_, ptrs=p, ws=p[10], nbytes=need: L.gdn_fwd_chunked_varlen(
        ctypes.byref(dd), cu_, *ptrs[:5], None, *ptrs[5:7], ws, nbytes, None)
    assert call(d, None) == 1                            # offsets missing
    assert call(d, P(cu.value + 2)) == 4                 # offsets misaligned
    assert call(d, cu, nbytes=need - 16) == 5
    bad = list(p)
    bad[5] = P(cu.value - 64)                            # o over the offsets
    assert call(d, cu, bad) == 1
    assert call(desc(B=5, T=1000, dk=64), cu) == 3
    # the conv form and the prologue
    d16 = desc(B=5, T=1000, qkv_dtype=gdn.F16)
    assert L.gdn_fwd_varlen_workspace_bytes(ctypes.byref(d16)) == need
    assert L.gdn_fwd_conv_varlen_workspace_bytes(ctypes.byref(d16), gdn.BF16) == \
        need + 2 * 1000 * 2 * 128 * 2                    # plus q and k after the prologue
    cneed = L.gdn_fwd_conv_varlen_workspace_bytes(ctypes.byref(d), gdn.BF16)
    assert L.gdn_fwd_chunked_conv_varlen(ctypes.byref(d), None, gdn.BF16, *p[:4], 1e-6, *p[4:6], None,
                                         *p[6:8], p[10], cneed, None) == 1
    assert L.gdn_prologue_varlen(ctypes.byref(d), cu, gdn.BF16, *p[:4], 1e-6, P(cu.value), *p[5:7],
                                 None) == 1              # q written over the offsets
    assert L.gdn_prologue_varlen(ctypes.byref(d), None, gdn.BF16, *p[:4], 1e-6, *p[4:7], None) == 1


def test_conv_cache_checks(L):
    P = ctypes.c_void_p
    p = [P(FAKE + i * (1 << 36)) for i in range(12)]
    d = desc(T=1)
    need = L.gdn_decode_conv_workspace_bytes(ctypes.byref(d))
    assert need == 2 * 2 * 2 * 128 * 2 + 2 * 6 * 128 * 2   # q, k (B 2, 2 heads) and v (6 heads), bf16
    # xq, xk, xv, conv_w | conv_state | g, beta, S, o | workspace
    call = lambda dd, ptrs=p, xt=gdn.BF16, nbytes=need: L.gdn_decode_step_conv(
        ctypes.byref(dd), xt, *ptrs[:4], 1e-6, ptrs[4], *ptrs[5:9], ptrs[9], nbytes, None)
    assert call(desc(T=2)) == 2                          # one token per sequence
    assert call(d, xt=gdn.F16) == 3                      # raw fp16 is not supported
    assert call(d, nbytes=need - 1) == 5
    bad = list(p)
    bad[4] = None
    assert call(d, bad) == 1                             # conv_state missing
    bad = list(p)
    bad[4] = P(p[7].value + 64)                          # conv_state over S
    assert call(d, bad) == 1
    assert L.gdn_conv_state(ctypes.byref(desc()), None, gdn.BF16, *p[:3], None, None) == 1
    assert L.gdn_conv_state(ctypes.byref(desc()), None, gdn.BF16, *p[:3], P(p[1].value + 16), None) == 1
    assert L.gdn_conv_state(ctypes.byref(desc()), P(p[5].value + 2), gdn.BF16, *p[:3], p[4], None) == 4


def test_bwd_checks(L):
    P = ctypes.c_void_p
    p = [P(FAKE + i * (1 << 36)) for i in range(16)]
    d = desc(qkv_dtype=gdn.F32, gate_dtype=gdn.F32)
    need = L.gdn_bwd_workspace_bytes(ctypes.byref(d))
    # head gate, per (batch, value head, chunk of 64): T and P^T [64][64], gamma and
    # beta [64], the state before the chunk and the state gradient after it [dv][dk],
    # U and E [64][dv], all fp32
    assert need == 2 * 6 * 2 * (2 * 64 * 64 + 2 * 64 + 2 * 128 * 128 + 2 * 64 * 128) * 4
    # at the prefill workload's size: one segment takes 2.8 GB; within 1 GB, four segments
    # of 16 chunks: T, gamma, beta for all 64 chunks, the states at the 4 segment starts,
    # P^T, S0, dS_C, U, E for one segment's 16 chunks (B 4, 48 value heads)
    dbig = desc(B=4, T=4096, Hk=16, Hv=48)
    per_chunk = 2 * 64 * 64 + 2 * 64 + 2 * 128 * 128 + 2 * 64 * 128
    assert L.gdn_bwd_workspace_bytes(ctypes.byref(dbig)) == 4 * 48 * 64 * per_chunk * 4
    assert L.gdn_bwd_workspace_bytes_within(ctypes.byref(dbig), 1 << 62) == 4 * 48 * 64 * per_chunk * 4
    units, sunits = 4 * 48 * 64, 4 * 48 * 16
    four = 4 * (units * (64 * 64 + 2 * 64) + 4 * 48 * 4 * 128 * 128
                + sunits * (64 * 64 + 2 * 128 * 128 + 2 * 64 * 128))
    assert four == 912261120
    assert L.gdn_bwd_workspace_bytes_within(ctypes.byref(dbig), 10 ** 9) == four
    # three segments (22, 22 and 20 chunks) need 1.145 GB
    three = 4 * (units * (64 * 64 + 2 * 64) + 4 * 48 * 3 * 128 * 128
                 + 4 * 48 * 22 * (64 * 64 + 2 * 128 * 128 + 2 * 64 * 128))
    assert L.gdn_bwd_workspace_bytes_within(ctypes.byref(dbig), three) == three
    # below the smallest plan (one chunk per segment) the call is refused
    smallest = L.gdn_bwd_workspace_bytes_within(ctypes.byref(dbig), 0)
    assert 0 < smallest < four
    # key-channel gate: as the head gate, with gamma [64][dk] per chunk in place of [64],
    # and K o e^gamma, Q o e^gamma, K o e^(gamma_C - gamma), [64][dk] each, per chunk
    dkey = desc(qkv_dtype=gdn.F32, gate_dtype=gdn.F32, gate=gdn.GATE_KEY_CHANNEL)
    assert L.gdn_bwd_workspace_bytes(ctypes.byref(dkey)) == 2 * 6 * 2 * (per_chunk - 64 + 4 * 64 * 128) * 4
    assert L.gdn_bwd_workspace_bytes_within(ctypes.byref(dkey), 0) < L.gdn_bwd_workspace_bytes(ctypes.byref(dkey))
    assert L.gdn_bwd_workspace_bytes(ctypes.byref(desc(dk=16))) == 0
    assert L.gdn_bwd_workspace_bytes(ctypes.byref(desc(dv=48))) == 0
    # q, k, v, g, beta | S0 | dO | dS_T | dq, dk, dv, dg, dbeta, dS0 | workspace
    call = lambda dd, ptrs=p, nbytes=need: L.gdn_bwd(ctypes.byref(dd), *ptrs[:5], None, ptrs[6], None,
                                                     *ptrs[8:14], ptrs[14], nbytes, None)
    assert call(desc(gate_dtype=gdn.F16)) == 3
    # without the delta correction: either gate, the same workspace as the delta rule
    dnd = desc(qkv_dtype=gdn.F32, gate_dtype=gdn.F32, rule=gdn.RULE_NO_DELTA)
    assert L.gdn_bwd_workspace_bytes(ctypes.byref(dnd)) == need
    knd = desc(qkv_dtype=gdn.F32, gate_dtype=gdn.F32, gate=gdn.GATE_KEY_CHANNEL, rule=gdn.RULE_NO_DELTA)
    assert L.gdn_bwd_workspace_bytes(ctypes.byref(knd)) == L.gdn_bwd_workspace_bytes(ctypes.byref(dkey))
    assert call(d, nbytes=L.gdn_bwd_workspace_bytes_within(ctypes.byref(d), 0) - 1) == 5
    assert call(dkey, nbytes=L.gdn_bwd_workspace_bytes_within(ctypes.byref(dkey), 0) - 1) == 5
    bad = list(p)
    bad[8] = None
    assert call(d, bad) == 1                             # dq missing
    bad = list(p)
    bad[10] = P(p[2].value + 64)                         # dv over v
    assert call(d, bad) == 1
    bad = list(p)
    bad[14] = P(p[13].value + 4096)                      # workspace over dS0
    assert call(d, bad) == 1
