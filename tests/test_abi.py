"""The C-ABI library on the host: it loads, exports every declared entry point, sizes the
workspace and the packed gradients, and rejects bad arguments before any launch.
No test here enqueues GPU work (every call below fails validation first)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def B():
    from gated_delta_rule_bwd_amd import binding
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(B):
    names = declared_functions()
    assert set(names) == set(B.EXPORTS), names
    for n in names:
        assert hasattr(B.lib, n), n


def problem(B, strides=None, **kw):
    d = dict(n_seqs=2, T=64, H_k=4, H_v=8, S=64, kda=True, C=8, scale=0.125,
             seq_lens=[64, 61], dtype=0, S_v=None)
    d.update(kw)
    override = strides or {}
    strides = {"q": (64 * 4 * 64, 4 * 64, 64), "k": (64 * 4 * 64, 4 * 64, 64),
               "v": (64 * 8 * 64, 8 * 64, 64), "g": (64 * 8 * 64, 8 * 64, 64),
               "beta": (64 * 8, 8, 1), "gy": (64 * 8 * 64, 8 * 64, 64),
               "y": (64 * 8 * 64, 8 * 64, 64)}
    strides.update(override)
    return B.Problem(d["n_seqs"], d["T"], d["H_k"], d["H_v"], d["S"], d["kda"], d["C"],
                     d["scale"], d["seq_lens"], strides, d["dtype"], d["S_v"])


def expected_ws(n, T, Hk, Hv, S, C, kda=True):
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    units = n * Hv
    if S == 128:                    # checkpoints on the 16-token block grid
        C = -(-C // 16) * 16
    n_ck = max(1, -(-T // C))
    tot = al(units * n_ck * S * S * 4)
    if S == 128:                    # matrix-core path, one workgroup per (sequence, head)
        rows = n * T * Hv
        nblk = -(-T // 16)
        tot = al(tot + n * nblk * Hv * 3 * 256 * 4)         # block matrices Bm, Te, Tb
        tot = al(tot + n * nblk * Hv * 4)                   # block flags
        tot = al(tot + rows * (S if kda else 1) * 4)        # running gate products
        tot = al(tot + rows * S * 4)                        # prediction errors
        nsl = 2 if units <= 128 else 1                      # row slabs of small launches
        # pieces of about 1024 tokens (at most 16, whole segments); beyond 4 pieces the chain's
        # results for the column pass live in a ring of 4 piece slots
        npt = min(16, max(1, T // 1024))
        piece = max(C, -(-(-(-T // npt)) // C) * C)
        npieces = -(-T // piece)
        slots, pbT = (4, piece) if npieces > 4 else (1, nblk * 16)
        pb_rows = n * pbT * Hv
        tot = al(tot + slots * pb_rows // 16 * nsl * 256 * 4)   # Grams G1
        tot = al(tot + slots * pb_rows // 16 * nsl * 256 * 4)   # Grams G2
        tot = al(tot + slots * (pb_rows * nsl if nsl > 1 else 0) * 4)   # dbeta per slab
        tot = al(tot + slots * pb_rows * S * 4)             # the chain's column sums X'^T delta
        tot = al(tot + units * n_ck * S * 4)                # dg at each segment's first token
        tot = al(tot + units * S * S * 4)                   # state / gradient between pieces
        return tot                                          # dq, dk summed in the column pass
    tot = al(tot + units * C * S * S * 4)
    tot = al(tot + units * C * S * 4)
    if Hv != Hk:
        part = n * T * Hv * S * 4
        tot = al(tot + part)
        tot = al(tot + part)
    return tot


def test_workspace_size(B):
    p = problem(B)
    assert B.workspace_size(p) == expected_ws(2, 64, 4, 8, 64, 8)
    # C = 0 selects ceil(sqrt(T)) = 8 here
    assert B.workspace_size(problem(B, C=0)) == expected_ws(2, 64, 4, 8, 64, 8)
    # no grouped heads: no partial buffers
    assert B.workspace_size(problem(B, H_v=4)) == expected_ws(2, 64, 4, 4, 64, 8)
    # layer shape, 4 x 4096 tokens, 48 value heads, S = 128, C = 64
    big = problem(B, n_seqs=4, T=4096, H_k=16, H_v=48, S=128, C=64, seq_lens=None)
    assert B.workspace_size(big) == expected_ws(4, 4096, 16, 48, 128, 64)
    # 65536 tokens, 48 value heads, scalar gate, C = 256: 16 pieces, the ring of 4 slots
    long = problem(B, n_seqs=1, T=65536, H_k=16, H_v=48, S=128, C=256, kda=False, seq_lens=None)
    assert B.workspace_size(long) == expected_ws(1, 65536, 16, 48, 128, 256, kda=False)
    assert B.workspace_size(long) < 4.0e9
    long = problem(B, n_seqs=1, T=65536, H_k=16, H_v=48, S=128, C=256, kda=False,
                   seq_lens=None)
    assert B.workspace_size(long) == expected_ws(1, 65536, 16, 48, 128, 256, kda=False)


def test_grad_layout(B):
    p = problem(B)
    total, lay = B.grad_layout(p)
    n, T, Hk, Hv, S = 2, 64, 4, 8, 64
    sizes = [n * T * Hk * S, n * T * Hk * S, n * T * Hv * S, n * T * Hv * S, n * T * Hv,
             n * Hv * S * S]
    offs = [0]
    for x in sizes[:-1]:
        offs.append(offs[-1] + x)
    assert [lay[k][0] for k in ("dq", "dk", "dv", "dg", "dbeta", "dstate")] == offs
    assert total == sum(sizes)
    total_s, lay_s = B.grad_layout(problem(B, kda=False))
    assert lay_s["dg"][1] == (n, T, Hv, 1)
    assert total_s == total - n * T * Hv * (S - 1)


def test_problem_rejects_length_count_mismatch(B):
    with pytest.raises(ValueError):
        problem(B, seq_lens=[64])


@pytest.mark.parametrize("kw,code", [
    (dict(S=48), -2), (dict(S=8), -2), (dict(S_v=8), -2), (dict(S_v=256), -2),
    (dict(H_k=3), -2), (dict(n_seqs=-1, seq_lens=None), -1),
    (dict(T=-1), -1), (dict(C=-1), -1), (dict(seq_lens=[65, 3]), -1),
    (dict(seq_lens=[-1, 3]), -1), (dict(scale=float("nan")), -1), (dict(H_k=0), -1),
    (dict(dtype=3), -1), (dict(dtype=-1), -1),
])
def test_invalid_problems(B, kw, code):
    p = problem(B, **kw)
    assert B.workspace_size(p) == 0
    assert B.lib.gdn_grad_packed_floats(p.c, None) == 0
    fake = ctypes.c_void_p(1 << 20)
    rc = B.lib.gdn_fwd(p.c, *([fake] * 8), fake, 1 << 40, None)
    assert rc == code


def _fwd(B, p, ptrs, ws_bytes):
    return B.lib.gdn_fwd(p.c, *[ctypes.c_void_p(x) if x else None for x in ptrs],
                         ws_bytes, None)


def _bwd(B, p, ptrs, ws_bytes, flags=0):
    return B.lib.gdn_bwd(p.c, *[ctypes.c_void_p(x) if x else None for x in ptrs],
                         ws_bytes, flags, None)


def layout_ptrs(p, B):
    """Disjoint fake device addresses for every argument of gdn_fwd / gdn_bwd."""
    base = 1 << 32
    step = 1 << 30
    names = ["q", "k", "v", "g", "beta", "state0", "y", "state_out", "ws", "gy", "dso", "grad"]
    return {n: base + i * step for i, n in enumerate(names)}


def test_fwd_argument_errors(B):
    p = problem(B)
    ws = B.workspace_size(p)
    a = layout_ptrs(p, B)
    good = [a[n] for n in ("q", "k", "v", "g", "beta", "state0", "y", "state_out", "ws")]
    for i in range(9):                       # each required pointer NULL
        bad = list(good)
        bad[i] = 0
        assert _fwd(B, p, bad, ws) == -1
    assert _fwd(B, p, good, ws - 1) == -3    # workspace too small
    mis = list(good)
    mis[0] += 2                              # q not 4-byte aligned
    assert _fwd(B, p, mis, ws) == -2
    ov = list(good)
    ov[6] = good[2] + 64                     # y overlapping v
    assert _fwd(B, p, ov, ws) == -1
    ov = list(good)
    ov[8] = good[7] + 256                    # workspace overlapping state_out
    assert _fwd(B, p, ov, ws) == -1
    # y as a self-overlapping view
    pbad = problem(B, strides={"y": (0, 8 * 64, 32)})
    assert _fwd(B, pbad, good, ws) == -1
    # negative stride
    pneg = problem(B, strides={"q": (-1, 256, 64)})
    assert _fwd(B, pneg, good, ws) == -2


def test_bwd_argument_errors(B):
    p = problem(B)
    ws = B.workspace_size(p)
    a = layout_ptrs(p, B)
    good = [a[n] for n in ("q", "k", "v", "g", "beta", "state0", "gy", "dso", "grad", "ws")]
    for i in range(10):
        if i == 7:
            continue                          # dstate_out may be NULL
        bad = list(good)
        bad[i] = 0
        assert _bwd(B, p, bad, ws) == -1, i
    assert _bwd(B, p, good, ws, flags=2) == -1
    assert _bwd(B, p, good, ws - 256) == -3
    ov = list(good)
    ov[8] = good[6] + 128                     # packed grads overlapping gy
    assert _bwd(B, p, ov, ws) == -1
    ov = list(good)
    ov[9] = good[0]                           # workspace overlapping q
    assert _bwd(B, p, ov, ws) == -1


def test_rectangular_heads_layout(B):
    """S_k != S_v: workspace (small-head path at every pair but 128 x 128) and the packed
    gradient regions (dq, dk, dg over S_k; dv over S_v; dstate S_v x S_k)."""
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    n, T, Hk, Hv, C = 2, 64, 4, 8, 8
    for Sk, Sv in ((64, 32), (32, 128), (128, 16), (16, 64)):
        for kda in (True, False):
            p = problem(B, S=Sk, S_v=Sv, kda=kda)
            units = n * Hv
            ws = al(units * -(-T // C) * Sv * Sk * 4)
            ws = al(ws + units * C * Sv * Sk * 4)
            ws = al(ws + units * C * Sv * 4)
            ws = al(al(ws + n * T * Hv * Sk * 4) + n * T * Hv * Sk * 4)
            assert B.workspace_size(p) == ws, (Sk, Sv, kda)
            total, lay = B.grad_layout(p)
            G = Sk if kda else 1
            assert lay["dq"][1] == (n, T, Hk, Sk) and lay["dv"][1] == (n, T, Hv, Sv)
            assert lay["dg"][1] == (n, T, Hv, G) and lay["dstate"][1] == (n, Hv, Sv, Sk)
            assert total == n * T * (2 * Hk * Sk + Hv * Sv + Hv * G + Hv) + n * Hv * Sv * Sk


def test_half_inputs_workspace_and_alignment(B):
    """fp16/bf16 inputs: the workspace gains their fp32 copies; input pointers need only
    2-byte alignment (the other buffers still 4)."""
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    n, T, Hk, Hv, S = 2, 64, 4, 8, 64
    for kda in (True, False):
        for dt in (1, 2):
            G = S if kda else 1
            widened = (2 * n * T * Hk * S + 2 * n * T * Hv * S + n * T * Hv * G + n * T * Hv) * 4
            ph = problem(B, dtype=dt, kda=kda)
            assert B.workspace_size(ph) == al(widened) + expected_ws(n, T, Hk, Hv, S, 8, kda=kda)
    # head size 128 reads half inputs directly: no copies, the fp32 workspace
    for dt in (1, 2):
        assert B.workspace_size(problem(B, dtype=dt, S=128, C=16)) == \
            B.workspace_size(problem(B, dtype=0, S=128, C=16))
    ph = problem(B, dtype=2)
    ws = B.workspace_size(ph)
    a = layout_ptrs(ph, B)
    good = [a[x] for x in ("q", "k", "v", "g", "beta", "state0", "y", "state_out", "ws")]
    odd = list(good)
    odd[0] += 1                               # q not 2-byte aligned
    assert _fwd(B, ph, odd, ws) == -2
    two = list(good)
    two[0] += 2                               # q 2-byte aligned: accepted, then ws too small
    assert _fwd(B, ph, two, ws - 1) == -3
    st = list(good)
    st[5] += 2                                # state0 stays fp32: 4-byte alignment
    assert _fwd(B, ph, st, ws) == -2
    gb = [a[x] for x in ("q", "k", "v", "g", "beta", "state0", "gy", "dso", "grad", "ws")]
    gb[6] += 1                                # gy not 2-byte aligned
    assert _bwd(B, ph, gb, ws) == -2


def test_status_strings(B):
    for c in (0, -1, -2, -3, -4):
        assert B.lib.gdn_status_string(c)


def _conv(B, fwd, n=2, T=16, D=8, K=4, sx_st=None, y_st=None, ptrs=None):
    sx_st = sx_st or ((T + K - 1) * D, D)
    y_st = y_st or (T * D, D)
    p = B.conv_problem(n, T, D, K, sx_st, y_st)
    a = ptrs or (1 << 32, 1 << 33, 1 << 34)
    f = B.lib.gdn_ssm_conv_fwd if fwd else B.lib.gdn_ssm_conv_bwd
    return f(ctypes.byref(p), *[ctypes.c_void_p(x) if x else None for x in a], None)


def test_conv_argument_errors(B):
    """The convolution entry points reject bad problems and pointers before any launch."""
    for fwd in (True, False):
        assert _conv(B, fwd, K=0) == -1
        assert _conv(B, fwd, K=9) == -2
        assert _conv(B, fwd, D=0) == -1
        assert _conv(B, fwd, T=-1) == -1
        assert _conv(B, fwd, sx_st=(-1, 8)) == -2
        for i in range(3):
            bad = [1 << 32, 1 << 33, 1 << 34]
            bad[i] = 0
            assert _conv(B, fwd, ptrs=bad) == -1
            bad = [1 << 32, 1 << 33, 1 << 34]
            bad[i] += 2
            assert _conv(B, fwd, ptrs=bad) == -2
        # the output overlapping the input, or the taps
        assert _conv(B, fwd, ptrs=(1 << 32, 1 << 33, (1 << 32) + 64)) == -1
        assert _conv(B, fwd, ptrs=(1 << 32, 1 << 33, (1 << 33) + 16)) == -1
    # a tensor with no elements may be NULL (and nothing is launched when no output row
    # exists); one that has elements may not
    assert _conv(B, True, T=0, ptrs=(1 << 32, 1 << 33, 0)) == 0
    assert _conv(B, True, n=0, ptrs=(0, 1 << 33, 0)) == 0
    assert _conv(B, False, n=0, ptrs=(0, 1 << 33, 0)) == 0
    assert _conv(B, True, T=0, ptrs=(0, 1 << 33, 1 << 34)) == -1     # 3 carried rows to read
    assert _conv(B, False, T=0, ptrs=(1 << 32, 1 << 33, 0)) == -1    # 3 carried rows to write
    # an output view whose rows overlap each other (row stride below the channel count):
    # y in the forward, d_sx in the backward
    assert _conv(B, True, y_st=(16 * 8, 4)) == -1
    assert _conv(B, False, sx_st=(19 * 8, 4)) == -1


def _l2(B, bwd, n=2, T=8, H=3, W=16, eps=1e-6, st=None, ptrs=None):
    """One l2norm call with fake device addresses; st = (x, dy, out) stride triples."""
    dense = (T * H * W, H * W, W)
    sx, sdy, so = st or (dense, dense, dense)
    p = B._L2Problem(n, T, H, W, eps, B._Strides(*sx), B._Strides(*sdy), B._Strides(*so))
    a = ptrs or (1 << 32, 1 << 33, 1 << 34)
    args = [ctypes.c_void_p(x) if x else None for x in a]
    if bwd:
        return B.lib.gdn_l2norm_bwd(ctypes.byref(p), args[0], args[1], args[2], None)
    return B.lib.gdn_l2norm_fwd(ctypes.byref(p), args[0], args[2], None)


def test_l2norm_argument_errors(B):
    """The normalisation entry points reject bad problems, pointers and overlaps before any
    launch; every call here fails validation."""
    dense = (8 * 3 * 16, 3 * 16, 16)
    for bwd in (False, True):
        assert _l2(B, bwd, W=0) == -1
        assert _l2(B, bwd, W=1025) == -2
        assert _l2(B, bwd, T=-1) == -1
        assert _l2(B, bwd, eps=-1.0) == -1
        assert _l2(B, bwd, eps=float("nan")) == -1
        assert _l2(B, bwd, eps=float("inf")) == -1
        assert _l2(B, bwd, st=((-1, 48, 16), dense, dense)) == -2
        assert _l2(B, bwd, ptrs=(0, 1 << 33, 1 << 34)) == -1            # x missing
        assert _l2(B, bwd, ptrs=(1 << 32, 1 << 33, 0)) == -1            # out missing
        assert _l2(B, bwd, ptrs=((1 << 32) + 2, 1 << 33, 1 << 34)) == -2
        # out overlapping x without being the same view
        assert _l2(B, bwd, ptrs=(1 << 32, 1 << 33, (1 << 32) + 64)) == -1
        assert _l2(B, bwd, st=(dense, dense, (48, 16, 16)), ptrs=(1 << 32, 1 << 33, 1 << 32)) == -1
        # out overlapping itself (head stride below the row width)
        assert _l2(B, bwd, st=(dense, dense, (8 * 3 * 8, 3 * 8, 8))) == -1
    assert _l2(B, True, ptrs=(1 << 32, 0, 1 << 34)) == -1               # dy missing
    assert _l2(B, True, ptrs=(1 << 32, 1 << 33, (1 << 33) + 32)) == -1  # out overlapping dy
    # no rows: NULL pointers are fine and nothing is launched
    assert _l2(B, False, T=0, ptrs=(0, 0, 0)) == 0
    assert _l2(B, True, n=0, ptrs=(0, 0, 0)) == 0


def _ssm(B, **kw):
    d = dict(n_seqs=2, T=20, H=4, P=8, N=32, G=2, a_per_state=0, dt_softplus=1)
    d.update(kw)
    return B._SsmProblem(*(d[k] for k in ("n_seqs", "T", "H", "P", "N", "G", "a_per_state",
                                          "dt_softplus")))


def test_ssm_sizes_and_layout(B):
    p = _ssm(B)
    ws = B.ssm_workspace_size(p)
    nwin = 3
    rows = 2 * 4 * 8
    assert ws >= 4 * (rows * nwin * 32 + rows // 16 * 20 * 2 * 32 + 2 * 20 * 4 * 8)
    total, lay = B.ssm_grad_layout(p)
    sizes = [2 * 4 * 8 * 32, 2 * 20 * 4 * 8, 2 * 20 * 4, 2 * 20 * 2 * 32, 2 * 20 * 2 * 32]
    assert total == sum(sizes)
    assert [lay[k][0] for k in ("ds", "dx", "ddt", "dB", "dC")] == [sum(sizes[:i]) for i in range(5)]


def test_ssm_chunked_workspace(B):
    """One decay per head with P = 64, N = 128: the chunked backward's workspace (the state before
    each 32-token chunk, the state gradient after each chunk, dB and dC per head slice; here two
    slices, one per head of a group), much smaller than the per-token form's."""
    up = lambda b: (b + 255) // 256 * 256
    n, T, H, P, N, G = 2, 100, 4, 64, 128, 2
    nc, rows = 4, n * H * P
    ws = B.ssm_workspace_size(_ssm(B, n_seqs=n, T=T, H=H, P=P, N=N, G=G))
    assert ws == up(4 * rows * nc * N) + up(4 * n * H * nc * P * N) + up(4 * 2 * 2 * n * T * G * N)
    per_token = B.ssm_workspace_size(_ssm(B, n_seqs=n, T=T, H=H, P=P, N=N, G=G, a_per_state=1))
    assert per_token >= 4 * (rows * 13 * N + rows // 16 * T * 2 * N + n * T * H * P) > ws


@pytest.mark.parametrize("kw,code", [
    (dict(H=4, G=3), -1), (dict(N=24), -2), (dict(N=256), -2), (dict(P=3, H=4, G=2), -2),
    (dict(a_per_state=2), -1), (dict(dt_softplus=-1), -1), (dict(T=-1), -1), (dict(P=0), -1),
    (dict(n_seqs=1 << 20, H=1 << 10, P=1 << 7, G=1), -2),    # 2^33 rows: beyond one launch
    (dict(n_seqs=1 << 12, T=1 << 20, H=1 << 4, P=64, N=128, G=1), -2),   # 2^31 chunks x heads
    (dict(n_seqs=1 << 14, T=1 << 20, H=1 << 8, P=1, N=16, G=1), -2),     # 2^32 windows x row blocks
])
def test_ssm_invalid_problems(B, kw, code):
    p = _ssm(B, **kw)
    assert B.lib.gdn_ssm_workspace_size(ctypes.byref(p)) == 0
    assert B.lib.gdn_ssm_fwd(ctypes.byref(p), *([None] * 8), None, 0, None) == code


def test_ssm_argument_errors(B):
    """Every call fails validation before any launch."""
    p = _ssm(B)
    ws = B.ssm_workspace_size(p)
    base = [1 << 32, 1 << 33, 1 << 34, 1 << 35, 1 << 36, 1 << 37]     # s0 x dt A B C
    y, s_out, w = 1 << 38, 1 << 39, 1 << 40

    def fwd(ins=base, y=y, s_out=s_out, w=w, wsb=ws):
        args = [ctypes.c_void_p(v) if v else None for v in list(ins) + [y, s_out, w]]
        return B.lib.gdn_ssm_fwd(ctypes.byref(p), *args, wsb, None)

    def bwd(ins=base, gy=1 << 41, gs=1 << 42, gp=1 << 43, w=w, wsb=ws, flags=0):
        args = [ctypes.c_void_p(v) if v else None for v in list(ins) + [gy, gs, gp, w]]
        return B.lib.gdn_ssm_bwd(ctypes.byref(p), *args, wsb, flags, None)

    for i in range(6):                                   # a required input missing
        bad = list(base)
        bad[i] = 0
        assert fwd(ins=bad) == -1 and bwd(ins=bad) == -1
    assert fwd(y=0) == -1 and fwd(s_out=0) == -1 and fwd(w=0) == -1
    assert bwd(gy=0) == -1 and bwd(gp=0) == -1 and bwd(w=0) == -1
    assert fwd(wsb=ws - 1) == -3 and bwd(wsb=ws - 1) == -3
    assert bwd(flags=2) == -1
    mis = list(base)
    mis[4] += 4                                          # B not 16-byte aligned
    assert fwd(ins=mis) == -2 and bwd(ins=mis) == -2
    assert fwd(s_out=s_out + 8) == -2 and bwd(gs=(1 << 42) + 4) == -2 and bwd(gp=(1 << 43) + 8) == -2
    assert fwd(y=base[1] + 64) == -1                     # y over x
    assert fwd(w=base[4]) == -1                          # workspace over B
    assert bwd(gp=base[0] + 16) == -1                    # gradients over s0
    assert bwd(gp=(1 << 41) + 16) == -1                  # gradients over gy
    assert bwd(w=(1 << 43) + 64) == -1                   # workspace over the gradients
