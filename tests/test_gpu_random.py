"""Seeded random problems across the supported envelope, each against the fp64 oracle on the
GPU: the recurrence over every head-size pair, both gates, grouped heads, ragged and empty
sequences, packed row views, checkpoint intervals, half-precision inputs and snapshot reuse;
the selective scan over both branches, state sizes and group shapes; the convolution and the
L2 normalisation over widths, taps and strided views.  Every case logs its seed first."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from compare import check  # noqa: E402
from gated_delta_rule_bwd_amd import inputs as I  # noqa: E402
from gpu_cases import REGIONS_BWD, REGIONS_FWD, log, oracle_results  # noqa: E402

SIZES = (16, 32, 64, 128)
HALF = {"bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_bwd_amd.device import DeviceCase
    return DeviceCase


def gdn_case(seed):
    r = np.random.default_rng(seed)
    n, T = int(r.integers(1, 4)), int(r.integers(1, 97))
    Hk = int(r.integers(1, 4))
    Hv = Hk * int(r.integers(1, 4))
    Sk, Sv = int(r.choice(SIZES)), int(r.choice(SIZES))
    kda = bool(r.random() < 0.5)
    C = 0 if r.random() < 0.4 else int(r.integers(1, T + 1))
    lens = tuple(int(x) for x in r.integers(0, T + 1, n)) if r.random() < 0.5 else None
    w = I.Workload(f"rand{seed}", n, T, Hk, Hv, Sk, kda, C, float(r.choice([-1.0, -0.3, -0.05])),
                   seq_lens=lens, packed=bool(r.random() < 0.5), seed=seed,
                   Sv=Sv if Sv != Sk else 0)
    return w, str(r.choice(["f32", "f32", "bf16", "f16"])), bool(r.random() < 0.7)


@pytest.mark.parametrize("seed", range(3000, 3024))
def test_random_gdn(dev, seed):
    w, dtype, reuse = gdn_case(seed)
    log(f"[random] seed={seed} n={w.n_seqs} T={w.T} Hk={w.H_k} Hv={w.H_v} Sk={w.S_k} Sv={w.S_v} "
        f"kda={w.kda} C={w.C} lens={w.lens} packed={w.packed} {dtype} reuse={reuse}")
    arrays, _ = I.make_all(w)
    kw = {}
    if dtype != "f32":
        arrays = I.round_inputs(arrays, dtype)
        kw["in_dtype"] = HALF[dtype]
    dc = dev(w, arrays, **kw)
    dc.fwd()
    dc.bwd(reuse=reuse)
    torch.cuda.synchronize()
    rep = check(dc.results_numpy(), oracle_results(w, arrays), REGIONS_FWD + REGIONS_BWD)
    log(f"[random] seed={seed}: " + ", ".join(f"{k} {v:.1e}" for k, v in rep.items()))


@pytest.mark.parametrize("seed", range(3100, 3112))
def test_random_ssm(seed):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_bwd_amd import binding as B
    from test_gpu_ssm import TOL, _arrays, _rel, oracle, run
    r = np.random.default_rng(seed)
    n, T = int(r.integers(1, 3)), int(r.integers(0, 61))
    N = int(r.choice(SIZES))
    P = int(r.choice([1, 2, 4, 8, 16, 32, 64]))
    G = int(r.choice([1, 2, 4]))
    hg = max(1, 16 // P) * int(r.integers(1, 3))     # heads per group: P * hg rows, a multiple of 16
    H = G * hg
    aps, softplus, with_gs = bool(r.random() < 0.5), bool(r.random() < 0.7), bool(r.random() < 0.7)
    log(f"[random] seed={seed} n={n} T={T} H={H} P={P} N={N} G={G} aps={aps} softplus={softplus}")
    arr = _arrays(n, T, H, P, N, G, aps, softplus, seed)
    y, sT, grads = run(B, arr, softplus, with_gs)
    ry, rsT, rg = oracle(arr, softplus, with_gs)
    errs = {"y": _rel(y, ry), "s_out": _rel(sT, rsT)}
    errs.update({k: _rel(grads[k], rg[k]) for k in rg})
    log(f"[random] seed={seed}: " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    assert all(v <= TOL for v in errs.values()), errs


@pytest.mark.parametrize("seed", range(3200, 3212))
def test_random_conv(seed):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_bwd_amd import binding as B
    from oracle import ssm_conv as C
    from test_gpu_conv import TOL, _data, _rel, run
    r = np.random.default_rng(seed)
    n, T, D, K = int(r.integers(1, 4)), int(r.integers(0, 51)), int(r.integers(1, 41)), int(r.integers(1, 9))
    wide = int(r.choice([0, 0, 4, 7, 12]))
    log(f"[random] seed={seed} n={n} T={T} D={D} K={K} wide={wide}")
    sx, c, dy = _data(seed, n, T, D, K)
    y, dsx = run(B, sx, c, dy, wide)
    ey, ed = _rel(y, C.conv_fwd(sx, c)), _rel(dsx, C.conv_bwd(dy, c))
    log(f"[random] seed={seed}: y {ey:.1e}, d_sx {ed:.1e}")
    assert ey <= TOL and ed <= TOL


@pytest.mark.parametrize("seed", range(3300, 3312))
def test_random_l2norm(seed):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_bwd_amd import binding as B
    from test_gpu_l2norm import _data, check, run
    r = np.random.default_rng(seed)
    n, T, H, W = int(r.integers(1, 3)), int(r.integers(0, 20)), int(r.integers(1, 5)), int(r.integers(1, 301))
    eps = float(r.choice([1e-6, 1e-3, 0.25]))
    pad = int(r.choice([0, 0, 8, 13]))
    shift = int(r.integers(0, pad + 1)) if pad else 0
    log(f"[random] seed={seed} n={n} T={T} H={H} W={W} eps={eps} pad={pad} shift={shift}")
    x, dy = _data(seed, (n, T, H, W))
    y, dx = run(B, x, dy, eps, pad, shift)
    check(x, dy, eps, y, dx, f"seed={seed}")
