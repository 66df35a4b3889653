"""gdn_bwd_noalloc (the backward on the library's static workspace) against gdn_bwd with a
caller workspace: two calls in a row, the second on a smaller problem, each bitwise equal to
the workspace call (same kernels and workspace layout) and within 2e-4 of the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gated_delta_rule_bwd_amd import inputs as I  # noqa: E402
from compare import check  # noqa: E402
from gpu_cases import REGIONS_BWD, log, oracle_results  # noqa: E402

CASES = [
    # larger first, then smaller: the second call runs on what the first left in the array
    I.Workload("noalloc_s128_kda", 2, 100, 2, 6, 128, True, 32, -0.3, seed=901, seq_lens=(100, 77)),
    I.Workload("noalloc_s64_scalar", 1, 40, 1, 2, 64, False, 8, -1.0, seed=902),
    I.Workload("noalloc_s128_scalar", 1, 37, 1, 1, 128, False, 16, -0.5, seed=903),
]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_bwd_amd.device import DeviceCase  # loads libgdn.so
    return DeviceCase


def test_noalloc_matches_workspace_call(dev):
    from gated_delta_rule_bwd_amd import binding as B
    for w in CASES:
        log(f"[noalloc] {w.name} lens={w.lens}")
        arrays, _ = I.make_all(w)
        dc = dev(w, arrays)
        assert B.workspace_size(dc.p) <= B.NOALLOC_SCRATCH_BYTES
        dc.bwd(reuse=False)
        torch.cuda.synchronize()
        ref_ws = {k: v.detach().cpu().numpy().copy() for k, v in dc.grads().items()}
        dc.grad.fill_(float("nan"))
        B.bwd_noalloc(dc.p, dc.q, dc.k, dc.v, dc.g, dc.beta, dc.state0, dc.gy, dc.dstate_out,
                      dc.grad)
        torch.cuda.synchronize()
        got = {k: v.detach().cpu().numpy() for k, v in dc.grads().items()}
        for name in REGIONS_BWD:
            assert np.array_equal(got[name], ref_ws[name]), (w.name, name)
        rep = check(got, oracle_results(w, arrays), REGIONS_BWD)
        log(f"[noalloc] {w.name}: " + ", ".join(f"{k} {v:.1e}" for k, v in rep.items()))


def test_noalloc_rejects_oversize(dev):
    from gated_delta_rule_bwd_amd import binding as B
    w = I.Workload("noalloc_big", 2, 4096, 2, 6, 128, True, 64, -0.3, seed=904)
    p = B.Problem(w.n_seqs, w.T, w.H_k, w.H_v, w.S, w.kda, w.C, w.scale)
    assert B.workspace_size(p) > B.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(1, device="cuda")
    ptr = B.ctypes.c_void_p(x.data_ptr())
    stream = B.ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = B.lib.gdn_bwd_noalloc(p.c, ptr, ptr, ptr, ptr, ptr, ptr, ptr, None, ptr, stream)
    assert rc == -3   # GDN_ERR_WORKSPACE, returned before anything is enqueued
