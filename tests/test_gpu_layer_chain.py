"""A hybrid layer's recurrence path chained from the C ABI's pieces, on the GPU, against the
same chain composed from the oracles.

Forward: the short convolution produces the mixed rows [q | k | v]; q and k are L2-normalised
from their row views into a packed buffer; the recurrence reads them there and v as a view of
the mixed rows.  Backward: the recurrence's gradients; the normalisation's backward writes dq
and dk straight into views of the mixed rows' gradient, dv is placed beside them, and the
convolution's backward gives the input gradient, carried state rows included."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_cases import log  # noqa: E402

TOL = 2e-4
EPS = 1e-6


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_bwd_amd import binding  # loads libgdn.so
    return binding


def _rel(x, r, name):
    """Worst error over (sequence, head) slices: per-token regions [n][T][H][..] slice on axes
    0 and 2, states [n][H][..] on 0 and 1, the input gradient [n][rows][D] per sequence and
    128-channel group."""
    from compare import slice_rel
    if name == "dsx":
        return slice_rel(x, r, (0,), 128 if r.shape[-1] % 128 == 0 else None)
    return slice_rel(x, r, (0, 1) if name in ("state_out", "dstate") else (0, 2))


def _inputs(seed, n, T, Hk, Hv, S, K):
    rng = np.random.default_rng(seed)
    D = 2 * Hk * S + Hv * S
    f = np.float32
    return {
        "sx": rng.standard_normal((n, T + K - 1, D)).astype(f),
        "c": (rng.standard_normal((D, K)) / np.sqrt(K)).astype(f),
        "g": rng.uniform(-0.5, 0.0, (n, T, Hv, S)).astype(f),
        "beta": rng.uniform(0.0, 1.0, (n, T, Hv)).astype(f),
        "state0": (0.1 * rng.standard_normal((n, Hv, S, S))).astype(f),
        "gy": rng.standard_normal((n, T, Hv, S)).astype(f),
        "dso": rng.standard_normal((n, Hv, S, S)).astype(f),
    }


def gpu_chain(B, a, n, T, Hk, Hv, S, C):
    cuda = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    sx, c = cuda(a["sx"]), cuda(a["c"])
    g, beta, state0, gy, dso = (cuda(a[k]) for k in ("g", "beta", "state0", "gy", "dso"))
    HkS = Hk * S
    D = sx.shape[2]
    mix = torch.empty((n, T, D), device="cuda")
    B.ssm_conv_fwd(sx, c, mix)
    qraw = mix[:, :, :HkS].unflatten(2, (Hk, S))
    kraw = mix[:, :, HkS:2 * HkS].unflatten(2, (Hk, S))
    v = mix[:, :, 2 * HkS:].unflatten(2, (Hv, S))
    qk = torch.empty((n, T, 2 * HkS), device="cuda")
    qn = qk[:, :, :HkS].unflatten(2, (Hk, S))
    kn = qk[:, :, HkS:].unflatten(2, (Hk, S))
    B.l2norm_fwd(qraw, qn, EPS)
    B.l2norm_fwd(kraw, kn, EPS)
    y = torch.empty((n, T, Hv, S), device="cuda")
    state_out = torch.empty((n, Hv, S, S), device="cuda")
    p = B.Problem.from_tensors(qn, kn, v, g, beta, C=C, scale=S ** -0.5, gy=gy, y=y)
    ws = torch.empty(max(B.workspace_size(p), 256), dtype=torch.uint8, device="cuda")
    B.fwd(p, qn, kn, v, g, beta, state0, y, state_out, ws)
    total, _ = B.grad_layout(p)
    grad = torch.empty(total, device="cuda")
    B.bwd(p, qn, kn, v, g, beta, state0, gy, dso, grad, ws, B.BWD_REUSE_SNAPSHOTS)
    G = B.unpack_grads(p, grad)
    dmix = torch.empty((n, T, D), device="cuda")
    B.l2norm_bwd(qraw, G["dq"], dmix[:, :, :HkS].unflatten(2, (Hk, S)), EPS)
    B.l2norm_bwd(kraw, G["dk"], dmix[:, :, HkS:2 * HkS].unflatten(2, (Hk, S)), EPS)
    dmix[:, :, 2 * HkS:].copy_(G["dv"].flatten(2))          # placement only
    dsx = torch.empty_like(sx)
    B.ssm_conv_bwd(dmix, c, dsx)
    torch.cuda.synchronize()
    out = {"y": y, "state_out": state_out, "dg": G["dg"], "dbeta": G["dbeta"],
           "dstate": G["dstate"], "dsx": dsx}
    return {k: t.cpu().numpy() for k, t in out.items()}


def oracle_chain(a, n, T, Hk, Hv, S, C):
    import oracle
    from oracle import l2norm as L
    from oracle import ssm_conv as CV
    HkS = Hk * S
    mix = CV.conv_fwd(a["sx"], a["c"])
    qraw = mix[:, :, :HkS].reshape(n, T, Hk, S)
    kraw = mix[:, :, HkS:2 * HkS].reshape(n, T, Hk, S)
    v = mix[:, :, 2 * HkS:].reshape(n, T, Hv, S)
    qn, kn = L.l2norm_fwd(qraw, EPS), L.l2norm_fwd(kraw, EPS)
    shape = dict(n_seqs=n, T=T, H_k=Hk, H_v=Hv, S_k=S, S_v=S, kda=True, C=C, scale=S ** -0.5,
                 seq_lens=[T] * n)
    orc = oracle.Oracle(threads=4)
    args = (qn, kn, v, a["g"], a["beta"], a["state0"])
    y, so = orc.fwd(shape, *args)
    d = orc.bwd(shape, *args, a["gy"], a["dso"])
    dmix = np.concatenate([L.l2norm_bwd(qraw, d["dq"], EPS).reshape(n, T, HkS),
                           L.l2norm_bwd(kraw, d["dk"], EPS).reshape(n, T, HkS),
                           d["dv"].reshape(n, T, Hv * S)], axis=2)
    return {"y": y, "state_out": so, "dg": d["dg"], "dbeta": d["dbeta"], "dstate": d["dstate"],
            "dsx": CV.conv_bwd(dmix, a["c"])}


@pytest.mark.parametrize("n,T,Hk,Hv,S,C", [
    (2, 40, 2, 4, 32, 0),      # small heads, two value heads per key head, ragged window
    (1, 24, 1, 2, 128, 8),     # the head size of the layer shape (matrix-core kernels)
])
def test_layer_chain(dev, n, T, Hk, Hv, S, C):
    a = _inputs(1700 + S + T, n, T, Hk, Hv, S, 4)
    got = gpu_chain(dev, a, n, T, Hk, Hv, S, C)
    ref = oracle_chain(a, n, T, Hk, Hv, S, C)
    errs = {k: _rel(got[k], ref[k].reshape(got[k].shape), k) for k in ref}
    log(f"[chain] n={n} T={T} Hk={Hk} Hv={Hv} S={S}: " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    assert all(v <= TOL for v in errs.values()), errs
