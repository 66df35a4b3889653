"""The L2-normalisation kernels (through the C ABI) against the fp64 oracle, on the GPU."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_cases import log  # noqa: E402


U = 2.0 ** -24


def tol(W):
    """Rounding steps of one row in fp32: a lane sums at most min(W, 16) products in order,
    then at most log2(64) = 6 butterfly levels; the root, the reciprocal, its cube and the
    final fma add a few more.  Four times that many unit roundoffs bounds each result
    against the magnitudes it is formed from."""
    return 4 * (min(W, 16) + 6 + 6) * U


def check(x, dy, eps, y, dx, tag):
    """Elementwise error bounds: y relative to itself, dx relative to the two terms it is the
    difference of, |dy_i| / n and |y_i| sum_j |y_j dy_j| / n.  The terms cancel when dy is
    nearly parallel to x (always, when W = 1), so a bound relative to dx itself, or to the
    largest dx of the block, does not hold in fp32; this one is the textbook bound for a
    difference of rounded terms."""
    from oracle import l2norm as L
    x64, dy64 = x.astype(np.float64), dy.astype(np.float64)
    ry, rdx = L.l2norm_fwd(x64, eps), L.l2norm_bwd(x64, dy64, eps)
    n = np.sqrt(np.sum(x64 * x64, axis=-1, keepdims=True) + eps)
    terms = (np.abs(dy64) + np.abs(ry) * np.sum(np.abs(ry * dy64), axis=-1, keepdims=True)) / n
    W = x.shape[-1]
    ey = float(np.max(np.abs(y - ry) / np.maximum(np.abs(ry), 1e-300))) if y.size else 0.0
    ed = float(np.max(np.abs(dx - rdx) / np.maximum(terms, 1e-300))) if dx.size else 0.0
    log(f"[l2norm] {tag}: y {ey:.1e}, dx {ed:.1e} (bound {tol(W):.1e} x unit roundoff-scaled terms)")
    assert ey <= tol(W) and ed <= tol(W)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_bwd_amd import binding  # loads libgdn.so
    return binding


def _data(seed, shape):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape).astype(np.float32),
            rng.standard_normal(shape).astype(np.float32))


def _view(a, pad, shift):
    """a [n, T, H, W] placed as a view into a buffer with `pad` extra floats per token (rows at
    float offset `shift` into each token)."""
    n, T, H, W = a.shape
    if not pad:
        return torch.from_numpy(a).cuda()
    buf = torch.zeros((n, T, H * W + pad), device="cuda")
    v = buf[:, :, shift:shift + H * W].unflatten(2, (H, W))
    v.copy_(torch.from_numpy(a))
    return v


def run(B, x, dy, eps, pad=0, shift=0):
    gx, gdy = _view(x, pad, shift), _view(dy, pad, shift)
    y = _view(np.zeros_like(x), pad, shift)
    dx = _view(np.zeros_like(x), pad, shift)
    B.l2norm_fwd(gx, y, eps)
    B.l2norm_bwd(gx, gdy, dx, eps)
    torch.cuda.synchronize()
    return y.cpu().numpy(), dx.cpu().numpy()


CASES = [
    # n, T, H, W, eps, pad, shift
    (2, 37, 4, 128, 1e-6, 0, 0),      # the recurrence's head size, dense
    (2, 37, 4, 16, 1e-6, 0, 0),       # four lanes per row
    (1, 19, 3, 20, 0.0, 0, 0),        # chunks not a power of two; eps = 0
    (1, 11, 2, 7, 1e-3, 0, 0),        # odd width: one float per lane
    (1, 9, 5, 1, 1e-6, 0, 0),         # width one: y = x / sqrt(x^2 + eps)
    (1, 4, 2, 1024, 1e-6, 0, 0),      # widest row: 64 lanes x 16 floats
    (1, 6, 2, 1000, 1e-6, 0, 0),      # wide, last chunks partly idle
    (2, 33, 6, 64, 1e-6, 96, 32),     # row views of a wider buffer, 16-byte aligned
    (2, 33, 6, 64, 1e-6, 96, 31),     # the same, misaligned: one float per lane
    (2, 0, 4, 128, 1e-6, 0, 0),       # no tokens
]


@pytest.mark.parametrize("n,T,H,W,eps,pad,shift", CASES)
def test_l2norm_parity(dev, n, T, H, W, eps, pad, shift):
    x, dy = _data(1200 + W + T + shift, (n, T, H, W))
    y, dx = run(dev, x, dy, eps, pad, shift)
    check(x, dy, eps, y, dx, f"n={n} T={T} H={H} W={W} eps={eps} pad={pad} shift={shift}")
    y2, dx2 = run(dev, x, dy, eps, pad, shift)
    assert np.array_equal(y, y2) and np.array_equal(dx, dx2)     # deterministic


def test_l2norm_zero_rows(dev):
    """An all-zero row maps to zero (eps > 0) and its gradient to dy / sqrt(eps)."""
    x, dy = _data(1300, (1, 3, 2, 32))
    x[0, 1] = 0.0
    y, dx = run(dev, x, dy, 1e-4)
    assert not np.any(y[0, 1])
    np.testing.assert_allclose(dx[0, 1], dy[0, 1] / np.sqrt(np.float32(1e-4)), rtol=1e-6)


def test_l2norm_in_place(dev):
    """Output over the input view (same pointer, same strides) gives the out-of-place bits."""
    B = dev
    x, dy = _data(1301, (2, 17, 4, 128))
    y_ref, dx_ref = run(B, x, dy, 1e-6)
    gx = torch.from_numpy(x).cuda()
    B.l2norm_fwd(gx, gx, 1e-6)
    gx2, gdy = torch.from_numpy(x).cuda(), torch.from_numpy(dy).cuda()
    B.l2norm_bwd(gx2, gdy, gdy, 1e-6)               # dx written over dy
    torch.cuda.synchronize()
    assert np.array_equal(gx.cpu().numpy(), y_ref)
    assert np.array_equal(gdy.cpu().numpy(), dx_ref)


def test_l2norm_layer_qk_rows(dev):
    """The layer shape's q and k rows as one view of the packed [4, 4096, 10240] buffer
    (32 heads of 128 at the start of each token), every row checked."""
    B = dev
    n, T, H, W = 4, 4096, 32, 128
    x, dy = _data(1302, (n, T, H, W))
    buf = torch.zeros((n, T, 10240), device="cuda")
    xv = buf[:, :, :H * W].unflatten(2, (H, W))
    xv.copy_(torch.from_numpy(x))
    gdy = torch.from_numpy(dy).cuda()
    y = torch.empty((n, T, H, W), device="cuda")
    dx = torch.empty_like(y)
    B.l2norm_fwd(xv, y, 1e-6)
    B.l2norm_bwd(xv, gdy, dx, 1e-6)
    torch.cuda.synchronize()
    check(x, dy, 1e-6, y.cpu().numpy(), dx.cpu().numpy(), "layer q|k rows")
