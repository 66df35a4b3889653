"""The convolution kernels (through the C ABI) against the fp64 oracle, on the GPU."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_cases import log  # noqa: E402

TOL = 1e-5   # fp32 taps summed in order against fp64: a few ulp of the largest term


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_bwd_amd import binding  # loads libgdn.so
    return binding


def _data(seed, n, T, D, K):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)  # noqa: E731
    return f(n, T + K - 1, D), f(D, K), f(n, T, D)


def _rel(x, r):
    """Worst error over slices: per sequence, and per group of 128 channels (a head of the
    mixed q/k/v rows) when the width is a multiple of 128."""
    from compare import slice_rel
    D = r.shape[-1] if r.ndim else 0
    return slice_rel(x, r, (0,), 128 if D and D % 128 == 0 else None)


def run(B, sx, c, dy, wide=0):
    """GPU y and d_sx; with wide > 0 the tensors are row views of wider buffers."""
    n, TT, D = sx.shape
    T = dy.shape[1]
    def view(a):
        if not wide:
            return torch.from_numpy(a).cuda()
        buf = torch.zeros((a.shape[0], a.shape[1], D + wide), device="cuda")
        v = buf[:, :, wide // 2: wide // 2 + D]
        v.copy_(torch.from_numpy(a))
        return v
    gsx, gdy, gc = view(sx), view(dy), torch.from_numpy(c).cuda()
    y = view(np.zeros((n, T, D), np.float32))
    dsx = view(np.zeros((n, TT, D), np.float32))
    B.ssm_conv_fwd(gsx, gc, y)
    B.ssm_conv_bwd(gdy, gc, dsx)
    torch.cuda.synchronize()
    return y.cpu().numpy(), dsx.cpu().numpy()


@pytest.mark.parametrize("n,T,D,K,wide", [
    (2, 37, 20, 4, 0),     # channels not a multiple of 4: one channel per thread
    (3, 100, 64, 4, 0),    # four channels per thread
    (1, 5, 8, 1, 0),       # no carried rows
    (2, 19, 12, 8, 0),     # the widest window
    (2, 64, 32, 3, 12),    # row views of wider buffers (strided rows, 16-byte misaligned)
    (2, 64, 32, 4, 8),     # row views, aligned
    (2, 0, 16, 4, 0),      # no tokens: the carried rows get a zero gradient
])
def test_conv_parity(dev, n, T, D, K, wide):
    from oracle import ssm_conv as C
    sx, c, dy = _data(900 + T + D + K, n, T, D, K)
    y, dsx = run(dev, sx, c, dy, wide)
    ry, rdsx = C.conv_fwd(sx, c), C.conv_bwd(dy, c)
    ey, ed = _rel(y, ry), _rel(dsx, rdsx)
    log(f"[conv] n={n} T={T} D={D} K={K} wide={wide}: y {ey:.1e}, d_sx {ed:.1e}")
    assert ey <= TOL and ed <= TOL
    if T == 0:
        assert not np.any(dsx)
    y2, dsx2 = run(dev, sx, c, dy, wide)
    assert np.array_equal(y, y2) and np.array_equal(dsx, dsx2)   # deterministic


def test_conv_layer_shape(dev):
    """The convolution that feeds the layer shape's mixed rows: 4 x 4096 tokens, 10240
    channels (2 x 16 x 128 + 48 x 128), 4 taps; the oracle checks sequence 0 in full."""
    from oracle import ssm_conv as C
    n, T, D, K = 4, 4096, 10240, 4
    sx, c, dy = _data(990, n, T, D, K)
    y, dsx = run(dev, sx, c, dy)
    ey = _rel(y[:1], C.conv_fwd(sx[:1], c))
    ed = _rel(dsx[:1], C.conv_bwd(dy[:1], c))
    log(f"[conv] layer shape, sequence 0: y {ey:.1e}, d_sx {ed:.1e}")
    assert ey <= TOL and ed <= TOL
