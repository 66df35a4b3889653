"""ctypes binding of the C ABI in include/gdn.h (argument marshalling only).

Every step of the computation runs in the HIP kernels of ``libgdn.so``; this module only
turns torch tensors into raw device pointers, strides and a stream handle.  Loading fails
loudly when the library has not been built: there is no other implementation to fall
back to.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is missing: build it with `python -m gated_delta_rule_bwd_amd.build` "
        "(or __graft_entry__.build())")
lib = ctypes.CDLL(_LIB_PATH)

STATUS = {0: "GDN_OK", -1: "GDN_ERR_ARG", -2: "GDN_ERR_UNSUPPORTED",
          -3: "GDN_ERR_WORKSPACE", -4: "GDN_ERR_DEVICE"}
GATE_SCALAR, GATE_KDA = 0, 1
DTYPE_F32, DTYPE_F16, DTYPE_BF16 = 0, 1, 2
_DTYPES = {torch.float32: DTYPE_F32, torch.float16: DTYPE_F16, torch.bfloat16: DTYPE_BF16}
BWD_REUSE_SNAPSHOTS = 1
EXPORTS = ("gdn_workspace_size", "gdn_grad_packed_floats", "gdn_fwd", "gdn_bwd", "gdn_bwd_noalloc",
           "gdn_ssm_conv_fwd", "gdn_ssm_conv_bwd", "gdn_l2norm_fwd", "gdn_l2norm_bwd",
           "gdn_ssm_workspace_size", "gdn_ssm_grad_packed_floats", "gdn_ssm_fwd", "gdn_ssm_bwd",
           "gdn_status_string")


class GdnError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {STATUS.get(code, code)} "
                         f"({lib.gdn_status_string(code).decode()})")
        self.code = code


class _Strides(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_int64), ("tok", ctypes.c_int64), ("head", ctypes.c_int64)]


class _Problem(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("T", ctypes.c_int32), ("H_k", ctypes.c_int32),
                ("H_v", ctypes.c_int32), ("S_k", ctypes.c_int32), ("S_v", ctypes.c_int32),
                ("gate", ctypes.c_int32), ("C", ctypes.c_int32), ("scale", ctypes.c_float),
                ("seq_lens", ctypes.POINTER(ctypes.c_int32))] + \
               [(n, _Strides) for n in ("q", "k", "v", "g", "beta", "gy", "y")] + \
               [("dtype", ctypes.c_int32)]


_VP = ctypes.c_void_p
lib.gdn_workspace_size.argtypes = [ctypes.POINTER(_Problem)]
lib.gdn_workspace_size.restype = ctypes.c_size_t
lib.gdn_grad_packed_floats.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(ctypes.c_size_t)]
lib.gdn_grad_packed_floats.restype = ctypes.c_size_t
lib.gdn_fwd.argtypes = [ctypes.POINTER(_Problem)] + [_VP] * 9 + [ctypes.c_size_t, _VP]
lib.gdn_fwd.restype = ctypes.c_int
lib.gdn_bwd.argtypes = [ctypes.POINTER(_Problem)] + [_VP] * 10 + [ctypes.c_size_t,
                                                                 ctypes.c_uint, _VP]
lib.gdn_bwd.restype = ctypes.c_int
lib.gdn_bwd_noalloc.argtypes = [ctypes.POINTER(_Problem)] + [_VP] * 9 + [_VP]
lib.gdn_bwd_noalloc.restype = ctypes.c_int
NOALLOC_SCRATCH_BYTES = 64 << 20   # GDN_NOALLOC_SCRATCH_BYTES
class _ConvProblem(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("T", ctypes.c_int32), ("d_inner", ctypes.c_int32),
                ("d_conv", ctypes.c_int32), ("sx_seq", ctypes.c_int64), ("sx_tok", ctypes.c_int64),
                ("y_seq", ctypes.c_int64), ("y_tok", ctypes.c_int64)]


for _f in (lib.gdn_ssm_conv_fwd, lib.gdn_ssm_conv_bwd):
    _f.argtypes = [ctypes.POINTER(_ConvProblem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_void_p]
    _f.restype = ctypes.c_int


class _L2Problem(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("W", ctypes.c_int32), ("eps", ctypes.c_float), ("x", _Strides), ("dy", _Strides),
                ("out", _Strides)]


lib.gdn_l2norm_fwd.argtypes = [ctypes.POINTER(_L2Problem), ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p]
lib.gdn_l2norm_fwd.restype = ctypes.c_int
lib.gdn_l2norm_bwd.argtypes = [ctypes.POINTER(_L2Problem), ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p]
lib.gdn_l2norm_bwd.restype = ctypes.c_int


class _SsmProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_seqs", "T", "H", "P", "N", "G", "a_per_state",
                                               "dt_softplus")]


lib.gdn_ssm_workspace_size.argtypes = [ctypes.POINTER(_SsmProblem)]
lib.gdn_ssm_workspace_size.restype = ctypes.c_size_t
lib.gdn_ssm_grad_packed_floats.argtypes = [ctypes.POINTER(_SsmProblem), ctypes.POINTER(ctypes.c_size_t)]
lib.gdn_ssm_grad_packed_floats.restype = ctypes.c_size_t
lib.gdn_ssm_fwd.argtypes = [ctypes.POINTER(_SsmProblem)] + [ctypes.c_void_p] * 9 + [ctypes.c_size_t,
                                                                                   ctypes.c_void_p]
lib.gdn_ssm_fwd.restype = ctypes.c_int
lib.gdn_ssm_bwd.argtypes = [ctypes.POINTER(_SsmProblem)] + [ctypes.c_void_p] * 10 + [
    ctypes.c_size_t, ctypes.c_uint, ctypes.c_void_p]
lib.gdn_ssm_bwd.restype = ctypes.c_int
lib.gdn_status_string.argtypes = [ctypes.c_int]
lib.gdn_status_string.restype = ctypes.c_char_p


def _tok_strides(t, name):
    """(seq, tok, head) strides of a [n, T, H, W] (or [n, T, H]) tensor; innermost must be 1."""
    if t is None:
        return (0, 0, 0)
    if t.dim() == 4:
        if t.shape[3] > 1 and t.stride(3) != 1:
            raise ValueError(f"{name}: innermost stride must be 1")
        return tuple(int(x) for x in t.stride()[:3])
    if t.dim() == 3:
        return tuple(int(x) for x in t.stride())
    raise ValueError(f"{name}: expected 3 or 4 dims, got {tuple(t.shape)}")


class Problem:
    """A gdn_problem: sizes, gate kind, interval, scale, lengths and the strides of the
    per-token tensors.  Use ``Problem.from_tensors``."""

    def __init__(self, n_seqs, T, H_k, H_v, S, kda, C, scale, seq_lens=None, strides=None,
                 dtype=DTYPE_F32, S_v=None):
        self.n_seqs, self.T, self.H_k, self.H_v, self.S = n_seqs, T, H_k, H_v, S
        self.S_k, self.S_v = S, (S if S_v is None else int(S_v))
        self.dtype = int(dtype)
        self.kda, self.C, self.scale = bool(kda), int(C), float(scale)
        self.seq_lens = None if seq_lens is None else [int(x) for x in seq_lens]
        if self.seq_lens is not None and len(self.seq_lens) != n_seqs:
            raise ValueError(f"seq_lens has {len(self.seq_lens)} entries for {n_seqs} sequences")
        self._lens = None
        self.strides = dict(strides or {})
        self._c = _Problem()
        self._fill()

    @classmethod
    def from_tensors(cls, q, k, v, g, beta, C=0, scale=None, seq_lens=None, gy=None, y=None):
        n, T, H_k, S = q.shape
        H_v, S_v = v.shape[2], v.shape[3]
        kda = g.dim() == 4 and g.shape[3] == S and S > 1
        strides = {"q": _tok_strides(q, "q"), "k": _tok_strides(k, "k"),
                   "v": _tok_strides(v, "v"), "g": _tok_strides(g, "g"),
                   "beta": _tok_strides(beta, "beta"), "gy": _tok_strides(gy, "gy"),
                   "y": _tok_strides(y, "y")}
        if scale is None:
            scale = S ** -0.5
        dts = {t.dtype for t in (q, k, v, g, beta, gy) if t is not None}
        if len(dts) != 1 or next(iter(dts)) not in _DTYPES:
            raise ValueError(f"q, k, v, g, beta, gy must share one of {list(_DTYPES)}: {dts}")
        return cls(n, T, H_k, H_v, S, kda, C, scale, seq_lens, strides,
                   _DTYPES[next(iter(dts))], S_v)

    def set_strides(self, **kw):
        for name, t in kw.items():
            self.strides[name] = _tok_strides(t, name) if isinstance(t, torch.Tensor) else tuple(t)
        self._fill()
        return self

    def _fill(self):
        c = self._c
        c.n_seqs, c.T, c.H_k, c.H_v = self.n_seqs, self.T, self.H_k, self.H_v
        c.S_k, c.S_v = self.S_k, self.S_v
        c.gate = GATE_KDA if self.kda else GATE_SCALAR
        c.C = self.C
        c.scale = self.scale
        c.dtype = self.dtype
        if self.seq_lens is not None:
            self._lens = (ctypes.c_int32 * max(1, len(self.seq_lens)))(*self.seq_lens)
            c.seq_lens = ctypes.cast(self._lens, ctypes.POINTER(ctypes.c_int32))
        else:
            self._lens = None
            c.seq_lens = None
        for name in ("q", "k", "v", "g", "beta", "gy", "y"):
            st = self.strides.get(name, (0, 0, 0))
            setattr(c, name, _Strides(*st))

    @property
    def c(self):
        return ctypes.byref(self._c)


def workspace_size(p: Problem) -> int:
    return int(lib.gdn_workspace_size(p.c))


def grad_layout(p: Problem):
    """(total floats, {region: (offset, shape)}) of the packed gradient buffer."""
    off = (ctypes.c_size_t * 6)()
    total = int(lib.gdn_grad_packed_floats(p.c, off))
    n, T, Hk, Hv, S, Sv = p.n_seqs, p.T, p.H_k, p.H_v, p.S_k, p.S_v
    G = S if p.kda else 1
    shapes = {"dq": (n, T, Hk, S), "dk": (n, T, Hk, S), "dv": (n, T, Hv, Sv),
              "dg": (n, T, Hv, G), "dbeta": (n, T, Hv), "dstate": (n, Hv, Sv, S)}
    return total, {name: (int(off[i]), shp) for i, (name, shp) in enumerate(shapes.items())}


def unpack_grads(p: Problem, grad_packed: torch.Tensor):
    _, lay = grad_layout(p)
    out = {}
    for name, (o, shp) in lay.items():
        cnt = 1
        for x in shp:
            cnt *= x
        out[name] = grad_packed[o:o + cnt].view(shp)
    return out


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_view(p: Problem, t, name):
    """t must have the (seq, tok, head) strides recorded in p for that tensor."""
    if t is not None and _tok_strides(t, name) != tuple(p.strides.get(name, (0, 0, 0))):
        raise ValueError(f"{name}: strides {tuple(t.stride())} differ from the problem's "
                         f"{p.strides.get(name)}")


def _check_state(p: Problem, t, name):
    """A state tensor must be contiguous [n_seqs][H_v][S_v][S_k]."""
    if t is None:
        return
    shape = (p.n_seqs, p.H_v, p.S_v, p.S_k)
    if tuple(t.shape) != shape or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {shape} tensor, got {tuple(t.shape)}")


def fwd(p: Problem, q, k, v, g, beta, state0, y, state_out, ws, stream=None):
    """gdn_fwd on device tensors (y must have the strides recorded in p for "y")."""
    _check_view(p, y, "y")
    _check_state(p, state0, "state0")
    _check_state(p, state_out, "state_out")
    rc = lib.gdn_fwd(p.c, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state0),
                     _ptr(y), _ptr(state_out), _ptr(ws), ws.numel() * ws.element_size(),
                     _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_fwd")


def bwd(p: Problem, q, k, v, g, beta, state0, gy, dstate_out, grad_packed, ws, flags=0,
        stream=None):
    """gdn_bwd on device tensors (gy must have the strides recorded in p for "gy")."""
    _check_view(p, gy, "gy")
    _check_state(p, state0, "state0")
    _check_state(p, dstate_out, "dstate_out")
    rc = lib.gdn_bwd(p.c, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state0),
                     _ptr(gy), _ptr(dstate_out), _ptr(grad_packed), _ptr(ws),
                     ws.numel() * ws.element_size(), int(flags), _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_bwd")


def bwd_noalloc(p: Problem, q, k, v, g, beta, state0, gy, dstate_out, grad_packed, stream=None):
    """gdn_bwd_noalloc: gdn_bwd on the library's own static workspace (no ws argument)."""
    _check_view(p, gy, "gy")
    _check_state(p, state0, "state0")
    _check_state(p, dstate_out, "dstate_out")
    rc = lib.gdn_bwd_noalloc(p.c, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state0),
                             _ptr(gy), _ptr(dstate_out), _ptr(grad_packed), _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_bwd_noalloc")


def conv_problem(n_seqs, T, d_inner, d_conv, sx_strides, y_strides) -> _ConvProblem:
    """A gdn_conv_problem; strides are (seq, row) in floats (the channel stride is 1)."""
    return _ConvProblem(n_seqs, T, d_inner, d_conv, sx_strides[0], sx_strides[1],
                        y_strides[0], y_strides[1])


def _taps(c):
    if c.dim() != 2 or not c.is_contiguous():
        raise ValueError("c: expected a contiguous [d_inner, d_conv] tensor")
    return _ptr(c)


def _rows(t, name):
    if t.dim() == 3 and t.numel() == 0:
        return (t.shape[1] * t.shape[2], t.shape[2])   # no element is addressed
    if t.dim() != 3 or (t.shape[2] > 1 and t.stride(2) != 1):
        raise ValueError(f"{name}: expected [n_seqs, rows, d_inner] with unit channel stride")
    return (t.stride(0), t.stride(1))


def ssm_conv_fwd(sx, c, y, stream=None):
    """gdn_ssm_conv_fwd: y [n, T, D] from sx [n, d_conv - 1 + T, D] and taps c [D, d_conv]."""
    n, D, K = sx.shape[0], sx.shape[2], c.shape[1]
    p = conv_problem(n, y.shape[1], D, K, _rows(sx, "sx"), _rows(y, "y"))
    rc = lib.gdn_ssm_conv_fwd(ctypes.byref(p), _ptr(sx), _taps(c), _ptr(y), _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_ssm_conv_fwd")


def ssm_conv_bwd(dy, c, d_sx, stream=None):
    """gdn_ssm_conv_bwd: d_sx [n, d_conv - 1 + T, D] from dy [n, T, D] and taps c [D, d_conv]."""
    n, D, K = dy.shape[0], dy.shape[2], c.shape[1]
    p = conv_problem(n, dy.shape[1], D, K, _rows(d_sx, "d_sx"), _rows(dy, "dy"))
    rc = lib.gdn_ssm_conv_bwd(ctypes.byref(p), _ptr(dy), _taps(c), _ptr(d_sx), _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_ssm_conv_bwd")


def _head_rows(t, name):
    """(seq, tok, head) strides of a [n, T, H, W] tensor with unit innermost stride."""
    if t.dim() != 4:
        raise ValueError(f"{name}: expected [n_seqs, T, H, W], got {tuple(t.shape)}")
    if t.numel() == 0:
        return (0, 0, 0)
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError(f"{name}: innermost stride must be 1")
    return tuple(int(x) for x in t.stride()[:3])


def l2norm_problem(x, eps, dy=None, out=None) -> _L2Problem:
    n, T, H, W = (int(v) for v in x.shape)
    return _L2Problem(n, T, H, W, eps, _Strides(*_head_rows(x, "x")),
                      _Strides(*(_head_rows(dy, "dy") if dy is not None else (0, 0, 0))),
                      _Strides(*(_head_rows(out, "out") if out is not None else (0, 0, 0))))


def l2norm_fwd(x, y, eps=1e-6, stream=None):
    """gdn_l2norm_fwd: y = x / sqrt(sum x^2 + eps) per row of [n, T, H, W] views."""
    if tuple(y.shape) != tuple(x.shape):
        raise ValueError("y must have the shape of x")
    p = l2norm_problem(x, eps, out=y)
    rc = lib.gdn_l2norm_fwd(ctypes.byref(p), _ptr(x), _ptr(y), _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_l2norm_fwd")


def l2norm_bwd(x, dy, dx, eps=1e-6, stream=None):
    """gdn_l2norm_bwd: dx = dy / n - x (x . dy) / n^3 per row, n = sqrt(sum x^2 + eps)."""
    if tuple(dy.shape) != tuple(x.shape) or tuple(dx.shape) != tuple(x.shape):
        raise ValueError("dy and dx must have the shape of x")
    p = l2norm_problem(x, eps, dy=dy, out=dx)
    rc = lib.gdn_l2norm_bwd(ctypes.byref(p), _ptr(x), _ptr(dy), _ptr(dx), _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_l2norm_bwd")


def ssm_problem(n_seqs, T, H, P, N, G, a_per_state, dt_softplus=True) -> _SsmProblem:
    return _SsmProblem(n_seqs, T, H, P, N, G, int(a_per_state), int(dt_softplus))


def ssm_problem_from(x, B, A, dt_softplus=True) -> _SsmProblem:
    """The problem of contiguous x [n, T, H, P], B [n, T, G, N] and A ([H, N] or [H])."""
    n, T, H, P = (int(v) for v in x.shape)
    G, N = int(B.shape[2]), int(B.shape[3])
    return ssm_problem(n, T, H, P, N, G, A.dim() == 2, dt_softplus)


def ssm_workspace_size(p: _SsmProblem) -> int:
    return int(lib.gdn_ssm_workspace_size(ctypes.byref(p)))


def ssm_grad_layout(p: _SsmProblem):
    """(total floats, {name: (offset, shape)}) of [d_s | d_x | d_dt | d_B | d_C]."""
    off = (ctypes.c_size_t * 5)()
    total = lib.gdn_ssm_grad_packed_floats(ctypes.byref(p), off)
    n, T, H, P, N, G = p.n_seqs, p.T, p.H, p.P, p.N, p.G
    shapes = {"ds": (n, H, P, N), "dx": (n, T, H, P), "ddt": (n, T, H), "dB": (n, T, G, N),
              "dC": (n, T, G, N)}
    return int(total), {k: (int(off[i]), shp) for i, (k, shp) in enumerate(shapes.items())}


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("the scan takes contiguous tensors")


def ssm_fwd(p: _SsmProblem, s0, x, dt, A, B, C, y, s_out, ws, stream=None):
    _contig(s0, x, dt, A, B, C, y, s_out)
    rc = lib.gdn_ssm_fwd(ctypes.byref(p), _ptr(s0), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                         _ptr(y), _ptr(s_out), _ptr(ws), ws.numel() * ws.element_size(),
                         _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_ssm_fwd")


def ssm_bwd(p: _SsmProblem, s0, x, dt, A, B, C, gy, gs_final, grad_packed, ws, flags=0,
            stream=None):
    _contig(s0, x, dt, A, B, C, gy, gs_final, grad_packed)
    rc = lib.gdn_ssm_bwd(ctypes.byref(p), _ptr(s0), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                         _ptr(gy), _ptr(gs_final) if gs_final is not None else None,
                         _ptr(grad_packed), _ptr(ws), ws.numel() * ws.element_size(), flags,
                         _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_ssm_bwd")
