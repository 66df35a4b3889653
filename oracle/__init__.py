"""Plain fp64 CPU oracle of the gated delta rule (forward and backward).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP product path
never imports it and shares no code with it.

The arithmetic lives in ``gdn_oracle.c`` (plain loops in double precision, written from
the pages' statement of the method: "metal: GATED_DELTA_NET_BACK" description and
reviews, and meTile's "Recurrent delta attention" section).  This module only compiles
that file with gcc and marshals numpy arrays through ctypes.

Arrays are taken in the logical contiguous layouts described in ``gdn_oracle.c``;
any float dtype is accepted and converted to float64 (fp32 inputs are read back exactly).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_NAME = "libgdn_oracle.so"
_lock = threading.Lock()
_libs: dict[int, ctypes.CDLL] = {}


class _Problem(ctypes.Structure):
    _fields_ = [
        ("n_seqs", ctypes.c_int), ("T", ctypes.c_int), ("H_k", ctypes.c_int),
        ("H_v", ctypes.c_int), ("S_k", ctypes.c_int), ("S_v", ctypes.c_int),
        ("kda", ctypes.c_int), ("C", ctypes.c_int),
        ("scale", ctypes.c_double),
        ("seq_lens", ctypes.POINTER(ctypes.c_int)),
    ]


_DP = ctypes.POINTER(ctypes.c_double)


class _IO(ctypes.Structure):
    _fields_ = [(n, _DP) for n in (
        "q", "k", "v", "g", "beta", "state0", "gy", "dstate_out",
        "y", "state_out", "dq", "dk", "dv", "dg", "dbeta", "dstate")]


def lib_path(mutation: int = 0, out_dir: str | None = None) -> str:
    if mutation == 0 and out_dir is None:
        return os.path.join(_HERE, _LIB_NAME)
    d = out_dir or os.path.join(_HERE, "_mutants")
    return os.path.join(d, f"libgdn_oracle_m{mutation}.so")


def build(mutation: int = 0, out_dir: str | None = None) -> str:
    """Compile the oracle (optionally with planted mutation ``mutation``) with gcc."""
    out = lib_path(mutation, out_dir)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-pthread", f"-DGDN_ORACLE_MUTATION={int(mutation)}", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load(mutation: int = 0, out_dir: str | None = None) -> ctypes.CDLL:
    """Load (building first if absent or stale) the oracle library."""
    with _lock:
        key = (mutation, out_dir)
        if key in _libs:
            return _libs[key]
        path = lib_path(mutation, out_dir)
        if (not os.path.exists(path)
                or os.path.getmtime(path) < os.path.getmtime(_SRC)):
            build(mutation, out_dir)
        lib = ctypes.CDLL(path)
        lib.gdn_oracle_fwd.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_IO), ctypes.c_int]
        lib.gdn_oracle_fwd.restype = ctypes.c_int
        lib.gdn_oracle_bwd.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_IO), ctypes.c_int]
        lib.gdn_oracle_bwd.restype = ctypes.c_int
        lib.gdn_oracle_default_C.argtypes = [ctypes.c_int]
        lib.gdn_oracle_default_C.restype = ctypes.c_int
        lib.gdn_oracle_mutation.restype = ctypes.c_int
        _libs[key] = lib
        return lib


def default_C(T: int) -> int:
    """ceil(sqrt(T)): the checkpoint interval the pages use when none is given."""
    return int(load().gdn_oracle_default_C(int(T)))


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(_DP) if a is not None else None


class Oracle:
    """Callable front end.  ``mutation`` selects a planted-mistake build (tests only)."""

    def __init__(self, mutation: int = 0, out_dir: str | None = None, threads: int | None = None):
        self.lib = load(mutation, out_dir)
        self.threads = threads or min(os.cpu_count() or 1, 16)

    @staticmethod
    def _problem(shape: dict):
        lens = shape.get("seq_lens")
        p = _Problem()
        p.n_seqs = shape["n_seqs"]
        p.T = shape["T"]
        p.H_k = shape["H_k"]
        p.H_v = shape["H_v"]
        p.S_k = shape["S_k"]
        p.S_v = shape["S_v"]
        p.kda = 1 if shape["kda"] else 0
        p.C = int(shape.get("C") or 0)
        p.scale = float(shape["scale"])
        keep = None
        if lens is not None:
            keep = (ctypes.c_int * len(lens))(*[int(x) for x in lens])
            p.seq_lens = ctypes.cast(keep, ctypes.POINTER(ctypes.c_int))
        return p, keep

    @staticmethod
    def _check(shape, q, k, v, g, beta, state0):
        n, T, Hk, Hv = shape["n_seqs"], shape["T"], shape["H_k"], shape["H_v"]
        Sk, Sv = shape["S_k"], shape["S_v"]
        G = Sk if shape["kda"] else 1
        assert q.shape == (n, T, Hk, Sk), q.shape
        assert k.shape == (n, T, Hk, Sk), k.shape
        assert v.shape == (n, T, Hv, Sv), v.shape
        assert g.shape == (n, T, Hv, G), g.shape
        assert beta.shape == (n, T, Hv), beta.shape
        assert state0.shape == (n, Hv, Sv, Sk), state0.shape

    def fwd(self, shape: dict, q, k, v, g, beta, state0):
        """Returns (y [n,T,H_v,S_v], state_out [n,H_v,S_v,S_k]) in float64."""
        q, k, v, g, beta, state0 = map(_f64, (q, k, v, g, beta, state0))
        g = g.reshape(g.shape[:3] + (-1,))
        self._check(shape, q, k, v, g, beta, state0)
        n, T, Hv, Sv, Sk = shape["n_seqs"], shape["T"], shape["H_v"], shape["S_v"], shape["S_k"]
        y = np.zeros((n, T, Hv, Sv))
        so = np.zeros((n, Hv, Sv, Sk))
        io = _IO()
        for name, arr in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta),
                          ("state0", state0), ("y", y), ("state_out", so)):
            setattr(io, name, _ptr(arr))
        p, keep = self._problem(shape)
        rc = self.lib.gdn_oracle_fwd(ctypes.byref(p), ctypes.byref(io), self.threads)
        del keep
        if rc != 0:
            raise RuntimeError(f"oracle forward failed ({rc})")
        return y, so

    def bwd(self, shape: dict, q, k, v, g, beta, state0, gy, dstate_out=None):
        """Returns dict dq, dk, dv, dg, dbeta, dstate (float64, logical layouts)."""
        q, k, v, g, beta, state0, gy, dso = map(_f64, (q, k, v, g, beta, state0, gy, dstate_out))
        g = g.reshape(g.shape[:3] + (-1,))
        self._check(shape, q, k, v, g, beta, state0)
        n, T, Hk, Hv = shape["n_seqs"], shape["T"], shape["H_k"], shape["H_v"]
        Sk, Sv = shape["S_k"], shape["S_v"]
        assert gy.shape == (n, T, Hv, Sv)
        if dso is not None:
            assert dso.shape == (n, Hv, Sv, Sk)
        out = dict(
            dq=np.zeros((n, T, Hk, Sk)), dk=np.zeros((n, T, Hk, Sk)),
            dv=np.zeros((n, T, Hv, Sv)), dg=np.zeros(g.shape),
            dbeta=np.zeros((n, T, Hv)), dstate=np.zeros((n, Hv, Sv, Sk)))
        io = _IO()
        for name, arr in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta),
                          ("state0", state0), ("gy", gy), ("dstate_out", dso)):
            setattr(io, name, _ptr(arr))
        for name, arr in out.items():
            setattr(io, name, _ptr(arr))
        p, keep = self._problem(shape)
        rc = self.lib.gdn_oracle_bwd(ctypes.byref(p), ctypes.byref(io), self.threads)
        del keep
        if rc != 0:
            raise RuntimeError(f"oracle backward failed ({rc})")
        return out


def workspace_formula_bytes(S_v: int, T: int, C: int | None = None) -> int:
    """The pages' per-(head, seq) scratch of the Metal backward: (n_ck + C + 3) S_v^2 4 bytes,
    with C = ceil(sqrt(T)) and n_ck = ceil(T / C) ("metal: GATED_DELTA_NET_BACK", approval
    review's sizing note).  Used only to pin the checkpoint-interval reading."""
    if C is None:
        C = math.isqrt(T - 1) + 1 if T > 0 else 1
    n_ck = -(-T // C)
    return (n_ck + C + 3) * S_v * S_v * 4
