"""Device placement of a workload: torch supplies the memory, the binding the calls.

``DeviceCase`` puts seeded inputs (``inputs.py``) on the GPU in the workload's layout
(contiguous, or q/k/v as row views of one packed buffer), allocates the outputs, the
packed gradient buffer and the workspace once, and runs the forward and backward through
the C ABI.  No arithmetic of the method happens here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B
from .inputs import Workload, pack_qkv


class DeviceCase:
    def __init__(self, w: Workload, arrays: dict, device="cuda", C=None, strided_gy=False,
                 packed=None, grad_offset=0, in_dtype=torch.float32):
        self.w = w
        n, T, Hk, Hv, S, Sv, G = w.n_seqs, w.T, w.H_k, w.H_v, w.S, w.S_v, w.G
        dev = torch.device(device)
        packed = w.packed if packed is None else packed

        def put(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        def put_in(a):   # q, k, v, g, beta, gy in the input element type (values must fit it)
            return put(a).to(in_dtype)

        if packed:
            self.qkv = put_in(pack_qkv(w, arrays["q"], arrays["k"], arrays["v"]))
            W = w.packed_width
            HkS = Hk * S
            self.q = self.qkv[:, :, :HkS].unflatten(2, (Hk, S))
            self.k = self.qkv[:, :, HkS:2 * HkS].unflatten(2, (Hk, S))
            self.v = self.qkv[:, :, 2 * HkS:].unflatten(2, (Hv, Sv))
            assert self.q.stride() == (T * W, W, S, 1)
        else:
            self.qkv = None
            self.q, self.k, self.v = put_in(arrays["q"]), put_in(arrays["k"]), put_in(arrays["v"])
        self.g = put_in(arrays["g"].reshape(n, T, Hv, G))
        self.beta = put_in(arrays["beta"])
        self.state0 = put(arrays["state0"])
        if strided_gy:
            # gy as a view with head-major order and a padded token stride
            base = torch.zeros((n, Hv, T, Sv + 8), dtype=in_dtype, device=dev)
            self.gy = base[..., :Sv].permute(0, 2, 1, 3)
            self.gy.copy_(put_in(arrays["gy"]))
        else:
            self.gy = put_in(arrays["gy"])
        self.dstate_out = put(arrays["dstate_out"]) if arrays.get("dstate_out") is not None else None
        self.y = torch.empty((n, T, Hv, Sv), dtype=torch.float32, device=dev)
        self.state_out = torch.empty((n, Hv, Sv, S), dtype=torch.float32, device=dev)
        self.p = B.Problem.from_tensors(self.q, self.k, self.v, self.g, self.beta,
                                        C=w.C if C is None else C, scale=w.scale,
                                        seq_lens=list(w.lens), gy=self.gy, y=self.y)
        self.ws = torch.empty(max(B.workspace_size(self.p), 256), dtype=torch.uint8, device=dev)
        total, _ = B.grad_layout(self.p)
        # grad_offset floats in: a packed gradient buffer that is only 4-byte aligned
        self.grad_all = torch.empty(max(total, 1) + grad_offset, dtype=torch.float32, device=dev)
        self.grad = self.grad_all[grad_offset:]

    def fwd(self, stream=None):
        B.fwd(self.p, self.q, self.k, self.v, self.g, self.beta, self.state0, self.y,
              self.state_out, self.ws, stream)

    def bwd(self, reuse=True, stream=None):
        B.bwd(self.p, self.q, self.k, self.v, self.g, self.beta, self.state0, self.gy,
              self.dstate_out, self.grad, self.ws,
              B.BWD_REUSE_SNAPSHOTS if reuse else 0, stream)

    def grads(self):
        return B.unpack_grads(self.p, self.grad)

    def results_numpy(self):
        """Everything the two calls produced, as float32 numpy arrays."""
        out = {"y": self.y, "state_out": self.state_out}
        out.update(self.grads())
        return {k: v.detach().cpu().numpy() for k, v in out.items()}
