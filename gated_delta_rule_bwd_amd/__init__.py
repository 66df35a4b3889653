"""Gated delta rule forward and checkpointed backward for MI355X (gfx950).

The compute path is the HIP library ``libgdn.so`` behind the C ABI in ``include/gdn.h``
(the recurrence, the short convolution and L2 normalisation around it, and the selective
state-space scan);
``binding`` marshals arguments to it through ctypes.  Importing this package does not load
the library; the first use of ``fwd``, ``bwd``, ``workspace_size`` or ``Problem`` does, and
raises if the library has not been built (there is no fallback path).
"""

_BINDING_NAMES = ("Problem", "workspace_size", "grad_layout", "unpack_grads", "fwd", "bwd", "bwd_noalloc",
                  "lib", "GdnError", "STATUS", "EXPORTS", "BWD_REUSE_SNAPSHOTS",
                  # the short convolution and the q/k normalisation around the recurrence
                  "ssm_conv_fwd", "ssm_conv_bwd", "l2norm_fwd", "l2norm_bwd",
                  # the selective scan
                  "ssm_problem", "ssm_problem_from", "ssm_workspace_size", "ssm_grad_layout",
                  "ssm_fwd", "ssm_bwd")


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
