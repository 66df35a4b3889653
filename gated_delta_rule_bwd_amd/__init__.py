"""Gated delta rule forward and checkpointed backward for MI355X (gfx950).

The compute path is the HIP library ``libgdn.so`` behind the C ABI in ``include/gdn.h``;
``binding`` marshals arguments to it through ctypes.  Importing this package does not load
the library; the first use of ``fwd``, ``bwd``, ``workspace_size`` or ``Problem`` does, and
raises if the library has not been built (there is no fallback path).
"""

_BINDING_NAMES = ("Problem", "workspace_size", "grad_layout", "unpack_grads", "fwd", "bwd",
                  "lib", "GdnError", "STATUS", "EXPORTS", "BWD_REUSE_SNAPSHOTS")


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
