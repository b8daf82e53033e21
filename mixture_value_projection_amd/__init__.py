"""MoVA routed value projection on MI355X (gfx950).

The compute path is the C-ABI library ``libmova.so`` built from ``csrc/``
(hand-written HIP); ``binding`` marshals torch tensors into it.  Importing this
package does not load the library; the first call into ``binding`` does, and
raises if it is missing.
"""
from . import accounting, inputs  # noqa: F401

__all__ = ["accounting", "inputs", "route", "value_forward", "workspace_bytes",
           "status_str", "load_library"]


def __getattr__(name):
    if name in ("route", "value_forward", "workspace_bytes", "status_str", "load_library",
                "MovaError"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
