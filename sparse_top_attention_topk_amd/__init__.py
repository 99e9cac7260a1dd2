"""libsmla: sparse top-k MLA attention (DeepSeek sparse attention) on MI355X.

The compute path is the HIP library ``libsmla.so`` (C ABI in include/smla.h);
``_lib`` is its thin ctypes binding.  ``workloads`` draws seeded synthetic
inputs.  Importing the binding requires the built library.
"""
__all__ = ["smla_fwd", "smla_bwd_preprocess", "smla_bwd_delta_exact", "smla_bwd_workspace_size",
           "smla_bwd", "smla_bwd_from_o"]


def __getattr__(name):
    if name in __all__:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
