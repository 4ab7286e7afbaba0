"""MI355X-native forward pass of the resolvent operator head.

The computation runs in hand-written HIP kernels for gfx950 behind the C ABI
declared in ``include/resolvent.h`` (library ``libresolvent.so`` in this
package directory).  ``resolvent_forward`` and its helpers below are the thin
Python binding: argument marshalling only.
"""
__all__ = ["resolvent_forward", "resolvent_workspace_bytes", "resolvent_status_str"]


def __getattr__(name):
    if name in __all__ or name in ("forward", "Status", "ResolventError", "library_path"):
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
