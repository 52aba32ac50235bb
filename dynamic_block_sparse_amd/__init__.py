"""MI355X (gfx950) Prism dynamic block-sparse attention.

    dynamic_block_sparse_amd.prism   ctypes binding of libprism.so (the C ABI)
    dynamic_block_sparse_amd.path    the hot path end to end on torch device tensors
    dynamic_block_sparse_amd.build   hipcc build of libprism.so

The binding is imported on first use so that the build step can run before
the library exists; using it without the library raises ImportError.
"""
import importlib

__all__ = ["prism", "path", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
