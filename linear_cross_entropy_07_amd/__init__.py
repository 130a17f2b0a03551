"""MI355X-native fused linear + cross-entropy (FLCE), forward and backward, in hand-written HIP.

`linear_cross_entropy_07_amd.flce` holds the Python binding of the C-ABI library
(libflce.so, built from `csrc/`); it is imported lazily so that `inputs` can be
used without loading the GPU library.
"""

__all__ = ["flce", "inputs"]


def __getattr__(name):
    if name in ("flce", "inputs"):
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    if name in ("flce_loss", "FLCE", "FlceError"):
        from . import flce

        return getattr(flce, name)
    raise AttributeError(name)
