"""MI355X-native packed varlen attention for vision encoder towers.

The compute path is ``libvit.so`` (hand-written HIP kernels for gfx950 behind a
C ABI, declared in ``include/vit.h``); ``ops`` wraps it for PyTorch tensors.
Importing this package does not load the library; the first op call does, and
fails loudly if it has not been built.
"""
from . import workloads  # noqa: F401  (pure NumPy, no device code)

__all__ = ["workloads", "ops"]


def __getattr__(name):
    if name == "ops":
        import importlib
        return importlib.import_module(".ops", __name__)
    raise AttributeError(name)
