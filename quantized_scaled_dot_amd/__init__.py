"""MI355X-native quantized attention forward (INT8 QK^T, FP8 P~V).

The compute path is the C-ABI library ``libsage.so`` built from ``csrc/``
(hand-written HIP kernels for gfx950); ``sage`` is its thin Python binding.
``synth`` draws the seeded synthetic inputs.
"""
import importlib

__all__ = ["sage", "synth"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(__name__ + "." + name)
    raise AttributeError(name)
