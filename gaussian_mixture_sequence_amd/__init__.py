"""MI355X-native Gaussian Mixture Attention (GMA) forward.

The compute path is ``libgma.so`` (HIP kernels for gfx950 behind a C ABI declared in
``include/gma.h``); ``gaussian_mixture_sequence_amd.binding`` marshals torch tensors
into that ABI.  The binding is imported lazily so that the seeded input generator
(``gaussian_mixture_sequence_amd.inputs``) can be used without loading the library.
"""
import importlib

__all__ = ["binding", "inputs"]


def __getattr__(name):
    if name in ("binding", "inputs"):
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
