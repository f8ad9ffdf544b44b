"""MI355X-native sequence-parallel tensor-parallel linear layer (one GPU's share).

The compute path lives in the HIP library ``libsptl.so`` (C ABI declared in
``include/sptl.h``); ``sp_transformer_linear_amd.sptl`` is its thin Python binding.  The
binding is imported lazily so that ``sp_transformer_linear_amd.synth`` (seeded inputs) can
be used without the library; any call into the layer raises if the library is missing.
"""
import importlib

__all__ = ["sptl", "synth"]


def __getattr__(name):
    if name in ("sptl", "synth"):
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
