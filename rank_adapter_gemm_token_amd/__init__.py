"""MI355X-native multi-LoRA adapter execution unit.

The compute path is liblora.so (hand-written HIP kernels for gfx950 behind a
C ABI, declared in include/lora.h); `rank_adapter_gemm_token_amd.lora` is its
thin ctypes binding.  Importing this package loads nothing: the binding loads
the library on first import and raises if it has not been built.
"""
import importlib

__all__ = ["lora", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
