"""MI355X-native block-causal linear-attention scan (liblinscan).

The library itself is the C-ABI shared object built from ``csrc/`` (HIP
kernels for gfx950 plus the host entry points declared in
``include/linscan.h``).  ``binding`` is a thin ctypes layer with the same entry
point names that marshals torch device tensors and the current stream; every
step of the scan runs in the HIP kernels.  ``inputs`` draws the seeded
synthetic workloads.

Submodules load lazily so that importing the package (for example to draw
inputs on a machine without a GPU) never touches the HIP runtime.
"""
import importlib

__all__ = ["binding", "inputs", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module("." + name, __name__)
    if name in ("ls_relu_block_forward", "ls_gdn_frame_forward", "ls_state_carry",
                "relu_block_forward", "gdn_frame_forward", "state_carry", "LinscanError"):
        return getattr(importlib.import_module(".binding", __name__), name)
    raise AttributeError(name)
