"""MI355X (gfx950) implementation of the Fast-dLLM block-cache decode step.

libdllm.so (HIP kernels + C ABI, include/dllm.h) does the work; ``binding`` is its
ctypes binding and ``engine`` owns device buffers through torch.
"""
from . import binding  # noqa: F401

__all__ = ["binding", "engine"]
