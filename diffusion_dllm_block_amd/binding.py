"""ctypes binding of libdllm (include/dllm.h, include/dllm_synth.h).

Argument marshalling only: every step of the decode path runs in the library's HIP
kernels.  torch is used here only to allocate device memory and to name the stream.
If the shared library is missing the import of a function fails loudly; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libdllm.so")
HEADERS = [os.path.join(ROOT, "include", "dllm.h"), os.path.join(ROOT, "include", "dllm_synth.h")]

F32, BF16 = 0, 1
CACHE_NONE, CACHE_PREFIX, CACHE_DUAL = 0, 1, 2

STATUS = {0: "DLLM_OK", -1: "DLLM_E_NULL", -2: "DLLM_E_SHAPE", -3: "DLLM_E_UNSUPPORTED",
          -4: "DLLM_E_WORKSPACE", -5: "DLLM_E_HIP", -6: "DLLM_E_STATE", -7: "DLLM_E_ARG"}

KERNEL_CLASSES = ["EMBED_NORM", "RMSNORM", "STEP_QKV", "STEP_ATTN", "STEP_O", "STEP_GATE_UP",
                  "STEP_DOWN", "LM_HEAD", "CONF_UNMASK", "REF_QKV", "REF_ATTN", "REF_O",
                  "REF_GATE_UP", "REF_DOWN", "SPLIT_REDUCE"]


class ModelDesc(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("d_ffn", C.c_int32),
                ("vocab", C.c_int32), ("mask_id", C.c_int32),
                ("rope_theta", C.c_float), ("norm_eps", C.c_float), ("logit_scale", C.c_float),
                ("dtype", C.c_int32),
                ("embed", C.c_void_p), ("final_norm", C.c_void_p), ("lm_head", C.c_void_p),
                ("attn_norm", C.POINTER(C.c_void_p)), ("w_qkv", C.POINTER(C.c_void_p)),
                ("w_o", C.POINTER(C.c_void_p)), ("ffn_norm", C.POINTER(C.c_void_p)),
                ("w_gate_up", C.POINTER(C.c_void_p)), ("w_down", C.POINTER(C.c_void_p))]


class SeqDesc(C.Structure):
    _fields_ = [("batch", C.c_int32), ("prompt_len", C.c_int32), ("gen_len", C.c_int32),
                ("block_len", C.c_int32), ("cache_mode", C.c_int32), ("threshold", C.c_float),
                ("tokens", C.c_void_p), ("kv_cache", C.c_void_p), ("kv_cache_bytes", C.c_size_t),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t)]


class Stats(C.Structure):
    _fields_ = [("steps", C.c_int32), ("refreshes", C.c_int32), ("tokens", C.c_int32),
                ("blocks", C.c_int32), ("ms_total", C.c_double), ("ms_refresh", C.c_double),
                ("ms_step", C.c_double), ("steps_per_block", C.POINTER(C.c_int32)),
                ("speculative_steps", C.c_int32), ("masked_at_step_start", C.c_int64)]


class DllmError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")
        self.status = status


_P = C.c_void_p
_I = C.c_int32
_SIGS = {
    "dllm_workspace_bytes": (C.c_size_t, [C.POINTER(ModelDesc), C.POINTER(SeqDesc)]),
    "dllm_kv_cache_bytes": (C.c_size_t, [C.POINTER(ModelDesc), C.POINTER(SeqDesc)]),
    "dllm_prefill_cache": (_I, [C.POINTER(ModelDesc), C.POINTER(SeqDesc), _P]),
    "dllm_refresh_cache": (_I, [C.POINTER(ModelDesc), C.POINTER(SeqDesc), _I, _P]),
    "dllm_cache_staleness": (_I, [C.POINTER(ModelDesc), C.POINTER(SeqDesc), _I, _P, C.c_size_t,
                                  _P, C.POINTER(C.c_double), _P]),
    "dllm_block_step": (_I, [C.POINTER(ModelDesc), C.POINTER(SeqDesc), _I, _P, _P, _P, _P, _P, _P]),
    "dllm_refresh_step": (_I, [C.POINTER(ModelDesc), C.POINTER(SeqDesc), _I, _P, _P, _P, _P, _P,
                               _P]),
    "dllm_generate": (_I, [C.POINTER(ModelDesc), C.POINTER(SeqDesc), _P, C.POINTER(Stats)]),
    "dllm_generate_graphs": (_I, [C.POINTER(ModelDesc), C.POINTER(SeqDesc), _P, C.POINTER(Stats)]),
    "dllm_kernel_workspace_bytes": (C.c_size_t, [_I] * 7),
    "dllm_kernel_block_attention": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P,
                                         C.c_size_t, _P]),
    "dllm_kernel_confidence_unmask": (_I, [_P, _I, _I, _I, _I, _I, C.c_float, _P, _I, _P, _P, _P,
                                           _P, _P, _P, C.c_size_t, _P]),
    "dllm_kernel_confidence_unmask_noalloc": (_I, [_P, _I, _I, _I, _I, _I, C.c_float, _P, _I, _P,
                                                   _P, _P, _P, _P, _P]),
    "dllm_linear_workspace_bytes": (C.c_size_t, [_I, _I, _I, _I]),
    "dllm_kernel_linear": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, C.c_float, _P, C.c_size_t, _P]),
    "dllm_status_string": (C.c_char_p, [_I]),
    "dllm_last_error": (C.c_char_p, []),
    "dllm_profile_select": (_I, [_I]),
    "dllm_profile_select_every": (_I, [_I, _I]),
    "dllm_profile_read": (_I, [C.POINTER(C.c_int32), C.POINTER(C.c_double)]),
    "dllm_synth_fill": (_I, [_P, C.c_int64, _I, C.c_uint64, C.c_uint32, C.c_double, _I, _P]),
}


def declared_functions() -> list[str]:
    """Names of every function the public headers declare."""
    names = []
    for h in HEADERS:
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"\b(dllm_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


class Lib:
    """The loaded library; functions raise DllmError on a non-zero status."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"{path} is missing: build it with `python -m diffusion_dllm_block_amd.build`")
        self.path = path
        self.cdll = C.CDLL(path)
        for name, (res, args) in _SIGS.items():
            f = getattr(self.cdll, name)
            f.restype = res
            f.argtypes = args

    def raw(self, name):
        return getattr(self.cdll, name)

    def check(self, status: int, where: str):
        if status != 0:
            raise DllmError(status, where, self.cdll.dllm_last_error().decode())

    def call(self, name: str, *args):
        st = getattr(self.cdll, name)(*args)
        self.check(st, name)
        return st


_LIB: Lib | None = None


def load(path: str = LIB_PATH) -> Lib:
    global _LIB
    if _LIB is None or _LIB.path != path:
        _LIB = Lib(path)
    return _LIB


def stream_handle(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def ptr(t) -> C.c_void_p:
    return C.c_void_p(t.data_ptr() if t is not None else 0)
