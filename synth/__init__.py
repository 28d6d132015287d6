"""Seeded synthetic inputs shared by the CPU oracle and the GPU tests/bench.

This module holds none of the method's arithmetic: it only turns (seed, tensor id,
element index) into numbers.  Everything is counter based so that any element of
any tensor can be produced on its own, in any order, on the host or on the device.

Generator
---------
SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014; the reference C code is Vigna's ``splitmix64.c``).
A SplitMix64 stream with state ``x0`` returns, as its i-th output (0-based),
``mix(x0 + (i + 1) * GAMMA)`` where ``GAMMA = 0x9e3779b97f4a7c15`` and ``mix`` is the
published 64-bit finaliser (xor-shift 30, multiply, xor-shift 27, multiply,
xor-shift 31).  All arithmetic wraps modulo 2**64.

Stream per tensor: ``x0 = mix(((seed XOR (tensor_id << 32)) + GAMMA) mod 2**64)``,
i.e. the first output of a SplitMix64 stream seeded with ``seed ^ (tensor_id << 32)``.

Normal deviates (Irwin-Hall, n = 4): the 64-bit output is cut into four 16-bit
fields u0..u3 (low to high).  ``z = (u0+u1+u2+u3 - 131070) * (sqrt(3)/65536)`` in
IEEE double has mean 0 and variance 1 (each 16-bit field has variance
(65536**2 - 1)/12).  The value is ``fp32(z * std)``: two double multiplies, each
rounded to nearest even, then one rounding to fp32; bf16 tensors round that fp32
value once more to bf16 (nearest even).  The device fill kernel in the library
implements exactly the same definition, so both sides get bit-identical values.

Uniform tokens: ``t = ((r >> 32) * n) >> 32`` for r the 64-bit output (multiply-shift
range reduction), uniform on [0, n).
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
SQRT3_OVER_65536 = math.sqrt(3.0) / 65536.0  # exact division by a power of two

_U64 = 0xFFFFFFFFFFFFFFFF


def _mix_np(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser on a uint64 array (wrapping arithmetic)."""
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def _mix_int(z: int) -> int:
    z &= _U64
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & _U64
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & _U64
    z ^= z >> 31
    return z


def stream_state(seed: int, tensor_id: int) -> int:
    """x0 of the SplitMix64 stream of one tensor (a Python int in [0, 2**64))."""
    s = (int(seed) ^ ((int(tensor_id) & 0xFFFFFFFF) << 32)) & _U64
    return _mix_int((s + 0x9E3779B97F4A7C15) & _U64)


def raw64(seed: int, tensor_id: int, idx: np.ndarray) -> np.ndarray:
    """64-bit outputs number ``idx`` (uint64 array) of the tensor's stream."""
    x0 = np.uint64(stream_state(seed, tensor_id))
    i = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = x0 + (i + np.uint64(1)) * GAMMA
        return _mix_np(z)


def _irwin_hall(r: np.ndarray) -> np.ndarray:
    """Sum of the four 16-bit fields minus the mean, as float64 (exact integers)."""
    m = np.uint64(0xFFFF)
    s = (r & m) + ((r >> np.uint64(16)) & m) + ((r >> np.uint64(32)) & m) + (r >> np.uint64(48))
    return s.astype(np.int64).astype(np.float64) - 131070.0


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def bf16_bits_to_fp32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_fp32(seed: int, tensor_id: int, idx: np.ndarray, std: float = 1.0) -> np.ndarray:
    """fp32 normal deviates for element indices ``idx`` of one tensor."""
    z = _irwin_hall(raw64(seed, tensor_id, idx)) * SQRT3_OVER_65536
    return (z * float(std)).astype(np.float32)


def normal_tensor(seed: int, tensor_id: int, shape, std: float = 1.0,
                  dtype: str = "f32", chunk: int = 1 << 22, threads: int | None = None) -> np.ndarray:
    """Whole tensor in row-major element order.

    dtype "f32" returns float32 values; "bf16" returns the uint16 bit patterns of
    the bf16 values (use :func:`bf16_bits_to_fp32` to read them).  Large tensors are
    produced by several threads (numpy releases the GIL); the values do not depend on
    the thread count.
    """
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)

    def part(a):
        b = min(n, a + chunk)
        v = normal_fp32(seed, tensor_id, np.arange(a, b, dtype=np.uint64), std)
        out[a:b] = v if dtype == "f32" else fp32_to_bf16_bits(v)

    starts = range(0, n, chunk)
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if n <= chunk or threads <= 1:
        for a in starts:
            part(a)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(part, starts))
    return out.reshape(shape)


def uniform_ints(seed: int, tensor_id: int, n: int, hi: int) -> np.ndarray:
    """n integers uniform on [0, hi), int64."""
    r = raw64(seed, tensor_id, np.arange(n, dtype=np.uint64))
    return (((r >> np.uint64(32)) * np.uint64(hi)) >> np.uint64(32)).astype(np.int64)


def uniform_unit(seed: int, tensor_id: int, n: int) -> np.ndarray:
    """n float64 values uniform on [0, 1) (top 53 bits of each output)."""
    r = raw64(seed, tensor_id, np.arange(n, dtype=np.uint64))
    return (r >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


# ---------------------------------------------------------------------------------
# Model and workload descriptions
# ---------------------------------------------------------------------------------

@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    rope_theta: float = 10000.0
    norm_eps: float = 1e-5
    logit_scale: float = 1.0
    dtype: str = "bf16"          # "f32" or "bf16": storage type of weights and cache

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    @property
    def qkv_rows(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape
    batch: int
    prompt_len: int
    gen_len: int
    block_len: int
    cache_mode: str               # "dual", "prefix" or "none" (no cache)
    threshold: float = 0.9
    model_seed: int = 1234
    prompt_seed: int = 5678
    norm_gain_std: float = 0.0    # 0: all norm gains exactly 1

    @property
    def seq_len(self) -> int:
        return self.prompt_len + self.gen_len


# Tensor ids of the model weights in the generator.
TID_EMBED = 0xE000
TID_FINAL_NORM = 0xE001
TID_LM_HEAD = 0xE002
TID_PROMPT = 0xF000
KIND_ATTN_NORM, KIND_QKV, KIND_O, KIND_FFN_NORM, KIND_GATE_UP, KIND_DOWN = range(6)


def layer_tid(layer: int, kind: int) -> int:
    return 16 * layer + kind


def weight_specs(m: ModelShape, norm_gain_std: float = 0.0):
    """List of (name, layer, tensor_id, shape, std, is_norm) for every weight.

    Projections are N(0, 1/fan_in); the embedding is N(0, 1); norm gains are 1, or
    1 + N(0, norm_gain_std) when norm_gain_std > 0 (used by tests only).
    """
    d, D = m.d_model, m.head_dim
    specs = [("embed", -1, TID_EMBED, (m.vocab, d), 1.0, False)]
    for l in range(m.n_layers):
        specs += [
            ("attn_norm", l, layer_tid(l, KIND_ATTN_NORM), (d,), norm_gain_std, True),
            ("w_qkv", l, layer_tid(l, KIND_QKV), (m.qkv_rows, d), 1.0 / math.sqrt(d), False),
            ("w_o", l, layer_tid(l, KIND_O), (d, m.n_heads * D), 1.0 / math.sqrt(m.n_heads * D), False),
            ("ffn_norm", l, layer_tid(l, KIND_FFN_NORM), (d,), norm_gain_std, True),
            ("w_gate_up", l, layer_tid(l, KIND_GATE_UP), (2 * m.d_ffn, d), 1.0 / math.sqrt(d), False),
            ("w_down", l, layer_tid(l, KIND_DOWN), (d, m.d_ffn), 1.0 / math.sqrt(m.d_ffn), False),
        ]
    specs += [("final_norm", -1, TID_FINAL_NORM, (d,), norm_gain_std, True),
              ("lm_head", -1, TID_LM_HEAD, (m.vocab, d), 1.0 / math.sqrt(d), False)]
    return specs


def norm_gain(seed: int, tensor_id: int, n: int, std: float, dtype: str) -> np.ndarray:
    """Norm gains: exactly 1 when std == 0, else fp32(1 + z*std) (rounded to bf16 if asked)."""
    if std == 0.0:
        g = np.ones(n, dtype=np.float32)
    else:
        z = _irwin_hall(raw64(seed, tensor_id, np.arange(n, dtype=np.uint64))) * SQRT3_OVER_65536
        g = (1.0 + z * std).astype(np.float32)
    return g if dtype == "f32" else fp32_to_bf16_bits(g)


def make_weight(wl: Workload, spec) -> np.ndarray:
    """One weight tensor: float32 values (f32 models) or uint16 bf16 bits (bf16 models)."""
    name, layer, tid, shape, std, is_norm = spec
    if is_norm:
        return norm_gain(wl.model_seed, tid, shape[0], std, wl.model.dtype)
    return normal_tensor(wl.model_seed, tid, shape, std, wl.model.dtype)


def make_weights(wl: Workload) -> dict:
    """All weights: dict name -> array (layer tensors under 'name.l')."""
    out = {}
    for spec in weight_specs(wl.model, wl.norm_gain_std):
        name, layer = spec[0], spec[1]
        out[name if layer < 0 else f"{name}.{layer}"] = make_weight(wl, spec)
    return out


def as_float(a: np.ndarray, dtype: str) -> np.ndarray:
    """Values of a generated array as float32 (bf16 bit patterns are decoded)."""
    return bf16_bits_to_fp32(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32)


def make_prompt(wl: Workload) -> np.ndarray:
    """int64 [B, P]: sequence i uses seed prompt_seed + i, tokens uniform on [0, V-1)."""
    V = wl.model.vocab
    rows = [uniform_ints(wl.prompt_seed + i, TID_PROMPT, wl.prompt_len, V - 1) for i in range(wl.batch)]
    return np.stack(rows) if rows else np.zeros((0, wl.prompt_len), np.int64)


# ---------------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------------

# Named workloads, one JSON file each in synth/workloads/ (shapes, batch, lengths, block,
# cache mode, threshold, seeds).  The logit scales of the random-init 8B/7B shapes are not
# in them: they are calibrated by the oracle (tests/golden/make_logit_scales.py) so that
# about 30 % of the masked positions of the first step reach confidence 0.9.
WORKLOAD_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workloads")


def workload_from_dict(d: dict) -> Workload:
    """A Workload from its JSON form (the keys of Workload, with "model" the keys of
    ModelShape); unknown keys are rejected so that a typo cannot pass silently."""
    d = dict(d)
    d.pop("description", None)
    m = dict(d.pop("model"))
    mk = set(ModelShape.__dataclass_fields__)
    wk = set(Workload.__dataclass_fields__) - {"model"}
    if set(m) - mk or set(d) - wk:
        raise ValueError(f"unknown workload keys: {sorted((set(m) - mk) | (set(d) - wk))}")
    return Workload(model=ModelShape(**m), **d)


def load_workload(path: str) -> Workload:
    import json
    with open(path) as f:
        return workload_from_dict(json.load(f))


def _load_named() -> dict:
    out = {}
    for fn in sorted(os.listdir(WORKLOAD_DIR)):
        if fn.endswith(".json"):
            wl = load_workload(os.path.join(WORKLOAD_DIR, fn))
            out[wl.name] = wl
    return out


WORKLOADS = _load_named()


def with_scale(wl: Workload, scale: float) -> Workload:
    from dataclasses import replace
    return replace(wl, model=replace(wl.model, logit_scale=float(scale)))


# ---------------------------------------------------------------------------------
# Kernel-only inputs (32 heads x 128, 32 block queries vs 1024 cached keys; and
# [32, 126464] block logits)
# ---------------------------------------------------------------------------------

TID_Q, TID_K, TID_V = 0xA000, 0xA001, 0xA002
TID_LOGITS, TID_BOOST_ID, TID_BOOST = 0xB000, 0xB001, 0xB002


def attention_inputs(seed: int, B: int, Hq: int, Hkv: int, R: int, S: int, D: int):
    """q [B,Hq,R,D], k [B,Hkv,S,D], v [B,Hkv,S,D], N(0,1), as bf16 bit patterns."""
    q = normal_tensor(seed, TID_Q, (B, Hq, R, D), 1.0, "bf16")
    k = normal_tensor(seed, TID_K, (B, Hkv, S, D), 1.0, "bf16")
    v = normal_tensor(seed, TID_V, (B, Hkv, S, D), 1.0, "bf16")
    return q, k, v


def boosted_logits(seed: int, rows: int, V: int, boost_hi: float, dtype: str = "bf16",
                   mask_id: int | None = None) -> np.ndarray:
    """N(0,1) logits with +U(0, boost_hi) added at one uniform vocab id per row.

    Returned as bf16 bit patterns (dtype "bf16") or float32 values (dtype "f32").
    """
    z = normal_tensor(seed, TID_LOGITS, (rows, V), 1.0, "f32").astype(np.float64)
    ids = uniform_ints(seed, TID_BOOST_ID, rows, V)
    amt = uniform_unit(seed, TID_BOOST, rows) * boost_hi
    z[np.arange(rows), ids] += amt
    z32 = z.astype(np.float32)
    return fp32_to_bf16_bits(z32) if dtype == "bf16" else z32
