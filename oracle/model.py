"""Oracle model: a LLaDA/Dream-style bidirectional transformer, written plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may use it).

What the pages fix, and what is a reading
-----------------------------------------
* The model is a masked-diffusion LLM whose attention is bidirectional: every position
  attends to every other, which is why an autoregressive KV cache does not apply as is
  (ccyt168.com Fast-dLLM article, opening paragraphs and section 1.1; techwalker.com
  explainer, "Core innovation: a KV cache suited to diffusion models").  Here: no causal
  mask anywhere.
* Architecture details are not on the pages (they only name LLaDA and Dream).  Reading:
  pre-norm blocks ``h = x + Attn(RMSNorm(x)); x' = h + FFN(RMSNorm(h))`` with a final
  RMSNorm, no biases, untied LM head, RoPE in rotate-half form (pairs i and i + D/2,
  inverse frequency theta**(-2j/D), absolute positions 0..S-1), RMSNorm eps 1e-5,
  attention scale 1/sqrt(D), SwiGLU FFN ``silu(gate) * up``; grouped-query attention
  maps query head h to KV head h // (Hq/Hkv).  The LM-head output is multiplied by a
  fixed logit scale.
* Block-wise approximate KV cache (both pages): before a block is generated, the KV of
  all positions is computed by a full forward and kept; while the block is decoded
  those entries are reused; after the block the KV of all positions is recomputed.
  DualCache keeps both the prefix and the masked suffix; prefix mode keeps only the
  prefix and recomputes the block and everything after it on every step (reading of
  the prefix-only variant: the pages describe it only as "caching the prefix").
* Storage precision (a reading; the pages state none).  fp32 models: no rounding, the
  oracle computes in float64.  bf16 models: weights and the KV cache are bf16; the
  residual stream and logits are fp32; the RMSNorm outputs, the post-RoPE q/k and v,
  the attention output and the SwiGLU output are rounded to bf16 (nearest even, via
  fp32).  Matmuls and softmax are evaluated in the oracle's compute dtype.

Pins (tests/test_oracle_model.py): RMSNorm, attention and SwiGLU against torch CPU
float64 library routines; RoPE against its closed form (norm preservation, relative
position property, position 0 identity); full forward against an independent torch
float64 re-composition; first cached step after a refresh equals the full forward
(both cache modes); refreshing before every step reproduces the no-cache algorithm;
layer-0 K/V of unchanged tokens equal fresh ones; with an empty prompt every prefix-mode
step of block 0 recomputes all rows, so each of them (not only the first) equals the full
forward, while DualCache drifts from the second step on (pins the suffix recompute of
prefix mode).  Later DualCache steps are defined by the cache-staleness reading only:
beyond those invariants their values have no external pin.
"""
from __future__ import annotations

import numpy as np

import synth


# ----------------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------------

def round_f32(x: np.ndarray) -> np.ndarray:
    """Round to fp32 storage (nearest even) and return in the input's dtype."""
    return np.asarray(x).astype(np.float32).astype(np.asarray(x).dtype)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bf16 storage: first to fp32 (nearest even), then to bf16 (nearest even)."""
    x = np.asarray(x)
    f = x.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    # nearest even on the low 16 bits
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    out = np.where(np.isfinite(f), out, f)
    return out.astype(x.dtype)


# ----------------------------------------------------------------------------------
# building blocks
# ----------------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_cos_sin(positions: np.ndarray, D: int, theta: float):
    """cos, sin [len(positions), D/2] in float64: angle = pos * theta**(-2j/D)."""
    j = np.arange(D // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / D)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE on the last axis; x [..., n, D], cos/sin [n, D/2]."""
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def softmax(z: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(z, axis=axis, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Non-causal attention. q [B,Hq,R,D], k/v [B,Hkv,S,D] -> o [B,Hq,R,D].

    Every query row sees every key (no mask); query head h reads KV head h // (Hq/Hkv).
    """
    B, Hq, R, D = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    o = np.empty_like(q)
    for b in range(B):
        for h in range(Hq):
            kv = h // group
            s = (q[b, h] @ k[b, kv].T) / np.sqrt(D)                # [R, S]
            o[b, h] = softmax(s, -1) @ v[b, kv]
    return o


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """x [..., K] . w[N, K]^T as one 2-D product (so the library GEMM is used)."""
    y = x.reshape(-1, x.shape[-1]) @ w.T
    return y.reshape(x.shape[:-1] + (w.shape[0],))


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


# ----------------------------------------------------------------------------------
# model container
# ----------------------------------------------------------------------------------

class OracleModel:
    """Weights as float arrays in the oracle's compute dtype, generated from ``synth``.

    Layers are generated on first use and kept only if ``keep`` is true, so a model of
    the 8B shapes can be evaluated layer by layer without holding every layer.
    """

    def __init__(self, wl: "synth.Workload", dtype=np.float64, keep: bool = True,
                 weights: dict | None = None):
        self.wl = wl
        self.m = wl.model
        self.dtype = dtype
        self.keep = keep
        self.bf16 = self.m.dtype == "bf16"
        self._specs = {(s[0], s[1]): s for s in synth.weight_specs(self.m, wl.norm_gain_std)}
        self._cache: dict = {}
        self._given = weights

    def _get(self, name: str, layer: int = -1) -> np.ndarray:
        key = (name, layer)
        if key in self._cache:
            return self._cache[key]
        if self._given is not None:
            raw = self._given[name if layer < 0 else f"{name}.{layer}"]
        else:
            raw = synth.make_weight(self.wl, self._specs[key])
        arr = synth.as_float(raw, self.m.dtype).astype(self.dtype)
        if self.keep or layer < 0:
            self._cache[key] = arr
        return arr

    def w(self, name: str, layer: int = -1) -> np.ndarray:
        return self._get(name, layer)

    # storage rounding points
    def rs(self, x):  # activations stored as bf16 (or unrounded for fp32 models)
        return round_bf16(x) if self.bf16 else x

    def rf(self, x):  # fp32 storage (residual stream, logits) for bf16 models
        return round_f32(x) if self.bf16 else x


# ----------------------------------------------------------------------------------
# one transformer layer over a set of rows
# ----------------------------------------------------------------------------------

def layer_qkv(M: OracleModel, l: int, x: np.ndarray, positions: np.ndarray):
    """Attention-norm + QKV projection + RoPE for rows x [B,R,d] at ``positions`` [R].

    Returns q [B,Hq,R,D], k [B,Hkv,R,D], v [B,Hkv,R,D] (bf16-rounded for bf16 models).
    """
    m = M.m
    B, R, _ = x.shape
    D, Hq, Hkv = m.head_dim, m.n_heads, m.n_kv_heads
    h = M.rs(rmsnorm(x, M.w("attn_norm", l), m.norm_eps))
    qkv = linear(h, M.w("w_qkv", l))                             # [B,R,(Hq+2Hkv)D]
    q = qkv[..., :Hq * D].reshape(B, R, Hq, D).transpose(0, 2, 1, 3)
    k = qkv[..., Hq * D:(Hq + Hkv) * D].reshape(B, R, Hkv, D).transpose(0, 2, 1, 3)
    v = qkv[..., (Hq + Hkv) * D:].reshape(B, R, Hkv, D).transpose(0, 2, 1, 3)
    cos, sin = rope_cos_sin(positions, D, m.rope_theta)
    # tables in the compute dtype: a float32 oracle stays in float32 (the tables are
    # then the fp32 values a float32 implementation stores); float64 is unchanged
    cos, sin = cos.astype(M.dtype), sin.astype(M.dtype)
    q = M.rs(apply_rope(q, cos, sin))
    k = M.rs(apply_rope(k, cos, sin))
    v = M.rs(v)
    return q, k, v


def layer_rest(M: OracleModel, l: int, x: np.ndarray, q: np.ndarray, K: np.ndarray,
               V: np.ndarray) -> np.ndarray:
    """Attention of q over keys K/V, output projection, residual, FFN, residual."""
    m = M.m
    B, R, d = x.shape
    o = M.rs(attention(q, K, V))                                 # [B,Hq,R,D]
    o = o.transpose(0, 2, 1, 3).reshape(B, R, m.n_heads * m.head_dim)
    x = M.rf(x + linear(o, M.w("w_o", l)))
    h = M.rs(rmsnorm(x, M.w("ffn_norm", l), m.norm_eps))
    gu = linear(h, M.w("w_gate_up", l))
    a = M.rs(silu(gu[..., :m.d_ffn]) * gu[..., m.d_ffn:])
    return M.rf(x + linear(a, M.w("w_down", l)))


def embed(M: OracleModel, tokens: np.ndarray) -> np.ndarray:
    return M.w("embed")[np.asarray(tokens)]


def lm_head(M: OracleModel, x: np.ndarray) -> np.ndarray:
    """Final RMSNorm, LM head, logit scale.  x [B,R,d] -> logits [B,R,V]."""
    m = M.m
    h = M.rs(rmsnorm(x, M.w("final_norm"), m.norm_eps))
    return M.rf(m.logit_scale * linear(h, M.w("lm_head")))


# ----------------------------------------------------------------------------------
# full forward (no cache) and the cached step
# ----------------------------------------------------------------------------------

class KVCache:
    """Per-layer post-RoPE K and V of every position: K[l], V[l] are [B,Hkv,S,D]."""

    def __init__(self, L: int, B: int, Hkv: int, S: int, D: int, dtype):
        self.K = [np.zeros((B, Hkv, S, D), dtype) for _ in range(L)]
        self.V = [np.zeros((B, Hkv, S, D), dtype) for _ in range(L)]


def full_forward(M: OracleModel, tokens: np.ndarray, logit_rows: slice | None = slice(None),
                 cache: KVCache | None = None):
    """Bidirectional forward over all S positions with nothing cached.

    Writes every layer's K/V into ``cache`` (created if None) and returns
    (cache, logits) where logits are for positions ``logit_rows`` ([B, R, V]) or None.
    """
    m = M.m
    tokens = np.asarray(tokens)
    B, S = tokens.shape
    if cache is None:
        cache = KVCache(m.n_layers, B, m.n_kv_heads, S, m.head_dim, M.dtype)
    x = embed(M, tokens)
    pos = np.arange(S)
    for l in range(m.n_layers):
        q, k, v = layer_qkv(M, l, x, pos)
        cache.K[l][...] = k
        cache.V[l][...] = v
        if l == m.n_layers - 1 and logit_rows is None:
            break                       # the cache does not need the last layer's tail
        x = layer_rest(M, l, x, q, k, v)
    logits = None if logit_rows is None else lm_head(M, x[:, logit_rows])
    return cache, logits


def step_rows(mode: str, s0: int, s1: int, S: int):
    """Rows recomputed by a cached step of the block [s0, s1)."""
    if mode == "dual":
        return s0, s1
    if mode == "prefix":
        return s0, S
    raise ValueError(mode)


def cached_step(M: OracleModel, tokens: np.ndarray, cache: KVCache, s0: int, s1: int,
                mode: str) -> np.ndarray:
    """One denoising step of block [s0, s1) against the block-wise approximate cache.

    DualCache: only the block rows are recomputed; every other position's K/V is the
    cached value from the last refresh.  Prefix: rows [s0, S) are recomputed and only
    [0, s0) comes from the cache.  The fresh rows' K/V replace the cache entries in
    place.  Returns the block rows' logits [B, s1 - s0, V].
    """
    m = M.m
    tokens = np.asarray(tokens)
    S = tokens.shape[1]
    r0, r1 = step_rows(mode, s0, s1, S)
    x = embed(M, tokens[:, r0:r1])
    pos = np.arange(r0, r1)
    for l in range(m.n_layers):
        q, k, v = layer_qkv(M, l, x, pos)
        cache.K[l][:, :, r0:r1] = k
        cache.V[l][:, :, r0:r1] = v
        x = layer_rest(M, l, x, q, cache.K[l], cache.V[l])
    return lm_head(M, x[:, : s1 - s0])
