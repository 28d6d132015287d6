"""Python-side ownership of device buffers for libdllm: a Model (weights) and a Session
(tokens, KV cache, workspace of one batch being generated).

torch provides the device allocations and the stream; every computation is a library
call (binding.py).
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import binding as bd

_WEIGHT_NAMES = ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate_up", "w_down")


def _torch():
    import torch
    return torch


def _tdtype(dtype: int):
    torch = _torch()
    return torch.float32 if dtype == bd.F32 else torch.bfloat16


class Model:
    """Weights on the device.  ``shape`` needs the attributes n_layers, d_model, n_heads,
    n_kv_heads, head_dim, d_ffn, vocab, mask_id, rope_theta, norm_eps, logit_scale and
    dtype ("f32" or "bf16")."""

    def __init__(self, lib: bd.Lib, shape, tensors: dict):
        self.lib, self.shape, self.t = lib, shape, tensors
        self.dtype = bd.F32 if shape.dtype == "f32" else bd.BF16
        L = shape.n_layers
        self._arrays = {}
        for n in _WEIGHT_NAMES:
            arr = (C.c_void_p * L)(*[tensors[f"{n}.{l}"].data_ptr() for l in range(L)])
            self._arrays[n] = arr
        self.desc = bd.ModelDesc(
            n_layers=L, d_model=shape.d_model, n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads,
            head_dim=shape.head_dim, d_ffn=shape.d_ffn, vocab=shape.vocab, mask_id=shape.mask_id,
            rope_theta=shape.rope_theta, norm_eps=shape.norm_eps, logit_scale=shape.logit_scale,
            dtype=self.dtype, embed=tensors["embed"].data_ptr(),
            final_norm=tensors["final_norm"].data_ptr(), lm_head=tensors["lm_head"].data_ptr(),
            **{n: C.cast(self._arrays[n], C.POINTER(C.c_void_p)) for n in _WEIGHT_NAMES})

    def with_logit_scale(self, scale: float) -> "Model":
        from dataclasses import replace
        return Model(self.lib, replace(self.shape, logit_scale=float(scale)), self.t)

    @staticmethod
    def from_host(lib: bd.Lib, shape, weights: dict, device="cuda") -> "Model":
        """Upload host arrays: float32 values (f32 models) or uint16 bf16 bit patterns."""
        torch = _torch()
        t = {}
        for k, a in weights.items():
            if shape.dtype == "f32":
                t[k] = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
            else:
                b = np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)
                t[k] = torch.from_numpy(b).view(torch.bfloat16).to(device)
        return Model(lib, shape, t)

    @staticmethod
    def synthetic(lib: bd.Lib, wl, device="cuda", stream=None) -> "Model":
        """Seeded random-init weights made on the device by the library's generator
        (bit-identical to the host generator in ``synth``)."""
        import synth
        torch = _torch()
        m = wl.model
        dt = bd.F32 if m.dtype == "f32" else bd.BF16
        st = bd.stream_handle(stream)
        t = {}
        for name, layer, tid, shape, std, is_norm in synth.weight_specs(m, wl.norm_gain_std):
            x = torch.empty(shape, dtype=_tdtype(dt), device=device)
            if is_norm:
                mode, s = (2, 1.0) if std == 0.0 else (1, std)
            else:
                mode, s = 0, std
            lib.call("dllm_synth_fill", bd.ptr(x), x.numel(), dt, wl.model_seed, tid, s, mode, st)
            t[name if layer < 0 else f"{name}.{layer}"] = x
        return Model(lib, m, t)


# Debug runs: bytes of guard band on each side of the KV cache and the workspace, and the
# 32-bit canary they hold.  The buffers themselves start filled with 0xFF bytes, a NaN in
# both fp32 and bf16, so that any read of a byte the library has not written first shows
# up as NaN in the results.
GUARD_BYTES = 1 << 16
CANARY = 0x5CA1AB1E


class Session:
    """Tokens, KV cache and workspace of one batch of sequences.

    With ``debug`` the KV cache and the workspace are NaN-poisoned before first use and
    framed by canary guard bands; ``check_guards()`` raises if a call wrote outside them."""

    def __init__(self, model: Model, prompt, gen_len: int, block_len: int, threshold: float,
                 mode: str, device="cuda", debug: bool = False):
        torch = _torch()
        self.model, self.lib = model, model.lib
        prompt = torch.as_tensor(np.asarray(prompt), dtype=torch.int32)
        B, P = prompt.shape
        self.B, self.P, self.G, self.K = B, P, gen_len, block_len
        self.S = P + gen_len
        self.n_blocks = gen_len // block_len if block_len > 0 else 0
        toks = torch.full((B, self.S), model.shape.mask_id, dtype=torch.int32)
        toks[:, :P] = prompt
        self.tokens = toks.to(device)
        modes = {"dual": bd.CACHE_DUAL, "prefix": bd.CACHE_PREFIX, "none": bd.CACHE_NONE}
        if mode not in modes:
            raise ValueError(f"cache mode {mode!r} not in {sorted(modes)}")
        self.mode = modes[mode]
        self.desc = bd.SeqDesc(batch=B, prompt_len=P, gen_len=gen_len, block_len=block_len,
                               cache_mode=self.mode, threshold=threshold,
                               tokens=self.tokens.data_ptr())
        mp, sp = C.byref(model.desc), C.byref(self.desc)
        cb = self.lib.raw("dllm_kv_cache_bytes")(mp, sp)
        wb = self.lib.raw("dllm_workspace_bytes")(mp, sp)
        if cb == 0 or wb == 0:
            # report why through a call that validates
            self.lib.check(self.lib.raw("dllm_prefill_cache")(mp, sp, None), "Session")
        self.debug = debug
        if debug:
            self._guarded = {}
            self.cache = self._guarded_buffer("kv_cache", cb, device)
            self.ws = self._guarded_buffer("workspace", wb, device)
        else:
            self.cache = torch.empty(cb, dtype=torch.uint8, device=device)
            self.ws = torch.empty(wb, dtype=torch.uint8, device=device)
        self.desc.kv_cache = self.cache.data_ptr()
        self.desc.kv_cache_bytes = cb
        self.desc.workspace = self.ws.data_ptr()
        self.desc.workspace_bytes = wb
        self.n_unmasked = torch.zeros(B, dtype=torch.int32, device=device)
        self.remaining = torch.zeros(B, dtype=torch.int32, device=device)

    def _guarded_buffer(self, name: str, nbytes: int, device):
        """A NaN-poisoned buffer of nbytes inside a larger allocation whose first and last
        GUARD_BYTES hold the canary; returns the view of the inner bytes."""
        torch = _torch()
        g = GUARD_BYTES // 4
        n4 = (nbytes + 3) // 4
        full = torch.full((2 * g + n4,), CANARY, dtype=torch.int32, device=device)
        full[g:g + n4] = -1                       # 0xFFFFFFFF: NaN as fp32 and as two bf16
        self._guarded[name] = (full, g, n4)
        return full.view(torch.uint8)[4 * g:4 * g + nbytes]

    def check_guards(self):
        """Raise if any byte of a guard band around the cache or the workspace changed."""
        if not self.debug:
            return
        torch = _torch()
        torch.cuda.synchronize(self.tokens.device)
        want = np.int32(CANARY)
        for name, (full, g, n4) in self._guarded.items():
            for side, band in (("before", full[:g]), ("after", full[g + n4:])):
                h = band.cpu().numpy()
                bad = np.nonzero(h != want)[0]
                if bad.size:
                    raise RuntimeError(f"{name}: guard band {side} the buffer overwritten at "
                                       f"{bad.size} words (first at word {int(bad[0])})")

    def _args(self):
        return C.byref(self.model.desc), C.byref(self.desc)

    def prefill(self, stream=None):
        self.lib.call("dllm_prefill_cache", *self._args(), bd.stream_handle(stream))

    def refresh(self, block: int, stream=None):
        self.lib.call("dllm_refresh_cache", *self._args(), block, bd.stream_handle(stream))

    def step(self, block: int, logits: bool = True, stream=None) -> dict:
        """One cached denoising step of `block` (dllm_block_step)."""
        return self._decode("dllm_block_step", block, logits, stream)

    def refresh_step(self, block: int, logits: bool = True, stream=None) -> dict:
        """The refresh of `block` (the prefill for block 0) fused with its first step
        (dllm_refresh_step)."""
        return self._decode("dllm_refresh_step", block, logits, stream)

    def staleness(self, block: int, stream=None) -> dict:
        """Cosine similarity of the cached K/V that a cached step of `block` would read now
        and the exact K/V of the current tokens (dllm_cache_staleness): per layer, the
        mean and minimum over the positions taken from the cache, for K and V; and the
        reuse ratio, the fraction of the S positions whose K/V the step takes from the
        cache (DualCache: all but the block's; prefix mode: those before the block)."""
        torch = _torch()
        dev = self.tokens.device
        fresh = torch.empty_like(self.cache)
        out = torch.empty((self.model.shape.n_layers, 2, 2), dtype=torch.float32, device=dev)
        reuse = C.c_double()
        self.lib.call("dllm_cache_staleness", *self._args(), block, bd.ptr(fresh),
                      fresh.numel(), bd.ptr(out), C.byref(reuse), bd.stream_handle(stream))
        torch.cuda.synchronize(dev)
        o = out.cpu().numpy()
        return {"k_mean": o[:, 0, 0], "k_min": o[:, 0, 1], "v_mean": o[:, 1, 0],
                "v_min": o[:, 1, 1], "reuse": reuse.value}

    def _decode(self, entry: str, block: int, logits: bool, stream) -> dict:
        torch = _torch()
        dev = self.tokens.device
        out = {"n_unmasked": self.n_unmasked, "remaining": self.remaining}
        lg = torch.empty((self.B * self.K, self.model.shape.vocab), dtype=torch.float32,
                         device=dev) if logits else None
        conf = torch.empty((self.B, self.K), dtype=torch.float32, device=dev)
        arg = torch.empty((self.B, self.K), dtype=torch.int32, device=dev)
        self.lib.call(entry, *self._args(), block, bd.stream_handle(stream),
                      bd.ptr(self.n_unmasked), bd.ptr(self.remaining), bd.ptr(lg), bd.ptr(conf),
                      bd.ptr(arg))
        out.update(logits=lg, conf=conf, argmax=arg)
        return out

    def generate(self, stream=None, graphs: bool = False):
        """Whole generation (dllm_generate; with graphs, dllm_generate_graphs: each
        block's cached steps replayed from a captured HIP graph)."""
        spb = (C.c_int32 * max(1, self.n_blocks))()
        st = bd.Stats(steps_per_block=spb)
        self.lib.call("dllm_generate_graphs" if graphs else "dllm_generate", *self._args(),
                      bd.stream_handle(stream), C.byref(st))
        stats = {"steps": st.steps, "refreshes": st.refreshes, "tokens": st.tokens,
                 "blocks": st.blocks, "ms_total": st.ms_total, "ms_refresh": st.ms_refresh,
                 "ms_step": st.ms_step, "steps_per_block": list(spb)[: self.n_blocks],
                 "speculative_steps": st.speculative_steps,
                 "masked_at_step_start": st.masked_at_step_start}
        return self.tokens[:, self.P:].cpu().numpy(), stats

    def reset_tokens(self, prompt=None):
        """Put the generated span back to mask tokens (and optionally a new prompt)."""
        torch = _torch()
        self.tokens[:, self.P:] = self.model.shape.mask_id
        if prompt is not None:
            self.tokens[:, :self.P] = torch.as_tensor(np.asarray(prompt), dtype=torch.int32,
                                                      device=self.tokens.device)
