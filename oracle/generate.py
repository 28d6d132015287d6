"""Oracle: block-wise generation with the approximate KV cache and threshold decoding.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may use it).

Control flow (techwalker.com explainer, "Core innovation: a KV cache suited to
diffusion models", steps 1 and 2; ccyt168.com Fast-dLLM article, sections 1.1-1.2):

* the sequence is prompt + G mask tokens; the G positions form blocks of K that are
  decoded left to right;
* before block 0 a full forward fills the cache (prefill); after each finished block
  a full forward recomputes every position's K/V (refresh), except after the last;
  the refresh decodes nothing (reading: the pages list it as a separate act);
* inside a block, cached steps run until no mask token is left in the block; each
  step unmasks by the threshold rule (``decode.unmask``);
* sequences of a batch move through blocks in lockstep; a sequence whose block is
  already complete gets no forced unmask (reading; the pages use batch 1);
* all G tokens are generated: no end-of-sequence handling (reading).

``Session`` exposes the same four operations as the GPU library (prefill, refresh,
step, generate) so tests can drive both sides from one token state.
"""
from __future__ import annotations

import numpy as np

from . import decode
from .model import KVCache, OracleModel, cached_step, full_forward


class Session:
    def __init__(self, M: OracleModel, prompt: np.ndarray, gen_len: int, block_len: int,
                 tau: float, mode: str):
        m = M.m
        prompt = np.asarray(prompt, dtype=np.int64)
        if gen_len % block_len:
            raise ValueError("gen_len must be a multiple of block_len")
        self.M, self.K, self.tau, self.mode = M, block_len, float(tau), mode
        self.P, self.G = prompt.shape[1], gen_len
        self.B = prompt.shape[0]
        self.S = self.P + self.G
        self.tokens = np.concatenate(
            [prompt, np.full((self.B, gen_len), m.mask_id, dtype=np.int64)], axis=1)
        self.cache = KVCache(m.n_layers, self.B, m.n_kv_heads, self.S, m.head_dim, M.dtype)
        self.n_blocks = gen_len // block_len

    def block_span(self, b: int):
        s0 = self.P + b * self.K
        return s0, s0 + self.K

    def refresh(self):
        """Full forward over every position; K/V into the cache.  Decodes nothing."""
        full_forward(self.M, self.tokens, logit_rows=None, cache=self.cache)

    prefill = refresh

    def step(self, b: int):
        """One cached denoising step of block b.  Returns a dict of what it produced."""
        s0, s1 = self.block_span(b)
        logits = cached_step(self.M, self.tokens, self.cache, s0, s1, self.mode)
        B, K, V = logits.shape
        conf, arg = decode.confidence_argmax(logits.reshape(B * K, V), self.M.m.mask_id)
        conf, arg = conf.reshape(B, K), arg.reshape(B, K)
        new, U, n_un, rem = decode.unmask(self.tokens[:, s0:s1], conf, arg,
                                          self.M.m.mask_id, self.tau)
        self.tokens[:, s0:s1] = new
        return {"logits": logits, "conf": conf, "argmax": arg, "U": U,
                "n_unmasked": n_un, "remaining": rem}

    def block_done(self, b: int) -> bool:
        s0, s1 = self.block_span(b)
        return not (self.tokens[:, s0:s1] == self.M.m.mask_id).any()

    def generate(self, on_step=None):
        """Whole generation.  Returns (generated tokens [B, G], stats)."""
        steps_per_block = []
        refreshes = 0
        for b in range(self.n_blocks):
            self.refresh()
            refreshes += 1
            n = 0
            while not self.block_done(b):
                out = self.step(b)
                n += 1
                if on_step is not None:
                    on_step(b, n, out)
                if n > self.K:
                    raise RuntimeError("a block took more steps than its length")
            steps_per_block.append(n)
        stats = {"steps": int(sum(steps_per_block)), "refreshes": refreshes,
                 "steps_per_block": steps_per_block, "tokens": self.B * self.G}
        return self.tokens[:, self.P:].copy(), stats


def generate(M: OracleModel, prompt: np.ndarray, gen_len: int, block_len: int, tau: float,
             mode: str):
    return Session(M, prompt, gen_len, block_len, tau, mode).generate()


def generate_nocache(M: OracleModel, prompt: np.ndarray, gen_len: int, block_len: int,
                     tau: float):
    """The same decoding with no cache: a full forward before every step.

    Used as the exact (no-approximation) counterpart of ``generate``.
    """
    s = Session(M, prompt, gen_len, block_len, tau, "dual")
    steps = 0
    for b in range(s.n_blocks):
        while not s.block_done(b):
            s0, s1 = s.block_span(b)
            _, logits = full_forward(M, s.tokens, logit_rows=slice(s0, s1))
            B, K, V = logits.shape
            conf, arg = decode.confidence_argmax(logits.reshape(B * K, V), M.m.mask_id)
            new, *_ = decode.unmask(s.tokens[:, s0:s1], conf.reshape(B, K),
                                    arg.reshape(B, K), M.m.mask_id, tau)
            s.tokens[:, s0:s1] = new
            steps += 1
    return s.tokens[:, s.P:].copy(), {"steps": steps}
