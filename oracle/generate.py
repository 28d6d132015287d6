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

Pins (tests/test_oracle_staleness.py): the cosine against its closed forms and scipy;
the statistics on a hand-built cache; the reused positions of both cache modes by hand;
every cosine is 1 right after a refresh, and layer 0 stays 1 after block-only token
changes while deeper layers move.

``Session`` exposes the same operations as the GPU library (prefill, refresh, step,
generate, and the staleness measure of the cache) so tests can drive both sides from
one token state.
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

    def reused_positions(self, b: int) -> np.ndarray:
        """Boolean [S]: the positions whose K/V a cached step of block b reads from the
        cache (DualCache: every position but the block's; prefix mode: those before it)."""
        s0, s1 = self.block_span(b)
        keep = np.zeros(self.S, dtype=bool)
        keep[:s0] = True
        if self.mode == "dual":
            keep[s1:] = True
        return keep

    def staleness(self, b: int):
        """How far the cache is from the exact K/V of the current tokens, at the positions
        a cached step of block b would take from it.  The pages justify the cache by the
        near-1 cosine similarity of K/V between adjacent denoising steps (ccyt168.com
        Fast-dLLM article, section 1.1, Figure 2; techwalker.com explainer, "Core
        innovation"); this measures that similarity for the live cache: a full forward
        over the current tokens gives the exact K/V, compared per layer by
        ``kv_cosine_stats``.  Returns ([L, 2 (K, V), 2 (mean, min)], reuse ratio), the
        ratio being the fraction of the S positions read from the cache."""
        fresh, _ = full_forward(self.M, self.tokens, logit_rows=None)
        keep = self.reused_positions(b)
        return kv_cosine_stats(self.cache, fresh, keep), keep.sum() / self.S

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


def cosine(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Cosine similarity of the vectors along the last axis, in fp64.  Two zero vectors
    count as identical (1), a zero and a non-zero vector as unrelated (0) (reading: the
    pages do not meet the case)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    dot = np.sum(a * b, axis=-1)
    na = np.sum(a * a, axis=-1)
    nb = np.sum(b * b, axis=-1)
    both = (na == 0) & (nb == 0)
    one = (na == 0) ^ (nb == 0)
    with np.errstate(invalid="ignore", divide="ignore"):
        c = dot / np.sqrt(na * nb)
    return np.where(both, 1.0, np.where(one, 0.0, c))


def kv_cosine_stats(cached: KVCache, fresh: KVCache, keep: np.ndarray) -> np.ndarray:
    """Per layer, for K and for V: the mean and the minimum, over every (sequence, KV
    head, position p with keep[p]), of the cosine similarity of the cached and the fresh
    D-vector.  [L, 2, 2]; a layer with no kept position reports (1, 1)."""
    L = len(cached.K)
    out = np.ones((L, 2, 2))
    keep = np.asarray(keep, dtype=bool)
    if not keep.any():
        return out
    for l in range(L):
        for j, (a, f) in enumerate(((cached.K[l], fresh.K[l]), (cached.V[l], fresh.V[l]))):
            c = cosine(a[:, :, keep, :], f[:, :, keep, :])
            out[l, j] = c.mean(), c.min()
    return out


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
