"""Oracle: confidence, argmax and the threshold-unmask rule.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may use it).

* Confidence is the probability the model assigns to the token it would emit
  (ccyt168.com Fast-dLLM article, section 1.2 "Confidence-Aware Parallel Decoding"):
  ``conf = max_v softmax(z)_v = 1 / sum_v exp(z_v - max z)``; the token is the argmax
  (greedy, no sampling; the article's theorem is stated for greedy decoding).
* Every masked position of the current block whose confidence is at or above the
  threshold (for example 0.9) is decoded in this step; the others wait for later steps
  (same section; techwalker.com explainer, "Solving the quality loss of parallel
  decoding": a threshold instead of a fixed number of tokens per step).
* Readings where the pages are silent: the mask token itself can never be emitted
  (its logit is excluded before the max, the sum and the argmax); ``>=`` is used at the
  threshold; argmax ties go to the lowest token id; if no masked position of a
  sequence reaches the threshold, the single most confident masked position is decoded
  (ties to the lowest position), so every step decodes at least one token per
  sequence that still has masked positions; decoded tokens are never masked again.

Pins (tests/test_oracle_decode.py): confidence against torch.softmax(...).max and
numpy.argmax (first occurrence) on random rows, uniform rows (conf = 1/(V-1), argmax
0), a two-value closed form; the unmask rule against a brute-force enumeration of all
2**K subsets for K <= 8 with the set definition; tau > 1 decodes exactly one token per
step; tau <= 0 decodes the whole block at once; monotone in tau.
"""
from __future__ import annotations

import numpy as np


def confidence_argmax(logits: np.ndarray, mask_id: int):
    """Per row: (conf float64 [R], argmax int64 [R]) with the mask id excluded."""
    z = np.array(logits, dtype=np.float64, copy=True)
    if z.ndim != 2:
        raise ValueError("logits must be [rows, V]")
    z[:, mask_id] = -np.inf
    m = z.max(axis=1)
    arg = np.argmax(z, axis=1)                  # first occurrence: lowest id on ties
    conf = 1.0 / np.exp(z - m[:, None]).sum(axis=1)
    return conf, arg.astype(np.int64)


def unmask(block_tokens: np.ndarray, conf: np.ndarray, argmax: np.ndarray, mask_id: int,
           tau: float):
    """Threshold unmask of one block for every sequence.

    block_tokens [B,K] int, conf [B,K], argmax [B,K].  Returns
    (new_tokens [B,K], U [B,K] bool, n_unmasked [B], remaining [B]).
    """
    tok = np.array(block_tokens, dtype=np.int64, copy=True)
    conf = np.asarray(conf, dtype=np.float64)
    B, K = tok.shape
    masked = tok == mask_id
    U = masked & (conf >= tau)
    for b in range(B):
        if masked[b].any() and not U[b].any():
            cand = np.where(masked[b], conf[b], -np.inf)
            U[b, int(np.argmax(cand))] = True  # lowest position on ties
    tok[U] = np.asarray(argmax)[U]
    n_unmasked = U.sum(axis=1).astype(np.int64)
    remaining = (masked & ~U).sum(axis=1).astype(np.int64)
    return tok, U, n_unmasked, remaining
