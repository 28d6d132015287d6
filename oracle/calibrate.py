"""Oracle: choice of the fixed logit scale for the random-init 8B/7B shapes.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may use it).

A random-init model has nearly flat next-token distributions, so no position would
ever reach a 0.9 confidence and the threshold rule would always fall back to one token
per step.  The workloads therefore multiply the LM-head output by a fixed scale,
chosen so that about 30 % of the masked positions of the first step of generation
reach the threshold.  Procedure (a reading; the pages have no random-init models):

1. one full forward over prompt + G mask tokens with scale 1 gives the unscaled
   logits z of every generated position;
2. for each position, conf(s) = 1 / sum_v exp(s (z_v - max z)) (mask id excluded) is
   non-decreasing in s >= 0, so bisection finds the s_i where conf(s_i) = tau;
3. the scale is the 30th percentile of {s_i}: at that scale 30 % of the positions
   reach the threshold.
tests/golden/make_logit_scales.py applies it to each 8B/7B workload.
"""
from __future__ import annotations

import numpy as np

from .model import OracleModel, full_forward


def conf_at_scale(z: np.ndarray, s: float) -> np.ndarray:
    """Max softmax probability of rows z (mask already excluded as -inf) at scale s."""
    d = z - z.max(axis=1, keepdims=True)
    return 1.0 / np.exp(s * d).sum(axis=1)


def scale_for_threshold(z: np.ndarray, tau: float, iters: int = 60) -> np.ndarray:
    """Per row, the scale s at which the row's confidence equals tau (bisection).

    A row whose maximum is attained k > 1 times never gets above 1/k, whatever the
    scale; if that is below tau the row's scale is +inf (it never passes)."""
    z = np.asarray(z, dtype=np.float64)
    ties = (z == z.max(axis=1, keepdims=True)).sum(axis=1)
    never = 1.0 / ties < tau
    zz = z[~never]
    lo = np.zeros(zz.shape[0])
    hi = np.ones(zz.shape[0])
    while True:                                   # grow hi until every row reaches tau
        c = conf_at_scale_rows(zz, hi)
        if (c >= tau).all():
            break
        hi = np.where(c >= tau, hi, hi * 2.0)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        c = conf_at_scale_rows(zz, mid)
        lo = np.where(c >= tau, lo, mid)
        hi = np.where(c >= tau, mid, hi)
    out = np.full(z.shape[0], np.inf)
    out[~never] = hi
    return out


def conf_at_scale_rows(z: np.ndarray, s: np.ndarray) -> np.ndarray:
    d = z - z.max(axis=1, keepdims=True)
    return 1.0 / np.exp(s[:, None] * d).sum(axis=1)


def calibrate_from_logits(z: np.ndarray, mask_id: int, tau: float = 0.9,
                          frac: float = 0.30) -> float:
    z = np.array(z, dtype=np.float64, copy=True)
    z[:, mask_id] = -np.inf
    s = scale_for_threshold(z, tau)
    return float(np.quantile(s, frac))


def calibrate(M: OracleModel, prompt: np.ndarray, gen_len: int, tau: float = 0.9,
              frac: float = 0.30) -> float:
    """Scale from one unscaled full forward over prompt + gen_len mask tokens."""
    if M.m.logit_scale != 1.0:
        raise ValueError("calibrate with a model whose logit scale is 1")
    prompt = np.asarray(prompt, dtype=np.int64)
    B, P = prompt.shape
    tokens = np.concatenate([prompt, np.full((B, gen_len), M.m.mask_id, np.int64)], axis=1)
    _, logits = full_forward(M, tokens, logit_rows=slice(P, P + gen_len))
    return calibrate_from_logits(logits.reshape(B * gen_len, -1), M.m.mask_id, tau, frac)
