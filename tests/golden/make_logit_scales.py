"""Writes tests/golden/logit_scales.json: the fixed LM-head logit scale of each random-init
8B/7B workload, chosen with the oracle so that about 30 % of the masked positions reach
confidence 0.9 per denoising step.

    python tests/golden/make_logit_scales.py [workload ...]

Procedure (oracle only; float32 here, since the result is one chosen constant):
1. one prefill forward fills the block-wise cache (it does not depend on the scale);
2. "first_step" scale: the 30th percentile of the per-position scales at which the
   first step's confidence reaches 0.9 (oracle.calibrate);
3. for a candidate scale, block 0 is decoded by the oracle's cached steps and the
   fraction of still-masked positions at or above 0.9 is averaged over its steps;
4. bisection on the scale until that per-step fraction is 0.30 (the value used).
Calls only the oracle and the seeded generator.
"""
import copy
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synth  # noqa: E402
from oracle import decode  # noqa: E402
from oracle.calibrate import calibrate_from_logits  # noqa: E402
from oracle.generate import Session  # noqa: E402
from oracle.model import OracleModel, cached_step, full_forward  # noqa: E402

OUT = os.path.join(HERE, "logit_scales.json")
DEFAULT = ["llada8b_dual_p1000_g1024", "llada8b_prefix_p256_g256", "dream7b_dual_b8_p512_g512"]
TARGET = 0.30


def block0_fraction(M, wl, prompt, cache0, scale):
    """Mean over block 0's cached steps of (#masked with conf >= tau) / (#masked)."""
    s = Session(M, prompt, wl.gen_len, wl.block_len, wl.threshold, wl.cache_mode)
    s.cache = copy.deepcopy(cache0)
    s0, s1 = s.block_span(0)
    fr = []
    steps = 0
    while not s.block_done(0):
        logits = cached_step(M, s.tokens, s.cache, s0, s1, wl.cache_mode) * scale
        B, K, V = logits.shape
        conf, arg = decode.confidence_argmax(logits.reshape(B * K, V), M.m.mask_id)
        conf, arg = conf.reshape(B, K), arg.reshape(B, K)
        masked = s.tokens[:, s0:s1] == M.m.mask_id
        fr.append(float(((conf >= wl.threshold) & masked).sum() / max(1, masked.sum())))
        new, *_ = decode.unmask(s.tokens[:, s0:s1], conf, arg, M.m.mask_id, wl.threshold)
        s.tokens[:, s0:s1] = new
        steps += 1
    return float(np.mean(fr)), steps


def main(names):
    res = json.load(open(OUT)) if os.path.exists(OUT) else {}
    for name in names:
        t = time.time()
        wl = synth.with_scale(synth.WORKLOADS[name], 1.0)
        M = OracleModel(wl, dtype=np.float32, keep=True)
        prompt = synth.make_prompt(wl)
        B, P = prompt.shape
        tokens = np.concatenate([prompt, np.full((B, wl.gen_len), M.m.mask_id, np.int64)], 1)
        cache0, logits = full_forward(M, tokens, logit_rows=slice(P, P + wl.gen_len))
        first = calibrate_from_logits(logits.reshape(B * wl.gen_len, -1), M.m.mask_id,
                                      wl.threshold, TARGET)
        print(name, "prefill + first-step scale", round(first, 4), round(time.time() - t, 1), "s",
              flush=True)
        lo, hi = first, None
        f_lo, _ = block0_fraction(M, wl, prompt, cache0, lo)
        trace = [(lo, f_lo)]
        print("  scale", round(lo, 4), "fraction", round(f_lo, 4), flush=True)
        s = lo
        while f_lo < TARGET and hi is None:       # bracket from above
            s = s * 1.6
            f, n = block0_fraction(M, wl, prompt, cache0, s)
            trace.append((s, f))
            print("  scale", round(s, 4), "fraction", round(f, 4), "steps", n, flush=True)
            if f >= TARGET:
                hi = s
            else:
                lo, f_lo = s, f
        for _ in range(6):                        # bisection
            mid = 0.5 * (lo + hi)
            f, n = block0_fraction(M, wl, prompt, cache0, mid)
            trace.append((mid, f))
            print("  scale", round(mid, 4), "fraction", round(f, 4), "steps", n, flush=True)
            if f >= TARGET:
                hi = mid
            else:
                lo = mid
        scale = hi
        res[name] = {"logit_scale": scale, "threshold": wl.threshold, "per_step_fraction": TARGET,
                     "first_step_scale": first, "trace": [[round(a, 5), round(b, 5)] for a, b in trace],
                     "oracle_dtype": "float32", "seconds": round(time.time() - t, 1)}
        print(name, res[name], flush=True)
        json.dump(res, open(OUT, "w"), indent=1, sort_keys=True)
        del M, cache0


if __name__ == "__main__":
    main(sys.argv[1:] or DEFAULT)
