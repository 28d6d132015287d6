"""Writes tests/golden/logit_scales.json: the fixed LM-head logit scale of each random-init
8B/7B workload, chosen with the oracle so that about 30 % of the masked positions reach
confidence 0.9 at the first denoising step.

    python tests/golden/make_logit_scales.py [workload ...]

Procedure (oracle only; float32 here, since the result is one chosen constant):
1. one prefill forward (prompt + G mask tokens, logit scale 1) gives the unscaled
   logits of every generated position;
2. for each position the scale at which its confidence reaches 0.9 is found by
   bisection (oracle.calibrate); the stored scale is the 30th percentile of those.
Later steps drift from 30 % (in these random-init models the blocks after the first few
see a repeated decoded token and become far less confident); the observed steps per
block are reported by the benchmark, not tuned here.

Also writes tests/golden/first_step_<workload>.json, a sample of the oracle's first
cached step at the chosen scale (by property (a) it equals the prefill's block rows):
for a few block rows of sequence 0 the unscaled logits of the 16 largest ids, the argmax
and the confidence at the chosen scale.  The GPU parity test at the full size compares
against it.  Calls only the oracle and the seeded generator.
"""
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
from oracle.model import OracleModel, full_forward  # noqa: E402

OUT = os.path.join(HERE, "logit_scales.json")
DEFAULT = ["llada8b_dual_p1000_g1024", "llada8b_prefix_p256_g256", "dream7b_dual_b8_p512_g512"]
TARGET = 0.30


def main(names):
    res = json.load(open(OUT)) if os.path.exists(OUT) else {}
    for name in names:
        t = time.time()
        wl = synth.with_scale(synth.WORKLOADS[name], 1.0)
        M = OracleModel(wl, dtype=np.float32, keep=True)
        prompt = synth.make_prompt(wl)
        B, P = prompt.shape
        tokens = np.concatenate([prompt, np.full((B, wl.gen_len), M.m.mask_id, np.int64)], 1)
        _, logits = full_forward(M, tokens, logit_rows=slice(P, P + wl.gen_len))
        z_all = logits.reshape(B * wl.gen_len, -1)
        scale = calibrate_from_logits(z_all, M.m.mask_id, wl.threshold, TARGET)
        sample = {"workload": name, "logit_scale": scale, "rows": []}
        z = logits.reshape(B, wl.gen_len, -1)[0].astype(np.float64)   # sequence 0
        for r in (0, 1, 17, wl.block_len - 1):
            zr = z[r].copy()
            zr[M.m.mask_id] = -np.inf
            top = np.argsort(-zr, kind="stable")[:16]
            conf, arg = decode.confidence_argmax(scale * zr[None, :], M.m.mask_id)
            sample["rows"].append({"row": r, "ids": [int(i) for i in top],
                                   "z": [float(zr[i]) for i in top],
                                   "argmax": int(arg[0]), "conf": float(conf[0])})
        json.dump(sample, open(os.path.join(HERE, f"first_step_{name}.json"), "w"), indent=1)
        res[name] = {"logit_scale": scale, "threshold": wl.threshold, "first_step_fraction": TARGET,
                     "oracle_dtype": "float32", "seconds": round(time.time() - t, 1)}
        print(name, res[name], flush=True)
        json.dump(res, open(OUT, "w"), indent=1, sort_keys=True)
        del M, logits, z_all


if __name__ == "__main__":
    main(sys.argv[1:] or DEFAULT)
