"""Writes tests/golden/logit_scales.json: the fixed LM-head logit scale of each random-init
8B/7B workload, chosen by the oracle (oracle.calibrate) so that about 30 % of the masked
positions reach confidence 0.9 at the first step of generation.

    python tests/golden/make_logit_scales.py [workload ...]

Calls only the oracle and the seeded generator.  The oracle runs in float32 here: the
result is a single chosen constant, not a parity value.
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synth  # noqa: E402
from oracle.calibrate import calibrate  # noqa: E402
from oracle.model import OracleModel  # noqa: E402

OUT = os.path.join(HERE, "logit_scales.json")
DEFAULT = ["llada8b_dual_p1000_g1024", "llada8b_prefix_p256_g256", "dream7b_dual_b8_p512_g512"]


def main(names):
    res = json.load(open(OUT)) if os.path.exists(OUT) else {}
    for name in names:
        wl = synth.with_scale(synth.WORKLOADS[name], 1.0)
        t = time.time()
        M = OracleModel(wl, dtype=np.float32, keep=False)
        s = calibrate(M, synth.make_prompt(wl), wl.gen_len, wl.threshold, 0.30)
        res[name] = {"logit_scale": s, "threshold": wl.threshold, "fraction": 0.30,
                     "oracle_dtype": "float32", "seconds": round(time.time() - t, 1)}
        print(name, res[name], flush=True)
        json.dump(res, open(OUT, "w"), indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:] or DEFAULT)
