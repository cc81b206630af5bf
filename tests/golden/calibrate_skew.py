"""Find the c5 skew strength beta and write tests/golden/skew_beta.json.

The c5 workload's expert bias is b_e = -beta * ln(rank_e) over a seeded
popularity ranking.  beta is chosen by bisection so that, on a separate
4096-token calibration batch (stream 11), the 10 hottest experts (3.9% of
256) receive 30% of the top-8 selections.  That matches the expert
popularity skew the pages measured for their host-side expert cache (about
one expert in 25 takes close to a third of the lookups; NeutronStar README,
"SSD streaming optimizations").  Routing is computed by
the CPU oracle only.

Run from the repository root:  python tests/golden/calibrate_skew.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from synth import configs  # noqa: E402
from oracle import Oracle  # noqa: E402

TARGET, HOT = 0.30, 10


def hot_share(orc, cfg, logits, ranks, beta):
    bias, _ = synth.zipf_bias(cfg["seed"], configs.S_BIAS, cfg["E"], beta)
    idx, _ = orc.select(cfg, logits, bias)
    return float(np.isin(idx, np.where(ranks <= HOT)[0]).mean())


def main():
    cfg = configs.get("c5")
    orc = Oracle()
    x = configs.gen_x(cfg, stream=configs.S_CALIB)
    logits, _, _ = orc.route(cfg, x, configs.gen_router(cfg), None)
    ranks = configs.skew_ranks(cfg)
    lo, hi = 0.0, 1.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if hot_share(orc, cfg, logits, ranks, mid) < TARGET:
            lo = mid
        else:
            hi = mid
    beta = float(np.float32(hi))
    share = hot_share(orc, cfg, logits, ranks, beta)
    out = dict(beta=beta, hot_experts=HOT, target_share=TARGET, achieved_share=share,
               calibration_tokens=int(x.shape[0]), stream=configs.S_CALIB,
               note="written by tests/golden/calibrate_skew.py from the CPU oracle's routing")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "skew_beta.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
