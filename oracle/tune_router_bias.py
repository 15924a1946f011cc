"""Find the router-bias strength beta of the skewed workloads with the oracle.

Writes nothing; prints the beta to record in ``workloads/configs.py``.  It
calls only the oracle (router logits, exact top-k, LIS) on the seeded inputs
of ``workloads``: the Switch-like layer targets LIS ~ 2 and the
DeepSeek-V2-Lite-like layer LIS ~ 4, the raw-routing values the
Replicate-and-Quantize page reports (its "Core claim").

    python -m oracle.tune_router_bias
"""
import sys

import numpy as np

import oracle
from workloads import CONFIGS
from workloads.gen import router_bias, _normal, TID_X, TID_WR, W_STD


def lis_for(cfg, x, w_r, beta):
    b = router_bias(cfg, beta)
    lg = oracle.router_logits(x, w_r, b)
    idx, _ = oracle.topk_gates(lg, cfg.k)
    return oracle.permute(idx, cfg.E)[4]


def tune(name, target, lo=0.0, hi=2.0, iters=12):
    cfg = CONFIGS[name]
    bf16 = cfg.dtype == "bf16"
    x = _normal(cfg.cfg_id, TID_X, 0, (cfg.T, cfg.d), 1.0, bf16)
    w_r = _normal(cfg.cfg_id, TID_WR, 0, (cfg.E, cfg.d), W_STD, bf16)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if lis_for(cfg, x, w_r, mid) < target:
            lo = mid
        else:
            hi = mid
    beta = round(0.5 * (lo + hi), 3)
    return beta, lis_for(cfg, x, w_r, beta)


if __name__ == "__main__":
    names = sys.argv[1:] or ["switch_bf16", "deepseek_v2_lite_bf16"]
    targets = {"switch_bf16": 2.0, "deepseek_v2_lite_bf16": 4.0}
    for n in names:
        beta, lis = tune(n, targets[n])
        print("%s: beta=%.3f LIS=%.6f" % (n, beta, lis))
