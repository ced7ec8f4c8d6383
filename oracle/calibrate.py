"""Calibrates the null-logit bias of the synthetic workloads and writes
``workloads/null_bias.json`` (test infrastructure; run by hand, output committed).

[Review] "expected active experts": with top-k_max routing at data sparsity rho
the expected number of chosen real experts per token is rho * k_max. An
untrained random router does not meet that on its own, so the scalar null bias b
is searched (bisection in float64 on the oracle's routing count) until the mean
number of chosen reals equals the target. For the modality-skewed workload two
biases (vision rows, text rows) are searched for target null fractions.

The count sum_t r_t(b) is a non-increasing step function of b; the script finds
the interval of b values where it equals the target exactly and stores its
midpoint rounded to float32, then re-checks the achieved mean with that value.

    python oracle/calibrate.py            # all calibrated workloads
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from oracle.moe_oracle import router_logits, select  # noqa: E402
from workloads import generate  # noqa: E402
from workloads.configs import CONFIGS, SWEEP, MATCHED_PAIR  # noqa: E402
from workloads.gen import BIAS_FILE, fingerprint  # noqa: E402


def real_count(real, null0, b, M, K):
    """r_t for every token at bias b (the closed form of the pool top-K:
    c = #{j : s_j > s_null}, r = min(K, max(c, K - M)))."""
    c = (real > (null0 + b)[:, None]).sum(axis=1)
    return np.minimum(K, np.maximum(c, K - M)) if M else np.full(len(real), K)


def solve_bias(real, null0, M, K, target_total):
    f = lambda b: int(real_count(real, null0, b, M, K).sum())  # noqa: E731
    lo, hi = -64.0, 64.0
    assert f(lo) >= target_total >= f(hi)

    def first_below_or_equal(level, strict):
        a, z = lo, hi
        for _ in range(200):
            mid = 0.5 * (a + z)
            ok = f(mid) < level if strict else f(mid) <= level
            if ok:
                z = mid
            else:
                a = mid
        return z

    b1 = first_below_or_equal(target_total, strict=False)   # start of {f <= target}
    b2 = first_below_or_equal(target_total, strict=True)    # start of {f <  target}
    return 0.5 * (b1 + b2), f(0.5 * (b1 + b2))


def calibrate(cfg):
    wl = generate(cfg, experts=False, bias=False)
    N, M, K, T = cfg.n_experts, cfg.n_null, cfg.top_k, cfg.T
    s = router_logits(wl.values("x"), wl.values("w_router"))
    real, null0 = s[:, :N], s[:, N]
    ent = {"x_fingerprint": fingerprint(wl.x), "router_fingerprint": fingerprint(wl.w_router)}
    if cfg.bias_mode == "calibrated":
        b, _ = solve_bias(real, null0, M, K, int(round(cfg.target_mean_r * T)))
        b = float(np.float32(b))
        s2 = s.copy()
        s2[:, N] += b
        _, r = select(s2, N, M, K)
        ent.update(null_bias=b, target_mean_r=cfg.target_mean_r, achieved_mean_r=float(r.mean()))
    elif cfg.bias_mode == "per_class":
        vT = int(round(cfg.vision_frac * T))
        out = {}
        for name, rows, frac in (("vision", slice(0, vT), cfg.class_null_frac[0]),
                                 ("text", slice(vT, T), cfg.class_null_frac[1])):
            n = rows.stop - rows.start
            b, _ = solve_bias(real[rows], null0[rows], M, K, int(round((1 - frac) * K * n)))
            out[name] = float(np.float32(b))
        btok = np.empty(T)
        btok[:vT], btok[vT:] = out["vision"], out["text"]
        s2 = s.copy()
        s2[:, N] += btok
        _, r = select(s2, N, M, K)
        ent.update(null_bias_vision=out["vision"], null_bias_text=out["text"],
                   target_null_frac=list(cfg.class_null_frac),
                   achieved_null_frac=[float(1 - r[:vT].mean() / K), float(1 - r[vT:].mean() / K)],
                   achieved_mean_r=float(r.mean()))
    return ent


def main():
    table = {}
    for tab in (CONFIGS, SWEEP, MATCHED_PAIR):
        for name, cfg in tab.items():
            if cfg.bias_mode != "zero":
                table[name] = calibrate(cfg)
                print(name, table[name], flush=True)
    with open(BIAS_FILE, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
        fh.write("\n")


if __name__ == "__main__":
    main()
