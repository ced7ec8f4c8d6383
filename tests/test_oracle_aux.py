"""Pins of the oracle's load-balance / z-loss statistics: hand-derived golden
values, the uniform-logit closed forms, the M = 0 reduction and invariants."""
import json
import math
import os

import numpy as np

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ev(v):
    return float(eval(v, {"log": math.log})) if isinstance(v, str) else float(v)


def test_golden_aux_cases():
    for c in json.load(open(os.path.join(GOLDEN, "aux_examples.json")))["cases"]:
        N, M, K = c["N"], c["M"], c["K"]
        s = np.array([[*map(_ev, c["real"]), _ev(c["null"])]])
        topk, _, _ = O.route(s, N, M, K)
        assert topk[0].tolist() == c["topk"], c["name"]
        a = O.aux_stats(s, topk, N, M, K)
        np.testing.assert_allclose(a["P"], [_ev(p) for p in c["P"]], rtol=1e-14, err_msg=c["name"])
        np.testing.assert_array_equal(a["f"], c["f"])
        assert abs(a["L_bal"] - _ev(c["L_bal"])) < 1e-14, c["name"]
        assert abs(a["L_z"] - _ev(c["L_z"])) < 1e-13, c["name"]


def test_uniform_logits_closed_forms():
    for N, M, K, T in ((8, 8, 2, 50), (64, 192, 8, 20), (64, 64, 4, 10)):
        s = np.zeros((T, N + 1))                  # W_g = 0 and b = 0
        topk, _, n_real = O.route(s, N, M, K)
        a = O.aux_stats(s, topk, N, M, K)
        assert (n_real == 0).all()
        np.testing.assert_allclose(a["P"], 1.0 / (N + M), rtol=1e-14)
        assert abs(a["L_z"] - math.log(N + M) ** 2) < 1e-12
        f = np.zeros(N + M)
        f[N:N + K] = 1.0
        np.testing.assert_array_equal(a["f"], f)
        assert abs(a["L_bal"] - N * K / (N + M)) < 1e-12


def test_invariants_and_null_copy_symmetry():
    rng = np.random.default_rng(8)
    N, M, K, T = 16, 16, 4, 500
    s = rng.standard_normal((T, N + 1))
    topk, _, n_real = O.route(s, N, M, K)
    a = O.aux_stats(s, topk, N, M, K)
    assert abs(a["P"].sum() - 1.0) < 1e-12
    assert abs(a["f"].sum() - K) < 1e-12
    assert a["counts"].sum() == T * K
    assert abs(a["mean_r"] - n_real.mean()) < 1e-15
    # L_bal does not depend on which null copies a token's null slots name
    rolled = topk.copy()
    for t in range(T):
        r = n_real[t]
        rolled[t, r:] = N + (np.arange(K - r) + t) % M
    b = O.aux_stats(s, rolled, N, M, K)
    assert abs(a["L_bal"] - b["L_bal"]) < 1e-12


def test_m0_reduction_to_plain_aux():
    """With M = 0 the pool is the N reals: L_bal = N sum_i f_i P_i with the plain
    router softmax, the E = N case of the switch/GShard auxiliary loss."""
    rng = np.random.default_rng(10)
    N, K, T = 8, 2, 300
    s = rng.standard_normal((T, N + 1))
    s[:, N] = 1e9                                     # ignored when M = 0
    topk, _, _ = O.route(s, N, 0, K)
    a = O.aux_stats(s, topk, N, 0, K)
    p = np.exp(s[:, :N]) / np.exp(s[:, :N]).sum(axis=1, keepdims=True)
    np.testing.assert_allclose(a["P"], p.mean(axis=0), rtol=1e-13)
    assert abs(a["L_z"] - np.mean(np.log(np.exp(s[:, :N]).sum(axis=1)) ** 2)) < 1e-12


def test_infinite_null_bias_closed_forms():
    """Every token's null logit at +inf (an infinite per-token bias): the pool softmax
    is its limit, 1/M per null copy and 0 per real; with M >= K the K slots are null
    copies N .. N+K-1, so L_bal = N K / M; every lse is +inf, so L_z = +inf."""
    rng = np.random.default_rng(12)
    for N, M, K, T in ((8, 8, 2, 40), (64, 192, 8, 16), (6, 3, 3, 9)):
        s = rng.standard_normal((T, N + 1))
        s[:, N] = np.inf
        topk, w, n_real = O.route(s, N, M, K)
        a = O.aux_stats(s, topk, N, M, K)
        assert (n_real == 0).all() and (w == 0).all()
        assert (a["P"][:N] == 0).all()
        np.testing.assert_allclose(a["P"][N:], 1.0 / M, rtol=1e-14)
        f = np.zeros(N + M)
        f[N:N + K] = 1.0
        np.testing.assert_array_equal(a["f"], f)
        assert abs(a["L_bal"] - N * K / M) < 1e-12
        assert a["L_z"] == np.inf and (a["lse"] == np.inf).all()
        assert a["mean_r"] == 0.0


def test_infinite_null_bias_is_the_large_bias_limit():
    """Some tokens' null logit at +inf: P, f, counts and L_bal equal those of a null
    logit of 1e4 (where exp(s - 1e4) already underflows to 0 in float64, so the finite
    path computes the limit itself), the other tokens' lse are unchanged, and only
    the L_z of the infinite tokens differs (+inf instead of 1e4 + log M)."""
    rng = np.random.default_rng(13)
    for N, M, K in ((16, 16, 4), (8, 2, 4)):          # 0 < M < K forces K - M reals
        T = 60
        s = rng.standard_normal((T, N + 1))
        inf_rows = np.arange(T) % 7 == 3
        s_inf, s_big = s.copy(), s.copy()
        s_inf[inf_rows, N] = np.inf
        s_big[inf_rows, N] = 1e4
        t_inf, w_inf, r_inf = O.route(s_inf, N, M, K)
        t_big, w_big, r_big = O.route(s_big, N, M, K)
        np.testing.assert_array_equal(t_inf, t_big)
        np.testing.assert_array_equal(w_inf, w_big)
        assert (r_inf[inf_rows] == max(0, K - M)).all()
        a, b = O.aux_stats(s_inf, t_inf, N, M, K), O.aux_stats(s_big, t_big, N, M, K)
        for key in ("P", "f", "counts"):
            np.testing.assert_array_equal(a[key], b[key], err_msg=key)
        assert a["L_bal"] == b["L_bal"]
        np.testing.assert_array_equal(a["lse"][~inf_rows], b["lse"][~inf_rows])
        np.testing.assert_allclose(b["lse"][inf_rows], 1e4 + np.log(M), rtol=1e-15)
        assert a["L_z"] == np.inf and np.isfinite(b["L_z"])
