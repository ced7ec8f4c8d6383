"""Pins of the oracle's routing (selection, weights, permutation) to things
other than itself: hand-derived golden cases, brute-force enumeration, the
M = 0 special case (plain top-K), closed forms and invariants."""
import json
import math
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ev(expr):
    return float(eval(expr, {"sigma": lambda z: 1.0 / (1.0 + math.exp(-z)), "log": math.log}))


def _logits(real, null):
    return np.array([[*map(_ev_num, real), _ev_num(null)]], dtype=np.float64)


def _ev_num(v):
    return _ev(v) if isinstance(v, str) else float(v)


def test_golden_routing_cases():
    cases = json.load(open(os.path.join(GOLDEN, "routing_examples.json")))["cases"]
    for c in cases:
        s = _logits(c["real"], c["null"])
        topk, w, n_real = O.route(s, c["N"], c["M"], c["K"])
        assert topk[0].tolist() == c["topk"], c["name"]
        assert int(n_real[0]) == c["n_real"], c["name"]
        np.testing.assert_allclose(w[0], [_ev(e) for e in c["weights"]], rtol=1e-15, atol=0, err_msg=c["name"])


def _random_pool(rng):
    N = int(rng.integers(1, 7))
    M = int(rng.integers(0, 5))
    K = int(rng.integers(1, (N if M == 0 else min(N + M, 5)) + 1))
    s = rng.integers(-2, 3, size=(1, N + 1)).astype(np.float64)   # integer logits: ties everywhere
    return s, N, M, K


def test_select_matches_brute_force_on_tie_heavy_pools():
    rng = np.random.default_rng(1234)
    for _ in range(1500):
        s, N, M, K = _random_pool(rng)
        topk, n_real = O.select(s, N, M, K)
        if M == 0:
            reals, n_null = brute.select_token(s[0, :N], 0.0, 0, K)
        else:
            reals, n_null = brute.select_token(s[0, :N], s[0, N], M, K)
        assert topk[0].tolist() == reals + [N + c for c in range(n_null)], (s, N, M, K)
        assert n_real[0] == len(reals)


def test_select_m0_is_plain_topk():
    rng = np.random.default_rng(7)
    s = rng.integers(-3, 4, size=(400, 9)).astype(np.float64)
    N, K = 8, 3
    topk, n_real = O.select(s, N, 0, K)
    ref = np.argsort(-s[:, :N], axis=1, kind="stable")[:, :K]   # textbook stable top-K
    assert (topk == ref).all()
    assert (n_real == K).all()


def test_select_threshold_closed_form_and_invariants():
    rng = np.random.default_rng(3)
    for N, M, K in ((8, 8, 2), (64, 64, 4), (64, 192, 8), (16, 3, 6), (5, 1, 5)):
        s = rng.standard_normal((300, N + 1))
        s[:50, N] = s[:50, 0]            # exact real/null ties
        topk, n_real = O.select(s, N, M, K)
        c = (s[:, :N] > s[:, N:N + 1]).sum(axis=1)
        assert (n_real == np.minimum(K, np.maximum(c, K - M))).all()
        for t in range(len(s)):
            r = n_real[t]
            reals = topk[t, :r]
            assert (reals < N).all() and (topk[t, r:] >= N).all()
            assert topk[t, r:].tolist() == list(range(N, N + K - r))
            if M >= K:   # every chosen real strictly beats the null
                assert (s[t, reals] > s[t, N]).all()
            unchosen = np.setdiff1d(np.arange(N), reals)
            if r and len(unchosen):
                assert s[t, reals].min() >= s[t, unchosen].max()


def test_weights_three_formulations_agree():
    rng = np.random.default_rng(5)
    for N, M, K in ((8, 8, 2), (64, 64, 4), (16, 4, 6)):
        s = rng.standard_normal((200, N + 1)) * 2
        topk, w, n_real = O.route(s, N, M, K)
        pool = np.concatenate([s[:, :N], np.repeat(s[:, N:N + 1], M, axis=1)], axis=1)
        p = np.exp(pool - pool.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        for t in range(len(s)):
            real = topk[t] < N
            if not real.any():
                assert (w[t] == 0).all()
                continue
            # (b) pool softmax restricted to the chosen reals, rescaled to sum 1
            pb = np.where(real, p[t, topk[t]], 0.0)
            pb /= pb.sum()
            # (c) MoE++ order: softmax over the K chosen pool logits, zero the null slots, renormalise
            g = np.exp(pool[t, topk[t]] - pool[t, topk[t]].max())
            g /= g.sum()
            g = np.where(real, g, 0.0)
            g /= g.sum()
            np.testing.assert_allclose(w[t], pb, rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(w[t], g, rtol=1e-12, atol=1e-15)
            assert abs(w[t].sum() - 1.0) < 1e-14


def test_k1_weight_is_one():
    s = np.random.default_rng(9).standard_normal((100, 9))
    topk, w, n_real = O.route(s, 8, 0, 1)
    assert (w[:, 0] == 1.0).all()


def test_permute_matches_counting_pass():
    rng = np.random.default_rng(11)
    for _ in range(60):
        N, M = int(rng.integers(1, 9)), int(rng.integers(0, 6))
        K = int(rng.integers(1, (N if M == 0 else N + M) + 1))
        T = int(rng.integers(0, 40))
        s = rng.integers(-2, 3, size=(T, N + 1)).astype(np.float64)
        topk, _ = O.select(s, N, M, K) if T else (np.zeros((0, K), np.int32), None)
        counts, offsets, perm_token, slot_pos = O.permute(topk, N)
        bc, bo, bp, bs = brute.counting_permute(topk.tolist(), N)
        assert counts.tolist() == bc and offsets.tolist() == bo
        assert perm_token.tolist() == bp and slot_pos.tolist() == bs


def test_permute_invariants():
    rng = np.random.default_rng(12)
    N, M, K, T = 64, 64, 4, 1000
    s = rng.standard_normal((T, N + 1))
    topk, n_real = O.select(s, N, M, K)
    counts, offsets, perm_token, slot_pos = O.permute(topk, N)
    R = int(offsets[-1])
    assert R == int(n_real.sum()) == int(counts.sum())
    assert (np.diff(offsets) >= 0).all()
    flat = slot_pos.reshape(-1)
    assert sorted(flat[flat >= 0].tolist()) == list(range(R))
    for t in range(T):
        for k in range(K):
            p = slot_pos[t, k]
            assert (p < 0) == (topk[t, k] >= N)
            if p >= 0:
                assert perm_token[p] == t
                assert offsets[topk[t, k]] <= p < offsets[topk[t, k] + 1]


def test_router_logits_closed_form():
    rng = np.random.default_rng(2)
    d, N = 16, 5
    w = rng.standard_normal((N + 1, d))
    x = np.eye(d)                                  # token t = unit vector e_t
    btok = rng.standard_normal(d)
    s = O.router_logits(x, w, 0.5, btok)
    np.testing.assert_array_equal(s[:, :N], w[:N].T)
    np.testing.assert_allclose(s[:, N], w[N] + 0.5 + btok, rtol=0, atol=1e-15)


def test_decisive_gap_examples():
    s = np.array([[3.0, 1.0, 2.0, 1.5]])           # N=3, null 1.5; M=2, K=2 -> chosen 0 and 2
    assert O.decisive_gap(s, 3, 2, 2)[0] == pytest.approx(0.5)
    s = np.array([[3.0, 1.5, 2.0, 1.5]])           # a real tied with the null
    assert O.decisive_gap(s, 3, 2, 3)[0] == 0.0


def test_decisive_gap_with_an_infinite_null_logit():
    """A +inf null logit: K null copies chosen and further copies left over, all the same
    infinity; no finite logit change moves the choice (no inf - inf = NaN)."""
    import warnings
    s = np.array([[3.0, 1.0, 2.0, np.inf], [3.0, 1.0, 2.0, 1.5]])
    with warnings.catch_warnings():
        warnings.simplefilter("error")
        g = O.decisive_gap(s, 3, 4, 2)
    assert g[0] == np.inf and g[1] == pytest.approx(0.5)   # chosen 3, 2 against the null 1.5
