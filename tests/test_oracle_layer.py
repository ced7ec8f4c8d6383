"""Pins of the oracle's expert FFN, combine and whole layer: a closed form of
SwiGLU, the dense routing-matrix form, solution-space preservation (bitwise),
the null-routed token, and the expected-real-count results."""
import math

import numpy as np

from oracle import moe_oracle as O
from oracle.calibrate import solve_bias
from workloads import generate, get_config
from workloads.configs import C0, Config


def test_silu_values():
    z = np.array([0.0, 1.0, -1.0, 20.0, -40.0, 2.5])
    ref = [v / (1.0 + math.exp(-v)) for v in z]
    np.testing.assert_allclose(O.silu(z), ref, rtol=1e-15, atol=0)
    assert O.silu(np.array([-1000.0]))[0] == 0.0


def test_swiglu_diagonal_closed_form():
    # gate = c I, up = I, down = I  ->  y_j = silu(c x_j) * x_j
    rng = np.random.default_rng(0)
    d, c = 12, 0.7
    a = rng.standard_normal((5, d))
    y = O.swiglu_ffn(a, c * np.eye(d), np.eye(d), np.eye(d))
    ref = [[(c * v) / (1 + math.exp(-c * v)) * v for v in row] for row in a]
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-300)


def test_swiglu_zero_gate_is_zero():
    a = np.random.default_rng(1).standard_normal((4, 8))
    assert (O.swiglu_ffn(a, np.zeros((6, 8)), np.ones((6, 8)), np.ones((8, 6))) == 0).all()


def _small_cfg(**kw):
    base = dict(name="small", T=96, d_model=32, n_experts=6, n_null=6, top_k=3, d_ff=24,
                d_ff_shared=16, dtype="f32", w_std=None)
    base.update(kw)
    return Config(**base)


def test_dense_form_equals_permuted_path():
    for cfg in (_small_cfg(), _small_cfg(n_null=0, top_k=2), _small_cfg(d_ff_shared=0, n_null=2, top_k=4), C0):
        wl = generate(cfg)
        out = O.layer_forward(wl)
        yd, topk, w = O.layer_dense(wl)
        np.testing.assert_array_equal(topk, out["topk_idx"])
        scale = np.sqrt((yd ** 2).mean())
        assert np.abs(out["y"] - yd).max() <= 1e-12 * scale


def test_dense_form_sampled_rows():
    wl = generate(_small_cfg())
    yd, _, _ = O.layer_dense(wl)
    rows = np.array([0, 5, 17, 95])
    ys, _, _ = O.layer_dense(wl, tokens=rows)
    np.testing.assert_allclose(ys, yd[rows], rtol=1e-13, atol=1e-15)


def test_solution_space_preservation_bitwise():
    """K=4 with exactly two reals above the null equals K=2 without nulls
    (the K^4_{0.5} vs K^2_{1.0} argument), bit for bit."""
    for M in (2, 4, 64):
        cfg = _small_cfg(top_k=4, n_null=M, n_experts=8)
        wl = generate(cfg)
        x, wr = wl.values("x"), wl.values("w_router")
        s = O.router_logits(x, wr)
        srt = np.sort(s[:, :8], axis=1)[:, ::-1]
        btok = 0.5 * (srt[:, 1] + srt[:, 2]) - s[:, 8]       # null between the 2nd and 3rd real
        wl.null_bias_tok = btok
        out4 = O.layer_forward(wl)
        assert (out4["n_real"] == 2).all()
        wl2 = generate(_small_cfg(top_k=2, n_null=0, n_experts=8))
        out2 = O.layer_forward(wl2)
        np.testing.assert_array_equal(out4["y"], out2["y"])
        np.testing.assert_array_equal(out4["topk_w"][:, :2], out2["topk_w"])


def test_null_routed_token_gives_shared_output_only():
    for fs in (16, 0):
        cfg = _small_cfg(d_ff_shared=fs)
        wl = generate(cfg)
        btok = np.zeros(cfg.T)
        btok[::3] = np.inf
        wl.null_bias_tok = btok
        out = O.layer_forward(wl)
        nul = btok == np.inf
        assert (out["n_real"][nul] == 0).all()
        ref = out["y_shared"][nul] if fs else np.zeros((nul.sum(), cfg.d_model))
        np.testing.assert_array_equal(out["y"][nul], ref)


def test_expected_real_count_closed_form_iid():
    """iid continuous logits, zero bias, M >= K: the null's rank among the N+1
    values is uniform, so E[r] = sum_{c=0}^{N} min(K, c) / (N + 1); 5/3 for N=8, K=2."""
    rng = np.random.default_rng(21)
    for N, M, K in ((8, 8, 2), (64, 64, 4)):
        T = 60000
        s = rng.standard_normal((T, N + 1))
        _, r = O.select(s, N, M, K)
        expect = sum(min(K, c) for c in range(N + 1)) / (N + 1)
        sd = np.sqrt(np.mean([(min(K, c) - expect) ** 2 for c in range(N + 1)]) / T)
        assert abs(r.mean() - expect) < 5 * sd
    assert abs(sum(min(2, c) for c in range(9)) / 9 - 5 / 3) < 1e-15


def test_calibrated_bias_reaches_rho_k():
    """E[K^{k_max}_rho] = rho * k_max: top-8 at rho = 0.5 expects 4 real experts."""
    rng = np.random.default_rng(4)
    N, M, K, T = 64, 64, 8, 20000
    s = rng.standard_normal((T, N + 1)) * 0.8
    b, total = solve_bias(s[:, :N], s[:, N], M, K, int(0.5 * K * T))
    s[:, N] += b
    _, r = O.select(s, N, M, K)
    assert r.sum() == total == 4 * T


def test_stored_calibration_reproduces_targets():
    from workloads.gen import fingerprint, load_bias_table
    table = load_bias_table()
    for name in ("qwen3_0p6b_rho0p5", "qwen3_1p7b_rho0p25", "modality_skew_rho0p5"):
        cfg = get_config(name)
        wl = generate(cfg, experts=False)
        ent = table[name]
        assert fingerprint(wl.x) == ent["x_fingerprint"]
        assert fingerprint(wl.w_router) == ent["router_fingerprint"]
        s = O.router_logits(wl.values("x"), wl.values("w_router"), wl.null_bias, wl.null_bias_tok)
        _, r = O.select(s, cfg.n_experts, cfg.n_null, cfg.top_k)
        if cfg.bias_mode == "calibrated":
            assert abs(r.mean() - cfg.target_mean_r) <= 0.05
        else:
            vT = int(cfg.vision_frac * cfg.T)
            assert abs((1 - r[:vT].mean() / cfg.top_k) - 0.70) <= 0.01
            assert abs((1 - r[vT:].mean() / cfg.top_k) - 0.30) <= 0.01


# ---------------------------------------------------------------- copy / constant null slots
def _all_null(kind):
    """Every slot null: a large null bias with M >= K."""
    wl = generate(_small_cfg(null_kind=kind, n_null=6, top_k=3))
    wl.null_bias = 1.0e4
    return wl


def test_copy_all_null_gives_token_plus_shared():
    """All K slots null with copy experts: K equal weights 1/K, so y = x + E_shared(x)."""
    wl = _all_null("copy")
    out = O.layer_forward(wl)
    assert (out["n_real"] == 0).all()
    np.testing.assert_allclose(out["topk_w"], 1.0 / 3.0, rtol=1e-15)
    x = wl.values("x")
    ref = x + O.swiglu_ffn(x, wl.ws_gate, wl.ws_up, wl.ws_down)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-13, atol=1e-13)


def test_copy_infinite_null_bias_is_the_large_bias_limit():
    """A null logit at +inf with copy experts: the weights are the limit of a large
    finite null bias (every chosen null copy equally, the reals 0), so with M >= K
    y = x + E_shared(x) exactly as with the 1e4 bias; with 0 < M < K the K - M forced
    reals get weight 0 and the M null copies 1/M each."""
    for M, K in ((6, 3), (2, 4)):
        wl = generate(_small_cfg(null_kind="copy", n_null=M, top_k=K))
        wl.null_bias = 1.0e4
        big = O.layer_forward(wl)
        wl.null_bias = np.inf
        inf = O.layer_forward(wl)
        np.testing.assert_array_equal(inf["topk_idx"], big["topk_idx"])
        np.testing.assert_array_equal(inf["topk_w"], big["topk_w"])
        np.testing.assert_array_equal(inf["y"], big["y"])
        w = np.where(inf["topk_idx"] >= wl.cfg.n_experts, 1.0 / min(M, K), 0.0)
        np.testing.assert_allclose(inf["topk_w"], w, rtol=1e-15)


def test_constant_all_null_gives_vector_plus_shared():
    wl = _all_null("constant")
    out = O.layer_forward(wl)
    x = wl.values("x")
    ref = wl.values("null_value")[None, :] + O.swiglu_ffn(x, wl.ws_gate, wl.ws_up, wl.ws_down)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-13, atol=1e-13)


def test_zero_kind_all_null_gives_shared_only():
    wl = _all_null("zero")
    out = O.layer_forward(wl)
    assert (out["topk_w"] == 0).all()
    x = wl.values("x")
    np.testing.assert_allclose(out["y"], O.swiglu_ffn(x, wl.ws_gate, wl.ws_up, wl.ws_down), rtol=1e-13)


def test_copy_equal_logits_is_one_minus_rho_x_plus_rho_mean():
    """All logits equal (router weights 0, null bias 0), M < K: the null logit wins
    every tie, so each token takes r = K - M reals (experts 0..r-1 by the index
    order) and M null copies, all with weight 1/K. Copy experts then give
    y = (1 - rho) x + rho * mean_{e < r} E_e(x) + E_shared(x) with rho = r / K,
    the table's (1 - rho) x + rho y_dense, exactly."""
    K, M = 4, 1
    wl = generate(_small_cfg(null_kind="copy", n_null=M, top_k=K, n_experts=6))
    wl.w_router = np.zeros_like(wl.w_router)
    wl.null_bias = 0.0
    out = O.layer_forward(wl)
    r = K - M
    assert (out["n_real"] == r).all()
    np.testing.assert_allclose(out["topk_w"], 1.0 / K, rtol=1e-15)
    x = wl.values("x")
    rho = r / K
    dense = sum(O.swiglu_ffn(x, wl.w_gate[e], wl.w_up[e], wl.w_down[e]) for e in range(r)) / r
    ref = (1 - rho) * x + rho * dense + O.swiglu_ffn(x, wl.ws_gate, wl.ws_up, wl.ws_down)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)
    # the dense form agrees
    yd, _, _ = O.layer_dense(wl)
    np.testing.assert_allclose(yd, out["y"], rtol=1e-12, atol=1e-12)


def test_chosen_weights_are_pool_softmax_over_the_chosen():
    """Copy-variant weights: softmax over the K chosen pool entries (null slots at
    the null logit), checked on a hand-made row."""
    s = np.array([[2.0, 0.5, 1.0, 1.5]])          # N = 3 reals, null logit 1.5
    topk, n_real = O.select(s, 3, 2, 3)           # reals 2.0 (e0) beat null; then null, null
    assert n_real[0] == 1 and list(topk[0]) == [0, 3, 4]
    w = O.chosen_weights(s, topk, 3)[0]
    e = np.exp(np.array([2.0, 1.5, 1.5]) - 2.0)
    np.testing.assert_allclose(w, e / e.sum(), rtol=1e-15)
