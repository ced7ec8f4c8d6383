"""Pins of the backward oracle: every gradient is checked against central finite
differences of the loss L = <dy, y> + alpha L_bal + beta L_z, which the forward
oracle evaluates (its own pins live in the other oracle tests). The layers are tiny
float64 ones whose routing decisions sit far from any tie, so a perturbation of
1e-6 cannot change them and L is smooth there; plus special cases with a closed form."""
import numpy as np
import pytest

from oracle import moe_backward as B
from oracle import moe_oracle as O
from workloads.configs import Config
from workloads.gen import Workload

EPS = 1e-6


def _layer(seed, T=20, d=9, N=5, M=5, K=3, d_ff=7, d_ffs=6, bias=0.0, tok_bias=None):
    cfg = Config(name="bwd", T=T, d_model=d, n_experts=N, n_null=M, top_k=K, d_ff=d_ff,
                 d_ff_shared=d_ffs, dtype="f32", w_std=None)
    rng = np.random.default_rng(seed)
    s = 1.0 / np.sqrt(d)
    wl = Workload(cfg=cfg, x=rng.standard_normal((T, d)), w_router=rng.standard_normal((N + 1, d)),
                  null_bias=bias, null_bias_tok=tok_bias,
                  w_gate=rng.standard_normal((N, d_ff, d)) * s, w_up=rng.standard_normal((N, d_ff, d)) * s,
                  w_down=rng.standard_normal((N, d, d_ff)) / np.sqrt(d_ff))
    if d_ffs:
        wl.ws_gate = rng.standard_normal((d_ffs, d)) * s
        wl.ws_up = rng.standard_normal((d_ffs, d)) * s
        wl.ws_down = rng.standard_normal((d, d_ffs)) / np.sqrt(d_ffs)
    dy = rng.standard_normal((T, d))
    return wl, dy


def _min_gap(wl):
    """Smallest distance between two of a token's N + 1 distinct logits (the reals
    and the null): above it no decision of the selection can move. Tokens routed
    only to null by an infinite bias are skipped."""
    cfg = wl.cfg
    s = O.router_logits(wl.values("x"), wl.values("w_router"), wl.null_bias, wl.null_bias_tok)
    s = s[np.isfinite(s).all(axis=1)]
    if cfg.n_null == 0:
        s = s[:, :-1]
    diff = np.abs(s[:, :, None] - s[:, None, :])
    iu = np.triu_indices(s.shape[1], 1)
    return float(diff[:, iu[0], iu[1]].min()) if len(s) else np.inf


def _fd(wl, dy, name, direction, alpha, beta, index=None):
    """Central difference of L along ``direction`` in parameter ``name`` (or in
    the slice ``index`` of it)."""
    base = getattr(wl, name).copy()

    def at(sign):
        p = base.copy()
        if index is None:
            p += sign * EPS * direction
        else:
            p[index] += sign * EPS * direction
        setattr(wl, name, p)
        return B.layer_loss(wl, dy, alpha, beta)

    v = (at(+1) - at(-1)) / (2 * EPS)
    setattr(wl, name, base)
    return v


PARAMS = [("x", "dx"), ("w_router", "dw_router"), ("w_gate", "dw_gate"), ("w_up", "dw_up"),
          ("w_down", "dw_down"), ("ws_gate", "dws_gate"), ("ws_up", "dws_up"), ("ws_down", "dws_down")]


@pytest.mark.parametrize("alpha,beta", [(0.0, 0.0), (2e-2, 1e-3), (0.7, 0.3)])
@pytest.mark.parametrize("seed,M,K", [(3, 5, 3), (11, 0, 2), (5, 2, 4)])
def test_gradients_match_finite_differences(seed, M, K, alpha, beta):
    wl, dy = _layer(seed, M=M, K=K)
    assert _min_gap(wl) > 2e-4, "test layer too close to a routing tie"
    g = B.layer_backward(wl, dy, alpha, beta)
    rng = np.random.default_rng(seed + 100)
    for name, gname in PARAMS:
        d = rng.standard_normal(getattr(wl, name).shape)
        fd = _fd(wl, dy, name, d, alpha, beta)
        an = float((g[gname] * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)


def test_single_expert_rows_and_router_entries():
    """Element-wise differences for a few single entries, so a gradient that is
    right on average along a random direction but misplaced (transposed, shifted to
    another expert or token) fails."""
    wl, dy = _layer(7, M=5, K=3)
    assert _min_gap(wl) > 2e-4
    g = B.layer_backward(wl, dy, 0.3, 0.2)
    T, d = wl.x.shape
    N, d_ff = wl.w_gate.shape[:2]
    for name, gname, idx in [("x", "dx", (3, 4)), ("x", "dx", (T - 1, 0)),
                             ("w_router", "dw_router", (N, 2)), ("w_router", "dw_router", (1, d - 1)),
                             ("w_gate", "dw_gate", (2, d_ff - 1, 3)), ("w_up", "dw_up", (4, 0, d - 1)),
                             ("w_down", "dw_down", (0, d - 2, 5)), ("ws_down", "dws_down", (1, 2))]:
        fd = _fd(wl, dy, name, 1.0, 0.3, 0.2, index=idx)
        assert abs(fd - g[gname][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, g[gname][idx])


def test_null_row_gets_nothing_without_null_copies():
    """With M = 0 the null row never enters the forward (plain top-K), so its
    gradient is exactly zero."""
    wl, dy = _layer(11, M=0, K=2)
    g = B.layer_backward(wl, dy, 0.5, 0.5)
    assert (g["dw_router"][-1] == 0).all()


def test_single_choice_router_gradient_only_from_aux():
    """K = 1 and M = 0: each token's one weight is softmax over one logit, exactly 1,
    so without auxiliary losses the router receives no gradient at all."""
    wl, dy = _layer(4, M=0, K=1)
    g = B.layer_backward(wl, dy, 0.0, 0.0)
    assert (g["dw_router"] == 0).all()
    assert (g["ds"] == 0).all()


def test_null_routed_tokens_pass_only_router_and_shared_gradient():
    """A large per-token null bias routes every slot of those tokens to null copies:
    their dx holds only the router and shared-expert terms, and no expert weight
    gradient depends on their dy."""
    T = 20
    tok = np.zeros(T)
    tok[:6] = 1e3
    wl, dy = _layer(9, T=T, M=5, K=3, tok_bias=tok)
    g = B.layer_backward(wl, dy, 0.0, 0.0)
    assert (g["fwd"]["topk_idx"][:6] >= wl.cfg.n_experts).all()
    dy2 = dy.copy()
    dy2[:6] *= -3.0
    g2 = B.layer_backward(wl, dy2, 0.0, 0.0)
    for k in ("dw_gate", "dw_up", "dw_down"):
        np.testing.assert_array_equal(g[k], g2[k])
    # their only routed-path term is zero: dx = shared-expert dx (router ds is 0 with K reals = 0)
    assert (g["ds"][:6] == 0).all()
    sh = B._swiglu_backward(wl.x[:6], wl.ws_gate, wl.ws_up, wl.ws_down, dy[:6])["da"]
    np.testing.assert_allclose(g["dx"][:6], sh, rtol=1e-13, atol=1e-13)


def test_expert_gradients_equal_dense_per_expert_autodiff_free_form():
    """Per expert, dW_down = sum over its slots of (g dy) h^T: check against an
    explicit per-token loop over the dense routing matrix (no permutation)."""
    wl, dy = _layer(2, M=5, K=3)
    g = B.layer_backward(wl, dy, 0.0, 0.0)
    fwd = g["fwd"]
    x = wl.x
    N = wl.cfg.n_experts
    ref = np.zeros_like(wl.w_down)
    for t in range(x.shape[0]):
        for k in range(wl.cfg.top_k):
            e = fwd["topk_idx"][t, k]
            if e >= N:
                continue
            h = O.silu(wl.w_gate[e] @ x[t]) * (wl.w_up[e] @ x[t])
            ref[e] += np.outer(fwd["topk_w"][t, k] * dy[t], h)
    np.testing.assert_allclose(g["dw_down"], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed,M,K", [(3, 5, 3), (11, 0, 2), (5, 2, 4)])
def test_sampled_backward_equals_full(seed, M, K):
    """The sampled form (used at full sizes) returns exactly the full oracle's rows
    and expert matrices."""
    wl, dy = _layer(seed, T=30, M=M, K=K)
    g = B.layer_backward(wl, dy, 0.4, 0.3)
    s = O.router_logits(wl.values("x"), wl.values("w_router"), wl.null_bias, wl.null_bias_tok)
    tokens = [0, 7, 29, 13]
    experts = [0, 2, 4]
    sb = B.sampled_backward(wl, dy, 0.4, 0.3, s, tokens, experts)
    np.testing.assert_allclose(sb["dx"], g["dx"][tokens], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sb["ds"], g["ds"][tokens], rtol=1e-12, atol=1e-14)
    for name in ("dw_gate", "dw_up", "dw_down"):
        for e in experts:
            np.testing.assert_allclose(sb[name][e], g[name][e], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("M,K", [(5, 3), (2, 4)])
def test_infinite_null_bias_token_gradient(M, K):
    """Tokens whose null logit is +inf: their logit gradient is the weight term alone
    (the z-loss term has no finite value and is taken as 0, and the balance term of a
    saturated pool softmax is 0). Against a null bias of 1e4, where the pool softmax
    already is the limit in float64: with beta = 0 every gradient is the same; with
    beta > 0 the infinite tokens' rows equal the beta = 0 ones, every other row is
    unchanged, and the router gradient stays finite."""
    T = 24
    inf_tok = np.zeros(T)
    inf_tok[::5] = np.inf
    big_tok = np.where(np.isinf(inf_tok), 1e4, 0.0)
    wl_inf, dy = _layer(21, T=T, M=M, K=K, tok_bias=inf_tok)
    wl_big, _ = _layer(21, T=T, M=M, K=K, tok_bias=big_tok)
    rows = np.isinf(inf_tok)
    g_inf0 = B.layer_backward(wl_inf, dy, 0.4, 0.0)
    g_big0 = B.layer_backward(wl_big, dy, 0.4, 0.0)
    for k in ("dx", "dw_router", "ds", "dw_gate", "dw_up", "dw_down"):
        np.testing.assert_allclose(g_inf0[k], g_big0[k], rtol=1e-13, atol=1e-14, err_msg=k)
    g_inf = B.layer_backward(wl_inf, dy, 0.4, 0.3)
    g_big = B.layer_backward(wl_big, dy, 0.4, 0.3)
    assert np.isfinite(g_inf["dw_router"]).all() and np.isfinite(g_inf["dx"]).all()
    np.testing.assert_allclose(g_inf["ds"][rows], g_big0["ds"][rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(g_inf["ds"][~rows], g_big["ds"][~rows], rtol=1e-13, atol=1e-14)
    if K <= M:   # no real slot: the whole row is zero (up to the rounding of f - fbar)
        assert np.abs(g_inf["ds"][rows]).max() <= 1e-15
