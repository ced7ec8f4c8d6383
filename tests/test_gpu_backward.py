"""GPU parity of moe_layer_backward against the float64 backward oracle.

The oracle routes with the GPU's float32 logits (the routing decision is held fixed
by both sides), so every gradient is compared element by element:
  * dx per token row, max |err| <= 2e-2 RMS(row) (the layer-output rule, TOL_BF16);
  * every weight gradient per expert matrix and the router gradient:
    RMS(err) <= TOL_RMS * RMS(ref) and max |err| <= TOL_MAX * RMS(ref); an expert
    that receives no token gets exactly zero; the router's null row exactly zero
    when M = 0.
Tolerances: the GPU rounds dY = g dy, h and [dg | du] to bf16 (the inputs of its
MFMA contractions) and accumulates in float32. A bf16 rounding (8 significant bits)
moves a value by at most 2^-8 relative, RMS 2^-8 / sqrt(3) = 0.23%; a gradient term
carries one or two of them, so the RMS error of a summed gradient is 0.2-0.3% of its
RMS (measured 0.15-0.32%): TOL_RMS = 1e-2 leaves a factor 3 and still fails any
systematic error (a lost term, a wrong scale or index). The largest single error is
a weaker statistic: a weight-gradient entry is a sum of products of two heavy-tailed
values, and for an expert with a handful of tokens it does not average at all, so one
term's rounding sets it (measured up to 5.6% of the RMS, for an expert with 3 rows):
TOL_MAX = 1e-1 bounds it."""
import numpy as np
import pytest
import torch

from oracle import moe_backward as B
from token_choice_routing_amd.layer import MoeLayer, to_device, to_host
from workloads import bf16_round, generate
from workloads.configs import Config
from tests.gpu_util import TOL_BF16, assert_rows_close, say, vals

pytestmark = pytest.mark.gpu

TOL_RMS = 1e-2
TOL_MAX = 1e-1

CASES = {
    # M >= K with a shared expert; d_ff a multiple of 32, not of 64
    "nullpool_shared": dict(T=200, d_model=128, n_experts=8, n_null=8, top_k=4, d_ff=96, d_ff_shared=64),
    # plain top-K (M = 0), no shared expert, K tails (72 = 64 + 8)
    "topk_m0": dict(T=150, d_model=64, n_experts=6, n_null=0, top_k=2, d_ff=72, d_ff_shared=0),
    # more tokens: several row tiles per expert, wgrad K over several 64-wide tiles
    "wide": dict(T=1024, d_model=256, n_experts=16, n_null=16, top_k=4, d_ff=192, d_ff_shared=128),
    # 0 < M < K and an expert count that leaves some experts empty
    "few_nulls": dict(T=40, d_model=64, n_experts=32, n_null=2, top_k=4, d_ff=64, d_ff_shared=32),
    # d_model, d_ff and d_ff_shared multiples of 8 but not of 64 or 32: ragged K tiles
    # in every contraction and ragged 64 x 64 tiles in every transpose
    "ragged_dims": dict(T=333, d_model=200, n_experts=12, n_null=4, top_k=3, d_ff=104, d_ff_shared=40),
    # 512 output rows per expert: the weight gradients take the 256 x 256 ping-pong
    # tiles (segments of ~150 rows: ragged K ranges of a few 32-wide K tiles)
    "pp_wgrad": dict(T=640, d_model=512, n_experts=8, n_null=8, top_k=2, d_ff=512, d_ff_shared=512),
    # 1024 rows per expert: the data gradients read the weights K-major on the 256 x 256
    # tiles (W_d for U; W_g then W_u, split at K = d_ff = 160, for da), partial column tiles
    "kmajor": dict(T=2048, d_model=256, n_experts=4, n_null=4, top_k=2, d_ff=160, d_ff_shared=96),
    # the same without a shared expert, d_model = 96 (K of U three K tiles, a partial
    # column tile of da)
    "kmajor_narrow": dict(T=1536, d_model=96, n_experts=2, n_null=2, top_k=2, d_ff=64, d_ff_shared=0),
    # weight gradients with both operands K-major (at least 512 output rows per group) on
    # ragged tiles: 520 and 544 rows (partial row and column tiles), segments of ~300 rows
    "kmajor_wgrad_ragged": dict(T=600, d_model=520, n_experts=4, n_null=4, top_k=2, d_ff=544, d_ff_shared=520),
}


def _run(case, alpha, beta, seed=0):
    cfg = Config(name=f"bwd_{case}", dtype="bf16", w_std=None, seed=seed, **CASES[case])
    wl = generate(cfg)
    say(f"  backward {case} T={cfg.T} d={cfg.d_model} N={cfg.n_experts} M={cfg.n_null} K={cfg.top_k} "
        f"alpha={alpha} beta={beta}")
    layer = MoeLayer(wl)
    layer.forward()
    out = layer.results()
    rng = np.random.default_rng(seed + 7)
    dy_bits = bf16_round(rng.standard_normal((cfg.T, cfg.d_model)).astype(np.float32))
    dy = to_device(dy_bits)
    g = layer.backward(dy, alpha, beta)
    torch.cuda.synchronize()
    got = {k: (to_host(v) if v is not None else None) for k, v in g.items()}
    ref = B.layer_backward(wl, vals(dy_bits), alpha, beta, logits=out["logits"].astype(np.float64))
    return cfg, layer, dy, got, ref


def _ratios(got, ref):
    """(RMS(err), max|err|) relative to RMS(ref)."""
    err = np.asarray(got, np.float64) - ref
    scale = max(float(np.sqrt((ref * ref).mean())), 1e-300)
    return float(np.sqrt((err * err).mean())) / scale, float(np.abs(err).max()) / scale


def _check_matrix(got, ref, what):
    r_rms, r_max = _ratios(got, ref)
    assert r_rms <= TOL_RMS and r_max <= TOL_MAX, f"{what}: RMS ratio {r_rms:.3e}, max ratio {r_max:.3e}"
    return r_rms, r_max


def _check(cfg, got, ref):
    N = cfg.n_experts
    assert_rows_close(got["dx"], ref["dx"], TOL_BF16, "dx")
    r = _check_matrix(got["dw_router"], ref["dw_router"], "dw_router")
    say(f"  dw_router: RMS(err)/RMS = {r[0]:.3e}, max|err|/RMS = {r[1]:.3e}")
    if cfg.n_null == 0:
        assert (got["dw_router"][N] == 0).all()
    counts = np.diff(ref["fwd"]["offsets"])
    for name in ("dw_gate", "dw_up", "dw_down"):
        worst = (0.0, 0.0)
        for e in range(N):
            if counts[e] == 0:
                assert (got[name][e] == 0).all(), f"{name}[{e}]: expert without tokens"
                continue
            r = _check_matrix(got[name][e], ref[name][e], f"{name}[{e}]")
            worst = (max(worst[0], r[0]), max(worst[1], r[1]))
        say(f"  {name}: worst per-expert RMS(err)/RMS = {worst[0]:.3e}, max|err|/RMS = {worst[1]:.3e} "
            f"over {int((counts > 0).sum())} experts")
    if cfg.d_ff_shared:
        for name in ("dws_gate", "dws_up", "dws_down"):
            r = _check_matrix(got[name], ref[name], name)
            say(f"  {name}: RMS(err)/RMS = {r[0]:.3e}, max|err|/RMS = {r[1]:.3e}")


@pytest.mark.parametrize("case", list(CASES))
def test_backward_matches_oracle(case):
    cfg, _, _, got, ref = _run(case, 2e-2, 1e-3)
    _check(cfg, got, ref)


def test_backward_strong_aux_terms():
    """Large loss weights make the router gradient dominated by L_bal and L_z."""
    cfg, _, _, got, ref = _run("nullpool_shared", 3.0, 0.5, seed=3)
    _check(cfg, got, ref)


def test_backward_deterministic():
    cfg, layer, dy, got, _ = _run("wide", 2e-2, 1e-3, seed=5)
    g2 = layer.backward(dy, 2e-2, 1e-3)
    torch.cuda.synchronize()
    for k, v in g2.items():
        if v is not None:
            np.testing.assert_array_equal(to_host(v), got[k], err_msg=k)


@pytest.mark.parametrize("name", ["qwen3_0p6b_rho1", "qwen3_1p7b_rho0p25"])
def test_backward_full_size_sampled(name):
    """Benchmark shapes at full size: dx of sampled tokens and the weight gradients of
    sampled experts (the first, a middle and the last expert that received rows)
    against the sampled oracle, routed with the GPU's logits; the router gradient
    and the shared expert's through the RMS criterion on sampled rows of dW."""
    from workloads import CONFIGS
    cfg = CONFIGS[name]
    say(f"  backward full size {name}")
    wl = generate(cfg)
    layer = MoeLayer(wl)
    layer.forward()
    out = layer.results()
    rng = np.random.default_rng(11)
    dy_bits = bf16_round(rng.standard_normal((cfg.T, cfg.d_model)).astype(np.float32))
    alpha, beta = 2e-2, 1e-3
    g = layer.backward(to_device(dy_bits), alpha, beta)
    torch.cuda.synchronize()
    counts = np.diff(out["offsets"])
    nonempty = np.nonzero(counts)[0]
    experts = sorted({int(nonempty[0]), int(nonempty[len(nonempty) // 2]), int(nonempty[-1])})
    tokens = np.sort(rng.choice(cfg.T, size=24, replace=False))
    ref = B.sampled_backward(wl, vals(dy_bits), alpha, beta, out["logits"].astype(np.float64), tokens, experts)
    assert_rows_close(to_host(g["dx"])[tokens], ref["dx"], TOL_BF16, f"dx sampled {name}")
    for nm in ("dw_gate", "dw_up", "dw_down"):
        full = to_host(g[nm])
        for e in experts:
            r = _check_matrix(full[e], ref[nm][e], f"{nm}[{e}]")
            say(f"  {nm}[{e}] ({counts[e]} rows): RMS(err)/RMS = {r[0]:.3e}, max|err|/RMS = {r[1]:.3e}")
        for e in np.nonzero(counts == 0)[0]:
            assert (full[e] == 0).all()


def _run_wl(wl, alpha, beta, seed=0):
    """_run for a workload prepared by the caller."""
    cfg = wl.cfg
    say(f"  backward {cfg.name} T={cfg.T} N={cfg.n_experts} M={cfg.n_null} K={cfg.top_k} alpha={alpha} beta={beta}")
    layer = MoeLayer(wl)
    layer.forward()
    out = layer.results()
    rng = np.random.default_rng(seed + 7)
    dy_bits = bf16_round(rng.standard_normal((cfg.T, cfg.d_model)).astype(np.float32))
    g = layer.backward(to_device(dy_bits), alpha, beta)
    torch.cuda.synchronize()
    got = {k: (to_host(v) if v is not None else None) for k, v in g.items()}
    ref = B.layer_backward(wl, vals(dy_bits), alpha, beta, logits=out["logits"].astype(np.float64))
    return got, ref


@pytest.mark.parametrize("shared", [64, 0])
def test_backward_every_token_null(shared):
    """A large per-token null bias sends every slot to a null copy (no routed rows):
    every expert gradient is exactly zero, and dx and the router gradient hold only
    the auxiliary-loss and shared-expert terms."""
    cfg = Config(name="bwd_all_null", dtype="bf16", w_std=None, seed=2,
                 **dict(CASES["nullpool_shared"], d_ff_shared=shared))
    wl = generate(cfg)
    wl.null_bias_tok = np.full(cfg.T, 1e3, dtype=np.float32)
    got, ref = _run_wl(wl, 2e-2, 1e-3)
    assert ref["fwd"]["offsets"][-1] == 0
    _check(cfg, got, ref)


@pytest.mark.parametrize("case", ["nullpool_shared", "few_nulls"])
def test_backward_infinite_null_bias(case):
    """Tokens whose per-token null bias is +inf (a valid input: with M >= K every slot
    null, with 0 < M < K the K - M forced reals): their lse is +inf, the z-loss term of
    their logit gradient is taken as 0 and the balance term is 0 by itself, so the
    router gradient stays finite and matches the oracle's limit."""
    cfg = Config(name=f"bwd_inf_{case}", dtype="bf16", w_std=None, seed=6, **CASES[case])
    wl = generate(cfg)
    btok = np.zeros(cfg.T, dtype=np.float32)
    btok[::4] = np.inf
    wl.null_bias_tok = btok
    got, ref = _run_wl(wl, 2e-2, 1e-3)
    assert np.isinf(ref["fwd"]["aux"]["L_z"])
    for k, v in got.items():
        if v is not None:
            assert np.isfinite(v).all(), k
    _check(cfg, got, ref)


@pytest.mark.parametrize("T", [1, 3, 65])
def test_backward_tiny_token_counts(T):
    """One token, a few tokens and one token past a 64-token tile."""
    cfg = Config(name=f"bwd_t{T}", dtype="bf16", w_std=None, seed=T, **dict(CASES["nullpool_shared"], T=T))
    got, ref = _run_wl(generate(cfg), 2e-2, 1e-3)
    _check(cfg, got, ref)


def test_backward_one_expert_takes_every_slot():
    """K = 1 and one expert wins every token: a single 700-row segment (a ragged last
    K tile of the weight gradient) and every other expert empty."""
    cfg = Config(name="bwd_one_expert", dtype="bf16", w_std=None, seed=4,
                 **dict(CASES["topk_m0"], T=700, top_k=1))
    wl = generate(cfg)
    wl.x[:, 0] = 0x3F80          # bf16 1.0 in column 0 of every token
    wl.w_router[3, 0] = 100.0    # expert 3 wins every token
    got, ref = _run_wl(wl, 2e-2, 1e-3)
    assert (ref["fwd"]["topk_idx"][:, 0] == 3).all()
    _check(cfg, got, ref)


def test_backward_empty_expert_ping_pong():
    """The ping-pong weight-gradient tiles with one expert that receives no rows (an
    empty K range: its weight gradients are exactly zero) between experts that do."""
    cfg = Config(name="bwd_pp_empty", dtype="bf16", w_std=None, seed=9, **CASES["pp_wgrad"])
    wl = generate(cfg)
    wl.x[:, 0] = 0x3F80          # bf16 1.0 in column 0 of every token
    wl.w_router[5, 0] = -100.0   # expert 5 loses every token
    got, ref = _run_wl(wl, 2e-2, 1e-3)
    off = ref["fwd"]["offsets"]
    assert off[6] == off[5] and off[-1] > 0
    for name in ("dw_gate", "dw_up", "dw_down"):
        assert (got[name][5] == 0).all(), name
    _check(cfg, got, ref)


def test_backward_at_the_size_limits():
    """N = 255, M = 3841 (the largest pool), K = 32, with a shared expert."""
    cfg = Config(name="bwd_limits", T=150, d_model=64, n_experts=255, n_null=3841, top_k=32, d_ff=64,
                 d_ff_shared=32, dtype="bf16", w_std=None, seed=12)
    got, ref = _run_wl(generate(cfg), 2e-2, 1e-3)
    _check(cfg, got, ref)


# moe_layer_forward_train + moe_layer_backward_saved against moe_layer_forward +
# moe_layer_backward, bit for bit: the gate/up launch keeping g and u on the 256 x 256
# tiles with the fused combine after it (keep_fused), on those tiles without a shared
# expert (the down projections and the combine launch), and off them (plain GEMMs for g
# and u, the layer's own gate/up for the half-precision h)
TRAIN_CASES = {
    "small": CASES["nullpool_shared"],
    "keep_fused": dict(T=4096, d_model=256, n_experts=8, n_null=8, top_k=2, d_ff=256, d_ff_shared=256),
    "keep_no_shared": dict(T=2048, d_model=256, n_experts=4, n_null=4, top_k=2, d_ff=160, d_ff_shared=0),
}


@pytest.mark.parametrize("case,null_bias", [(c, None) for c in TRAIN_CASES] +
                         [("keep_fused", 1e3), ("keep_fused", np.inf)])
def test_forward_train_and_backward_saved_match_the_stateless_pair(case, null_bias):
    """(null_bias: a per-token null bias for every token; 1e3 and +inf send every slot
    to a null copy, so there are no routed rows)"""
    cfg = Config(name=f"train_{case}", dtype="bf16", w_std=None, seed=3, **TRAIN_CASES[case])
    say(f"  training pair {case} T={cfg.T} d={cfg.d_model} N={cfg.n_experts} Fs={cfg.d_ff_shared} "
        f"null bias {null_bias}")
    wl = generate(cfg)
    if null_bias is not None:
        wl.null_bias_tok = np.full(cfg.T, null_bias, dtype=np.float32)
    layer = MoeLayer(wl)
    layer.forward()
    y_ref = layer.y.clone()
    aux_ref = {k: getattr(layer, k).clone() for k in ("counts", "P", "scalars")}
    rng = np.random.default_rng(11)
    dy = to_device(bf16_round(rng.standard_normal((cfg.T, cfg.d_model)).astype(np.float32)))
    g_ref = {k: v.clone() for k, v in layer.backward(dy, 2e-2, 1e-3).items() if v is not None}
    layer.y.zero_()
    for k in aux_ref:
        getattr(layer, k).zero_()
    layer.forward_train()
    torch.cuda.synchronize()
    assert torch.equal(layer.y, y_ref), "forward_train y differs from the forward's"
    for k, v in aux_ref.items():
        # (equal_nan: with a +inf null logit the z-loss scalar is +inf, others may be NaN-free)
        assert torch.equal(getattr(layer, k), v) or torch.allclose(getattr(layer, k), v, rtol=0, atol=0,
                                                                   equal_nan=True), k
    for v in layer.grads.values():
        if v is not None:
            v.fill_(float("nan"))
    layer.backward_saved(dy, 2e-2, 1e-3)
    torch.cuda.synchronize()
    for k, v in g_ref.items():
        assert torch.equal(layer.grads[k], v), k
    # a second backward from the same state gives the same gradients (it reads the state
    # only)
    layer.backward_saved(dy, 2e-2, 1e-3)
    torch.cuda.synchronize()
    for k, v in g_ref.items():
        assert torch.equal(layer.grads[k], v), k


def test_training_pair_full_size_headline_shape():
    """The training pair at the Qwen3-1.7B rho = 0.25 shape (16384 tokens, 64 experts,
    K = 8 of 64 + 192, shared expert): y and every gradient equal the stateless pair's."""
    from workloads import CONFIGS
    cfg = CONFIGS["qwen3_1p7b_rho0p25"]
    say(f"  training pair full size {cfg.name}")
    layer = MoeLayer(generate(cfg))
    layer.forward(aux=False)
    y_ref = layer.y.clone()
    g = torch.Generator(device="cuda").manual_seed(5)
    dy = torch.randn((layer.T, cfg.d_model), generator=g, device="cuda").to(torch.bfloat16)
    g_ref = {k: v.clone() for k, v in layer.backward(dy, 2e-2, 1e-3).items() if v is not None}
    layer.forward_train()
    torch.cuda.synchronize()
    assert torch.equal(layer.y, y_ref)
    layer.backward_saved(dy, 2e-2, 1e-3)
    torch.cuda.synchronize()
    for k, v in g_ref.items():
        assert torch.equal(layer.grads[k], v), k


def test_forward_train_refuses_routing_outputs():
    from token_choice_routing_amd import AuxOut, MoeError, moe_layer_forward_train
    cfg = Config(name="train_refuse", dtype="bf16", w_std=None, seed=3, **CASES["topk_m0"])
    layer = MoeLayer(generate(cfg))
    layer._backward_buffers()
    bad = AuxOut(layer.logits.data_ptr(), None, None, None, None, None, None, None, None)
    with pytest.raises(MoeError):
        moe_layer_forward_train(layer.dims, layer.params, layer.y, bad, layer.ws_bwd)

