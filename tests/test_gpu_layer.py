"""End-to-end GPU parity of moe_layer_forward against the CPU oracle.

Every config runs at full size. Configs the oracle finishes in seconds are
compared on every output element; the large ones on a seeded sample of tokens
(plus whole-array checks of routing, permutation and statistics, which are
cheap). Also: determinism, solution-space preservation, null-routed tokens."""
import copy

import numpy as np
import pytest
import torch

import token_choice_routing_amd as tcr
from oracle import moe_oracle as O
from token_choice_routing_amd.layer import MoeLayer, to_device, to_host
from workloads import CONFIGS, generate
from workloads.configs import Config
from tests.gpu_util import FLIP_GAP, TOL_BF16, TOL_F32, assert_layer_close, empty, say, vals
from workloads import bf16_round

pytestmark = pytest.mark.gpu


def sub_workload(wl, rows):
    """Same weights, a subset of the tokens (in the given order)."""
    w2 = copy.copy(wl)
    w2.x = np.ascontiguousarray(wl.x[rows])
    if wl.null_bias_tok is not None:
        w2.null_bias_tok = np.ascontiguousarray(wl.null_bias_tok[rows])
    w2.cfg = copy.copy(wl.cfg)
    object.__setattr__(w2.cfg, "T", len(rows))
    return w2


def run_layer(wl):
    say(f"  layer forward T={wl.x.shape[0]} {wl.cfg.name}")
    layer = MoeLayer(wl)
    layer.forward()
    return layer, layer.results()


def check_routing(wl, out, rows=None, stats=True):
    """Logits against float64, routing bit-exact from the GPU logits, flips only at tiny gaps."""
    cfg = wl.cfg
    N, M, K = cfg.n_experts, cfg.n_null, cfg.top_k
    gl = out["logits"]
    ot, ow, on = O.route(gl.astype(np.float64), N, M, K, cfg.null_kind)
    np.testing.assert_array_equal(out["topk_idx"], ot)
    np.testing.assert_array_equal(out["n_real"], on)
    np.testing.assert_allclose(out["topk_w"], ow, rtol=1e-6, atol=0)
    rows = np.arange(gl.shape[0]) if rows is None else rows
    btok = None if wl.null_bias_tok is None else wl.null_bias_tok[rows].astype(np.float64)
    ref = O.router_logits(wl.values("x")[rows], wl.values("w_router"), wl.null_bias, btok)
    fin = np.isfinite(ref)
    err = (np.abs(gl[rows][fin] - ref[fin]) / np.maximum(1.0, np.abs(ref[fin]))).max()
    say(f"  max |logit err| / max(1, |logit|) = {err:.3e}")
    assert err < 1e-6
    ft, _, _ = O.route(ref, N, M, K)
    flips = np.nonzero((np.sort(ft, 1) != np.sort(ot[rows], 1)).any(1))[0]
    gap = O.decisive_gap(ref, N, M, K)
    say(f"  tokens routed differently from the float64 logits: {len(flips)}")
    assert (gap[flips] < FLIP_GAP).all()
    # permutation offsets and the statistics from the same routing
    _, off, _, _ = O.permute(out["topk_idx"], N)
    np.testing.assert_array_equal(out["offsets"], off)
    if not stats:
        return gl
    a = O.aux_stats(gl.astype(np.float64), out["topk_idx"], N, M, K)
    np.testing.assert_array_equal(out["counts"], a["counts"])
    np.testing.assert_allclose(out["P"], a["P"], rtol=1e-4, atol=1e-12)
    np.testing.assert_allclose(out["f"], a["f"], rtol=1e-6)
    for i, key in enumerate(("L_bal", "L_z", "mean_r")):
        if np.isinf(a[key]):   # L_z with a null logit at +inf
            assert out["scalars"][i] == a[key], key
        else:
            assert abs(out["scalars"][i] - a[key]) <= 1e-4 * abs(a[key]) + 1e-12, key
    return gl


def tol(cfg):
    return TOL_BF16 if cfg.dtype == "bf16" else TOL_F32


def check_full(wl, stats=True):
    layer, out = run_layer(wl)
    gl = check_routing(wl, out, stats=stats)
    ref = O.layer_forward(wl, logits=gl.astype(np.float64))
    assert_layer_close(out["y"], ref["y"], tol(wl.cfg), wl.cfg.dtype == "bf16", f"y {wl.cfg.name}")
    nul = out["n_real"] == 0
    if nul.any() and not wl.cfg.d_ff_shared and wl.cfg.null_kind == "zero":
        assert (vals(out["y"])[nul] == 0).all()
    return out


@pytest.mark.parametrize("name", ["tiny_f32", "qwen3_0p6b_rho1"])
def test_layer_full_compare(name):
    say(f"layer full compare {name}")
    check_full(generate(CONFIGS[name]))


@pytest.mark.parametrize("name,rows", [
    ("qwen3_0p6b_rho0p5", np.arange(1500)),
    ("qwen3_1p7b_rho0p25", np.arange(777)),
    ("modality_skew_rho0p5", np.r_[0:500, 16384 - 524:16384]),   # both token classes
])
def test_layer_token_subset_full_compare(name, rows):
    say(f"layer subset compare {name} T={len(rows)}")
    check_full(sub_workload(generate(CONFIGS[name]), rows))


@pytest.mark.parametrize("name", ["qwen3_0p6b_rho0p5", "qwen3_1p7b_rho0p25", "modality_skew_rho0p5"])
def test_layer_full_size_sampled(name):
    cfg = CONFIGS[name]
    say(f"layer full size, sampled rows: {name}")
    wl = generate(cfg)
    layer, out = run_layer(wl)
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(cfg.T, size=384, replace=False))
    gl = check_routing(wl, out, rows=rows)
    if cfg.bias_mode == "calibrated":
        assert abs(out["n_real"].mean() - cfg.target_mean_r) <= 0.05
    yd, _, _ = O.layer_dense(wl, logits=gl.astype(np.float64), tokens=rows)
    assert_layer_close(vals(out["y"])[rows], yd, TOL_BF16, True, f"y sampled {name}")
    # second run in the same launch configuration is bitwise identical
    y1 = out["y"].copy()
    layer.forward()
    np.testing.assert_array_equal(to_host(layer.y), y1)


def _small(**kw):
    base = dict(name="small_bf16", T=600, d_model=256, n_experts=16, n_null=16, top_k=4, d_ff=128,
                d_ff_shared=64, dtype="bf16", w_std=0.05)
    base.update(kw)
    return Config(**base)


def test_solution_space_preservation_bitwise():
    """K=4 with the null logit put between each token's 2nd and 3rd real logit
    gives the K=2, M=0 layer output bit for bit."""
    say("solution-space preservation on the GPU")
    wl4 = generate(_small(top_k=4, n_null=2))
    s = O.router_logits(wl4.values("x"), wl4.values("w_router"))
    srt = np.sort(s[:, :16], axis=1)[:, ::-1]
    wl4.null_bias_tok = (0.5 * (srt[:, 1] + srt[:, 2]) - s[:, 16]).astype(np.float32)
    _, o4 = run_layer(wl4)
    assert (o4["n_real"] == 2).all()
    _, o2 = run_layer(generate(_small(top_k=2, n_null=0)))
    np.testing.assert_array_equal(o4["y"], o2["y"])
    np.testing.assert_array_equal(o4["topk_w"][:, :2], o2["topk_w"])


@pytest.mark.parametrize("shared", [64, 0])
def test_null_routed_tokens_give_shared_output(shared):
    say(f"null-routed tokens, shared={shared}")
    wl = generate(_small(d_ff_shared=shared))
    btok = np.zeros(wl.cfg.T, dtype=np.float32)
    btok[::3] = np.inf
    wl.null_bias_tok = btok
    layer, out = run_layer(wl)
    nul = np.isinf(btok)
    assert (out["n_real"][nul] == 0).all()
    if shared:
        dims = layer.dims
        ys = empty((wl.cfg.T, wl.cfg.d_model), torch.float32)
        ws = empty((tcr.expert_ffn_workspace_bytes(dims, shared, wl.cfg.T),), torch.uint8)
        tcr.moe_expert_ffn(dims, 1, shared, wl.cfg.T, layer.x, None, layer.ws_gate, layer.ws_up,
                           layer.ws_down, ys, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out["y"][nul], bf16_round(to_host(ys)[nul]))
    else:
        assert (vals(out["y"])[nul] == 0).all()
    check_routing(wl, out)
    assert out["scalars"][1] == np.inf


@pytest.mark.parametrize("shared", [64, 0])
def test_every_token_null(shared):
    say(f"every token null (R = 0), shared={shared}")
    wl = generate(_small(d_ff_shared=shared))
    wl.null_bias_tok = np.full(wl.cfg.T, np.inf, dtype=np.float32)
    _, out = run_layer(wl)
    assert out["offsets"][-1] == 0
    if not shared:
        assert (vals(out["y"]) == 0).all()
    check_routing(wl, out)
    assert out["scalars"][1] == np.inf and np.isfinite(out["scalars"][0])


def test_one_expert_takes_every_slot():
    say("one expert holds every real slot")
    wl = generate(_small(top_k=1, n_null=0, T=700))
    wl.x[:, 0] = 0x3F80                      # bf16 1.0 in column 0 of every token
    wl.w_router[5, 0] = 100.0                # expert 5 wins every token
    out = check_full(wl)
    assert (out["topk_idx"][:, 0] == 5).all()


@pytest.mark.parametrize("T", [1, 2, 63, 65, 129])
def test_tiny_token_counts(T):
    say(f"T = {T}")
    check_full(sub_workload(generate(_small()), np.arange(T)))


@pytest.mark.parametrize("kind", ["copy", "constant"])
def test_copy_and_constant_null_slots(kind):
    """Copy / constant zero-compute experts: full compare on a small shape and on
    1500 tokens of the rho = 0.5 Qwen3-0.6B shape (about half the slots null)."""
    say(f"layer with {kind} null slots")
    out = check_full(generate(_small(null_kind=kind)))
    assert (out["n_real"] < 4).any()
    from dataclasses import replace
    cfg = replace(CONFIGS["qwen3_0p6b_rho0p5"], null_kind=kind)
    out = check_full(sub_workload(generate(cfg), np.arange(1500)))
    assert (out["topk_w"][out["topk_idx"] >= cfg.n_experts] > 0).any()


@pytest.mark.parametrize("T", [1, 16, 64])
def test_decode_token_counts_headline_shape(T):
    """Decode-size batches at the Qwen3-0.6B shape (few rows per expert: the
    grouped GEMMs take the skinny path up to 32 rows per group)."""
    say(f"decode T = {T}")
    check_full(sub_workload(generate(CONFIGS["qwen3_0p6b_rho1"]), np.arange(T)))


@pytest.mark.parametrize("N,M,K,T,kind", [
    (255, 3841, 32, 4, "zero"),   # the size limits: 256 logits, 32 slots (a 256-thread workgroup)
    (8, 0, 2, 3, "zero"),         # plain top-K, the router's null row unused
    (16, 4, 8, 4, "zero"),        # 0 < M < K: forced reals
    (64, 64, 8, 2, "copy"),
    (16, 16, 4, 1, "constant"),
])
def test_few_tokens_route_and_sort_in_one_workgroup(N, M, K, T, kind):
    """Up to 4 tokens: scoring (float64 dot products), selection, the permutation and
    the statistics run in one workgroup of one launch; full compare with statistics."""
    say(f"few tokens N={N} M={M} K={K} T={T} {kind}")
    check_full(generate(_small(n_experts=N, n_null=M, top_k=K, T=T, null_kind=kind)))


def test_few_tokens_infinite_null_bias():
    """The one-workgroup routing with some tokens' null bias at +inf: their slots are
    all null, L_z is +inf, the other statistics take the limit."""
    say("few tokens with +inf null biases")
    wl = generate(_small(T=4))
    btok = np.zeros(4, dtype=np.float32)
    btok[::3] = np.inf
    wl.null_bias_tok = btok
    out = check_full(wl)
    assert (out["n_real"][::3] == 0).all() and np.isinf(out["scalars"][1])


@pytest.mark.parametrize("N,M,K,T", [(100, 28, 6, 300), (255, 1, 8, 130), (24, 0, 3, 200)])
def test_expert_counts_across_router_tilings(N, M, K, T):
    """Full layer where the router spreads a token tile over several scoring
    workgroups (N > 64, up to the 255-expert limit) and where one 32-expert
    tile covers every expert (N <= 32)."""
    say(f"layer with N={N} M={M} K={K} T={T}")
    check_full(generate(_small(n_experts=N, n_null=M, top_k=K, T=T)))


def test_layer_forward_and_backward_replay_in_a_hip_graph():
    """The layer forward and backward enqueue only kernels on the caller's stream (no
    allocation, copy, fill or host synchronisation), so both can be captured in a
    HIP graph: every replay, with eager calls and synchronisations in between, gives
    the eager results bit for bit."""
    from workloads.configs import Config
    say("forward + backward captured in a HIP graph")
    cfg = Config(name="graph", T=300, d_model=128, n_experts=8, n_null=8, top_k=4, d_ff=96,
                 d_ff_shared=64, dtype="bf16", w_std=None, seed=9)
    layer = MoeLayer(generate(cfg))
    rng = np.random.default_rng(1)
    dy = to_device(bf16_round(rng.standard_normal((cfg.T, cfg.d_model)).astype(np.float32)))
    layer.forward()
    grads = layer.backward(dy, 2e-2, 1e-3)
    torch.cuda.synchronize()
    ref_y = layer.y.clone()
    ref_g = {k: v.clone() for k, v in grads.items() if v is not None}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on a side stream, as capture requires
        layer.forward(stream=side)
        layer.backward(dy, 2e-2, 1e-3, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cs = torch.cuda.current_stream()
        layer.forward(stream=cs)
        layer.backward(dy, 2e-2, 1e-3, stream=cs)
    torch.cuda.synchronize()
    for i in range(3):
        layer.y.zero_()
        for v in grads.values():
            if v is not None:
                v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.y, ref_y), f"replay {i}: y"
        for k, v in ref_g.items():
            assert torch.equal(grads[k], v), f"replay {i}: {k}"
        layer.forward()                 # eager work between replays
        layer.backward(dy, 2e-2, 1e-3)
        torch.cuda.synchronize()
        assert torch.equal(layer.y, ref_y)
    del graph


def test_training_pair_replays_in_a_hip_graph():
    """moe_layer_forward_train + moe_layer_backward_saved enqueue only kernels as well:
    captured in one HIP graph (on the 256 x 256 keep launch with the fused combine), every
    replay with eager calls in between gives the stateless pair's y and gradients."""
    from workloads.configs import Config
    say("forward_train + backward_saved captured in a HIP graph")
    cfg = Config(name="graph_train", T=4096, d_model=256, n_experts=8, n_null=8, top_k=2, d_ff=256,
                 d_ff_shared=256, dtype="bf16", w_std=None, seed=4)
    layer = MoeLayer(generate(cfg))
    rng = np.random.default_rng(2)
    dy = to_device(bf16_round(rng.standard_normal((cfg.T, cfg.d_model)).astype(np.float32)))
    layer.forward()
    grads = layer.backward(dy, 2e-2, 1e-3)
    torch.cuda.synchronize()
    ref_y = layer.y.clone()
    ref_g = {k: v.clone() for k, v in grads.items() if v is not None}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward_train(stream=side)
        layer.backward_saved(dy, 2e-2, 1e-3, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cs = torch.cuda.current_stream()
        layer.forward_train(stream=cs)
        layer.backward_saved(dy, 2e-2, 1e-3, stream=cs)
    torch.cuda.synchronize()
    for i in range(3):
        layer.y.zero_()
        for v in grads.values():
            if v is not None:
                v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.y, ref_y), f"replay {i}: y"
        for k, v in ref_g.items():
            assert torch.equal(grads[k], v), f"replay {i}: {k}"
        layer.forward()                 # eager work between replays
        layer.backward(dy, 2e-2, 1e-3)
        torch.cuda.synchronize()
    del graph


def test_validate_inputs_finds_nan_and_inf():
    """moe_validate_inputs: a clean layer passes; a NaN in x, an infinity in an expert
    weight or in the router, or a NaN null bias is found; an infinite per-token null
    bias (a valid input: all slots of that token null) passes."""
    say("moe_validate_inputs")
    cfg = Config(name="validate", T=200, d_model=128, n_experts=8, n_null=8, top_k=4, d_ff=96,
                 d_ff_shared=64, dtype="bf16", w_std=None, seed=3)
    wl = generate(cfg)
    wl.null_bias_tok = np.zeros(cfg.T, dtype=np.float32)
    layer = MoeLayer(wl)
    assert layer.validate()

    def planted(t, index, value):
        old = t.view(-1)[index].clone()
        t.view(-1)[index] = value
        ok = layer.validate()
        t.view(-1)[index] = old
        assert layer.validate()
        return ok

    nan16, inf16 = torch.tensor(0x7FC0, dtype=torch.int16), torch.tensor(0x7F80, dtype=torch.int16)
    assert not planted(layer.x.view(torch.int16), 1234, nan16)
    assert not planted(layer.w_up.view(torch.int16), layer.w_up.numel() - 1, inf16)
    assert not planted(layer.ws_down.view(torch.int16), 7, inf16)
    assert not planted(layer.w_router, 5, float("inf"))
    assert not planted(layer.null_bias_tok, 17, float("nan"))
    assert planted(layer.null_bias_tok, 17, float("inf"))
    assert planted(layer.null_bias_tok, 18, float("-inf"))


def test_layer_at_the_size_limits():
    """The largest pool the library takes: N = 255 experts (MOE_MAX_EXPERTS), M = 3841
    null copies (N + M = MOE_MAX_POOL) and K = 32 (MOE_MAX_TOPK), with a shared
    expert: routing, permutation over 255 segments, 256 GEMM groups and a 32-slot
    combine against the oracle."""
    say("layer at N = 255, M = 3841, K = 32")
    cfg = Config(name="limits", T=150, d_model=64, n_experts=255, n_null=3841, top_k=32, d_ff=64,
                 d_ff_shared=32, dtype="bf16", w_std=None, seed=12)
    check_full(generate(cfg))


def _fused_shape(**kw):
    """Shapes whose down projections both take the 256 x 256 tiles (at least 512 rows per
    expert if every slot were real, and at least 512 tokens), so the layer stores the
    routed outputs token-major and the shared expert's down projection adds them in its
    epilogue instead of a separate combine."""
    base = dict(name="fused_bf16", T=2100, d_model=256, n_experts=4, n_null=4, top_k=2, d_ff=128,
                d_ff_shared=64, dtype="bf16", w_std=0.05)
    base.update(kw)
    return Config(**base)


def _workspace(cfg, **kw):
    from dataclasses import replace
    return tcr.workspace_bytes(tcr.dims_from_config(replace(cfg, **kw), cfg.T), tcr.MOE_WS_LAYER)


@pytest.mark.parametrize("kw", [
    dict(),                                   # T = 2100: a ragged last tile of 256 tokens
    dict(T=1100, top_k=8, n_null=8),          # K > N: at most min(K, N) = 4 reals per token
    dict(T=1100, n_null=0),                   # M = 0: every slot real
    dict(T=4100, d_model=320, d_ff=96, d_ff_shared=160, n_experts=8, top_k=1, n_null=0),
    dict(T=512, n_experts=1, top_k=1, n_null=1),           # one expert, exactly 512 rows of it
    dict(T=700, d_model=64, d_ff=64, d_ff_shared=32, n_experts=1, top_k=2, n_null=3),  # narrow rows
])
def test_shared_down_projection_with_the_combine(kw):
    """The shared expert's down projection with the combine in its epilogue: full
    compare against the oracle; a third of the tokens routed to null entirely (+inf
    null bias) give exactly the shared expert's own output (the standalone FFN, rounded
    once), as in the path with a separate combine."""
    cfg = _fused_shape(**kw)
    say(f"fused combine {kw}")
    assert _workspace(cfg) < _workspace(cfg, null_kind="copy")   # the fused layout was chosen
    wl = generate(cfg)
    out = check_full(wl)
    if cfg.n_null == 0:          # (the null logit takes no part without null copies)
        assert (out["n_real"] == cfg.top_k).all()
        return
    btok = np.zeros(cfg.T, dtype=np.float32)
    btok[::3] = np.inf
    wl.null_bias_tok = btok
    layer, out = run_layer(wl)
    nul = np.isinf(btok)
    assert (out["n_real"][nul] == 0).all() and (out["n_real"][~nul] > 0).any()
    dims = layer.dims
    ys = empty((cfg.T, cfg.d_model), torch.float32)
    ws = empty((tcr.expert_ffn_workspace_bytes(dims, cfg.d_ff_shared, cfg.T),), torch.uint8)
    tcr.moe_expert_ffn(dims, 1, cfg.d_ff_shared, cfg.T, layer.x, None, layer.ws_gate, layer.ws_up,
                       layer.ws_down, ys, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["y"][nul], bf16_round(to_host(ys)[nul]))
    check_routing(wl, out)
    ref = O.layer_forward(wl, logits=out["logits"].astype(np.float64))
    assert_layer_close(out["y"], ref["y"], TOL_BF16, True, "y with null-routed tokens")


def test_shared_down_projection_with_the_combine_every_token_null():
    """No routed rows at all (R = 0): the routed down projection has nothing to do and
    the shared expert's epilogue adds nothing."""
    cfg = _fused_shape(T=1100)
    wl = generate(cfg)
    wl.null_bias_tok = np.full(cfg.T, np.inf, dtype=np.float32)
    _, out = run_layer(wl)
    assert out["offsets"][-1] == 0
    ref = O.layer_forward(wl, logits=out["logits"].astype(np.float64))
    assert_layer_close(out["y"], ref["y"], TOL_BF16, True, "y, every token null")
