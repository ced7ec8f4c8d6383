"""GPU parity of each entry point against the CPU oracle, called through the C ABI.

Routing and permutation are compared bit for bit from identical float32
inputs; the expert FFN, combine and statistics within the stated tolerances."""
import numpy as np
import pytest
import torch

import token_choice_routing_amd as tcr
from oracle import moe_oracle as O
from token_choice_routing_amd.layer import to_device, to_host
from workloads import CONFIGS, bf16_round, generate
from tests.gpu_util import (TOL_BF16, TOL_F32, assert_close_rms, assert_rows_close, empty,
                            route_from_logits, say, vals)

pytestmark = pytest.mark.gpu

ROUTE_CASES = [(8, 8, 2), (8, 0, 2), (8, 1, 3), (8, 3, 8), (64, 64, 4), (64, 192, 8), (64, 0, 2),
               (64, 64, 8), (100, 28, 16), (255, 4000 - 255, 32), (1, 0, 1), (3, 5, 7), (33, 2, 1)]


@pytest.mark.parametrize("N,M,K", ROUTE_CASES)
def test_route_from_logits_bit_exact_on_ties(N, M, K):
    say(f"route_from_logits ties N={N} M={M} K={K}")
    rng = np.random.default_rng(N * 1000 + M * 10 + K)
    T = 4099
    s = rng.integers(-3, 4, size=(T, N + 1)).astype(np.float32)
    s[::7] = rng.standard_normal((len(s[::7]), N + 1)).astype(np.float32)
    s[5, :] = 0.0                      # everything tied
    s[6, N] = np.inf                   # all-null
    s[8, N] = -np.inf                  # all-real
    topk, w, nr = route_from_logits(s, N, M, K)
    ot, ow, onr = O.route(s.astype(np.float64), N, M, K)
    np.testing.assert_array_equal(topk, ot)
    np.testing.assert_array_equal(nr, onr)
    np.testing.assert_allclose(w, ow, rtol=1e-6, atol=0)
    say(f"  weights: {int((w != ow.astype(np.float32)).sum())} of {w.size} differ from the float32-rounded oracle")


@pytest.mark.parametrize("N,M,K", [(8, 8, 2), (8, 3, 8), (64, 192, 8), (100, 28, 16), (64, 0, 2)])
def test_route_weights_over_all_chosen(N, M, K):
    """Copy / constant null slots: the weights are a softmax over all K chosen pool
    entries (null slots at the null logit); the selection is unchanged."""
    say(f"route weights over all K N={N} M={M} K={K}")
    rng = np.random.default_rng(N + 7 * M + K)
    s = (rng.standard_normal((3001, N + 1)) * 2).astype(np.float32)
    s[5, :] = 0.0
    topk, w, nr = route_from_logits(s, N, M, K, tcr.MOE_NULL_COPY)
    ot, ow, onr = O.route(s.astype(np.float64), N, M, K, "copy")
    np.testing.assert_array_equal(topk, ot)
    np.testing.assert_array_equal(nr, onr)
    np.testing.assert_allclose(w, ow, rtol=1e-6, atol=0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_route_from_config_logits_bit_exact(name):
    cfg = CONFIGS[name]
    say(f"route_from_logits config {name}")
    wl = generate(cfg, experts=False)
    s = O.router_logits(wl.values("x"), wl.values("w_router"), wl.null_bias, wl.null_bias_tok).astype(np.float32)
    topk, w, nr = route_from_logits(s, cfg.n_experts, cfg.n_null, cfg.top_k)
    ot, ow, onr = O.route(s.astype(np.float64), cfg.n_experts, cfg.n_null, cfg.top_k)
    np.testing.assert_array_equal(topk, ot)
    np.testing.assert_array_equal(nr, onr)
    np.testing.assert_allclose(w, ow, rtol=1e-6, atol=0)


def _router_case(T, d, N, M, K, dtype, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    w = (rng.standard_normal((N + 1, d)) * 0.02).astype(np.float32)
    if dtype == "bf16":
        xs = bf16_round(x)
        xv = vals(xs)
    else:
        xs, xv = x, x.astype(np.float64)
    btok = (rng.standard_normal(T) * 0.1).astype(np.float32)
    return xs, xv, w, 0.25, btok


@pytest.mark.parametrize("T,d,N,M,K,dtype", [
    (1000, 1024, 64, 64, 4, "bf16"), (777, 2048, 64, 192, 8, "bf16"), (300, 200, 40, 8, 3, "bf16"),
    (130, 24, 8, 8, 2, "bf16"), (256, 64, 8, 8, 2, "f32"), (65, 1032, 100, 0, 6, "bf16"),
    (1, 512, 64, 64, 8, "bf16"),
    # from 128 token tiles on, one workgroup per tile scores and selects (eight
    # wavefronts for up to 8 slots): ragged token tails, a K tail, experts past N
    (8200, 2048, 64, 192, 8, "bf16"), (8250, 200, 40, 8, 3, "bf16"), (8192, 1024, 64, 0, 2, "bf16"),
    (8193, 512, 64, 64, 16, "bf16")])
def test_route_gemm_logits_and_flip_rule(T, d, N, M, K, dtype):
    say(f"route GEMM T={T} d={d} N={N} M={M} K={K} {dtype}")
    xs, xv, w, b, btok = _router_case(T, d, N, M, K, dtype, T + d)
    dims = tcr.make_dims(T, d, N, M, K, 64, 0, tcr.MOE_BF16 if dtype == "bf16" else tcr.MOE_F32)
    logits = empty((T, N + 1), torch.float32)
    topk = empty((T, K), torch.int32)
    tw = empty((T, K), torch.float32)
    nr = empty((T,), torch.int32)
    ws = empty((max(tcr.workspace_bytes(dims, tcr.MOE_WS_ROUTE), 16),), torch.uint8)
    tcr.moe_route(dims, to_device(xs), to_device(w), b, to_device(btok), None, logits, topk, tw, nr, ws)
    torch.cuda.synchronize()
    gl, gt, gw, gn = to_host(logits), to_host(topk), to_host(tw), to_host(nr)
    ref = O.router_logits(xv, w.astype(np.float64), b, btok.astype(np.float64))
    err = (np.abs(gl - ref) / np.maximum(1.0, np.abs(ref))).max()
    say(f"  max |logit err| / max(1, |logit|) = {err:.3e}")
    assert err < 1e-6
    # routing from the GPU's own logits is the oracle's routing of those logits, bit for bit
    ot, ow, on = O.route(gl.astype(np.float64), N, M, K)
    np.testing.assert_array_equal(gt, ot)
    np.testing.assert_array_equal(gn, on)
    np.testing.assert_allclose(gw, ow, rtol=1e-6, atol=0)
    # against the float64 logits, a token may only differ where the decisive gap is below 1e-5
    ft, _, _ = O.route(ref, N, M, K)
    diff = np.nonzero((np.sort(ft, 1) != np.sort(gt, 1)).any(1))[0]
    gap = O.decisive_gap(ref, N, M, K)
    say(f"  tokens routed differently from the float64 oracle: {len(diff)}")
    assert (gap[diff] < 1e-5).all()


def _perm_check(topk, N, M, K, d=64, dtype="bf16", seed=0):
    T = topk.shape[0]
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    xs = bf16_round(x) if dtype == "bf16" else x
    dims = tcr.make_dims(T, d, N, M, K, 64, 0, tcr.MOE_BF16 if dtype == "bf16" else tcr.MOE_F32)
    R_max = T * min(K, N)
    counts = empty((N,), torch.int32)
    offsets = empty((N + 1,), torch.int32)
    perm = torch.full((max(R_max, 1),), -7, dtype=torch.int32, device="cuda")
    slot = empty((T, K), torch.int32)
    xp = torch.zeros((max(R_max, 1), d), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    ws = empty((max(tcr.workspace_bytes(dims, tcr.MOE_WS_PERMUTE), 16),), torch.uint8)
    tcr.moe_permute(dims, to_device(np.ascontiguousarray(topk, dtype=np.int32)), to_device(xs), counts,
                    offsets, perm, slot, xp, ws)
    torch.cuda.synchronize()
    oc, oo, op, osl = O.permute(topk, N)
    R = int(oo[-1])
    np.testing.assert_array_equal(to_host(counts), oc)
    np.testing.assert_array_equal(to_host(offsets), oo)
    np.testing.assert_array_equal(to_host(perm)[:R], op)
    np.testing.assert_array_equal(to_host(slot), osl)
    np.testing.assert_array_equal(to_host(xp)[:R], xs[op])
    return R


@pytest.mark.parametrize("T,N,M,K", [(3000, 64, 64, 4), (1, 8, 8, 2), (5, 3, 0, 3), (2048, 64, 192, 8),
                                     (4097, 255, 100, 7), (700, 1, 3, 4), (513, 64, 0, 2)])
def test_permute_bit_exact(T, N, M, K):
    say(f"permute T={T} N={N} M={M} K={K}")
    rng = np.random.default_rng(T + N + M + K)
    s = rng.standard_normal((T, N + 1))
    s[:, N] += rng.uniform(-1, 2, T)
    topk, _ = O.select(s, N, M, K)
    R = _perm_check(topk, N, M, K, seed=T)
    say(f"  R = {R}")


def test_permute_skewed_and_empty():
    say("permute: every slot on one expert; every slot null")
    T, N, K = 5000, 64, 2
    topk = np.zeros((T, K), dtype=np.int32)
    topk[:, 1] = 64 + 3            # null
    assert _perm_check(topk, N, 8, K) == T
    topk[:, 0] = 64
    assert _perm_check(topk, N, 8, K) == 0


def test_permute_full_size_c3():
    cfg = CONFIGS["qwen3_1p7b_rho0p25"]
    say("permute at the C3 shape (T=16384, K=8)")
    wl = generate(cfg, experts=False)
    s = O.router_logits(wl.values("x"), wl.values("w_router"), wl.null_bias, wl.null_bias_tok)
    topk, _ = O.select(s, cfg.n_experts, cfg.n_null, cfg.top_k)
    _perm_check(topk, cfg.n_experts, cfg.n_null, cfg.top_k, d=cfg.d_model)


def _ffn_run(lengths, d, f, dtype="bf16", seed=0, slack=7, offsets=None):
    rng = np.random.default_rng(seed)
    G = len(lengths)
    rows = int(np.sum(lengths)) + slack
    a = rng.standard_normal((rows, d)).astype(np.float32)
    wg = (rng.standard_normal((G, f, d)) * 0.05).astype(np.float32)
    wu = (rng.standard_normal((G, f, d)) * 0.05).astype(np.float32)
    wd = (rng.standard_normal((G, d, f)) * 0.05).astype(np.float32)
    conv = bf16_round if dtype == "bf16" else (lambda z: z)
    A, Wg, Wu, Wd = conv(a), conv(wg), conv(wu), conv(wd)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32) if offsets is None else offsets
    dims = tcr.make_dims(max(rows, 1), d, max(G, 1), 0, 1, f, 0, tcr.MOE_BF16 if dtype == "bf16" else tcr.MOE_F32)
    out = torch.full((rows, d), 3.0, dtype=torch.float32, device="cuda")  # sentinel outside the segments
    ws = empty((max(tcr.expert_ffn_workspace_bytes(dims, f, rows), 16),), torch.uint8)
    tcr.moe_expert_ffn(dims, G, f, rows, to_device(A), to_device(off), to_device(Wg), to_device(Wu),
                       to_device(Wd), out, ws)
    torch.cuda.synchronize()
    got = vals(to_host(out))
    ref = O.expert_ffn_grouped(vals(A), off, Wg, Wu, Wd)
    R = int(off[-1])
    return got, ref, R, rows


@pytest.mark.parametrize("lengths,d,f", [
    ([0, 1, 17, 128, 129, 300, 0, 5], 256, 192),
    ([513], 1024, 768),
    # at least 512 rows per group (the 256 x 256 ping-pong tiles): ragged K (264, 200)
    # and output columns (200 of a 128-column gate/up tile, 264 of a 256-column down
    # tile), empty and one-row groups, K loops shorter than the three-tile prologue
    ([700, 0, 1, 1400], 264, 200),
    ([513, 511, 1030], 2048, 1536),
    ([2600], 128, 64),
    ([4000, 5000], 64, 32),
    ([0, 0, 0], 128, 64),
    ([37, 250, 3, 0, 128], 136, 72),            # K and N tails (not multiples of 64)
    ([64] * 64, 512, 384),
    ([1, 2, 3, 4, 1000, 5], 2048, 1536),
    # segments ending in a tile of exactly 128 rows (the launch of half-full last
    # tiles), of 129 rows (a full-tile launch) and a single 128-row segment
    ([384, 385, 128, 1200], 256, 128),
])
def test_expert_ffn_segments_bf16(lengths, d, f):
    say(f"expert_ffn bf16 lengths={lengths[:8]} d={d} d_ff={f}")
    got, ref, R, rows = _ffn_run(lengths, d, f, "bf16", seed=d + f)
    if R:
        assert_close_rms(got[:R], ref[:R], TOL_BF16, "segments")
    assert (got[R:] == 3.0).all(), "rows outside the segments were written"


@pytest.mark.parametrize("lengths,d,f", [
    ([0, 1, 17, 0, 5], 256, 192),               # a group over 16 rows: two row blocks
    ([3, 16, 2], 136, 72),                      # K not a multiple of 32, n_out of 16
    ([25], 2048, 1536),
    ([1] * 20, 1024, 768),
    ([0, 0, 1], 64, 8),
])
def test_expert_ffn_few_rows(lengths, d, f):
    """At most 32 rows per group: the skinny kernel (16 x 16 blocks, K split over
    the wavefronts, registers only)."""
    say(f"expert_ffn few rows lengths={lengths[:8]} d={d} d_ff={f}")
    got, ref, R, rows = _ffn_run(lengths, d, f, "bf16", seed=d + 2 * f)
    assert rows <= 32
    if R:
        assert_close_rms(got[:R], ref[:R], TOL_BF16, "segments")
    assert (got[R:] == 3.0).all(), "rows outside the segments were written"


def test_expert_ffn_f32():
    say("expert_ffn f32 (tiny workload shape)")
    got, ref, R, rows = _ffn_run([27, 0, 31, 26, 30, 1, 60, 38], 64, 128, "f32", seed=3)
    assert_close_rms(got[:R], ref[:R], TOL_F32, "segments f32")
    assert (got[R:] == 3.0).all()


def test_expert_ffn_clamps_bad_offsets():
    say("expert_ffn with an offset past the buffer: the segment is clamped to max_rows")
    off = np.array([0, 40, 10_000_000], dtype=np.int32)
    got, ref, R, rows = _ffn_run([40, 10], 128, 64, "bf16", seed=5, slack=0, offsets=off)
    assert rows == 50
    assert_rows_close(got, ref, TOL_BF16, "clamped segments")   # numpy slicing clamps the same way


@pytest.mark.parametrize("T,K,d,shared", [(1000, 4, 1024, True), (333, 8, 2048, False), (64, 2, 64, False)])
def test_combine(T, K, d, shared):
    say(f"combine T={T} K={K} d={d} shared={shared}")
    rng = np.random.default_rng(T + K)
    N, M = 64, 64
    s = rng.standard_normal((T, N + 1))
    s[:, N] += 1.0
    topk, w, _ = O.route(s, N, M, K)
    _, off, _, slot = O.permute(topk, N)
    Rmax = T * min(K, N)
    yp = rng.standard_normal((Rmax, d)).astype(np.float32)
    ys = rng.standard_normal((T, d)).astype(np.float32) if shared else None
    w32 = w.astype(np.float32)
    dims = tcr.make_dims(T, d, N, M, K, 64, 64 if shared else 0, tcr.MOE_BF16)
    y = empty((T, d), torch.bfloat16)
    tcr.moe_combine(dims, to_device(yp), to_device(slot), to_device(w32), to_device(ys) if shared else None, y)
    torch.cuda.synchronize()
    ref = O.combine(yp.astype(np.float64), slot, w32.astype(np.float64),
                    ys.astype(np.float64) if shared else None, d_model=d)
    got = vals(to_host(y))
    assert_rows_close(got, ref, TOL_BF16, "combine")
    # float32 accumulation + one bf16 rounding: within one bf16 half-ulp plus accumulation noise
    assert (np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6).all()


@pytest.mark.parametrize("kind", ["copy", "constant"])
def test_combine_null_sources(kind):
    """Null slots add w x (copy) or w v (constant), in slot order with the reals."""
    say(f"combine with {kind} null slots")
    rng = np.random.default_rng(11)
    T, K, d, N, M = 700, 4, 512, 64, 64
    s = rng.standard_normal((T, N + 1))
    s[:, N] += 0.8
    topk, w, _ = O.route(s, N, M, K, kind)
    _, off, _, slot = O.permute(topk, N)
    assert (slot < 0).any() and (slot >= 0).any()
    yp = rng.standard_normal((T * K, d)).astype(np.float32)
    ys = rng.standard_normal((T, d)).astype(np.float32)
    src = bf16_round(rng.standard_normal((T, d) if kind == "copy" else (d,)).astype(np.float32))
    w32 = w.astype(np.float32)
    dims = tcr.make_dims(T, d, N, M, K, 64, 64, tcr.MOE_BF16, tcr.NULL_KINDS[kind])
    y = empty((T, d), torch.bfloat16)
    tcr.moe_combine(dims, to_device(yp), to_device(slot), to_device(w32), to_device(ys), y,
                    null_src=to_device(src))
    torch.cuda.synchronize()
    ref = O.combine(yp.astype(np.float64), slot, w32.astype(np.float64), ys.astype(np.float64),
                    d_model=d, null_src=vals(src))
    got = vals(to_host(y))
    assert_rows_close(got, ref, TOL_BF16, f"combine {kind}")
    assert (np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6).all()


@pytest.mark.parametrize("N,M,K,T", [(64, 192, 8, 5000), (8, 8, 2, 128), (64, 0, 2, 2048), (255, 1000, 32, 300)])
def test_aux_stats(N, M, K, T):
    check_aux_stats(N, M, K, T, inf_every=0)


@pytest.mark.parametrize("N,M,K,T,inf_every", [(64, 192, 8, 3000, 7), (16, 2, 4, 500, 3), (8, 8, 2, 64, 1)])
def test_aux_stats_infinite_null_logit(N, M, K, T, inf_every):
    """Tokens whose null logit is +inf (an infinite per-token null bias): P takes the
    limit (1/M per null copy, reals 0), f and L_bal stay finite and L_z = +inf."""
    check_aux_stats(N, M, K, T, inf_every)


def check_aux_stats(N, M, K, T, inf_every):
    say(f"aux_stats N={N} M={M} K={K} T={T} null at +inf every {inf_every}")
    rng = np.random.default_rng(N + M + K + T)
    s = (rng.standard_normal((T, N + 1)) * 1.5).astype(np.float32)
    if inf_every:
        s[::inf_every, N] = np.inf
    topk, _, _ = O.route(s.astype(np.float64), N, M, K)
    dims = tcr.make_dims(T, 64, N, M, K, 64, 0, tcr.MOE_BF16)
    P = N + M
    f_, P_, c_, sc = empty((P,), torch.float32), empty((P,), torch.float32), empty((P,), torch.int32), empty((3,), torch.float32)
    ws = empty((tcr.workspace_bytes(dims, tcr.MOE_WS_AUX),), torch.uint8)
    tcr.moe_aux_stats(dims, to_device(s), to_device(topk), f_, P_, c_, sc, ws)
    torch.cuda.synchronize()
    a = O.aux_stats(s.astype(np.float64), topk, N, M, K)
    np.testing.assert_array_equal(to_host(c_), a["counts"])
    np.testing.assert_allclose(to_host(f_), a["f"], rtol=1e-6)
    np.testing.assert_allclose(to_host(P_), a["P"], rtol=1e-4, atol=1e-12)
    g = to_host(sc)
    for i, key in enumerate(("L_bal", "L_z", "mean_r")):
        if np.isinf(a[key]):
            assert g[i] == a[key], (key, g[i], a[key])
        else:
            assert abs(g[i] - a[key]) <= 1e-4 * abs(a[key]) + 1e-12, (key, g[i], a[key])
