"""How close the layer-output tolerance (max |err| <= 2e-2 RMS(y) over the whole
tensor, bf16 outputs) lets any bf16 implementation come, on the exact rows the GPU
tests compare (CPU only; the float64 oracle's output is rounded here, nothing runs on
a GPU).

  floor_out: the exact output rounded once to bf16, the least error any bf16 layer
             output has;
  floor_h16: the same with the SwiGLU intermediate h rounded to IEEE half before the
             down projection, as the kernels store it;
  floor_hbf: the same with h rounded to bf16 instead.

The whole-tensor rule is reachable where floor_out < 2e-2: every workload but the
modality-skewed one, whose vision rows are ~17x larger than its text rows (its floor
is about 3.9%, so there the GPU tests hold each token row to 2e-2 of its own RMS).
Rounding h to bf16 would push the Qwen3-1.7B workload past the rule (2.10%), half
precision leaves it at the output floor; the kernels' half-precision h is checked
here to stay within the rule with room to spare."""
import copy

import numpy as np
import pytest

from oracle import moe_oracle as O
from workloads import CONFIGS, bf16_bits_to_f32, bf16_round, generate

TOL = 2e-2


def _rb(a):
    return bf16_bits_to_f32(bf16_round(np.asarray(a, np.float32))).astype(np.float64)


def _rh(a):
    return np.asarray(a, np.float64).astype(np.float16).astype(np.float64)


def _layer_rows(wl, rows, hround):
    """Layer output at the given token rows, with the whole batch's routing, h passed
    through hround before the down projection (float64 otherwise)."""
    cfg = wl.cfg
    N = cfg.n_experts
    x = wl.values("x")
    s = O.router_logits(x, wl.values("w_router"), wl.null_bias, wl.null_bias_tok)[rows]
    topk, w, _ = O.route(s, N, cfg.n_null, cfg.top_k)
    xs = x[rows]

    def ffn(a, wg, wu, wd):
        h = O.silu(a @ O._vals(wg).T) * (a @ O._vals(wu).T)
        return hround(h) @ O._vals(wd).T

    y = ffn(xs, wl.ws_gate, wl.ws_up, wl.ws_down) if cfg.d_ff_shared else np.zeros((len(rows), cfg.d_model))
    for e in range(N):
        sel = np.nonzero(topk == e)
        if len(sel[0]):
            y[sel[0]] += w[sel][:, None] * ffn(xs[sel[0]], wl.w_gate[e], wl.w_up[e], wl.w_down[e])
    return y


def _sub(wl, rows):
    w2 = copy.copy(wl)
    w2.x = np.ascontiguousarray(wl.x[rows])
    if wl.null_bias_tok is not None:
        w2.null_bias_tok = np.ascontiguousarray(wl.null_bias_tok[rows])
    return w2


def _ratio(y, ref):
    return float(np.abs(y - ref).max() / np.sqrt(np.mean(ref * ref)))


# (workload, token rows of the subset the layer tests compare in full, or None for all)
SUBSETS = [
    ("qwen3_0p6b_rho1", None),
    ("qwen3_0p6b_rho0p5", np.arange(1500)),
    ("qwen3_1p7b_rho0p25", np.arange(777)),
    ("modality_skew_rho0p5", np.r_[0:500, 16384 - 524:16384]),
]


@pytest.mark.parametrize("name,rows", SUBSETS)
def test_tolerance_floor_on_the_compared_subsets(name, rows):
    wl = generate(CONFIGS[name])
    if rows is not None:
        wl = _sub(wl, rows)
    idx = np.arange(wl.x.shape[0])
    exact = _layer_rows(wl, idx, lambda h: h)
    floor_out = _ratio(_rb(exact), exact)
    floor_h16 = _ratio(_rb(_layer_rows(wl, idx, _rh)), exact)
    floor_hbf = _ratio(_rb(_layer_rows(wl, idx, _rb)), exact)
    print(f"{name}: floor_out {floor_out:.4e}  floor_h16 {floor_h16:.4e}  floor_hbf {floor_hbf:.4e}")
    if name.startswith("modality_skew"):
        assert floor_out > TOL          # the whole-tensor rule is out of reach for bf16 outputs
    else:
        assert floor_out < TOL and floor_h16 < 0.95 * TOL
    if name == "qwen3_1p7b_rho0p25":
        assert floor_hbf > TOL          # bf16 h would not meet the rule here


@pytest.mark.parametrize("name", ["qwen3_0p6b_rho0p5", "qwen3_1p7b_rho0p25", "modality_skew_rho0p5"])
def test_tolerance_floor_on_the_sampled_rows(name):
    """The 384 rows the full-size GPU test samples (seed 1), routed with the whole batch."""
    cfg = CONFIGS[name]
    wl = generate(cfg)
    rows = np.sort(np.random.default_rng(1).choice(cfg.T, size=384, replace=False))
    exact = _layer_rows(wl, rows, lambda h: h)
    floor_out = _ratio(_rb(exact), exact)
    floor_h16 = _ratio(_rb(_layer_rows(wl, rows, _rh)), exact)
    print(f"{name} sampled: floor_out {floor_out:.4e}  floor_h16 {floor_h16:.4e}")
    if name.startswith("modality_skew"):
        assert floor_out > TOL
    else:
        assert floor_out < TOL and floor_h16 < 0.95 * TOL
