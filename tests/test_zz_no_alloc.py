"""moe_layer_forward_noalloc (the entry point for callers that cannot allocate)
against moe_layer_forward with a caller workspace: the same kernels on the same
inputs, so every output is compared bit for bit, on two calls in a row, the second
with a smaller batch (the static workspace keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import token_choice_routing_amd as tcr
from token_choice_routing_amd.layer import MoeLayer, to_host
from workloads import CONFIGS, generate
from workloads.configs import Config
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

NAMES = ("y", "logits", "topk_idx", "topk_w", "n_real", "offsets", "counts", "f", "P", "scalars")


def _outputs(layer):
    torch.cuda.synchronize()
    return {n: to_host(getattr(layer, n)).copy() for n in NAMES}


def _clear(layer):
    for n in NAMES:
        getattr(layer, n).zero_()


@pytest.mark.parametrize("first,second", [
    (("qwen3_0p6b_rho1", 1500), ("qwen3_0p6b_rho1", 333)),
    (("small_null_pool", 900), ("small_null_pool", 1)),
    # the shared expert's down projection with the combine (2100 tokens), then the
    # separate combine (600 tokens: too few rows per expert for the large tiles)
    (("fused_combine", 2100), ("fused_combine", 600)),
])
def test_noalloc_matches_workspace_forward(first, second):
    local = {
        "small_null_pool": Config(name="small_null_pool", T=900, d_model=256, n_experts=16, n_null=48, top_k=6,
                                  d_ff=192, d_ff_shared=64, dtype="bf16", w_std=0.05, seed=4),
        "fused_combine": Config(name="fused_combine", T=2100, d_model=256, n_experts=4, n_null=4, top_k=2,
                                d_ff=128, d_ff_shared=64, dtype="bf16", w_std=0.05, seed=6),
    }
    for name, T in (first, second):
        cfg = local.get(name) or CONFIGS[name]
        say(f"noalloc {name} T={T}")
        wl = generate(cfg, T=min(T, cfg.T))
        if name == "small_null_pool":
            wl.null_bias = 0.3
        layer = MoeLayer(wl, T=T)
        assert tcr.workspace_bytes(layer.dims, tcr.MOE_WS_LAYER) <= tcr.MOE_NOALLOC_MAX_WS_BYTES
        layer.forward()
        ref = _outputs(layer)
        _clear(layer)
        tcr.moe_layer_forward_noalloc(layer.dims, layer.params, layer.y, layer.aux_full)
        got = _outputs(layer)
        for n in NAMES:
            np.testing.assert_array_equal(got[n], ref[n], err_msg=f"{name} T={T}: {n}")
        # y alone, no statistics requested
        layer.y.zero_()
        tcr.moe_layer_forward_noalloc(layer.dims, layer.params, layer.y, None)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(layer.y), ref["y"])


def test_noalloc_refuses_layers_past_its_workspace():
    cfg = CONFIGS["qwen3_1p7b_rho0p25"]
    dims = tcr.dims_from_config(cfg)
    assert tcr.workspace_bytes(dims, tcr.MOE_WS_LAYER) > tcr.MOE_NOALLOC_MAX_WS_BYTES
    p = tcr.LayerParams()
    with pytest.raises(tcr.MoeError) as e:
        tcr.moe_layer_forward_noalloc(dims, p, 0x7f0000001000)
    assert e.value.status == tcr.MOE_ERR_UNSUPPORTED
