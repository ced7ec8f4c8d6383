"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, sizes workspaces, and rejects bad arguments with the documented
status before anything reaches the GPU (these calls never launch a kernel, so
they run without a GPU)."""
import ctypes

import pytest

import token_choice_routing_amd as tcr
from token_choice_routing_amd import (MOE_BF16, MOE_ERR_ALIGN, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED,
                                      MOE_ERR_WORKSPACE, MOE_F32, MOE_OK, MOE_WS_AUX, MOE_WS_LAYER,
                                      MOE_WS_PERMUTE, MOE_WS_ROUTE, make_dims)
from workloads import CONFIGS

FAKE = 0x7f0000001000        # 16-byte aligned, never dereferenced: validation fails first
MIS = FAKE + 4               # misaligned


@pytest.fixture(scope="module")
def lib():
    return tcr.load_library()


def test_exports_every_declared_function(lib):
    names = tcr.header_functions()
    assert {"moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_aux_stats",
            "moe_layer_forward", "moe_workspace_bytes", "moe_status_str"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert tcr.version() >= 100


def test_status_strings(lib):
    for s in range(6):
        assert tcr.status_str(s)
    assert tcr.status_str(99) == "unknown status"


def test_workspace_sizes_cover_the_worst_case():
    for cfg in CONFIGS.values():
        d = tcr.dims_from_config(cfg)
        e = 2 if cfg.dtype == "bf16" else 4
        R = cfg.T * min(cfg.top_k, cfg.n_experts)
        total = tcr.workspace_bytes(d, MOE_WS_LAYER)
        assert total >= R * cfg.d_model * 4 + R * cfg.d_ff * e   # float32 expert outputs + h
        assert tcr.workspace_bytes(d, MOE_WS_PERMUTE) > 0
        assert tcr.workspace_bytes(d, MOE_WS_AUX) > 0
        assert (tcr.workspace_bytes(d, MOE_WS_ROUTE) > 0) == (cfg.dtype == "bf16")
        assert tcr.expert_ffn_workspace_bytes(d, cfg.d_ff, R) == R * cfg.d_ff * e


BAD_DIMS = [
    dict(T=-1), dict(n_experts=0), dict(n_null=-1), dict(top_k=0), dict(top_k=17, n_null=8),
    dict(n_null=0, top_k=9), dict(d_model=12), dict(d_ff=4), dict(d_ff_shared=-8), dict(dtype=7),
    dict(null_kind=3), dict(null_kind=-1),
]
UNSUPPORTED_DIMS = [dict(n_experts=256, top_k=2), dict(top_k=33, n_null=64), dict(n_null=5000),
                    dict(T=1 << 30, top_k=2)]


def _dims(**kw):
    base = dict(T=64, d_model=64, n_experts=8, n_null=8, top_k=2, d_ff=64, d_ff_shared=0, dtype=MOE_BF16)
    base.update(kw)
    return make_dims(**base)


@pytest.mark.parametrize("kw", BAD_DIMS)
def test_invalid_dims_rejected(lib, kw):
    d = _dims(**kw)
    assert tcr.workspace_bytes(d, MOE_WS_LAYER) == 0
    st = lib.moe_route(ctypes.byref(d), FAKE, FAKE, 0.0, None, None, None, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert st == MOE_ERR_ARG


@pytest.mark.parametrize("kw", UNSUPPORTED_DIMS)
def test_unsupported_dims_rejected(lib, kw):
    d = _dims(**kw)
    st = lib.moe_combine(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, None)
    assert st == MOE_ERR_UNSUPPORTED


def test_null_and_misaligned_pointers(lib):
    d = _dims()
    b = ctypes.byref(d)
    big = 1 << 34
    assert lib.moe_route(b, FAKE, FAKE, 0.0, None, None, None, None, FAKE, None, FAKE, big, None) == MOE_ERR_ARG
    assert lib.moe_route(b, FAKE, FAKE, 0.0, None, None, None, MIS, FAKE, None, FAKE, big, None) == MOE_ERR_ALIGN
    assert lib.moe_route(b, None, FAKE, 0.0, None, None, None, FAKE, FAKE, None, FAKE, big, None) == MOE_ERR_ARG
    assert lib.moe_permute(b, FAKE, None, FAKE, None, FAKE, FAKE, None, FAKE, big, None) == MOE_ERR_ARG
    assert lib.moe_permute(b, FAKE, MIS, FAKE, FAKE, FAKE, FAKE, None, FAKE, big, None) == MOE_ERR_ALIGN
    assert lib.moe_combine(b, FAKE, FAKE, FAKE, MIS, None, FAKE, None) == MOE_ERR_ALIGN
    assert lib.moe_combine(b, None, FAKE, FAKE, None, None, FAKE, None) == MOE_ERR_ARG
    assert lib.moe_aux_stats(b, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, big, None) == MOE_ERR_ARG
    assert lib.moe_expert_ffn(b, 0, 64, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == MOE_ERR_ARG
    assert lib.moe_expert_ffn(b, 2, 64, 10, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == MOE_ERR_ARG
    assert lib.moe_expert_ffn(b, 2, 60, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == MOE_ERR_ARG
    p = tcr.LayerParams(FAKE, FAKE, 0.0, None, FAKE, FAKE, None, None, None, None)
    assert lib.moe_layer_forward(b, ctypes.byref(p), FAKE, None, FAKE, big, None) == MOE_ERR_ARG
    assert lib.moe_layer_forward(b, None, FAKE, None, FAKE, big, None) == MOE_ERR_ARG
    # copy / constant null slots: combine needs the null source, the layer the vector
    dc = _dims(null_kind=tcr.MOE_NULL_COPY)
    assert lib.moe_combine(ctypes.byref(dc), FAKE, FAKE, FAKE, None, None, FAKE, None) == MOE_ERR_ARG
    assert lib.moe_combine(ctypes.byref(dc), FAKE, FAKE, FAKE, None, MIS, FAKE, None) == MOE_ERR_ALIGN
    dk = _dims(null_kind=tcr.MOE_NULL_CONSTANT)
    p = tcr.LayerParams(FAKE, FAKE, 0.0, None, FAKE, FAKE, FAKE, None, None, None, None)
    assert lib.moe_layer_forward(ctypes.byref(dk), ctypes.byref(p), FAKE, None, FAKE, big, None) == MOE_ERR_ARG
    ds = _dims(d_ff_shared=64)
    p = tcr.LayerParams(FAKE, FAKE, 0.0, None, FAKE, FAKE, FAKE, None, None, None)
    assert lib.moe_layer_forward(ctypes.byref(ds), ctypes.byref(p), FAKE, None, FAKE, big, None) == MOE_ERR_ARG


def test_bf16_operands_past_4g_unsupported(lib):
    """bf16 GEMM operands are read at 32-bit byte offsets that may run one row past
    the end: a group's weight matrix and the gathered activation matrix, plus a row,
    must fit in 4 GB; larger ones are refused before anything is launched."""
    d = make_dims(T=16, d_model=32768, n_experts=4, n_null=0, top_k=2, d_ff=65536, dtype=MOE_BF16)
    b = ctypes.byref(d)
    big = 1 << 40
    assert lib.moe_grouped_gemm(b, 0, 1, 65536, 32768, 10, FAKE, None, FAKE, FAKE, FAKE, None) == MOE_ERR_UNSUPPORTED
    assert lib.moe_expert_ffn(b, 1, 65536, 10, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == MOE_ERR_UNSUPPORTED
    d2 = make_dims(T=70000, d_model=32768, n_experts=4, n_null=0, top_k=2, d_ff=64, dtype=MOE_BF16)
    p = tcr.LayerParams(FAKE, FAKE, 0.0, None, FAKE, FAKE, FAKE, None, None, None)
    assert lib.moe_layer_forward(ctypes.byref(d2), ctypes.byref(p), FAKE, None, FAKE, big, None) == MOE_ERR_UNSUPPORTED


def test_short_workspace(lib):
    d = _dims()
    b = ctypes.byref(d)
    need = tcr.workspace_bytes(d, MOE_WS_LAYER)
    p = tcr.LayerParams(FAKE, FAKE, 0.0, None, FAKE, FAKE, FAKE, None, None, None)
    assert lib.moe_layer_forward(b, ctypes.byref(p), FAKE, None, FAKE, need - 1, None) == MOE_ERR_WORKSPACE
    assert lib.moe_layer_forward(b, ctypes.byref(p), FAKE, None, None, need, None) == MOE_ERR_WORKSPACE
    assert lib.moe_route(b, FAKE, FAKE, 0.0, None, None, None, FAKE, FAKE, None, FAKE,
                         tcr.workspace_bytes(d, MOE_WS_ROUTE) - 1, None) == MOE_ERR_WORKSPACE
    assert lib.moe_permute(b, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == MOE_ERR_WORKSPACE
    assert lib.moe_aux_stats(b, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                             tcr.workspace_bytes(d, MOE_WS_AUX) - 1, None) == MOE_ERR_WORKSPACE
    ffn_need = tcr.expert_ffn_workspace_bytes(d, 64, 10)
    assert lib.moe_expert_ffn(b, 2, 64, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ffn_need - 1,
                              None) == MOE_ERR_WORKSPACE


def test_empty_inputs_are_noops(lib):
    """T = 0 and zero rows validate and return OK without launching anything."""
    d = _dims(T=0)
    b = ctypes.byref(d)
    big = 1 << 34
    assert lib.moe_route(b, FAKE, FAKE, 0.0, None, None, None, FAKE, FAKE, None, FAKE, big, None) == MOE_OK
    assert lib.moe_combine(b, FAKE, FAKE, FAKE, None, None, FAKE, None) == MOE_OK
    assert lib.moe_permute(b, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == MOE_OK
    p = tcr.LayerParams(FAKE, FAKE, 0.0, None, FAKE, FAKE, FAKE, None, None, None)
    assert lib.moe_layer_forward(b, ctypes.byref(p), FAKE, None, FAKE, big, None) == MOE_OK
    d1 = _dims()
    assert lib.moe_expert_ffn(ctypes.byref(d1), 3, 64, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                              None) == MOE_OK
    assert tcr.workspace_bytes(_dims(dtype=MOE_F32), MOE_WS_ROUTE) == 0


def test_backward_argument_checks(lib):
    """moe_layer_backward refuses what it does not cover and bad pointers or
    workspaces with the documented status, before anything is launched; T = 0 is a
    no-op."""
    big = 1 << 40
    grads = tcr.LayerGrads(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None)
    p = tcr.LayerParams(FAKE, FAKE, 0.0, None, FAKE, FAKE, FAKE, None, None, None)

    def call(d, params=p, dy=FAKE, g=grads, ws=FAKE, nbytes=big):
        return lib.moe_layer_backward(ctypes.byref(d), ctypes.byref(params) if params else None, dy,
                                      ctypes.c_float(0.02), ctypes.c_float(0.001),
                                      ctypes.byref(g) if g else None, ws, ctypes.c_size_t(nbytes), None)

    d = _dims()
    assert call(_dims(dtype=MOE_F32)) == MOE_ERR_UNSUPPORTED
    assert call(_dims(null_kind=tcr.MOE_NULL_COPY)) == MOE_ERR_UNSUPPORTED
    assert call(d, params=None) == MOE_ERR_ARG
    assert call(d, g=None) == MOE_ERR_ARG
    assert call(d, dy=None) == MOE_ERR_ARG
    assert call(d, dy=MIS) == MOE_ERR_ALIGN
    assert call(d, g=tcr.LayerGrads(FAKE, FAKE, FAKE, None, FAKE, None, None, None)) == MOE_ERR_ARG
    assert call(d, g=tcr.LayerGrads(FAKE, FAKE, FAKE, FAKE, MIS, None, None, None)) == MOE_ERR_ALIGN
    # a shared expert needs its weights and its three gradients
    ds = _dims(d_ff_shared=64)
    assert call(ds) == MOE_ERR_ARG
    ps = tcr.LayerParams(FAKE, FAKE, 0.0, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert call(ds, params=ps) == MOE_ERR_ARG
    need = tcr.workspace_bytes(d, tcr.MOE_WS_BACKWARD)
    assert need > tcr.workspace_bytes(d, MOE_WS_LAYER)
    assert call(d, nbytes=need - 1) == MOE_ERR_WORKSPACE
    assert call(d, ws=None, nbytes=need) == MOE_ERR_WORKSPACE
    # bf16 operands past the 32-bit offsets (transposed activations included)
    assert call(make_dims(T=70000, d_model=32768, n_experts=4, n_null=0, top_k=2, d_ff=64,
                          dtype=MOE_BF16)) == MOE_ERR_UNSUPPORTED
    assert call(_dims(T=0)) == MOE_OK


def test_training_pair_argument_checks(lib):
    """moe_layer_forward_train and moe_layer_backward_saved refuse what the backward does
    not cover and bad pointers or workspaces like moe_layer_backward, before anything is
    launched; the training forward also refuses the aux routing outputs and f (they stay
    in the workspace). T = 0 is a no-op for both."""
    big = 1 << 40
    p = tcr.LayerParams(FAKE, FAKE, 0.0, None, FAKE, FAKE, FAKE, None, None, None)
    d = _dims()
    need = tcr.workspace_bytes(d, tcr.MOE_WS_BACKWARD)

    def fwd(d, params=p, y=FAKE, aux=None, ws=FAKE, nbytes=big):
        return lib.moe_layer_forward_train(ctypes.byref(d), ctypes.byref(params) if params else None, y,
                                           ctypes.byref(aux) if aux else None, ws, ctypes.c_size_t(nbytes), None)

    assert fwd(_dims(dtype=MOE_F32)) == MOE_ERR_UNSUPPORTED
    assert fwd(_dims(null_kind=tcr.MOE_NULL_COPY)) == MOE_ERR_UNSUPPORTED
    assert fwd(d, params=None) == MOE_ERR_ARG
    assert fwd(d, y=None) == MOE_ERR_ARG
    assert fwd(d, y=MIS) == MOE_ERR_ALIGN
    assert fwd(d, nbytes=need - 1) == MOE_ERR_WORKSPACE
    assert fwd(d, ws=None, nbytes=need) == MOE_ERR_WORKSPACE
    for name in ("logits", "topk_idx", "topk_w", "n_real", "offsets", "f"):
        a = tcr.AuxOut()
        setattr(a, name, FAKE)
        assert fwd(d, aux=a) == MOE_ERR_ARG, name
    a = tcr.AuxOut()
    a.P = MIS
    assert fwd(d, aux=a) == MOE_ERR_ALIGN
    assert fwd(_dims(T=0)) == MOE_OK

    grads = tcr.LayerGrads(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None)

    def bwd(d, dy=FAKE, g=grads, ws=FAKE, nbytes=big):
        return lib.moe_layer_backward_saved(ctypes.byref(d), ctypes.byref(p), dy, ctypes.c_float(0.02),
                                            ctypes.c_float(0.001), ctypes.byref(g) if g else None, ws,
                                            ctypes.c_size_t(nbytes), None)

    assert bwd(_dims(dtype=MOE_F32)) == MOE_ERR_UNSUPPORTED
    assert bwd(d, g=None) == MOE_ERR_ARG
    assert bwd(d, dy=None) == MOE_ERR_ARG
    assert bwd(d, dy=MIS) == MOE_ERR_ALIGN
    assert bwd(d, nbytes=need - 1) == MOE_ERR_WORKSPACE
    assert bwd(_dims(T=0)) == MOE_OK


def test_binding_refuses_host_and_strided_tensors():
    """The binding passes device addresses only: a host tensor or a strided view would be
    read as a dense device array, so it is refused before the call."""
    import torch
    with pytest.raises(ValueError):
        tcr._ptr(torch.zeros(4))


def test_binding_refuses_host_workspace():
    """A workspace tensor in host memory is refused by the binding like any other
    host tensor (its address would otherwise reach device kernels)."""
    import torch
    with pytest.raises(ValueError):
        tcr._ws(torch.zeros(256, dtype=torch.uint8))
    d = _dims()
    with pytest.raises(ValueError):
        tcr.moe_aux_stats(d, FAKE, FAKE, FAKE, FAKE, None, FAKE, torch.zeros(4096, dtype=torch.uint8))


def test_validate_inputs_argument_checks(lib):
    """moe_validate_inputs checks pointers and workspace like the forward, and a NaN
    host-side null bias is reported before anything is launched."""
    d = _dims()
    b = ctypes.byref(d)
    p = tcr.LayerParams(FAKE, FAKE, 0.0, None, FAKE, FAKE, FAKE, None, None, None)
    assert lib.moe_validate_inputs(b, None, FAKE, 256, None) == MOE_ERR_ARG
    assert lib.moe_validate_inputs(b, ctypes.byref(tcr.LayerParams(None, FAKE, 0.0, None, FAKE, FAKE, FAKE,
                                                                   None, None, None)), FAKE, 256, None) == MOE_ERR_ARG
    assert lib.moe_validate_inputs(b, ctypes.byref(p), FAKE, 8, None) == MOE_ERR_WORKSPACE
    assert lib.moe_validate_inputs(b, ctypes.byref(p), MIS, 256, None) == MOE_ERR_ALIGN
    pn = tcr.LayerParams(FAKE, FAKE, float("nan"), None, FAKE, FAKE, FAKE, None, None, None)
    assert lib.moe_validate_inputs(b, ctypes.byref(pn), FAKE, 256, None) == tcr.MOE_ERR_NONFINITE
    assert lib.moe_status_str(tcr.MOE_ERR_NONFINITE).decode().startswith("non-finite")


def test_noalloc_entry_checks(lib):
    """moe_layer_forward_noalloc: bad dims, a NULL params struct, and a layer whose
    workspace exceeds the static array are refused before anything touches a GPU."""
    d = _dims()
    assert lib.moe_layer_forward_noalloc(ctypes.byref(_dims(top_k=0)), None, FAKE, None, None) == MOE_ERR_ARG
    assert lib.moe_layer_forward_noalloc(ctypes.byref(d), None, FAKE, None, None) == MOE_ERR_ARG
    big = tcr.dims_from_config(CONFIGS["qwen3_1p7b_rho0p25"])
    assert tcr.workspace_bytes(big, MOE_WS_LAYER) > tcr.MOE_NOALLOC_MAX_WS_BYTES
    p = tcr.LayerParams(FAKE, FAKE, 0.0, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert lib.moe_layer_forward_noalloc(ctypes.byref(big), ctypes.byref(p), FAKE, None, None) == MOE_ERR_UNSUPPORTED
