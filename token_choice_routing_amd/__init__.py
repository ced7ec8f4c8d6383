"""Python binding of libmoe_mi355x.so (C ABI in include/moe.h).

Argument marshalling only: every function passes torch tensors' device
pointers and torch's current HIP stream to the C entry point of the same name
and raises ``MoeError`` on a non-zero status. No step of the layer runs here.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (one runtime per process: streams and
pointers are shared). The library must have been built
(``python -m token_choice_routing_amd.build``); importing the package does not
fall back to anything when it is missing.
"""
import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe.h")

MOE_OK, MOE_ERR_ARG, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP, MOE_ERR_NONFINITE = range(7)
MOE_F32, MOE_BF16 = 0, 1
MOE_NULL_ZERO, MOE_NULL_COPY, MOE_NULL_CONSTANT = 0, 1, 2
NULL_KINDS = {"zero": MOE_NULL_ZERO, "copy": MOE_NULL_COPY, "constant": MOE_NULL_CONSTANT}
MOE_WS_LAYER, MOE_WS_ROUTE, MOE_WS_PERMUTE, MOE_WS_AUX, MOE_WS_BACKWARD = range(5)
MOE_GEMM_GATE_UP, MOE_GEMM_DOWN = 0, 1


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_str(status)})")


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("n_null", ctypes.c_int32), ("top_k", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("d_ff_shared", ctypes.c_int32), ("dtype", ctypes.c_int32), ("null_kind", ctypes.c_int32)]


class LayerParams(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("w_router", ctypes.c_void_p), ("null_bias", ctypes.c_float),
                ("null_bias_tok", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p), ("ws_gate", ctypes.c_void_p),
                ("ws_up", ctypes.c_void_p), ("ws_down", ctypes.c_void_p), ("null_value", ctypes.c_void_p)]


class AuxOut(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("logits", "topk_idx", "topk_w", "n_real", "offsets", "counts", "f", "P", "scalars")]


class LayerGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dx", "dw_router", "dw_gate", "dw_up", "dw_down", "dws_gate", "dws_up", "dws_down")]


_lib = None
_P = ctypes.c_void_p


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m token_choice_routing_amd.build`")
    lib = ctypes.CDLL(path)
    D = ctypes.POINTER(Dims)
    sig = {
        "moe_route": [D, _P, _P, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
        "moe_permute": [D, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
        "moe_expert_ffn": [D, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, _P, _P, _P, _P, _P, _P,
                           _P, ctypes.c_size_t, _P],
        "moe_combine": [D, _P, _P, _P, _P, _P, _P, _P],
        "moe_expert_gate_up": [D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
        "moe_grouped_gemm": [D, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                             ctypes.c_int64, _P, _P, _P, _P, _P, _P],
        "moe_aux_stats": [D, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
        "moe_layer_forward": [D, ctypes.POINTER(LayerParams), _P, ctypes.POINTER(AuxOut), _P,
                              ctypes.c_size_t, _P],
        "moe_layer_forward_noalloc": [D, ctypes.POINTER(LayerParams), _P, ctypes.POINTER(AuxOut), _P],
        "moe_layer_backward": [D, ctypes.POINTER(LayerParams), _P, ctypes.c_float, ctypes.c_float,
                               ctypes.POINTER(LayerGrads), _P, ctypes.c_size_t, _P],
        "moe_layer_forward_train": [D, ctypes.POINTER(LayerParams), _P, ctypes.POINTER(AuxOut), _P,
                                    ctypes.c_size_t, _P],
        "moe_layer_backward_saved": [D, ctypes.POINTER(LayerParams), _P, ctypes.c_float, ctypes.c_float,
                                     ctypes.POINTER(LayerGrads), _P, ctypes.c_size_t, _P],
        "moe_validate_inputs": [D, ctypes.POINTER(LayerParams), _P, ctypes.c_size_t, _P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.moe_workspace_bytes.argtypes = [D, ctypes.c_int32]
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_expert_ffn_workspace_bytes.argtypes = [D, ctypes.c_int32, ctypes.c_int64]
    lib.moe_expert_ffn_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_status_str.argtypes = [ctypes.c_int]
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_version.argtypes = []
    lib.moe_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def header_functions(path: str = HEADER):
    """Names of the functions include/moe.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)) - {"moe_stream"})


def _ptr(t):
    """Device address of a tensor argument (an int is taken as an address as is).
    The library reads every array as a dense row-major block in device memory, so a
    host tensor or a strided view is refused here rather than read wrongly there."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if t.device.type != "cuda":
        raise ValueError(f"expected a device tensor, got one on {t.device}")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor (the library reads dense row-major arrays)")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, where):
    if status != MOE_OK:
        raise MoeError(status, where)


def _ws(ws):
    """(device address, bytes) of a workspace tensor, checked like every other
    tensor argument (device memory, contiguous); a tuple is taken as given."""
    if ws is None:
        return None, 0
    if isinstance(ws, tuple):
        return ws
    return _ptr(ws), ws.numel() * ws.element_size()


def status_str(status: int) -> str:
    return load_library().moe_status_str(int(status)).decode()


def version() -> int:
    return load_library().moe_version()


def make_dims(T, d_model, n_experts, n_null, top_k, d_ff, d_ff_shared=0, dtype=MOE_BF16,
              null_kind=MOE_NULL_ZERO) -> Dims:
    return Dims(int(T), int(d_model), int(n_experts), int(n_null), int(top_k), int(d_ff),
                int(d_ff_shared), int(dtype), int(null_kind))


def dims_from_config(cfg, T=None) -> Dims:
    return make_dims(cfg.T if T is None else T, cfg.d_model, cfg.n_experts, cfg.n_null, cfg.top_k,
                     cfg.d_ff, cfg.d_ff_shared, MOE_BF16 if cfg.dtype == "bf16" else MOE_F32,
                     NULL_KINDS[cfg.null_kind])


def workspace_bytes(dims: Dims, which: int = MOE_WS_LAYER) -> int:
    return load_library().moe_workspace_bytes(ctypes.byref(dims), which)


def expert_ffn_workspace_bytes(dims: Dims, d_ff: int, max_rows: int) -> int:
    return load_library().moe_expert_ffn_workspace_bytes(ctypes.byref(dims), d_ff, max_rows)


def moe_route(dims, x, w_router, null_bias=0.0, null_bias_tok=None, logits_in=None,
              logits_out=None, topk_idx=None, topk_w=None, n_real=None, ws=None, stream=None):
    wp, wb = _ws(ws)
    _check(load_library().moe_route(ctypes.byref(dims), _ptr(x), _ptr(w_router), float(null_bias),
                                     _ptr(null_bias_tok), _ptr(logits_in), _ptr(logits_out),
                                     _ptr(topk_idx), _ptr(topk_w), _ptr(n_real), wp, wb,
                                     _stream(stream)), "moe_route")


def moe_permute(dims, topk_idx, x, counts, offsets, perm_token, slot_pos, x_perm, ws, stream=None):
    wp, wb = _ws(ws)
    _check(load_library().moe_permute(ctypes.byref(dims), _ptr(topk_idx), _ptr(x), _ptr(counts),
                                       _ptr(offsets), _ptr(perm_token), _ptr(slot_pos),
                                       _ptr(x_perm), wp, wb, _stream(stream)), "moe_permute")


def moe_expert_ffn(dims, n_groups, d_ff, max_rows, a, offsets, w_gate, w_up, w_down, out, ws,
                   stream=None):
    wp, wb = _ws(ws)
    _check(load_library().moe_expert_ffn(ctypes.byref(dims), int(n_groups), int(d_ff), int(max_rows),
                                          _ptr(a), _ptr(offsets), _ptr(w_gate), _ptr(w_up),
                                          _ptr(w_down), _ptr(out), wp, wb, _stream(stream)),
           "moe_expert_ffn")


def moe_grouped_gemm(dims, op, n_groups, n_out, k_dim, rows, a, offsets, b0, b1, out, stream=None):
    _check(load_library().moe_grouped_gemm(ctypes.byref(dims), int(op), int(n_groups), int(n_out),
                                            int(k_dim), int(rows), _ptr(a), _ptr(offsets), _ptr(b0),
                                            _ptr(b1), _ptr(out), _stream(stream)), "moe_grouped_gemm")


def moe_expert_gate_up(dims, x, perm_token, offsets, w_gate, w_up, ws_gate, ws_up, h, hs, stream=None):
    _check(load_library().moe_expert_gate_up(ctypes.byref(dims), _ptr(x), _ptr(perm_token), _ptr(offsets),
                                              _ptr(w_gate), _ptr(w_up), _ptr(ws_gate), _ptr(ws_up), _ptr(h),
                                              _ptr(hs), _stream(stream)), "moe_expert_gate_up")


def moe_combine(dims, y_perm, slot_pos, topk_w, y_shared, y, stream=None, null_src=None):
    """null_src: the rows a null slot adds (x for copy experts, v for constant)."""
    _check(load_library().moe_combine(ctypes.byref(dims), _ptr(y_perm), _ptr(slot_pos),
                                       _ptr(topk_w), _ptr(y_shared), _ptr(null_src), _ptr(y),
                                       _stream(stream)),
           "moe_combine")


def moe_aux_stats(dims, logits, topk_idx, f, P, counts, scalars, ws, stream=None):
    wp, wb = _ws(ws)
    _check(load_library().moe_aux_stats(ctypes.byref(dims), _ptr(logits), _ptr(topk_idx), _ptr(f),
                                         _ptr(P), _ptr(counts), _ptr(scalars), wp, wb,
                                         _stream(stream)), "moe_aux_stats")


def moe_layer_forward(dims, params: LayerParams, y, aux: AuxOut = None, ws=None, stream=None):
    wp, wb = _ws(ws)
    _check(load_library().moe_layer_forward(ctypes.byref(dims), ctypes.byref(params), _ptr(y),
                                             ctypes.byref(aux) if aux is not None else None, wp, wb,
                                             _stream(stream)), "moe_layer_forward")


MOE_NOALLOC_MAX_WS_BYTES = 64 << 20


def moe_layer_forward_noalloc(dims, params: LayerParams, y, aux: AuxOut = None, stream=None):
    """moe_layer_forward with the library's static per-device workspace (no allocation)."""
    _check(load_library().moe_layer_forward_noalloc(ctypes.byref(dims), ctypes.byref(params), _ptr(y),
                                                     ctypes.byref(aux) if aux is not None else None,
                                                     _stream(stream)), "moe_layer_forward_noalloc")


def moe_layer_backward(dims, params: LayerParams, dy, alpha: float, beta: float, grads: LayerGrads,
                       ws=None, stream=None):
    wp, wb = _ws(ws)
    _check(load_library().moe_layer_backward(ctypes.byref(dims), ctypes.byref(params), _ptr(dy),
                                              float(alpha), float(beta), ctypes.byref(grads), wp, wb,
                                              _stream(stream)), "moe_layer_backward")


def moe_layer_forward_train(dims, params: LayerParams, y, aux: AuxOut = None, ws=None, stream=None):
    """The layer forward that leaves its routing and expert pre-activations in ws (the
    backward's workspace) for moe_layer_backward_saved."""
    wp, wb = _ws(ws)
    _check(load_library().moe_layer_forward_train(ctypes.byref(dims), ctypes.byref(params), _ptr(y),
                                                   ctypes.byref(aux) if aux is not None else None, wp, wb,
                                                   _stream(stream)), "moe_layer_forward_train")


def moe_layer_backward_saved(dims, params: LayerParams, dy, alpha: float, beta: float, grads: LayerGrads,
                             ws=None, stream=None):
    """moe_layer_backward from the state a moe_layer_forward_train call left in ws."""
    wp, wb = _ws(ws)
    _check(load_library().moe_layer_backward_saved(ctypes.byref(dims), ctypes.byref(params), _ptr(dy),
                                                    float(alpha), float(beta), ctypes.byref(grads), wp, wb,
                                                    _stream(stream)), "moe_layer_backward_saved")


def moe_validate_inputs(dims, params: LayerParams, ws, stream=None) -> bool:
    """True when the layer's inputs hold no NaN or infinity (null biases may be
    infinite), False when they do; synchronises the stream. ws: >= 16 device bytes."""
    wp, wb = _ws(ws)
    status = load_library().moe_validate_inputs(ctypes.byref(dims), ctypes.byref(params), wp, wb,
                                                _stream(stream))
    if status == MOE_ERR_NONFINITE:
        return False
    _check(status, "moe_validate_inputs")
    return True


from .layer import MoeLayer  # noqa: E402,F401
