"""Device-side holder for one layer call: uploads a workload's tensors once,
owns the workspace and output buffers, and calls ``moe_layer_forward`` (and
``moe_layer_backward``). Marshalling only; the layer itself runs in the HIP library."""
import numpy as np
import torch

from . import (AuxOut, LayerGrads, LayerParams, MOE_BF16, MOE_WS_BACKWARD, MOE_WS_LAYER, dims_from_config,
               moe_layer_backward, moe_layer_backward_saved, moe_layer_forward, moe_layer_forward_train,
               workspace_bytes)


def to_device(a, device="cuda"):
    """numpy storage array (uint16 bf16 bit patterns or float32/int32) -> torch tensor."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def to_host(t):
    """torch tensor -> numpy (bf16 becomes uint16 bit patterns)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class MoeLayer:
    WEIGHTS = ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down", "null_value")

    def __init__(self, workload, device="cuda", T=None, weights_from=None):
        """weights_from: another MoeLayer whose device weights are reused (same arrays)."""
        cfg = workload.cfg
        self.cfg = cfg
        self.T = cfg.T if T is None else T
        self.dims = dims_from_config(cfg, self.T)
        self.bf16 = self.dims.dtype == MOE_BF16
        dt = torch.bfloat16 if self.bf16 else torch.float32
        dev = device
        self.x = to_device(workload.x[: self.T], dev)
        self.null_bias = float(workload.null_bias)
        self.null_bias_tok = (to_device(workload.null_bias_tok[: self.T], dev)
                              if workload.null_bias_tok is not None else None)
        for name in self.WEIGHTS:
            arr = getattr(workload, name)
            if weights_from is not None and arr is not None:
                t = getattr(weights_from, name)
                assert t is not None and tuple(t.shape) == arr.shape
            else:
                t = to_device(arr, dev)
            setattr(self, name, t)
        N, M, K = cfg.n_experts, cfg.n_null, cfg.top_k
        T_ = self.T
        self.y = torch.empty((T_, cfg.d_model), dtype=dt, device=dev)
        i32, f32 = torch.int32, torch.float32
        self.logits = torch.empty((T_, N + 1), dtype=f32, device=dev)
        self.topk_idx = torch.empty((T_, K), dtype=i32, device=dev)
        self.topk_w = torch.empty((T_, K), dtype=f32, device=dev)
        self.n_real = torch.empty((T_,), dtype=i32, device=dev)
        self.offsets = torch.empty((N + 1,), dtype=i32, device=dev)
        self.counts = torch.empty((N + M,), dtype=i32, device=dev)
        self.f = torch.empty((N + M,), dtype=f32, device=dev)
        self.P = torch.empty((N + M,), dtype=f32, device=dev)
        self.scalars = torch.empty((3,), dtype=f32, device=dev)
        self.ws = torch.empty((max(workspace_bytes(self.dims, MOE_WS_LAYER), 256),), dtype=torch.uint8,
                              device=dev)
        p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
        self.params = LayerParams(p(self.x), p(self.w_router), self.null_bias, p(self.null_bias_tok),
                                  p(self.w_gate), p(self.w_up), p(self.w_down), p(self.ws_gate),
                                  p(self.ws_up), p(self.ws_down), p(self.null_value))
        self.aux_full = AuxOut(p(self.logits), p(self.topk_idx), p(self.topk_w), p(self.n_real),
                               p(self.offsets), p(self.counts), p(self.f), p(self.P), p(self.scalars))

    def forward(self, aux=True, stream=None):
        moe_layer_forward(self.dims, self.params, self.y, self.aux_full if aux else None, self.ws,
                          stream=stream)
        return self.y

    GRADS = ("dx", "dw_router", "dw_gate", "dw_up", "dw_down", "dws_gate", "dws_up", "dws_down")

    def _backward_buffers(self):
        if getattr(self, "grads", None) is None:
            cfg, dev, f32 = self.cfg, self.x.device, torch.float32
            N, d, F, Fs = cfg.n_experts, cfg.d_model, cfg.d_ff, cfg.d_ff_shared
            shapes = dict(dx=(self.T, d), dw_router=(N + 1, d), dw_gate=(N, F, d), dw_up=(N, F, d),
                          dw_down=(N, d, F), dws_gate=(Fs, d), dws_up=(Fs, d), dws_down=(d, Fs))
            self.grads = {k: torch.empty(v, dtype=f32, device=dev) if (Fs or not k.startswith("dws")) else None
                          for k, v in shapes.items()}
            p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
            self.grads_struct = LayerGrads(*(p(self.grads[k]) for k in self.GRADS))
            self.ws_bwd = torch.empty((max(workspace_bytes(self.dims, MOE_WS_BACKWARD), 256),),
                                      dtype=torch.uint8, device=dev)
            self.aux_train = AuxOut(None, None, None, None, None, p(self.counts), None, p(self.P),
                                    p(self.scalars))

    def backward(self, dy, alpha=0.0, beta=0.0, stream=None):
        """Gradients of <dy, y> + alpha L_bal + beta L_z (float32 device tensors,
        allocated on the first call and reused)."""
        self._backward_buffers()
        moe_layer_backward(self.dims, self.params, dy, alpha, beta, self.grads_struct, self.ws_bwd,
                           stream=stream)
        return self.grads

    def forward_train(self, stream=None):
        """The forward that keeps its routing and pre-activations in the backward's
        workspace (counts, P and scalars are written too; the routing outputs are not)."""
        self._backward_buffers()
        moe_layer_forward_train(self.dims, self.params, self.y, self.aux_train, self.ws_bwd, stream=stream)
        return self.y

    def backward_saved(self, dy, alpha=0.0, beta=0.0, stream=None):
        """backward() from the state of the last forward_train() call."""
        self._backward_buffers()
        moe_layer_backward_saved(self.dims, self.params, dy, alpha, beta, self.grads_struct, self.ws_bwd,
                                 stream=stream)
        return self.grads

    def validate(self):
        """True when x, the router, the expert weights and the null biases are free of
        NaN (and, except for the null biases, of infinities); synchronises."""
        from . import moe_validate_inputs
        return moe_validate_inputs(self.dims, self.params, self.ws)

    def results(self):
        """Host copies of every output (synchronises)."""
        torch.cuda.synchronize()
        names = ("y", "logits", "topk_idx", "topk_w", "n_real", "offsets", "counts", "f", "P", "scalars")
        return {n: to_host(getattr(self, n)) for n in names}
