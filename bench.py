#!/usr/bin/env python3
"""Throughput of the null-expert token-choice MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-sweep] [--no-cpu]

A step is one moe_layer_forward call (route, permute, gather, grouped SwiGLU
GEMMs, shared expert, combine, statistics) over one batch of synthetic tokens
already resident in HBM. The headline workload is the Qwen3-1.7B-shaped layer at
rho = 0.25 (T=16384, d_model=2048, N=64 experts of d_ff=1536, shared expert
d_ff=1536, K=8, M=192, null bias calibrated to 2 real experts per token), the
shape the rho sweep runs at. Real-expert FLOPs count only the slots routed to real
experts (6 d d_ff per slot); the shared expert's FLOPs (6 d d_ff_shared per
token) are reported beside them.

Besides the JSON line's required fields it reports, per kernel, the average
launch time measured with HIP events on the launch stream and the algorithmic
bytes / FLOPs per launch; the rho sweep and the other workloads (timed only);
the decode regime; the backward pass; and the CPU oracle's throughput on a
bounded sample. Prints exactly one JSON line on stdout.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-sweep", action="store_true", help="skip the rho sweep and other workloads")
    ap.add_argument("--with-backward", action="store_true",
                    help="time the backward pass even with --no-sweep (it runs with the sweep anyway)")
    ap.add_argument("--with-decode", action="store_true",
                    help="time the decode regime even with --no-sweep (it runs with the sweep anyway)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--kernel-iters", type=int, default=20)
    ap.add_argument("--workload", default="qwen3_1p7b_rho0p25",
                    help="configuration of the timed layer and kernel table (the headline by default; "
                         "another one for profiling runs)")
    ap.add_argument("--copy-ref", action="store_true",
                    help="also run three 256 MiB device copies: the reference that scales the "
                         "FETCH_SIZE / WRITE_SIZE counters (token_choice_routing_amd.traffic)")
    return ap.parse_args()


COPY_REF_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timer:
    """Launch timing with HIP events recorded on torch's current stream (the stream
    every entry point is given). The events are created with
    hipEventDisableSystemFence: a default timing event makes its release a
    system-scope fence (L2 write-back and invalidate), which lands inside a
    single-launch measurement. The runtime is the libamdhip64 that torch loaded."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, torch):
        import ctypes
        self.torch = torch
        self.ct = ctypes
        torch.cuda.init()
        with open("/proc/self/maps") as f:
            paths = [ln.split()[-1] for ln in f if "libamdhip64.so" in ln]
        if not paths:
            raise RuntimeError("libamdhip64 is not loaded")
        self.hip = ctypes.CDLL(paths[0])
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def _events(self, n):
        evs = []
        for _ in range(n):
            e = self.ct.c_void_p()
            if self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            evs.append(e)
        return evs

    def _elapsed_us(self, a, b):
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value * 1e3

    def _record(self, e):
        if self.hip.hipEventRecord(e, self.ct.c_void_p(self.torch.cuda.current_stream().cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def _free(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)

    def run(self, fn, iters, warmup=2):
        torch = self.torch
        for _ in range(warmup):
            fn()
        a, b = self._events(2)
        torch.cuda.synchronize()
        self._record(a)
        for _ in range(iters):
            fn()
        self._record(b)
        torch.cuda.synchronize()
        us = self._elapsed_us(a, b) / iters
        self._free([a, b])
        return us   # microseconds per call

    def run_cold(self, fn, iters, flush):
        """Average of single launches, each after a flush (outside the timed events)."""
        torch = self.torch
        fn()
        evs = self._events(2 * iters)
        for i in range(iters):
            flush()
            self._record(evs[2 * i])
            fn()
            self._record(evs[2 * i + 1])
        torch.cuda.synchronize()
        us = sum(self._elapsed_us(evs[2 * i], evs[2 * i + 1]) for i in range(iters)) / iters
        self._free(evs)
        return us


class Flush:
    """Evicts earlier data from the caches by reading 512 MB, twice the 256 MB
    last-level cache, with one reduction kernel. A read leaves clean lines behind; a
    write flush would leave the last-level cache full of dirty lines, and the next
    kernel would then pay for writing them back to HBM (measured: the routed gate/up
    launch goes from ~53 us to ~89 us at 2048 tokens), which is not its own traffic."""

    def __init__(self, torch):
        self.buf = torch.ones((128 << 20,), dtype=torch.float32, device="cuda")
        self.sink = torch.empty((), dtype=torch.float32, device="cuda")
        self.torch = torch

    def __call__(self):
        self.torch.sum(self.buf, dim=0, out=self.sink)


def routed_flops(cfg, R):
    """Real-expert FLOPs of the routed slots: 6 d d_ff per real slot (gate, up, down)."""
    return 6.0 * cfg.d_model * cfg.d_ff * R


def shared_flops(cfg, T):
    return 6.0 * cfg.d_model * cfg.d_ff_shared * T


def time_layer(torch, layer, steps, warmup):
    for _ in range(warmup):
        layer.forward()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(s)
    for _ in range(steps):
        layer.forward()
    b.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return a.elapsed_time(b) / steps, wall * 1e3 / steps


def kernel_table(torch, tcr, layer, iters):
    """Each stage through its own entry point, on the layer's own inputs."""
    cfg, dims = layer.cfg, layer.dims
    T, d, N, M, K, f, fs = layer.T, cfg.d_model, cfg.n_experts, cfg.n_null, cfg.top_k, cfg.d_ff, cfg.d_ff_shared
    Rmax = T * min(K, N)
    dev, i32, f32, bf = "cuda", torch.int32, torch.float32, torch.bfloat16
    E = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)  # noqa: E731
    logits, topk, tw, nr = E((T, N + 1), f32), E((T, K), i32), E((T, K), f32), E((T,), i32)
    ws_r = E((max(tcr.workspace_bytes(dims, tcr.MOE_WS_ROUTE), 16),), torch.uint8)
    counts, offsets = E((N,), i32), E((N + 1,), i32)
    perm, slot = E((Rmax,), i32), E((T, K), i32)
    xp = E((Rmax, d), bf)
    ws_p = E((max(tcr.workspace_bytes(dims, tcr.MOE_WS_PERMUTE), 16),), torch.uint8)
    h, yp = E((Rmax, f), bf), E((Rmax, d), f32)
    hs = E((T, max(fs, 8)), bf)
    ys = E((T, d), f32) if fs else None
    y = E((T, d), bf)
    P = N + M
    fo, Po, co, sc = E((P,), f32), E((P,), f32), E((P,), i32), E((3,), f32)
    ws_a = E((tcr.workspace_bytes(dims, tcr.MOE_WS_AUX),), torch.uint8)

    def route():
        tcr.moe_route(dims, layer.x, layer.w_router, layer.null_bias, layer.null_bias_tok, None, logits,
                      topk, tw, nr, ws_r)

    def permute():
        tcr.moe_permute(dims, topk, None, counts, offsets, perm, slot, None, ws_p)

    def permute_gather():
        tcr.moe_permute(dims, topk, layer.x, counts, offsets, perm, slot, xp, ws_p)

    def gate_up_layer():
        tcr.moe_expert_gate_up(dims, layer.x, perm, offsets, layer.w_gate, layer.w_up, layer.ws_gate,
                               layer.ws_up, h, hs if fs else None)

    def gemm1():
        tcr.moe_grouped_gemm(dims, tcr.MOE_GEMM_GATE_UP, N, f, d, Rmax, xp, offsets, layer.w_gate,
                             layer.w_up, h)

    def gemm2():
        tcr.moe_grouped_gemm(dims, tcr.MOE_GEMM_DOWN, N, d, f, Rmax, h, offsets, layer.w_down, None, yp)

    def sgemm1():
        tcr.moe_grouped_gemm(dims, tcr.MOE_GEMM_GATE_UP, 1, fs, d, T, layer.x, None, layer.ws_gate,
                             layer.ws_up, hs)

    def sgemm2():
        tcr.moe_grouped_gemm(dims, tcr.MOE_GEMM_DOWN, 1, d, fs, T, hs, None, layer.ws_down, None, ys)

    def combine():
        tcr.moe_combine(dims, yp, slot, tw, ys, y)

    def aux():
        tcr.moe_aux_stats(dims, logits, topk, fo, Po, co, sc, ws_a)

    tm = Timer(torch)
    flush = Flush(torch)
    route()
    permute_gather()
    torch.cuda.synchronize()
    off_h = offsets.cpu().numpy()
    R = int(off_h[-1])
    active = int((off_h[1:] > off_h[:-1]).sum())
    rows = {}

    def add(name, us, nbytes, flops=0.0, launches=1, us_warm=None):
        rows[name] = {"us": round(us, 3), "bytes": int(nbytes), "flops": float(flops),
                      "GB_s": round(nbytes / us / 1e3, 1), "TFLOP_s": round(flops / us / 1e6, 2),
                      "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                      "mfma_frac": round(flops / us / 1e6 / BF16_PEAK_TFLOPS, 4), "launches": launches}
        if us_warm is not None:
            rows[name]["us_warm"] = round(us_warm, 3)
            rows[name]["mfma_frac_warm"] = round(flops / us_warm / 1e6 / BF16_PEAK_TFLOPS, 4)

    t_route = tm.run(route, iters)
    add("route", t_route, T * d * 2 + 4 * (N + 1) * d + 4 * T * (N + 1) + 8 * T * K + 4 * T,
        2.0 * T * d * (N + 1), 2)
    t_perm = tm.run(permute, iters)
    add("permute", t_perm, 4 * T * K + 4 * R + 4 * T * K + 4 * (2 * N + 1), 0, 3)
    t_pg = tm.run(permute_gather, iters)
    add("gather", max(t_pg - t_perm, 1e-3), 2 * R * d * 2 + 4 * R)
    # GEMMs: "us" after a last-level-cache flush (the roofline figure), "us_warm" back to back
    add("gate_up_layer", tm.run_cold(gate_up_layer, iters, flush),
        T * d * 2 + active * 2 * f * d * 2 + R * f * 2 + (2 * fs * d * 2 + T * fs * 2 if fs else 0),
        4.0 * R * d * f + 4.0 * T * d * fs, us_warm=tm.run(gate_up_layer, iters))
    add("gemm_gate_up", tm.run_cold(gemm1, iters, flush), R * d * 2 + active * 2 * f * d * 2 + R * f * 2,
        4.0 * R * d * f, us_warm=tm.run(gemm1, iters))
    add("gemm_down", tm.run_cold(gemm2, iters, flush), R * f * 2 + active * d * f * 2 + R * d * 4,
        2.0 * R * d * f, us_warm=tm.run(gemm2, iters))
    if fs:
        add("shared_gate_up", tm.run_cold(sgemm1, iters, flush), T * d * 2 + 2 * fs * d * 2 + T * fs * 2,
            4.0 * T * d * fs, us_warm=tm.run(sgemm1, iters))
        add("shared_down", tm.run_cold(sgemm2, iters, flush), T * fs * 2 + d * fs * 2 + T * d * 4,
            2.0 * T * d * fs, us_warm=tm.run(sgemm2, iters))
    add("combine", tm.run(combine, iters), R * d * 4 + (T * d * 4 if fs else 0) + T * d * 2 + 8 * T * K)
    add("aux_stats", tm.run(aux, iters), 4 * T * (N + 1) + 4 * T * K, 0, 3)
    return rows, R


def roofline(k):
    """Dominant-kernel roofline object from one kernel_table row."""
    ai = k["flops"] / max(k["bytes"], 1)
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai >= ridge:
        return {"bound": "mfma", "achieved": k["TFLOP_s"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(k["TFLOP_s"] / BF16_PEAK_TFLOPS, 4), "traffic": None}
    return {"bound": "hbm", "achieved": k["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(k["GB_s"] / HBM_PEAK_GBS, 4), "traffic": None}


def traffic_from_profiles(kernel, workload):
    """(HBM bytes per launch, profiled kernel name) measured with rocprofv3 counters,
    when a summary for this launch and workload is committed under profiles/ (else
    None, None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None, None
    try:
        ent = json.load(open(path)).get(f"{kernel}@{workload}")
    except (ValueError, OSError):
        return None, None
    return (None, None) if ent is None else (ent.get("bytes_per_launch"), ent.get("kernel"))


def cpu_baseline(wl_full, budget_s=15.0, Ts=512):
    """The CPU oracle as it stands, on the first Ts tokens of the headline workload
    (same weights, same per-token biases), repeated until about budget_s seconds of
    CPU work. NumPy's BLAS runs on its default thread pool; the threads it used,
    the host cores this process may run on and the BLAS library are reported."""
    import copy
    import numpy as np
    from oracle import moe_oracle as O
    blas, threads = "unknown", 1
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if pools:
            threads = max(int(i.get("num_threads", 1)) for i in pools)
            blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in pools}))
    except Exception:  # noqa: BLE001
        pass
    wl = copy.copy(wl_full)
    wl.x = np.ascontiguousarray(wl_full.x[:Ts])
    if wl_full.null_bias_tok is not None:
        wl.null_bias_tok = np.ascontiguousarray(wl_full.null_bias_tok[:Ts])
    O.layer_forward(wl)            # warm caches
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        O.layer_forward(wl)
        n += 1
    el = time.perf_counter() - t0
    return {"value": round(n * Ts / el, 1), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "host_cores_available": len(os.sched_getaffinity(0)), "blas": blas,
            "sample": f"first {Ts} tokens of the headline workload {wl_full.cfg.name} (same weights and "
                      f"null bias), float64 NumPy oracle (whole layer: router, selection, sort, "
                      f"expert FFNs, combine, statistics), {n} layer forwards in {el:.1f} s"}


def sweep(torch, tcr, steps, warmup, base=None):
    """Other workloads, timed only: the rho sweep at the Qwen3-1.7B shape, the
    matched-FLOPs pair at T=8192, the modality-skewed mix, and the rho = 0.5
    Qwen3-0.6B shape with copy and with constant null slots (the zero-compute
    variants that add w x or w v in the combine)."""
    import copy
    from token_choice_routing_amd.layer import MoeLayer
    from workloads import CONFIGS, MATCHED_PAIR, SWEEP, generate
    from workloads.gen import null_bias_for
    out = []
    base = base if base is not None else generate(CONFIGS["qwen3_1p7b_rho0p25"])
    base_layer = None
    names = list(SWEEP) + ["modality_skew_rho0p5"]
    for name in names:
        cfg = SWEEP.get(name) or CONFIGS[name]
        if cfg.x_kind == "modality":
            wl = generate(cfg, experts=False)
            wl.w_gate, wl.w_up, wl.w_down = base.w_gate, base.w_up, base.w_down
        else:
            wl = copy.copy(base)
            wl.cfg = cfg
            wl.null_bias, wl.null_bias_tok = null_bias_for(cfg)
        layer = MoeLayer(wl, weights_from=base_layer)
        if base_layer is None:
            base_layer = layer
        out.append(measure(torch, layer, steps, warmup))
        log(f"  {name}: {out[-1]}")
    c1 = generate(CONFIGS["qwen3_0p6b_rho0p5"])
    l1 = None
    for name in ("matched_k2_rho1", "matched_k4_rho0p5"):
        cfg = MATCHED_PAIR[name]
        wl = copy.copy(c1)
        wl.cfg = cfg
        wl.null_bias, wl.null_bias_tok = null_bias_for(cfg)
        layer = MoeLayer(wl, weights_from=l1)
        l1 = l1 or layer
        out.append(measure(torch, layer, steps, warmup))
        log(f"  {name}: {out[-1]}")
    from dataclasses import replace
    for kind in ("zero", "copy", "constant"):
        cfg = replace(CONFIGS["qwen3_0p6b_rho0p5"], null_kind=kind, name=f"qwen3_0p6b_rho0p5_{kind}")
        wl = generate(cfg, experts=False, bias=False)
        wl.w_gate, wl.w_up, wl.w_down = c1.w_gate, c1.w_up, c1.w_down
        wl.ws_gate, wl.ws_up, wl.ws_down = c1.ws_gate, c1.ws_up, c1.ws_down
        wl.null_bias, wl.null_bias_tok = null_bias_for(CONFIGS["qwen3_0p6b_rho0p5"])
        layer = MoeLayer(wl)
        out.append(measure(torch, layer, steps, warmup))
        log(f"  {cfg.name}: {out[-1]}")
        del layer
    return out


def measured_peaks(torch):
    """This GPU's attainable rates: a 1 GiB device copy (bytes read + written), a
    large bf16 GEMM through torch (hipBLASLt), and hipBLASLt on one dense GEMM with
    the FLOPs of the headline layer's routed gate/up (32768 x 3072 x 2048)."""
    tm = Timer(torch)
    n = 1 << 30
    a = torch.ones((n,), dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    us_c = tm.run(lambda: b.copy_(a), 10)
    del a, b
    m = 8192
    x = torch.randn((m, m), device="cuda").to(torch.bfloat16).contiguous()
    y = torch.randn((m, m), device="cuda").to(torch.bfloat16).contiguous()
    us_g = tm.run(lambda: torch.matmul(x, y), 10)
    del x, y
    a = torch.randn((32768, 2048), device="cuda").to(torch.bfloat16)
    b = torch.randn((3072, 2048), device="cuda").to(torch.bfloat16)
    bt = b.t()
    us_s = tm.run(lambda: torch.matmul(a, bt), 10)
    del a, b, bt
    torch.cuda.empty_cache()
    return {"copy_GB_s": round(2 * n / us_c / 1e3, 1), "copy": "1 GiB device-to-device copy, read + write",
            "bf16_gemm_TFLOP_s": round(2.0 * m ** 3 / us_g / 1e6, 1),
            "gemm": "8192 x 8192 x 8192 bf16 torch.matmul (hipBLASLt)",
            "bf16_gemm_gate_up_shape_TFLOP_s": round(2.0 * 32768 * 3072 * 2048 / us_s / 1e6, 1),
            "gemm_gate_up_shape": "32768 x 2048 times 2048 x 3072 bf16 torch.matmul (hipBLASLt), one dense "
                                  "GEMM with the routed gate/up FLOPs of the headline layer",
            "datasheet": {"hbm_GB_s": HBM_PEAK_GBS, "bf16_TFLOP_s": BF16_PEAK_TFLOPS}}


def decode_sweep(torch, base, main_layer, steps):
    """Small token counts at the headline shape (the decode regime): few rows per
    expert, so the layer reads the weights of the experts it touches. Reported as
    the rate on those weight bytes, with the last-level cache flushed before every
    call (weights come from HBM, as when the other layers of a model ran in between)
    and back to back."""
    from token_choice_routing_amd.layer import MoeLayer
    out = []
    flush = Flush(torch)
    tm = Timer(torch)
    cfg = base.cfg
    for Ts in (1, 16, 64, 256):
        layer = MoeLayer(base, T=Ts, weights_from=main_layer)
        layer.forward()
        torch.cuda.synchronize()
        off = layer.offsets.cpu().numpy()
        active = int((off[1:] > off[:-1]).sum())
        wbytes = (active * 3 * cfg.d_model * cfg.d_ff + 3 * cfg.d_model * cfg.d_ff_shared) * 2 \
            + 4 * (cfg.n_experts + 1) * cfg.d_model
        cold = tm.run_cold(layer.forward, steps, flush)
        warm = tm.run(layer.forward, steps)
        out.append({"workload": f"decode_T{Ts}", "T": Ts, "active_experts": active,
                    "weight_bytes": wbytes, "us_cold": round(cold, 2), "us_warm": round(warm, 2),
                    "weight_GB_s_cold": round(wbytes / cold / 1e3, 1),
                    "hbm_frac_cold": round(wbytes / cold / 1e3 / HBM_PEAK_GBS, 4)})
        log(f"  decode T={Ts}: {out[-1]}")
    return out


def backward_bench(torch, layers, steps, warmup):
    """moe_layer_backward (gradients of <dy, y> + 2e-2 L_bal + 1e-3 L_z, routing and
    expert pre-activations recomputed from x) on each layer, timed with events on the
    current stream; beside it the training pair moe_layer_forward_train +
    moe_layer_backward_saved (the forward keeps that state, the backward reads it). TFLOP/s are counted on the gradient contractions of the real
    slots and the shared expert (2 x the forward's: data and weight gradients,
    12 d d_ff per row); the recomputation (the forward's gate/up for routed rows and
    for the shared expert) is reported as executed FLOPs beside them."""
    out = []
    for layer in layers:
        cfg = layer.cfg
        g = torch.Generator(device="cuda").manual_seed(0)
        dy = torch.randn((layer.T, cfg.d_model), generator=g, device="cuda").to(torch.bfloat16)
        for _ in range(warmup):
            layer.backward(dy, 2e-2, 1e-3)
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        for _ in range(steps):
            layer.backward(dy, 2e-2, 1e-3)
        b.record(s)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        fwd_ms, _ = time_layer(torch, layer, steps, 2)  # also fills the holder's offsets
        R = int(layer.offsets[-1].item())
        d, F, Fs, T = cfg.d_model, cfg.d_ff, cfg.d_ff_shared, layer.T

        def timed(fn):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            a.record(s)
            for _ in range(steps):
                fn()
            b.record(s)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / steps

        # the training pair: a forward that keeps its routing and pre-activations, and the
        # backward that reads them instead of recomputing (each timed alone, then as a step)
        train_fwd_ms = timed(lambda: layer.forward_train())
        saved_ms = timed(lambda: layer.backward_saved(dy, 2e-2, 1e-3))
        train_step_ms = timed(lambda: (layer.forward_train(), layer.backward_saved(dy, 2e-2, 1e-3)))
        useful = 12.0 * d * F * R + 12.0 * d * Fs * T
        executed = useful + 4.0 * d * F * R + 4.0 * d * Fs * T
        out.append({"workload": cfg.name, "T": T, "real_slots": R, "ms": round(ms, 4),
                    "forward_ms": round(fwd_ms, 4), "tokens_per_s": round(T / ms * 1e3, 1),
                    "grad_tflops": round(useful / ms / 1e9, 2),
                    "grad_mfma_frac": round(useful / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
                    "executed_tflops": round(executed / ms / 1e9, 2),
                    "saved": {"forward_train_ms": round(train_fwd_ms, 4), "backward_saved_ms": round(saved_ms, 4),
                              "train_step_ms": round(train_step_ms, 4),
                              "stateless_step_ms": round(fwd_ms + ms, 4),
                              "grad_tflops": round(useful / saved_ms / 1e9, 2),
                              "grad_mfma_frac": round(useful / saved_ms / 1e9 / BF16_PEAK_TFLOPS, 4)}})
        log(f"  backward {cfg.name}: {out[-1]}")
    return out


def measure(torch, layer, steps, warmup):
    ms, _ = time_layer(torch, layer, steps, warmup)
    cfg = layer.cfg
    R = int(layer.offsets[-1].item())
    fl = routed_flops(cfg, R)
    fs = shared_flops(cfg, layer.T)
    seg = layer.offsets.diff().double()
    out = {"workload": cfg.name, "T": layer.T, "K": cfg.top_k, "M": cfg.n_null,
           "rho_nominal": round(cfg.rho_nominal, 4), "rho_realised": round(R / (layer.T * cfg.top_k), 4),
           "real_slots": R, "ms": round(ms, 4), "tokens_per_s": round(layer.T / ms * 1e3, 1),
           "real_expert_tflops": round(fl / ms / 1e9, 2),
           "real_expert_mfma_frac": round(fl / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
           "executed_tflops": round((fl + fs) / ms / 1e9, 2),
           "executed_mfma_frac": round((fl + fs) / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
           # expert segment lengths (rows per expert): the grouped GEMM's load balance
           "segments": {"min": int(seg.min().item()), "max": int(seg.max().item()),
                        "cv": round(float((seg.std(unbiased=False) / seg.mean().clamp(min=1e-9)).item()), 3)}}
    if cfg.x_kind == "modality":
        # compute intensity r / K per class (the first round(vision_frac T) tokens are vision)
        vT = int(round(cfg.vision_frac * layer.T))
        r = layer.n_real.double()
        out["intensity"] = {"vision": round(float(r[:vT].mean().item()) / cfg.top_k, 4),
                            "text": round(float(r[vT:].mean().item()) / cfg.top_k, 4)}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path is built and measured for one GPU's share).", file=sys.stderr)
        sys.exit(2)
    import torch

    import token_choice_routing_amd as tcr
    from token_choice_routing_amd.layer import MoeLayer
    from workloads import CONFIGS, generate

    if args.workload not in CONFIGS:
        print(f"unknown workload {args.workload}; one of {sorted(CONFIGS)}", file=sys.stderr)
        sys.exit(2)
    tcr.load_library()
    torch.cuda.set_device(0)
    cfg = CONFIGS[args.workload]
    log(f"bench: generating {cfg.name}")
    wl = generate(cfg)
    layer = MoeLayer(wl)
    log("bench: warmup + timed steps")
    ms, wall_ms = time_layer(torch, layer, args.steps, args.warmup)
    R = int(layer.offsets[-1].item())
    T = layer.T
    tok_s = T / ms * 1e3
    fl, fs = routed_flops(cfg, R), shared_flops(cfg, T)
    log(f"bench: {ms:.4f} ms/step (events), {wall_ms:.4f} ms/step (wall), R={R}")
    if args.copy_ref:
        src = torch.ones((COPY_REF_BYTES,), dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log("bench: per-kernel timing")
    kernels, _ = kernel_table(torch, tcr, layer, args.kernel_iters)
    dom = "gate_up_layer"
    rl = roofline(kernels[dom])
    traffic, kname = traffic_from_profiles(dom, cfg.name)
    rl["kernel"] = (f"{kname or 'grouped GEMM <0, 2>'}: the layer's gate/up + SwiGLU launch (routed rows "
                    "of x read through perm_token, and the shared expert) through moe_expert_gate_up, "
                    "caches flushed by a 512 MB read before each timed launch")
    rl["flops_per_launch"] = kernels[dom]["flops"]
    rl["us_per_launch"] = kernels[dom]["us"]
    rl["traffic"] = traffic
    line = {
        "metric": "MoE-layer tokens/s + real-expert TFLOP/s (% bf16 MFMA peak) vs rho",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights, fp32 router)",
        "config": {"workload": f"{cfg.name}: T={T}, d_model={cfg.d_model}, N={cfg.n_experts}, "
                               f"M={cfg.n_null}, K={cfg.top_k}, d_ff={cfg.d_ff}, shared d_ff={cfg.d_ff_shared}",
                   "T": T, "d_model": cfg.d_model, "n_experts": cfg.n_experts, "n_null": cfg.n_null,
                   "top_k": cfg.top_k, "d_ff": cfg.d_ff, "d_ff_shared": cfg.d_ff_shared,
                   "parallelism": "single GPU"},
        "real_slots": R,
        "real_expert_tflops": round(fl / ms / 1e9, 2),
        "real_expert_mfma_frac": round(fl / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
        "shared_expert_tflops": round(fs / ms / 1e9, 2),
        "executed_tflops": round((fl + fs) / ms / 1e9, 2),
        "executed_mfma_frac": round((fl + fs) / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
        "flop_counting": "real_expert_tflops: 6 d d_ff per real slot (routed experts only); "
                         "executed adds the shared expert's 6 d d_ff_shared per token",
        "wall_ms_per_step": round(wall_ms, 4),
        "roofline": rl,
        "kernels": kernels,
    }
    c3 = "qwen3_1p7b_rho0p25"
    if not args.no_sweep:
        log("bench: rho sweep and other workloads")
        line["workloads"] = sweep(torch, tcr, max(5, args.steps // 2), 3, base=wl if cfg.name == c3 else None)
    small = small_layer = None
    if not args.no_sweep or args.with_decode or args.with_backward:
        small = generate(CONFIGS["qwen3_0p6b_rho1"])
        small_layer = MoeLayer(small)
    if not args.no_sweep or args.with_decode:
        log("bench: decode regime (Qwen3-0.6B shape)")
        line["decode"] = decode_sweep(torch, small, small_layer, max(5, args.steps // 2))
    if not args.no_sweep or args.with_backward:
        log("bench: backward")
        big = layer if cfg.name == c3 else MoeLayer(generate(CONFIGS[c3]))
        line["backward"] = backward_bench(torch, [small_layer, big], max(5, args.steps // 2), 2)
        del big
        torch.cuda.empty_cache()
    if not args.no_sweep:
        log("bench: measured peaks")
        line["measured_peaks"] = measured_peaks(torch)
    if not args.no_cpu:
        log("bench: CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
