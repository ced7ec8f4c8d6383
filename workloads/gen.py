"""Seeded input generation. No routing or expert arithmetic lives here.

Every tensor has its own PCG64 stream keyed by (seed, tensor id), so a caller
can draw the activations and the router without drawing the expert weights.
Normals are drawn in float32, scaled by the init std in float32 and rounded
once, round-to-nearest-even, to the storage type (bf16 bit patterns held in
uint16 arrays, or float32). Both the oracle and the HIP path read exactly these
arrays.
"""
import hashlib
import json
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import Config

_TID = {"x": 1, "w_router": 2, "w_gate": 3, "w_up": 4, "w_down": 5,
        "ws_gate": 6, "ws_up": 7, "ws_down": 8,
        "vision_basis": 9, "vision_z": 10, "vision_noise": 11, "null_value": 12}

BIAS_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "null_bias.json")


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TID[name]])))


def _normal(seed: int, name: str, shape, std: float, dtype: str) -> np.ndarray:
    rng = _rng(seed, name)
    if len(shape) == 3:   # one expert at a time keeps peak memory at one matrix
        out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
        for e in range(shape[0]):
            z = rng.standard_normal(shape[1:], dtype=np.float32)
            z *= np.float32(std)
            out[e] = bf16_round(z) if dtype == "bf16" else z
        return out
    z = rng.standard_normal(shape, dtype=np.float32)
    z *= np.float32(std)
    return bf16_round(z) if dtype == "bf16" else z


def _modality_x(cfg: Config) -> np.ndarray:
    """Vision rows [0, vT): z B + 0.1 eps with z ~ N(0, I_16), B_ij ~ N(0, 1/16)
    (unit per-coordinate variance, like the text rows); text rows ~ N(0, 1).
    Computed in float64, rounded to float32 and then to the storage type."""
    T, d = cfg.T, cfg.d_model
    vT = int(round(cfg.vision_frac * T))
    basis = _rng(cfg.seed, "vision_basis").standard_normal((16, d)) * 0.25
    z = _rng(cfg.seed, "vision_z").standard_normal((vT, 16))
    noise = _rng(cfg.seed, "vision_noise").standard_normal((vT, d))
    x = np.empty((T, d), dtype=np.float32)
    x[:vT] = (z @ basis + 0.1 * noise).astype(np.float32)
    x[vT:] = _rng(cfg.seed, "x").standard_normal((T - vT, d), dtype=np.float32)
    return bf16_round(x) if cfg.dtype == "bf16" else x


def fingerprint(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


def load_bias_table() -> dict:
    if not os.path.exists(BIAS_FILE):
        return {}
    with open(BIAS_FILE) as f:
        return json.load(f)


@dataclass
class Workload:
    cfg: Config
    x: np.ndarray                      # [T, d]   uint16 (bf16 bits) or float32
    w_router: np.ndarray               # [N+1, d] float32, row N = null logit
    null_bias: float                   # scalar added to the null logit (float32 value)
    null_bias_tok: Optional[np.ndarray]  # [T] float32 or None
    w_gate: Optional[np.ndarray] = None  # [N, d_ff, d]
    w_up: Optional[np.ndarray] = None    # [N, d_ff, d]
    w_down: Optional[np.ndarray] = None  # [N, d, d_ff]
    ws_gate: Optional[np.ndarray] = None  # [d_ffs, d]
    ws_up: Optional[np.ndarray] = None
    ws_down: Optional[np.ndarray] = None  # [d, d_ffs]
    null_value: Optional[np.ndarray] = None  # [d] the constant expert's vector (null_kind "constant")

    def values(self, name: str) -> Optional[np.ndarray]:
        """float64 copy of the exact stored values of one tensor."""
        a = getattr(self, name)
        if a is None:
            return None
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def null_bias_for(cfg: Config, table: Optional[dict] = None):
    """(scalar bias, per-token bias or None) for a workload, from the stored table."""
    if cfg.bias_mode == "zero":
        return 0.0, None
    table = load_bias_table() if table is None else table
    if cfg.name not in table:
        raise KeyError(f"no calibrated null bias stored for {cfg.name}; run oracle/calibrate.py")
    ent = table[cfg.name]
    if cfg.bias_mode == "calibrated":
        return float(np.float32(ent["null_bias"])), None
    vT = int(round(cfg.vision_frac * cfg.T))
    tok = np.empty(cfg.T, dtype=np.float32)
    tok[:vT] = np.float32(ent["null_bias_vision"])
    tok[vT:] = np.float32(ent["null_bias_text"])
    return 0.0, tok


def generate(cfg: Config, experts: bool = True, bias: bool = True, T: Optional[int] = None) -> Workload:
    """Draw one workload. ``experts=False`` skips the expert weights (router-only
    uses); ``bias=False`` leaves the null bias at zero (calibration input);
    ``T`` truncates the token dimension to the first T rows (same values)."""
    dt = cfg.dtype
    x = _modality_x(cfg) if cfg.x_kind == "modality" else _normal(cfg.seed, "x", (cfg.T, cfg.d_model), 1.0, dt)
    w_router = _normal(cfg.seed, "w_router", (cfg.n_experts + 1, cfg.d_model), cfg.weight_std, "f32")
    b, btok = null_bias_for(cfg) if bias else (0.0, None)
    wl = Workload(cfg, x, w_router, b, btok)
    if T is not None:
        wl.x = np.ascontiguousarray(x[:T])
        if btok is not None:
            wl.null_bias_tok = np.ascontiguousarray(btok[:T])
    if experts:
        N, d, f, fs, s = cfg.n_experts, cfg.d_model, cfg.d_ff, cfg.d_ff_shared, cfg.weight_std
        wl.w_gate = _normal(cfg.seed, "w_gate", (N, f, d), s, dt)
        wl.w_up = _normal(cfg.seed, "w_up", (N, f, d), s, dt)
        wl.w_down = _normal(cfg.seed, "w_down", (N, d, f), s, dt)
        if fs:
            wl.ws_gate = _normal(cfg.seed, "ws_gate", (fs, d), s, dt)
            wl.ws_up = _normal(cfg.seed, "ws_up", (fs, d), s, dt)
            wl.ws_down = _normal(cfg.seed, "ws_down", (d, fs), s, dt)
    if cfg.null_kind == "constant":
        wl.null_value = _normal(cfg.seed, "null_value", (cfg.d_model,), 1.0, dt)
    return wl
