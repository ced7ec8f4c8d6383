"""Workload shapes of the null-expert MoE layer.

Sources (the pages describing arXiv:2601.15370, "Improving MoE Compute
Efficiency by Composing Weight and Data Sparsity"):
  * Section "Null Expert mechanism" (core formulas) fixes the pool: N real
    experts plus one null logit duplicated M times, top-K over the pool.
  * The training-configuration table (Section "Experimental results") names the
    model family: Qwen3 dense 0.6B / 1.7B upcycled to 64 experts.
  * The "expected active experts" paragraph defines E[K] = rho * k_max, and the
    "solution space preservation" paragraph pairs K^4_{0.5} with K^2_{1.0}.

rho is the expected fraction of selected slots that are real; nominally
rho = N / (N + M). The null-logit bias of the calibrated workloads is stored in
``null_bias.json`` next to this file (written by ``oracle/calibrate.py``).
"""
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    T: int                 # tokens
    d_model: int
    n_experts: int         # N real experts
    n_null: int            # M null copies
    top_k: int             # K
    d_ff: int              # routed expert hidden size
    d_ff_shared: int       # 0 = no shared expert
    dtype: str             # "f32" or "bf16" (activations and expert weights)
    w_std: Optional[float]  # None = 1/sqrt(d_model)
    x_kind: str = "normal"  # "normal" or "modality"
    bias_mode: str = "zero"  # "zero" | "calibrated" | "per_class"
    target_mean_r: Optional[float] = None       # calibrated: mean real experts per token
    class_null_frac: Tuple[float, float] = (0.0, 0.0)  # per_class: (vision, text) null fraction
    vision_frac: float = 0.0
    seed: int = 0
    note: str = ""
    null_kind: str = "zero"  # output of a null slot: "zero", "copy" (the token) or "constant" (a vector)

    @property
    def rho_nominal(self) -> float:
        return self.n_experts / (self.n_experts + self.n_null)

    @property
    def max_rows(self) -> int:
        """Worst-case number of real slots T * min(K, N)."""
        return self.T * min(self.top_k, self.n_experts)

    @property
    def weight_std(self) -> float:
        return self.w_std if self.w_std is not None else self.d_model ** -0.5


C0 = Config("tiny_f32", T=128, d_model=64, n_experts=8, n_null=8, top_k=2, d_ff=128,
            d_ff_shared=0, dtype="f32", w_std=None, bias_mode="zero",
            note="fp32 throughout; x~N(0,1); W~N(0,1/d); null bias 0")
C1 = Config("qwen3_0p6b_rho1", T=2048, d_model=1024, n_experts=64, n_null=0, top_k=2,
            d_ff=768, d_ff_shared=768, dtype="bf16", w_std=0.02, bias_mode="zero",
            note="K^2_{1.0}: plain top-2, shared expert, bf16 with fp32 router")
C2 = Config("qwen3_0p6b_rho0p5", T=8192, d_model=1024, n_experts=64, n_null=64, top_k=4,
            d_ff=768, d_ff_shared=768, dtype="bf16", w_std=0.02, bias_mode="calibrated",
            target_mean_r=2.0, note="K^4_{0.5}: matched expected FLOPs with K^2_{1.0}")
C3 = Config("qwen3_1p7b_rho0p25", T=16384, d_model=2048, n_experts=64, n_null=192, top_k=8,
            d_ff=1536, d_ff_shared=1536, dtype="bf16", w_std=0.02, bias_mode="calibrated",
            target_mean_r=2.0, note="K^8_{0.25}, E[K]=2, 256-slot pool")
C4 = Config("modality_skew_rho0p5", T=16384, d_model=2048, n_experts=64, n_null=64, top_k=8,
            d_ff=1536, d_ff_shared=0, dtype="bf16", w_std=0.02, x_kind="modality",
            bias_mode="per_class", class_null_frac=(0.70, 0.30), vision_frac=0.75,
            note="75% rank-16 'vision' rows routed ~70% to null, 25% text rows ~30%")

CONFIGS = {c.name: c for c in (C0, C1, C2, C3, C4)}
ORDER = [C0.name, C1.name, C2.name, C3.name, C4.name]

# rho sweep at the C3 shape: M = N (1 - rho) / rho, mean real experts calibrated to rho * K.
SWEEP = {}
for _rho, _m in ((1.0, 0), (0.67, 32), (0.5, 64), (0.25, 192)):
    _c = replace(C3, name=f"sweep_rho{_rho:g}", n_null=_m,
                 bias_mode="zero" if _m == 0 else "calibrated",
                 target_mean_r=None if _m == 0 else 8 * (64 / (64 + _m)),
                 note=f"C3 shape at rho={_rho:g}")
    SWEEP[_c.name] = _c

# Matched expected FLOPs at equal T: K^2_{1.0} versus K^4_{0.5} (the C2 workload).
MATCHED_PAIR = {
    "matched_k2_rho1": replace(C1, name="matched_k2_rho1", T=8192, note="K^2_{1.0} at T=8192"),
    "matched_k4_rho0p5": replace(C2, name="matched_k4_rho0p5"),
}


def get_config(name: str) -> Config:
    for table in (CONFIGS, SWEEP, MATCHED_PAIR):
        if name in table:
            return table[name]
    aliases = {f"C{i}": ORDER[i] for i in range(5)}
    if name in aliases:
        return CONFIGS[aliases[name]]
    raise KeyError(name)
