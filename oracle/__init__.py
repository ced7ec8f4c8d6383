"""CPU oracle for the null-expert token-choice MoE layer forward.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, float64 NumPy
statement of what the layer computes. It is imported only by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``.
The HIP library never calls it, and it shares no code with the HIP path: the
only module both sides use is ``workloads`` (seeded input draws, no routing
arithmetic).

Sources, cited by page title and section:
  [Review]  "Improving MoE Compute Efficiency by Composing Weight and Data
            Sparsity" -- paper review of arXiv:2601.15370 (xllm-io), section 3
            "Technical architecture": core formulas, null-expert mechanism,
            expected active experts, threshold interpretation, load-balance
            loss, z-loss, solution-space preservation, implementation.
  [Summary] sciencestack page for arXiv:2601.15370: abstract; captions of
            Figure 3 (rho = real fraction of selected slots) and Figure 4
            (compute intensity = fraction of top-K slots that are real).
  [Primer]  "MoE: sparse activation ..." (quant67 Transformer series, part 44):
            section 3 "router and top-k", section 4.2 auxiliary loss,
            section 4.3 router z-loss.
  [MoE++]   MoE++ zero-computation experts page (pomoai): "Gating mechanism"
            section (top-k, softmax over the k, zero the zero-compute slots,
            renormalise).

Every function is pinned by ``tests/test_oracle_*.py`` against values that do
not come from the oracle itself (brute force, closed forms, hand-derived golden
fixtures under ``tests/golden/``, invariants).
"""
from .moe_oracle import (  # noqa: F401
    router_logits, select, renorm_weights, route, permute, silu, swiglu_ffn,
    expert_ffn_grouped, combine, pool_softmax, aux_stats, layer_forward, layer_dense,
    decisive_gap,
)
