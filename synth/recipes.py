"""Workload recipes: shapes, seeds and value laws of the synthetic inputs.

Shapes follow the Beam MoE block: hidden 5120, 256 routed experts in 8 groups of
32, best 4 groups kept, top-8 experts, expert intermediate 2560, routed scaling
2.5, RMSNorm eps 1e-6 (Transformers "Beam" model page, BeamConfig defaults and
Overview; archdb "Beam-1.0-501B-A23B" fact sheet, MoE and normalisation rows).
The value laws are synthetic by design: no trained weights are used anywhere.

Every tensor is addressed by (seed, tensor id, flat element index) and produced
by the counter-based generator in this package, on the host or on the GPU.
"""
from __future__ import annotations

from dataclasses import dataclass
import math

# Tensor ids: one independent Philox stream per tensor.
TID_X = 1        # hidden states entering the layer, [T, d] bf16
TID_WR = 2       # router weight, [d, E] fp32
TID_BIAS = 3     # per-expert selection bias, [E] fp32
TID_WG = 4       # gate projections, [E, I, d] bf16
TID_WU = 5       # up projections, [E, I, d] bf16
TID_WD = 6       # down projections, [E, d, I] bf16
TID_H = 7        # pre-norm hidden states (large-chunk workload), [T, d] bf16
TID_NORMW = 8    # pre-MLP RMSNorm weight, [d] bf16
TID_HOT = 9      # permutation that picks the hot experts (skewed workload)
TID_RESID = 10   # residual stream entering the post-MLP add, [T, d] fp32
TID_POSTW = 11   # post-MLP RMSNorm weight, [d] bf16


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    T: int
    d: int
    E: int
    n_group: int
    topk_group: int
    top_k: int
    I: int
    scale: float = 2.5
    norm_topk_prob: bool = True
    eps: float = 1e-6
    bias_lo: float = -0.1
    bias_hi: float = 0.1
    hot_experts: int = 0
    hot_bias: float = 0.0
    prenorm: bool = False      # x = RMSNorm(h) fused into the routing read
    seed_base: int = 1000

    @property
    def seed(self) -> int:
        return self.seed_base + self.cfg_id

    @property
    def pairs(self) -> int:
        return self.T * self.top_k

    @property
    def std_in(self) -> float:
        """Standard deviation of Wr, Wg and Wu: 1/sqrt(fan_in) with fan_in = d."""
        return 1.0 / math.sqrt(self.d)

    @property
    def std_down(self) -> float:
        """Standard deviation of Wd: 1/sqrt(fan_in) with fan_in = I."""
        return 1.0 / math.sqrt(self.I)

    def with_T(self, T: int) -> "Workload":
        from dataclasses import replace
        return replace(self, T=T)


_BEAM = dict(d=5120, E=256, n_group=8, topk_group=4, top_k=8, I=2560)

WORKLOADS = {
    0: Workload(0, "tiny", T=128, d=256, E=16, n_group=4, topk_group=2, top_k=4, I=128),
    1: Workload(1, "beam_decode_T64", T=64, **_BEAM),
    2: Workload(2, "beam_prefill_T8192", T=8192, **_BEAM),
    3: Workload(3, "beam_skewed_T4096", T=4096, hot_experts=16, hot_bias=0.5, **_BEAM),
    4: Workload(4, "beam_chunk_T32768_prenorm", T=32768, prenorm=True, **_BEAM),
}


@dataclass(frozen=True)
class DenseWorkload:
    """One dense SwiGLU MLP (the first layers of the model): y = Wd . bf16(silu(Wg . x) * (Wu . x)).
    Inputs use the MoE tensor ids (x: TID_X, Wg: TID_WG, Wu: TID_WU, Wd: TID_WD) under this
    workload's own seed; Wg, Wu are [I, d] and Wd is [d, I]."""
    cfg_id: int
    name: str
    T: int
    d: int
    I: int
    seed_base: int = 1000

    @property
    def seed(self) -> int:
        return self.seed_base + self.cfg_id

    @property
    def std_in(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def std_down(self) -> float:
        return 1.0 / math.sqrt(self.I)

    def with_T(self, T: int) -> "DenseWorkload":
        from dataclasses import replace
        return replace(self, T=T)


DENSE_WORKLOADS = {
    10: DenseWorkload(10, "beam_dense_prefill_T8192", T=8192, d=5120, I=20480),
    11: DenseWorkload(11, "beam_dense_decode_T64", T=64, d=5120, I=20480),
    12: DenseWorkload(12, "dense_mid_T300", T=300, d=512, I=2048),
}
