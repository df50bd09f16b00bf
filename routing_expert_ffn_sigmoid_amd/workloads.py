"""Workload presets for the DeepSeekMoE layer forward.

Each preset fixes the layer's shapes, routing rule and input distributions.
Shapes follow the pages:
  * V3 routing: 256 routed experts in 8 groups of 32, keep 4 groups, top-8
    ("DeepSeek-V3的Group-Limited Expert Routing与负载均衡优化实践" §1);
    256 routed / 8 active ("DeepSeek MoE：从v1到v3的演进" §DeepSeek-v3 table).
  * v1: softmax gate, fine-grained routed experts plus always-on shared
    experts ("DeepSeek MoE：从v1到v3的演进" §DeepSeek-v1).
  * capacity factor and dropping ("DeepSeek MoE：从v1到v3的演进" §GShard).
  * v2: 160 routed / 6 active experts ("DeepSeek MoE：从v1到v3的演进"
    §DeepSeek-v3 table), device-limited routing over 8 devices keeping the
    3 best, and device-level token dropping at the average device load
    (§DeepSeek-v2).
Sizes not printed on the pages (hidden, intermediate, token counts, weight
scales, the v2 device count and kept-device count) are the workload
definitions of this library's benchmark.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

SOFTMAX, SIGMOID = 0, 1
F32, BF16 = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    N: int
    k: int
    n_groups: int
    topk_groups: int
    group_topn: int
    score_fn: int
    norm_topk: int
    route_scale: float
    capacity: int
    I: int
    n_shared: int
    I_shared: int
    act_dtype: int
    w_dtype: int
    router_dtype: int
    x_std: float
    wg_std: float
    w_std: float
    bias_kind: str  # "none" | "uniform" | "zipf"
    bias_param: float  # half-width of the uniform bias, or the Zipf exponent
    seed: int = 0
    group_capacity: int = 0  # device-level drop: 0 off, -1 average group load

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def assignments(self) -> int:
        return self.T * self.k

    @property
    def w_layout(self) -> int:
        """Expert weight layout the library reads: tiled for bf16, rows for fp32."""
        return 1 if self.w_dtype == BF16 else 0


def capacity_for(T: int, k: int, N: int, factor_num: int = 5, factor_den: int = 4) -> int:
    """Per-expert capacity ceil(factor * T * k / N) in integer arithmetic
    (GShard-style capacity factor, here 1.25 = 5/4)."""
    num = factor_num * T * k
    den = factor_den * N
    return (num + den - 1) // den


TINY = Workload(
    name="tiny_fp32_T64_H128_N16_k4_G4of2", T=64, H=128, N=16, k=4,
    n_groups=4, topk_groups=2, group_topn=2, score_fn=SIGMOID, norm_topk=1,
    route_scale=1.0, capacity=0, I=64, n_shared=1, I_shared=64,
    act_dtype=F32, w_dtype=F32, router_dtype=F32,
    x_std=1.0, wg_std=0.02, w_std=0.02, bias_kind="uniform", bias_param=0.1)

V1 = Workload(
    name="v1_bf16_T4096_H2048_N64_k6_softmax", T=4096, H=2048, N=64, k=6,
    n_groups=1, topk_groups=1, group_topn=2, score_fn=SOFTMAX, norm_topk=0,
    route_scale=1.0, capacity=0, I=1408, n_shared=2, I_shared=1408,
    act_dtype=BF16, w_dtype=BF16, router_dtype=BF16,
    x_std=1.0, wg_std=0.006, w_std=0.006, bias_kind="none", bias_param=0.0)

V3_PREFILL = Workload(
    name="v3_prefill_bf16_T8192_H7168_N256_k8_G8of4", T=8192, H=7168, N=256, k=8,
    n_groups=8, topk_groups=4, group_topn=2, score_fn=SIGMOID, norm_topk=1,
    route_scale=2.5, capacity=0, I=2048, n_shared=1, I_shared=2048,
    act_dtype=BF16, w_dtype=BF16, router_dtype=F32,
    x_std=1.0, wg_std=0.006, w_std=0.006, bias_kind="uniform", bias_param=0.05)

V3_DECODE = V3_PREFILL.with_(name="v3_decode_bf16_T128_H7168_N256_k8_G8of4", T=128)

V3_SKEW = V3_PREFILL.with_(
    name="v3_skew_bf16_T16384_H7168_N256_k8_G8of4_C640", T=16384,
    capacity=capacity_for(16384, 8, 256), bias_kind="zipf", bias_param=1.2)

# v2-shaped routing: softmax gate (raw probability), device-limited routing
# (group score = the group's best logit, 3 of 8 devices kept), device-level
# dropping at the average device load; expert widths as v1.
V2 = Workload(
    name="v2_bf16_T4096_H2048_N160_k6_dev8of3_drop", T=4096, H=2048, N=160, k=6,
    n_groups=8, topk_groups=3, group_topn=1, score_fn=SOFTMAX, norm_topk=0,
    route_scale=1.0, capacity=0, I=1408, n_shared=2, I_shared=1408,
    act_dtype=BF16, w_dtype=BF16, router_dtype=BF16,
    x_std=1.0, wg_std=0.006, w_std=0.006, bias_kind="none", bias_param=0.0,
    group_capacity=-1)

PRESETS = {w.name: w for w in (TINY, V1, V2, V3_PREFILL, V3_DECODE, V3_SKEW)}
SHORT = {"tiny": TINY, "v1": V1, "v2": V2, "v3_prefill": V3_PREFILL,
         "v3_decode": V3_DECODE, "v3_skew": V3_SKEW}


def group_capacity_for(wl: Workload) -> int:
    """The per-group cap a workload's group_capacity stands for (0 = off)."""
    if wl.group_capacity >= 0:
        return wl.group_capacity
    return (wl.T * wl.k + wl.n_groups - 1) // wl.n_groups


def get(name: str) -> Workload:
    if name in SHORT:
        return SHORT[name]
    return PRESETS[name]
