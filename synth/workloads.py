"""The five synthetic MoE-layer workloads and their input distributions.

Shapes follow the models the pages evaluate on (GPT-2, BERT-Large, Mixtral,
DeepSeek-V2 families in the FlowMoE notes' results table and the FSMoE
abstract); the data are i.i.d. synthetic tensors because no dataset or
trained weights are used:

* x ~ N(0, 1), every weight ~ N(0, 0.02^2) (0.02 is the standard deviation),
  upstream gradient dy ~ N(0, 1);
* only the BERT-Large-shaped workload is imbalanced, through a fixed router
  bias b_e = 2 ln p_e with p the Zipf(s=1.2) law over the E experts (expert 0
  most popular), added to the gate logits.  It stands in for the load
  imbalance that the tutorial's "设备间负载不均衡" and "All-to-All 通信模式 /
  五、性能瓶颈与挑战" parts discuss.

Gating names:
  "softmax_topk"        g_j = softmax(l)[e_j]
  "softmax_topk_renorm" g_j = softmax(l)[e_j] / sum over the chosen k
  "topk_softmax"        g_j = softmax over the k chosen logits
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                      # tokens (batch x sequence, row-major flatten)
    d: int                      # model width
    ffn: int                    # routed expert hidden width
    E: int                      # routed experts
    k: int                      # experts per token
    capacity_factor: float      # > 0: capacity ceil(cf*k*T/E); <= 0: dropless
    gating: str                 # see module docstring
    act: str                    # "gelu" | "swiglu"
    dtype: str                  # "f32" | "bf16"
    ep_ranks: int = 1           # expert-parallel ranks of the send layout
    placement: str = "contiguous"   # | "round_robin"
    n_shared: int = 0           # always-on shared experts
    ffn_shared: int = 0         # hidden width of each shared expert
    zipf_s: float = 0.0         # > 0: router bias 2 ln Zipf(s) probabilities
    aux_coef: float = 0.0       # != 0: balance loss coefficient (loss_coef)
    seed: int = 0x4D6F45        # base seed of the workload's tensors
    w_std: float = 0.02         # weight standard deviation

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def has_bias(self) -> bool:
        return self.zipf_s > 0.0


def _seed(idx: int) -> int:
    return (0x4D6F45 ^ (idx << 32)) & 0xFFFFFFFFFFFFFFFF


WORKLOADS = {
    "switch_tiny_f32": Workload(
        name="switch_tiny_f32", T=512, d=128, ffn=256, E=4, k=1,
        capacity_factor=1.25, gating="softmax_topk", act="gelu", dtype="f32",
        seed=_seed(0)),
    "gpt2s_bf16": Workload(
        name="gpt2s_bf16", T=8 * 1024, d=768, ffn=3072, E=8, k=2,
        capacity_factor=1.25, gating="softmax_topk_renorm", act="gelu",
        dtype="bf16", seed=_seed(1)),
    "bertl_skew_bf16": Workload(
        name="bertl_skew_bf16", T=32 * 512, d=1024, ffn=4096, E=16, k=2,
        capacity_factor=1.0, gating="softmax_topk_renorm", act="gelu",
        dtype="bf16", zipf_s=1.2, seed=_seed(2)),
    "mixtral_bf16": Workload(
        name="mixtral_bf16", T=4 * 4096, d=4096, ffn=14336, E=8, k=2,
        capacity_factor=0.0, gating="topk_softmax", act="swiglu",
        dtype="bf16", seed=_seed(3)),
    "dsv2lite_bf16": Workload(
        name="dsv2lite_bf16", T=16384, d=2048, ffn=1408, E=64, k=6,
        capacity_factor=0.0, gating="softmax_topk", act="swiglu",
        dtype="bf16", ep_ranks=8, n_shared=2, ffn_shared=1408,
        seed=_seed(4)),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def zipf_bias(E: int, s: float):
    """Router bias b_e = 2 ln p_e, p_e = (e+1)^-s / sum_{i=1..E} i^-s.

    Computed in double precision and returned as a list of Python floats;
    callers round to fp32.
    """
    z = sum(i ** (-s) for i in range(1, E + 1))
    return [2.0 * math.log(((e + 1) ** (-s)) / z) for e in range(E)]
