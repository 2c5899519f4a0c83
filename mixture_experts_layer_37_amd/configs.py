"""The five MoE-layer workloads this library is measured and tested on.

Shapes follow the pages' own workloads:
  * tiny     -- a fp32 correctness case small enough for a pure CPU check;
  * small    -- 8 x FFN(2048, 8192), top-2: the ``moe.ExpertParallel`` usage example
                (hnwysp.cn/news/132341, section 3.2);
  * mixtral  -- x[1024*8, 4096] with expert weights [8, 4096, 14336]: the fused-operator
                example and the MindSpeed Mixtral flags (lshu.cn/news/82007, sections 3-4);
  * cap32    -- "MoE-32E" with top-2 routing (gitcode.csdn.net, "ops-transformer 仓库 - MoE
                算子优化实战", Step 2 config.json and Step 4 results) with capacity_factor 1.2
                (hnwysp.cn/news/132341, section 3.2);
  * fine     -- batch 8 x seq 4096 (same gitcode page, Step 4 benchmark command) on a
                128-expert, top-8 layer (the 128-expert example of that page's introduction).
"""
from dataclasses import dataclass, field, replace
from typing import Optional

SWIGLU = "swiglu"
GELU = "gelu"
BF16 = "bf16"
F32 = "f32"


@dataclass(frozen=True)
class MoEConfig:
    name: str
    tokens: int
    hidden: int
    inter: int
    experts: int
    top_k: int
    activation: str = SWIGLU
    dtype: str = BF16
    capacity_factor: float = 0.0      # <= 0: no capacity limit
    renormalize: bool = True
    # gate-bias recipe: None, ("normal", variance) or ("zipf", s)
    bias: Optional[tuple] = None
    router_std: Optional[float] = None  # default 1/sqrt(hidden)
    # "topk", or "threshold": experts with softmax score > threshold (<= 0: 1/E), at most
    # top_k of them
    routing: str = "topk"
    threshold: float = 0.0
    # expert weight layout handed to the library: "plain" (row-major) or "packed" (repacked
    # once into MFMA operand order by moe_pack_expert_weight; bf16 forward only)
    weights: str = "plain"
    # auxiliary load-balancing loss coefficient of the backward (0: off)
    aux_loss_coeff: float = 0.0
    description: str = field(default="", compare=False)

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)

    @property
    def assignments(self) -> int:
        return self.tokens * self.top_k


TINY = MoEConfig(
    "tiny", tokens=64, hidden=64, inter=128, experts=8, top_k=2, activation=GELU, dtype=F32,
    description="tiny fp32 GELU layer, 64 tokens, 8 experts, top-2")
SMALL = MoEConfig(
    "small", tokens=4096, hidden=2048, inter=8192, experts=8, top_k=2,
    bias=("normal", 0.5),
    description="4096 tokens, H 2048, I 8192, 8 experts, top-2, SwiGLU, gate bias N(0,0.5)")
MIXTRAL = MoEConfig(
    "mixtral", tokens=8192, hidden=4096, inter=14336, experts=8, top_k=2,
    description="8192 tokens (8 x 1024), H 4096, I 14336, 8 experts, top-2, SwiGLU")
CAP32 = MoEConfig(
    "cap32", tokens=8192, hidden=4096, inter=14336, experts=32, top_k=2, capacity_factor=1.2,
    bias=("zipf", 1.1),
    description="8192 tokens, H 4096, I 14336, 32 experts, top-2, capacity factor 1.2, "
                "Zipf(1.1) expert-popularity gate bias")
FINE = MoEConfig(
    "fine", tokens=32768, hidden=2048, inter=1408, experts=128, top_k=8, bias=("normal", 1.0),
    description="32768 tokens (8 x 4096), H 2048, I 1408, 128 experts, top-8, SwiGLU, "
                "gate bias N(0,1)")

# Threshold routing on the Mixtral shape: every expert whose softmax score exceeds 1/E,
# uncapped (top_k = E slots), renormalised (intelliparadigm.com page, section 3.2.1).
MIXTRAL_THRESHOLD = MIXTRAL.with_(
    name="mixtral_threshold", top_k=8, routing="threshold",
    description="8192 tokens (8 x 1024), H 4096, I 14336, 8 experts, threshold routing "
                "(score > 1/E, uncapped), SwiGLU")

CONFIGS = {c.name: c for c in (TINY, SMALL, MIXTRAL, CAP32, FINE, MIXTRAL_THRESHOLD)}


def get(name: str) -> MoEConfig:
    return CONFIGS[name]
