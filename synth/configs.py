"""Workload shapes for the MoE expert layer.

Shape sources (the pages):
  * LatentMoE expert width 2048, 512 experts, top-22: Nemotron 3 Ultra
    interview notes, "concepts" list (LatentMoE item).
  * Skewed load, max/mean expert load about 12 with upper bound 512/22:
    same notes, paragraph after the divergence table (MaxVio).
  * 4 local experts per GPU: same notes, follow-up on the long-context
    parallelism (EP128 -> 4 experts per rank).
Token counts, expert MLP width and the ReLU^2 activation are workload
choices of this library (the pages state none of them).
"""
from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class Config:
    name: str
    tokens: int
    d_model: int
    d_ffn: int
    num_experts: int
    top_k: int
    expert_begin: int
    num_local: int
    dtype: str            # "f32" or "bf16": storage dtype of x, W, dy, h, y, dx
    combine: int          # 1: token-layout outputs (full layer); 0: row-layout (expert shard)
    seed: int
    skew: Optional[str] = None   # None or "zipf"
    zipf_beta: Optional[float] = None  # None: the calibrated value (zipf_beta.json)
    zipf_empty: int = 8          # lowest-ranked experts pushed to -30 (no tokens)
    x_std: float = 0.02
    w_std: float = 0.02

    @property
    def rows_cap(self) -> int:
        """Upper bound on routed rows held by this GPU (each token picks distinct experts)."""
        return self.tokens * min(self.top_k, self.num_local)

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    "tiny_fp32": Config("tiny_fp32", 64, 64, 128, 4, 2, 0, 4, "f32", 1, 1),
    "bf16_e8k2": Config("bf16_e8k2", 4096, 1024, 2048, 8, 2, 0, 8, "bf16", 1, 2),
    "latent_e512k22": Config("latent_e512k22", 4096, 2048, 2048, 512, 22, 0, 512, "bf16", 1, 3),
    "skewed_e512k22": Config("skewed_e512k22", 4096, 2048, 2048, 512, 22, 0, 512, "bf16", 1, 4, "zipf"),
    "shard_e512k22_l4": Config("shard_e512k22_l4", 16384, 2048, 2048, 512, 22, 0, 4, "bf16", 0, 5),
}


def get_config(name: str) -> Config:
    return CONFIGS[name]
