"""The five workload configurations of the sparse LoRA linear path.

Sizes follow the LLaMA-family shapes the SparseLoRA pages evaluate on
(paper-graph summary, §5 "Evaluation Methodology": LLaMA2-7B/13B, LLaMA3-8B;
§3.4 "Token Sensitivity": output tokens are a contiguous tail of each
sequence).  Sparsity ratios are exact rationals ``(num, den)`` so that the
number of kept channels can be formed in integer arithmetic by the caller.
"""
from dataclasses import dataclass, field
from fractions import Fraction
from typing import Dict, List, Optional, Tuple


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    kind: str                 # "ffn" | "attn" | "layer" | "stack"
    dtype: str                # "f32" | "bf16"
    batch: int
    seq: int
    out_per_seq: int          # output (dense) tokens at the tail of each sequence
    hidden: int
    inter: int = 0            # FFN intermediate size F (0 when no FFN)
    n_q_heads: int = 0
    n_kv_heads: int = 0
    head_dim: int = 0
    lora_rank: int = 16
    est_rank: int = 16
    lora_alpha: int = 32      # scale = alpha / rank
    ffn_sparsity: Tuple[int, int] = (0, 1)
    qk_sparsity: Tuple[int, int] = (0, 1)
    vo_sparsity: Tuple[int, int] = (0, 1)
    n_layers: int = 1
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def out_tokens(self) -> int:
        return self.batch * self.out_per_seq

    @property
    def ctx_tokens(self) -> int:
        return self.tokens - self.out_tokens

    @property
    def lora_scale(self) -> float:
        return self.lora_alpha / self.lora_rank

    def layer_sparsity(self, layer: int) -> Tuple[int, int]:
        """Per-layer sparsity of the 32-layer stack: 0 for layers 0..3, then a
        linear ramp reaching 4/5 at layer 31, i.e. s = 4*(l-3) / (5*28)."""
        if self.kind != "stack":
            return self.ffn_sparsity
        if layer <= 3:
            return (0, 1)
        f = Fraction(4 * (layer - 3), 5 * 28)
        return (f.numerator, f.denominator)


CONFIGS: Dict[int, Config] = {
    1: Config(1, "ffn-tiny-f32", "ffn", "f32", batch=2, seq=64, out_per_seq=16,
              hidden=256, inter=688, lora_rank=8, est_rank=8, lora_alpha=16,
              ffn_sparsity=(1, 2), seed=1001),
    2: Config(2, "llama3-8b-ffn", "ffn", "bf16", batch=8, seq=512, out_per_seq=128,
              hidden=4096, inter=14336, lora_rank=16, est_rank=16, lora_alpha=32,
              ffn_sparsity=(7, 10), seed=1002),
    3: Config(3, "llama3-8b-attn-proj", "attn", "bf16", batch=8, seq=512, out_per_seq=128,
              hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, lora_rank=16,
              est_rank=16, lora_alpha=32, qk_sparsity=(1, 2), vo_sparsity=(1, 2), seed=1003),
    4: Config(4, "llama2-13b-layer", "layer", "bf16", batch=4, seq=1024, out_per_seq=204,
              hidden=5120, inter=13824, n_q_heads=40, n_kv_heads=40, head_dim=128,
              lora_rank=32, est_rank=16, lora_alpha=64, ffn_sparsity=(7, 10),
              qk_sparsity=(1, 2), vo_sparsity=(1, 2), seed=1004),
    5: Config(5, "llama3-8b-stack32", "stack", "bf16", batch=4, seq=2048, out_per_seq=512,
              hidden=4096, inter=14336, n_q_heads=32, n_kv_heads=8, head_dim=128,
              lora_rank=16, est_rank=16, lora_alpha=32, n_layers=32, seed=1005),
}


def get_config(cid: int) -> Config:
    return CONFIGS[cid]


def scaled(cfg: Config, **over) -> Config:
    """A copy of ``cfg`` with some fields replaced (used for small test shapes)."""
    d = dict(cfg.__dict__)
    d.update(over)
    return Config(**d)
