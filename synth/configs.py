"""The decode-step workloads: the pages' toy GQA layer and four model-shaped steps.

Each shape is named for what it is. ``lengths`` gives the cached tokens per
sequence *before* the step; a step appends one token and attends T_b + 1.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

from .gen import ELEM_BYTES, ragged_lengths


@dataclass(frozen=True)
class ToyConfig:
    """One GQA layer of the glossary page's runnable experiment: B=1, hidden 16,
    H_q=4, H_kv=2, D=4, fp32, prompt 8 then 5 decode steps (final cache
    [1, 2, 13, 4])."""
    name: str = "toy_gqa"
    batch: int = 1
    hidden: int = 16
    n_q_heads: int = 4
    n_kv_heads: int = 2
    head_dim: int = 4
    prompt: int = 8
    decode: int = 5
    dtype: str = "fp32"


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    batch: int
    dtype: str
    fixed_len: int | None = None          # every sequence holds this many tokens
    ragged: tuple[int, int] | None = None  # inclusive [low, high] uniform lengths
    description: str = ""

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    def lengths(self, seed: int = 7) -> torch.Tensor:
        """Cached tokens per sequence before the step, int32 [B] on the host."""
        if self.fixed_len is not None:
            return torch.full((self.batch,), self.fixed_len, dtype=torch.int32)
        lo, hi = self.ragged
        return ragged_lengths(self.batch, lo, hi, seed, self.name)

    def kv_read_bytes(self, lengths: torch.Tensor, extra_tokens: int = 1) -> int:
        """K+V bytes one step reads: 2*L*H_kv*D*s*sum_b(T_b + extra)."""
        tok = int(lengths.to(torch.int64).sum()) + extra_tokens * self.batch
        return 2 * self.n_layers * self.n_kv_heads * self.head_dim * self.elem_bytes * tok


CONFIGS: dict[str, object] = {
    "toy_gqa": ToyConfig(),
    "mha_7b": DecodeConfig(
        "mha_7b", n_layers=32, n_q_heads=32, n_kv_heads=32, head_dim=128, batch=1,
        dtype="fp16", fixed_len=4096,
        description="Llama-2-7B-shaped MHA step: 32 layers, 32/32 heads, D=128, B=1, T=4096, fp16"),
    "gqa_8b": DecodeConfig(
        "gqa_8b", n_layers=32, n_q_heads=32, n_kv_heads=8, head_dim=128, batch=16,
        dtype="bf16", fixed_len=2048,
        description="8B-shaped GQA step: 32 layers, 32/8 heads, D=128, B=16, T=2048, bf16"),
    "ragged_long": DecodeConfig(
        "ragged_long", n_layers=32, n_q_heads=32, n_kv_heads=32, head_dim=128, batch=24,
        dtype="fp16", ragged=(3000, 6000),
        description="long-session batch: 32 layers, 32/32 heads, D=128, B=24, T_b~U[3000,6000], fp16"),
    "gqa_70b": DecodeConfig(
        "gqa_70b", n_layers=80, n_q_heads=64, n_kv_heads=8, head_dim=128, batch=32,
        dtype="bf16", fixed_len=8192,
        description="70B-shaped GQA step: 80 layers, 64/8 heads, D=128, B=32, T=8192, bf16"),
    "mqa_70b": DecodeConfig(
        "mqa_70b", n_layers=80, n_q_heads=64, n_kv_heads=1, head_dim=128, batch=32,
        dtype="bf16", fixed_len=8192,
        description="70B-shaped MQA step: 80 layers, 64/1 heads, D=128, B=32, T=8192, bf16"),
}
