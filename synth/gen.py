"""Counter-keyed random tensors (no attention arithmetic here)."""

from __future__ import annotations

import zlib

import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
ELEM_BYTES = {"fp32": 4, "fp16": 2, "bf16": 2}

_MASK64 = (1 << 64) - 1


def _splitmix64(x: int) -> int:
    """One SplitMix64 output step (Steele, Lea, Flood 2014)."""
    x = (x + 0x9E3779B97F4A7C15) & _MASK64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def derive_seed(seed: int, *names) -> int:
    """Mix a base seed and a tuple of names/ints into one 63-bit seed."""
    h = _splitmix64(int(seed) & _MASK64)
    for n in names:
        key = zlib.crc32(str(n).encode("utf-8"))
        h = _splitmix64(h ^ key)
    return h & ((1 << 63) - 1)


def _generator(device, seed: int, names) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(derive_seed(seed, *names))
    return g


def normal(shape, dtype: str, seed: int, *names, device="cpu", std: float = 1.0,
           out: torch.Tensor | None = None) -> torch.Tensor:
    """N(0, std^2) drawn in fp32, rounded (RNE) to ``dtype``.

    With ``out`` given, the values are written into that tensor (any strides),
    which lets a large cache be filled in place, one layer at a time.
    """
    g = _generator(device if out is None else out.device, seed, names)
    if out is not None:
        tmp = torch.empty(out.shape, dtype=torch.float32, device=out.device)
        tmp.normal_(0.0, 1.0, generator=g)
        if std != 1.0:
            tmp.mul_(std)
        out.copy_(tmp)
        return out
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t.to(DTYPES[dtype])


def uniform_int(shape, low: int, high_inclusive: int, seed: int, *names,
                device="cpu") -> torch.Tensor:
    g = _generator(device, seed, names)
    return torch.randint(low, high_inclusive + 1, tuple(shape), generator=g,
                         dtype=torch.int64, device=device).to(torch.int32)


def ragged_lengths(batch: int, low: int, high_inclusive: int, seed: int, *names) -> torch.Tensor:
    """Per-sequence cached lengths, integers uniform in [low, high_inclusive]."""
    return uniform_int((batch,), low, high_inclusive, seed, "lens", *names)
