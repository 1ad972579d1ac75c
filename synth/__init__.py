"""Seeded synthetic inputs for the KV-cache decode step.

This package only draws random numbers and rounds them to a storage dtype. It
holds none of the attention arithmetic, so both the CPU oracle's tests and the
GPU library's tests and benchmark can take their inputs from it without the two
sides sharing any step of the method.

Every tensor is keyed by ``(seed, *names)``: the names are mixed into one 63-bit
generator seed with SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), and torch's own Philox/MT
generator on the requested device draws the values. Normal draws are made in
fp32 and converted to the storage dtype with torch's round-to-nearest-even.
"""

from .gen import (  # noqa: F401
    DTYPES,
    ELEM_BYTES,
    derive_seed,
    normal,
    ragged_lengths,
    uniform_int,
)
from .configs import CONFIGS, DecodeConfig, ToyConfig  # noqa: F401
