"""Helpers for the GPU parity tests: build seeded caches on the device and the
matching host copies the oracle reads. Only torch's RNG and plain copies are
used here; nothing is computed by libkvc."""

from __future__ import annotations

import torch

import synth

TOL = {"fp32": 1e-5, "fp16": 2e-3, "bf16": 2e-3}   # max-abs vs the fp64 oracle


def poison_(t: torch.Tensor) -> torch.Tensor:
    """Fill with a quiet NaN of the tensor's dtype: any read of it shows up in the output."""
    return t.fill_(float("nan"))


class DecodeCase:
    """One layer: cache [B, H_kv, T_max, D] holding T_b generated tokens per
    sequence, NaN past them; k_new/v_new/q drawn fresh. Host copies are taken
    before any libkvc call touches the device buffers."""

    def __init__(self, *, batch, n_q, n_kv, head_dim, dtype, lengths, t_max=None, seed=7, tag="case",
                 device="cuda", layout="bhtd", host_rows=None):
        self.batch, self.n_q, self.n_kv, self.head_dim, self.dtype = batch, n_q, n_kv, head_dim, dtype
        self.lengths = torch.as_tensor(lengths, dtype=torch.int32)
        self.t_max = int(t_max if t_max is not None else int(self.lengths.max()) + 1)
        tdt = synth.DTYPES[dtype]
        shape = (batch, n_kv, self.t_max, head_dim)
        if layout == "bhtd":
            self.k = torch.empty(shape, dtype=tdt, device=device)
            self.v = torch.empty(shape, dtype=tdt, device=device)
        else:  # [B, T, H, D] storage viewed as [B, H, T, D]
            self.k = torch.empty((batch, self.t_max, n_kv, head_dim), dtype=tdt, device=device).transpose(1, 2)
            self.v = torch.empty((batch, self.t_max, n_kv, head_dim), dtype=tdt, device=device).transpose(1, 2)
        poison_(self.k)
        poison_(self.v)
        tmax_b = int(self.lengths.max()) if batch else 0
        for name, dst in (("K", self.k), ("V", self.v)):
            full = synth.normal((batch, n_kv, max(tmax_b, 1), head_dim), dtype, seed, tag, name, device=device)
            for b in range(batch):
                n = int(self.lengths[b])
                if n > 0:
                    dst[b, :, :n].copy_(full[b, :, :n])
        self.q = synth.normal((batch, n_q, head_dim), dtype, seed, tag, "q", device=device)
        self.k_new = synth.normal((batch, n_kv, head_dim), dtype, seed, tag, "k_new", device=device)
        self.v_new = synth.normal((batch, n_kv, head_dim), dtype, seed, tag, "v_new", device=device)
        self.seq_lens = self.lengths.to(device)
        # Host copies for the oracle. host_rows=None copies everything; otherwise
        # only the listed (b, g) units are copied (large caches).
        self.host = {}
        units = host_rows if host_rows is not None else [(b, g) for b in range(batch) for g in range(n_kv)]
        for b, g in units:
            n = int(self.lengths[b])
            self.host[(b, g)] = (self.k[b, g, :n].cpu(), self.v[b, g, :n].cpu(),
                                 self.k_new[b, g].cpu(), self.v_new[b, g].cpu())
        self.q_host = self.q.cpu()

    def oracle_inputs(self, b: int, g: int):
        """K, V rows [0, T_b] of unit (b, g) after the step's append, on the host."""
        k_old, v_old, kn, vn = self.host[(b, g)]
        return torch.cat([k_old, kn[None]]), torch.cat([v_old, vn[None]])
