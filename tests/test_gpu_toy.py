"""The glossary page's runnable experiment on the GPU path: one GQA layer, fp32,
B=1, hidden 16, H_q=4, H_kv=2, D=4; prefill 8 tokens, then 5 decode steps.

Path B runs on libkvc (kvc_prefill_fill, then per token kvc_append,
kvc_decode_attn, kvc_seq_lens_advance); the host only projects with fp64
matmuls rounded to fp32 (the page's dtype) and applies W_o. The oracle's path A
(full-prefix causal recompute in fp64) is the reference: the glossary's bar is
rtol 1e-4 / atol 1e-5 per step, the tighter max-abs 1e-5 is used here. The
final cache must be [1, 2, 13, 4] and hold the projected K/V rows bit for bit.
"""

import math

import numpy as np
import pytest
import torch

import kv_cache_append_amd as kvc
import oracle
import synth

pytestmark = pytest.mark.gpu


def _inputs(cfg, seed=7):
    std = 1.0 / math.sqrt(cfg.hidden)
    t = cfg.prompt + cfg.decode
    wq = synth.normal((cfg.hidden, cfg.n_q_heads * cfg.head_dim), "fp32", seed, "toy", "wq", std=std)
    wk = synth.normal((cfg.hidden, cfg.n_kv_heads * cfg.head_dim), "fp32", seed, "toy", "wk", std=std)
    wv = synth.normal((cfg.hidden, cfg.n_kv_heads * cfg.head_dim), "fp32", seed, "toy", "wv", std=std)
    wo = synth.normal((cfg.n_q_heads * cfg.head_dim, cfg.hidden), "fp32", seed, "toy", "wo", std=std)
    x = synth.normal((t, cfg.hidden), "fp32", seed, "toy", "x")
    return x, wq, wk, wv, wo


def _proj_fp32(x, w, heads, d):
    """Host-side projection of the harness: fp64 product, one rounding to fp32,
    laid out [heads, T, D] (head h owns columns [hD, (h+1)D))."""
    y = (x.double() @ w.double()).float()
    return y.reshape(x.shape[0], heads, d).transpose(0, 1).contiguous()


def run_toy_on_gpu(cfg, x, wq, wk, wv, wo, device):
    t_total = cfg.prompt + cfg.decode
    q_all = _proj_fp32(x, wq, cfg.n_q_heads, cfg.head_dim)       # [H_q, T, D]
    k_all = _proj_fp32(x, wk, cfg.n_kv_heads, cfg.head_dim)      # [H_kv, T, D]
    v_all = _proj_fp32(x, wv, cfg.n_kv_heads, cfg.head_dim)
    kc = torch.full((1, cfg.n_kv_heads, t_total, cfg.head_dim), float("nan"), device=device)
    vc = torch.full_like(kc, float("nan"))
    lens = torch.zeros(1, dtype=torch.int32, device=device)
    status = torch.zeros(1, dtype=torch.int32, device=device)
    kvc.prefill_fill(kc, vc, lens, k_all[None, :, :cfg.prompt].to(device), v_all[None, :, :cfg.prompt].to(device),
                     status=status)
    kvc.seq_lens_advance(lens, cfg.prompt)
    ws = kvc.workspace(kc, vc, cfg.n_q_heads)
    contexts = []
    for t in range(cfg.prompt, t_total):
        k_new = k_all[:, t][None].to(device)
        v_new = v_all[:, t][None].to(device)
        q = q_all[:, t][None].contiguous().to(device)
        out = torch.empty((1, cfg.n_q_heads, cfg.head_dim), device=device)
        kvc.append(kc, vc, lens, k_new, v_new, status=status)
        kvc.decode_attn(kc, vc, lens, q, out, ws, n_pending=1, status=status)
        kvc.seq_lens_advance(lens, 1)
        contexts.append(out[0].cpu())
    torch.cuda.synchronize()
    return torch.stack(contexts), kc.cpu(), vc.cpu(), int(lens.item()), int(status.item()), (q_all, k_all, v_all)


def test_toy_incremental_decode_matches_full_recompute(gpu):
    cfg = synth.CONFIGS["toy_gqa"]
    x, wq, wk, wv, wo = _inputs(cfg)
    ctx_gpu, kc, vc, final_len, status, (q_all, k_all, v_all) = run_toy_on_gpu(cfg, x, wq, wk, wv, wo, gpu)
    assert status == 0 and final_len == 13
    # final cache: shape [1, 2, 13, 4], rows are the projected K/V bit for bit
    assert tuple(kc.shape) == (1, 2, 13, 4) and tuple(vc.shape) == (1, 2, 13, 4)
    assert torch.equal(kc[0].view(torch.int32), k_all.view(torch.int32))
    assert torch.equal(vc[0].view(torch.int32), v_all.view(torch.int32))
    # against the oracle's path A (fp64 full-prefix causal recompute)
    out_a, ctx_a = oracle.toy_path_a(x, wq, wk, wv, wo, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.prompt)
    ctx = ctx_gpu.double().numpy()
    assert np.abs(ctx - ctx_a).max() <= 1e-5
    out_b = ctx.reshape(cfg.decode, -1) @ oracle.widen(wo)
    assert np.abs(out_b - out_a).max() <= 1e-5
    assert np.allclose(out_b, out_a, rtol=1e-4, atol=1e-5)
    # against the oracle's decode on the identical fp32 inputs, step by step
    for j in range(cfg.decode):
        t = cfg.prompt + j
        ref = oracle.decode_attention(q_all[:, t][None], k_all[None, :, :t + 1], v_all[None, :, :t + 1],
                                      np.array([t]), n_pending=1)[0]
        assert np.abs(ctx[j] - ref).max() <= 1e-5
