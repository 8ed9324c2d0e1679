"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no SFA arithmetic: it only draws random tensors with the
shapes, dtypes and distributions of the workloads (attention shapes of
Qwen2.5-0.5B and Qwen2.5-7B, the models the pages evaluate).  Each tensor has
its own ``torch.Generator`` seeded from (workload seed, tensor index), so a
tensor never depends on the draw order of another.  bf16 tensors are drawn in
fp32, scaled, then rounded to bf16 (round-to-nearest-even) once; the GPU path
and the CPU oracle both consume exactly these values.

Workloads (ids 1..5):
  1 tiny fp32 prefill        B=1, Hq=Hkv=1, d=64, n=256, W=16, γ=0.9, α=0.1, N(0,1)
  2 0.5B-shaped prefill      B=4, n=4096, Hq=14, Hkv=2, d=64, bf16 N(0,1)·0.5,
                             γ ~ U(0.90,0.99) per KV head, α ~ U(0,0.2) per query head
  3 7B-shaped decode step    L=28, B=256, Hq=28, Hkv=4, d=128, W=16, bf16 N(0,1)
                             q/k_new/v_new/ring, fp32 N(0,1) state, pos ~ U{128..8192}
  4 7B-shaped 64K prefill    B=1, n=65536, Hq=28, Hkv=4, d=128, bf16 N(0,1)·0.5,
                             γ=0.98, α=0.1, W=16; one independent draw per layer
  5 triple-channel enhance   L=24, T=4096, H=1024, bf16 N(0,1) attention output,
                             64-slot fp32 pool N(0,1) L2-normalised per slot
"""
from __future__ import annotations

import torch

WINDOW = 16


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, seed: int, std: float = 1.0, dtype=torch.bfloat16, device="cpu"):
    """N(0,1)·std drawn in fp32, then rounded once to ``dtype``."""
    x = torch.randn(shape, generator=_gen(seed, device), dtype=torch.float32, device=device)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def uniform(shape, lo: float, hi: float, seed: int, device="cpu"):
    x = torch.rand(shape, generator=_gen(seed, device), dtype=torch.float32, device=device)
    return x.mul_(hi - lo).add_(lo)


def randint(shape, lo: int, hi_inclusive: int, seed: int, device="cpu"):
    return torch.randint(lo, hi_inclusive + 1, shape, generator=_gen(seed, device),
                         dtype=torch.int32, device=device)


def prefill_inputs(B, n, Hq, Hkv, d, *, seed, std=0.5, dtype=torch.bfloat16,
                   gamma=(0.90, 0.99), alpha=(0.0, 0.2), device="cpu"):
    """Q/K/V in BNHD layout plus per-KV-head γ and per-query-head α.

    ``gamma``/``alpha`` are either a (lo, hi) uniform range or a scalar.
    """
    s = int(seed) * 16
    q = normal((B, n, Hq, d), s + 0, std, dtype, device)
    k = normal((B, n, Hkv, d), s + 1, std, dtype, device)
    v = normal((B, n, Hkv, d), s + 2, std, dtype, device)
    if isinstance(gamma, tuple):
        gm = uniform((Hkv,), gamma[0], gamma[1], s + 3, device)
    else:
        gm = torch.full((Hkv,), float(gamma), dtype=torch.float32, device=device)
    if isinstance(alpha, tuple):
        al = uniform((Hq,), alpha[0], alpha[1], s + 4, device)
    else:
        al = torch.full((Hq,), float(alpha), dtype=torch.float32, device=device)
    return dict(q=q, k=k, v=v, gamma=gm, alpha=al, window=WINDOW)


def decode_inputs(L, B, Hq, Hkv, d, *, seed, W=WINDOW, dtype=torch.bfloat16,
                  pos_range=(128, 8192), std=1.0, device="cpu"):
    """One decode step's inputs and a ring/state cache pre-filled with N(0,1)."""
    s = int(seed) * 16
    return dict(
        q=normal((L, B, Hq, d), s + 0, std, dtype, device),
        k_new=normal((L, B, Hkv, d), s + 1, std, dtype, device),
        v_new=normal((L, B, Hkv, d), s + 2, std, dtype, device),
        ring_k=normal((L, B, Hkv, W, d), s + 3, std, dtype, device),
        ring_v=normal((L, B, Hkv, W, d), s + 4, std, dtype, device),
        state=normal((L, B, Hkv, d), s + 5, 1.0, torch.float32, device),
        pos=randint((B,), pos_range[0], pos_range[1], s + 6, device),
        gamma=uniform((L, Hkv), 0.90, 0.99, s + 7, device),
        alpha=uniform((L, Hq), 0.0, 0.2, s + 8, device),
        window=W,
    )


def enhance_inputs(L, T, H, *, seed, n_slots=64, dtype=torch.bfloat16, device="cpu"):
    """Attention output [L,T,H] and a per-layer pool of unit-norm slots."""
    s = int(seed) * 16
    attn = normal((L, T, H), s + 0, 1.0, dtype, device)
    pool = normal((L, n_slots, H), s + 1, 1.0, torch.float32, device)
    pool = pool / pool.norm(dim=-1, keepdim=True)
    return dict(attn=attn, pool=pool.contiguous())


def workload(wid: int, device="cpu", layer: int = 0):
    """Inputs of workload ``wid`` (1..5); ``layer`` selects the per-layer draw of 4."""
    seed = 1000 + int(wid)
    if wid == 1:
        d = prefill_inputs(1, 256, 1, 1, 64, seed=seed, std=1.0, dtype=torch.float32,
                           gamma=0.9, alpha=0.1, device=device)
    elif wid == 2:
        d = prefill_inputs(4, 4096, 14, 2, 64, seed=seed, device=device)
    elif wid == 3:
        d = decode_inputs(28, 256, 28, 4, 128, seed=seed, device=device)
    elif wid == 4:
        d = prefill_inputs(1, 65536, 28, 4, 128, seed=seed * 64 + layer, gamma=0.98,
                           alpha=0.1, device=device)
    elif wid == 5:
        d = enhance_inputs(24, 4096, 1024, seed=seed, device=device)
        d.update(alpha_base=0.1, cross_decay=0.8, ema_gamma=0.98, temperature=0.07,
                 clip=0.5, ring_size=16, t0=0)
    else:
        raise ValueError(f"unknown workload {wid}")
    return d
