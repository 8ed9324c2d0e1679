"""GPU parity of the prefill past 64 tiles per sequence, in every far-field mode.

The carry scan splits a sequence's 64-token tiles into 64 parts; up to 4096
tokens every part folds at most one tile.  These cases make each part fold
several tiles (and, for the 64K layer, 16), in the three modes the library
exports: S per KV head (sfa_prefill), γ and S per query head (sfa_prefill_qh)
and the running mean of the keys that have left the window (sfa_prefill_rm).
They cover a full 65,536-token 7B-shaped layer in the launch configuration the
bench times (bf16 in, bf16 out), ragged lengths (one past 65,536 tokens, where
a part folds more tiles than the scan keeps in registers), a second chunk
continuing a first one, and continuations from per-sequence positions beyond
64 tiles.
Tolerances are those of tests/parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
import windowed_ewma_state_amd as sfa
from windowed_ewma_state_amd import inputs
from tests.parity import check_exact, check_output, check_state, log

pytestmark = pytest.mark.gpu

MODES = ["kv", "qh", "rm"]


def _kw(mode):
    return {"gamma_per_query_head": mode == "qh", "running_mean": mode == "rm"}


def _okw(mode):
    return {"s_per_query": mode == "qh", "running_mean": mode == "rm"}


def _state_shape(mode, B, Hq, Hkv, d):
    if mode == "qh":
        return (B, Hq, d)
    if mode == "rm":
        return (B, Hkv, 2, d)
    return (B, Hkv, d)


def _inputs(mode, B, n, Hq, Hkv, hd, seed, dtype=torch.bfloat16, device="cpu"):
    d = inputs.prefill_inputs(B, n, Hq, Hkv, hd, seed=seed, dtype=dtype, device=device)
    if mode == "qh":
        d["gamma"] = inputs.uniform((Hq,), 0.90, 0.99, seed * 16 + 9, device=device)
    return d


def _cpu(d):
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def _gpu(d):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


@pytest.mark.parametrize("mode", ["qh", "rm"])
def test_prefill_mode_7b_64k_one_layer(mode):
    """One full 65,536-token 7B-shaped layer (1,024 tiles: each carry part folds
    16), bf16 in and bf16 out as the bench runs it, plus fp32 out; γ per query
    head drawn as U(0.90, 0.99) for the per-query-head mode."""
    log(f"prefill {mode} 7B-shaped 64K layer")
    d = inputs.workload(4, device="cuda", layer=0)
    if mode == "qh":
        d["gamma"] = inputs.uniform((28,), 0.90, 0.99, 77)
    c = _cpu(d)
    ref = oracle.prefill(c["q"], c["k"], c["v"], c["gamma"], c["alpha"], 16, **_okw(mode))
    g = _gpu(d)
    for od in (torch.bfloat16, torch.float32):
        out, rk, rv, st = sfa.prefill(g["q"], g["k"], g["v"], g["gamma"], g["alpha"], window=16,
                                      out_dtype=od, **_kw(mode))
        torch.cuda.synchronize()
        check_output(out, ref[0], True, f"out[{od}]")
        check_exact(rk, ref[1], "ring_k")
        check_exact(rv, ref[2], "ring_v")
        check_state(st, ref[3])
        del out


RAGGED = [  # (B, n, Hq, Hkv, hd, W, dtype)
    (2, 8192 + 37, 14, 2, 64, 16, torch.bfloat16),
    (1, 8192 + 37, 28, 4, 128, 16, torch.bfloat16),
    (2, 4096 + 64 * 9 + 1, 7, 1, 128, 5, torch.bfloat16),
    (1, 4700, 4, 2, 64, 16, torch.float32),
    (1, 6000 + 3, 8, 2, 128, 16, torch.float32),
    (1, 65536 + 4096 + 37, 2, 1, 64, 16, torch.bfloat16),  # 1,089 tiles: 18 per carry part
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "B{}n{}H{}-{}d{}W{}-{}".format(*c[:6], str(c[6])[6:]))
def test_prefill_ragged_past_64_tiles(case, mode):
    B, n, Hq, Hkv, hd, W, dt = case
    log(f"prefill {mode} ragged {case}")
    d = _inputs(mode, B, n, Hq, Hkv, hd, seed=n + Hq + W, dtype=dt)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W, **_okw(mode))
    g = _gpu(d)
    for od in (torch.float32, torch.bfloat16):
        out, rk, rv, st = sfa.prefill(g["q"], g["k"], g["v"], g["gamma"], g["alpha"], window=W,
                                      out_dtype=od, **_kw(mode))
        torch.cuda.synchronize()
        check_output(out, ref[0], dt == torch.bfloat16, f"out[{od}]")
        check_exact(rk, ref[1], "ring_k")
        check_exact(rv, ref[2], "ring_v")
        check_state(st, ref[3])


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("hd", [64, 128])
def test_prefill_two_long_chunks_equal_one(mode, hd):
    """GPU prefill of 5,000 tokens, then a continued GPU prefill of 4,500
    (pos0 = 5,000: both chunks span more than 64 tiles) == oracle prefill of
    9,500 tokens."""
    B, Hq, Hkv, W, n1, n2 = 2, 8, 2, 16, 5000, 4500
    log(f"prefill {mode} two chunks {n1}+{n2} d {hd}")
    d = _inputs(mode, B, n1 + n2, Hq, Hkv, hd, seed=31 + hd)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W, **_okw(mode))
    c = _gpu(d)
    o1, rk, rv, st = sfa.prefill(c["q"][:, :n1].contiguous(), c["k"][:, :n1].contiguous(),
                                 c["v"][:, :n1].contiguous(), c["gamma"], c["alpha"], window=W,
                                 out_dtype=torch.float32, **_kw(mode))
    o2, rk, rv, st = sfa.prefill(c["q"][:, n1:].contiguous(), c["k"][:, n1:].contiguous(),
                                 c["v"][:, n1:].contiguous(), c["gamma"], c["alpha"], window=W,
                                 out_dtype=torch.float32, ring_k=rk, ring_v=rv, state=st,
                                 pos0=torch.full((B,), n1, dtype=torch.int32, device="cuda"),
                                 **_kw(mode))
    torch.cuda.synchronize()
    check_output(torch.cat([o1, o2], 1), ref[0], True, "out")
    check_exact(rk, ref[1], "ring_k")
    check_exact(rv, ref[2], "ring_v")
    check_state(st, ref[3])


@pytest.mark.parametrize("mode", MODES)
def test_prefill_continuation_from_positions_past_64_tiles(mode):
    """Each sequence continues from its own position (0, 4,500, 5,013 and 70,001
    tokens already cached; the carried ring and state come from the oracle) over
    a 4,200-token chunk."""
    B, Hq, Hkv, hd, W, n2 = 4, 6, 2, 128, 16, 4200
    hist = [0, 4500, 5013, 70001]
    log(f"prefill {mode} continuation from {hist}")
    d = _inputs(mode, B, n2, Hq, Hkv, hd, seed=57)
    rk = np.zeros((B, Hkv, W, hd))
    rv = np.zeros((B, Hkv, W, hd))
    st = np.zeros(_state_shape(mode, B, Hq, Hkv, hd))
    for b, h in enumerate(hist):
        if h == 0:
            continue
        if h > 10000:
            # a long history stands in for its last W tokens and a state drawn
            # at random (the state is an input of the continued call)
            rk[b] = inputs.normal((Hkv, W, hd), 900 + b, 0.5, torch.bfloat16).double().numpy()
            rv[b] = inputs.normal((Hkv, W, hd), 950 + b, 0.5, torch.bfloat16).double().numpy()
            st[b] = inputs.normal(st.shape[1:], 990 + b, 0.3, torch.float32).double().numpy()
            continue
        hb = _inputs(mode, 1, h, Hq, Hkv, hd, seed=200 + b)
        _, rk1, rv1, st1 = oracle.prefill(hb["q"], hb["k"], hb["v"], d["gamma"], d["alpha"], W,
                                          **_okw(mode))
        rk[b], rv[b], st[b] = rk1[0], rv1[0], st1[0]
    rk = torch.from_numpy(rk).to(torch.bfloat16)
    rv = torch.from_numpy(rv).to(torch.bfloat16)
    st = torch.from_numpy(st).float()
    pos0 = torch.tensor(hist, dtype=torch.int32)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W, ring_k=rk, ring_v=rv,
                         state=st, pos0=pos0, **_okw(mode))
    g_rk, g_rv, g_st = rk.cuda(), rv.cuda(), st.cuda()
    out, *_ = sfa.prefill(d["q"].cuda(), d["k"].cuda(), d["v"].cuda(), d["gamma"].cuda(),
                          d["alpha"].cuda(), window=W, out_dtype=torch.float32, ring_k=g_rk,
                          ring_v=g_rv, state=g_st, pos0=pos0.cuda(), **_kw(mode))
    torch.cuda.synchronize()
    check_output(out, ref[0], True, "out")
    check_exact(g_rk, ref[1], "ring_k")
    check_exact(g_rv, ref[2], "ring_v")
    check_state(g_st, ref[3])


# ---------------------------------------------------------------------------
# decode: GQA groups of 9..16 query heads (16 query rows per MFMA tile, the
# store epilogue without the row rotation), in every mode
# ---------------------------------------------------------------------------
DECODE_GROUPS = [  # (L, B, Hq, Hkv, hd, W)
    (2, 5, 24, 2, 128, 16),  # group 12
    (2, 5, 32, 2, 64, 16),   # group 16
    (2, 5, 9, 1, 128, 16),   # group 9
    (1, 5, 30, 3, 64, 7),    # group 10
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", DECODE_GROUPS, ids=lambda c: "L{}B{}H{}-{}d{}W{}".format(*c))
def test_decode_groups_9_to_16(case, mode):
    L, B, Hq, Hkv, hd, W = case
    log(f"decode {mode} group {Hq // Hkv} case {case}")
    seed = L * 100 + Hq + W
    d = inputs.decode_inputs(L, B, Hq, Hkv, hd, seed=seed, W=W)
    if mode == "qh":
        d["state"] = inputs.normal((L, B, Hq, hd), seed * 16 + 9, 1.0, torch.float32)
        d["gamma"] = inputs.uniform((L, Hq), 0.90, 0.99, seed * 16 + 10)
    elif mode == "rm":
        d["state"] = inputs.normal((L, B, Hkv, 2, hd), seed * 16 + 11, 1.0, torch.float32)
    d["pos"] = torch.tensor([0, 1, W - 1, W, 5000][:B], dtype=torch.int32)
    ref = oracle.decode_step(d["q"], d["k_new"], d["v_new"], d["ring_k"], d["ring_v"], d["state"],
                             d["pos"], d["gamma"], d["alpha"], **_okw(mode))
    for od in (torch.float32, torch.bfloat16):
        rk, rv, st = d["ring_k"].cuda().clone(), d["ring_v"].cuda().clone(), d["state"].cuda().clone()
        out = sfa.decode_step(d["q"].cuda(), d["k_new"].cuda(), d["v_new"].cuda(), rk, rv, st,
                              d["pos"].cuda(), d["gamma"].cuda(), d["alpha"].cuda(), out_dtype=od,
                              **_kw(mode))
        torch.cuda.synchronize()
        check_output(out, ref[0], True, f"out[{od}]")
        check_exact(rk, ref[1], "ring_k")
        check_exact(rv, ref[2], "ring_v")
        check_state(st, ref[3])
