"""GPU parity of the running-mean far field (sfa_prefill_rm, sfa_decode_step_rm):
the EWMA input is the mean of every key that has left the window; checked
against the oracle's same mode."""
import pytest
import torch

import oracle
import windowed_ewma_state_amd as sfa
from windowed_ewma_state_amd import inputs
from tests.parity import check_exact, check_output, check_state, log

pytestmark = pytest.mark.gpu

PREFILL = [  # (B, n, Hq, Hkv, hd, W)
    (1, 1, 2, 1, 64, 16), (2, 63, 4, 2, 64, 5), (1, 130, 14, 2, 64, 16), (2, 300, 8, 2, 128, 3),
    (1, 1000, 7, 1, 128, 16), (3, 65, 6, 3, 64, 1), (1, 17, 4, 4, 128, 16),
    # groups of 20, 1 and 5; positions from 1 to past 16 blocks
    (1, 200, 20, 1, 64, 16), (2, 150, 3, 3, 128, 16), (1, 257, 10, 2, 128, 7),
]


def _gpu(d):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: "B{}n{}H{}-{}d{}W{}".format(*c))
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_prefill_rm_small(case, dt):
    B, n, Hq, Hkv, hd, W = case
    log(f"prefill_rm case {case} {dt}")
    d = inputs.prefill_inputs(B, n, Hq, Hkv, hd, seed=n * 5 + Hq, dtype=dt)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W, running_mean=True)
    c = _gpu(d)
    for od in (torch.float32, torch.bfloat16):
        out, rk, rv, st = sfa.prefill(c["q"], c["k"], c["v"], c["gamma"], c["alpha"], window=W,
                                      out_dtype=od, running_mean=True)
        torch.cuda.synchronize()
        check_output(out, ref[0], dt == torch.bfloat16, f"out[{od}]")
        w = min(n, W)
        check_exact(rk[:, :, :w], ref[1][:, :, :w], "ring_k")
        check_state(st, ref[3])


def test_prefill_rm_workload_05b():
    """0.5B-shaped prefill (B 4, n 4096, 14/2 heads, d 64, bf16) with the running mean."""
    log("prefill_rm 0.5B-shaped workload")
    d = inputs.workload(2)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], 16, running_mean=True)
    c = _gpu(d)
    out, rk, rv, st = sfa.prefill(c["q"], c["k"], c["v"], c["gamma"], c["alpha"], window=16,
                                  out_dtype=torch.float32, running_mean=True)
    torch.cuda.synchronize()
    check_output(out, ref[0], True, "out")
    check_state(st, ref[3])


@pytest.mark.parametrize("n1,n2,W", [(100, 77, 16), (9, 200, 16), (300, 5, 4)])
def test_prefill_rm_two_chunks_equal_one(n1, n2, W):
    B, Hq, Hkv, hd = 2, 7, 1, 128
    log(f"prefill_rm two chunks {n1}+{n2} W {W}")
    d = inputs.prefill_inputs(B, n1 + n2, Hq, Hkv, hd, seed=6 + n1)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W, running_mean=True)
    c = _gpu(d)
    o1, rk, rv, st = sfa.prefill(c["q"][:, :n1].contiguous(), c["k"][:, :n1].contiguous(),
                                 c["v"][:, :n1].contiguous(), c["gamma"], c["alpha"], window=W,
                                 out_dtype=torch.float32, running_mean=True)
    o2, rk, rv, st = sfa.prefill(c["q"][:, n1:].contiguous(), c["k"][:, n1:].contiguous(),
                                 c["v"][:, n1:].contiguous(), c["gamma"], c["alpha"], window=W,
                                 out_dtype=torch.float32, ring_k=rk, ring_v=rv, state=st,
                                 pos0=torch.full((B,), n1, dtype=torch.int32, device="cuda"),
                                 running_mean=True)
    torch.cuda.synchronize()
    check_output(torch.cat([o1, o2], 1), ref[0], True, "out")
    check_exact(rk, ref[1], "ring_k")
    check_state(st, ref[3])


def _decode_inputs(L, B, Hq, Hkv, hd, W, seed, dtype=torch.bfloat16):
    d = inputs.decode_inputs(L, B, Hq, Hkv, hd, seed=seed, W=W, dtype=dtype)
    d["state"] = inputs.normal((L, B, Hkv, 2, hd), seed * 16 + 11, 1.0, torch.float32)
    return d


DECODE = [  # (L, B, Hq, Hkv, hd, W, in_dtype)
    (2, 5, 8, 2, 64, 16, torch.bfloat16),
    (2, 5, 8, 2, 128, 16, torch.bfloat16),
    (1, 5, 4, 4, 128, 4, torch.bfloat16),
    (3, 5, 6, 1, 64, 1, torch.bfloat16),
    (2, 5, 36, 2, 128, 16, torch.bfloat16),  # 18 query heads per KV head: the VALU kernel
    (2, 5, 24, 2, 128, 16, torch.bfloat16),  # 12 query heads per KV head: 16-row query tiles (d 128)
    (2, 5, 32, 2, 64, 16, torch.bfloat16),  # 16 query heads per KV head: 16-row query tiles (d 64)
    (2, 5, 8, 2, 128, 16, torch.float32),
    (1, 5, 3, 3, 64, 7, torch.float32),
]


def _decode_check(d, out_dtype):
    ref = oracle.decode_step(d["q"], d["k_new"], d["v_new"], d["ring_k"], d["ring_v"], d["state"],
                             d["pos"], d["gamma"], d["alpha"], running_mean=True)
    rk, rv, st = d["ring_k"].cuda().clone(), d["ring_v"].cuda().clone(), d["state"].cuda().clone()
    out = sfa.decode_step(d["q"].cuda(), d["k_new"].cuda(), d["v_new"].cuda(), rk, rv, st,
                          d["pos"].cuda(), d["gamma"].cuda(), d["alpha"].cuda(), out_dtype=out_dtype,
                          running_mean=True)
    torch.cuda.synchronize()
    check_output(out, ref[0], d["q"].dtype == torch.bfloat16, "out")
    check_exact(rk, ref[1], "ring_k")
    check_exact(rv, ref[2], "ring_v")
    check_state(st, ref[3])


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "L{}B{}H{}-{}d{}W{}-{}".format(*c[:6], str(c[6])[6:]))
def test_decode_rm_small(case):
    L, B, Hq, Hkv, hd, W, dt = case
    log(f"decode_rm case {case}")
    d = _decode_inputs(L, B, Hq, Hkv, hd, W, seed=L * 10 + Hq + W, dtype=dt)
    d["pos"] = torch.tensor([0, 1, W - 1, W, 5000][:B], dtype=torch.int32)
    for od in (torch.float32, torch.bfloat16):
        _decode_check(d, od)


def test_decode_rm_workload_7b_28_layers():
    """7B-shaped decode step (28 layers x 256 sequences, 28/4 heads, d 128, bf16), running mean."""
    log("decode_rm 7B-shaped 28 layers")
    d = _decode_inputs(28, 256, 28, 4, 128, 16, seed=1013)
    _decode_check(d, torch.float32)


def test_decode_rm_continues_a_gpu_prefill_rm():
    """prefill_rm(n) then decode_rm steps == prefill_rm(n + steps) (oracle)."""
    B, Hq, Hkv, hd, W, n, m = 2, 8, 2, 128, 16, 40, 6
    log("decode_rm after prefill_rm")
    d = inputs.prefill_inputs(B, n + m, Hq, Hkv, hd, seed=19)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W, running_mean=True)
    c = _gpu(d)
    _, rk, rv, st = sfa.prefill(c["q"][:, :n].contiguous(), c["k"][:, :n].contiguous(),
                                c["v"][:, :n].contiguous(), c["gamma"], c["alpha"], window=W,
                                running_mean=True)
    rk, rv, st = rk[None], rv[None], st[None]
    for i in range(m):
        t = n + i
        o = sfa.decode_step(c["q"][None, :, t].contiguous(), c["k"][None, :, t].contiguous(),
                            c["v"][None, :, t].contiguous(), rk, rv, st,
                            torch.full((B,), t, dtype=torch.int32, device="cuda"),
                            c["gamma"][None], c["alpha"][None], out_dtype=torch.float32,
                            running_mean=True)
        check_output(o[0], ref[0][:, t], True, f"step {t}")
    torch.cuda.synchronize()
    check_exact(rk[0], ref[1], "ring_k")
    check_state(st[0], ref[3])


def test_decode_rm_negative_position_skips_the_sequence():
    L, B, Hq, Hkv, hd, W = 2, 4, 8, 2, 128, 16
    log("decode_rm skip case")
    d = _decode_inputs(L, B, Hq, Hkv, hd, W, seed=23)
    d["pos"] = torch.tensor([30, -5, 16, 3], dtype=torch.int32)
    sentinel = torch.full(d["q"].shape, 7.25, dtype=torch.float32)
    out = sentinel.cuda()
    rk, rv, st = d["ring_k"].cuda(), d["ring_v"].cuda(), d["state"].cuda()
    sfa.decode_step(d["q"].cuda(), d["k_new"].cuda(), d["v_new"].cuda(), rk, rv, st, d["pos"].cuda(),
                    d["gamma"].cuda(), d["alpha"].cuda(), out=out, running_mean=True)
    ref = oracle.decode_step(d["q"], d["k_new"], d["v_new"], d["ring_k"], d["ring_v"], d["state"],
                             d["pos"], d["gamma"], d["alpha"], running_mean=True)
    torch.cuda.synchronize()
    assert torch.equal(out[:, 1].cpu(), sentinel[:, 1])
    assert torch.equal(st[:, 1].cpu(), d["state"][:, 1])
    assert torch.equal(rk[:, 1].cpu(), d["ring_k"][:, 1])
    keep = [0, 2, 3]
    check_output(out[:, keep], ref[0][:, keep], True, "out (kept)")
    check_state(st[:, keep], ref[3][:, keep])
