"""GPU parity of the per-query-head far field (sfa_prefill_qh, sfa_decode_step_qh):
γ and S belong to each query head; checked against the oracle's same mode."""
import numpy as np
import pytest
import torch

import oracle
import windowed_ewma_state_amd as sfa
from windowed_ewma_state_amd import inputs
from tests.parity import check_exact, check_output, check_state, log

pytestmark = pytest.mark.gpu


def _prefill_inputs(B, n, Hq, Hkv, hd, seed, dtype=torch.bfloat16):
    d = inputs.prefill_inputs(B, n, Hq, Hkv, hd, seed=seed, dtype=dtype)
    d["gamma"] = inputs.uniform((Hq,), 0.90, 0.99, seed * 16 + 9)  # one decay per query head
    return d


PREFILL = [  # (B, n, Hq, Hkv, hd, W)
    (1, 1, 2, 1, 64, 16), (2, 63, 4, 2, 64, 5), (1, 130, 14, 2, 64, 16), (2, 300, 8, 2, 128, 3),
    (1, 1000, 7, 1, 128, 16), (3, 65, 6, 3, 64, 1),
    # groups of 20 (more heads than the query slots and a 16-row MFMA tile), 1 and 5
    (1, 200, 20, 1, 64, 16), (2, 150, 3, 3, 128, 16), (1, 257, 10, 2, 128, 7),
]


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: "B{}n{}H{}-{}d{}W{}".format(*c))
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_prefill_qh_small(case, dt):
    B, n, Hq, Hkv, hd, W = case
    log(f"prefill_qh case {case} {dt}")
    d = _prefill_inputs(B, n, Hq, Hkv, hd, seed=n * 7 + Hq, dtype=dt)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W, s_per_query=True)
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    for od in (torch.float32, torch.bfloat16):
        out, rk, rv, st = sfa.prefill(c["q"], c["k"], c["v"], c["gamma"], c["alpha"], window=W,
                                      out_dtype=od, gamma_per_query_head=True)
        torch.cuda.synchronize()
        check_output(out, ref[0], dt == torch.bfloat16, f"out[{od}]")
        w = min(n, W)
        check_exact(rk[:, :, :w], ref[1][:, :, :w], "ring_k")
        check_state(st, ref[3])


def test_prefill_qh_workload_05b():
    """0.5B-shaped prefill (B 4, n 4096, 14/2 heads, d 64, bf16) with a decay per query head."""
    log("prefill_qh 0.5B-shaped workload")
    d = _prefill_inputs(4, 4096, 14, 2, 64, seed=1002)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], 16, s_per_query=True)
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    out, rk, rv, st = sfa.prefill(c["q"], c["k"], c["v"], c["gamma"], c["alpha"], window=16,
                                  out_dtype=torch.float32, gamma_per_query_head=True)
    torch.cuda.synchronize()
    check_output(out, ref[0], True, "out")
    check_state(st, ref[3])


def test_prefill_qh_two_chunks_equal_one():
    B, Hq, Hkv, hd, W, n1, n2 = 2, 7, 1, 128, 16, 100, 77
    log("prefill_qh two chunks")
    d = _prefill_inputs(B, n1 + n2, Hq, Hkv, hd, seed=5)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W, s_per_query=True)
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    o1, rk, rv, st = sfa.prefill(c["q"][:, :n1].contiguous(), c["k"][:, :n1].contiguous(),
                                 c["v"][:, :n1].contiguous(), c["gamma"], c["alpha"], window=W,
                                 out_dtype=torch.float32, gamma_per_query_head=True)
    o2, rk, rv, st = sfa.prefill(c["q"][:, n1:].contiguous(), c["k"][:, n1:].contiguous(),
                                 c["v"][:, n1:].contiguous(), c["gamma"], c["alpha"], window=W,
                                 out_dtype=torch.float32, ring_k=rk, ring_v=rv, state=st,
                                 pos0=torch.full((B,), n1, dtype=torch.int32, device="cuda"),
                                 gamma_per_query_head=True)
    torch.cuda.synchronize()
    check_output(torch.cat([o1, o2], 1), ref[0], True, "out")
    check_exact(rk, ref[1], "ring_k")
    check_state(st, ref[3])


def _decode_inputs(L, B, Hq, Hkv, hd, W, seed, dtype=torch.bfloat16):
    d = inputs.decode_inputs(L, B, Hq, Hkv, hd, seed=seed, W=W, dtype=dtype)
    s = seed * 16
    d["state"] = inputs.normal((L, B, Hq, hd), s + 9, 1.0, torch.float32)
    d["gamma"] = inputs.uniform((L, Hq), 0.90, 0.99, s + 10)
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
                             d["pos"], d["gamma"], d["alpha"], s_per_query=True)
    rk, rv, st = d["ring_k"].cuda().clone(), d["ring_v"].cuda().clone(), d["state"].cuda().clone()
    out = sfa.decode_step(d["q"].cuda(), d["k_new"].cuda(), d["v_new"].cuda(), rk, rv, st,
                          d["pos"].cuda(), d["gamma"].cuda(), d["alpha"].cuda(), out_dtype=out_dtype,
                          gamma_per_query_head=True)
    torch.cuda.synchronize()
    check_output(out, ref[0], d["q"].dtype == torch.bfloat16, "out")
    check_exact(rk, ref[1], "ring_k")
    check_exact(rv, ref[2], "ring_v")
    check_state(st, ref[3])


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "L{}B{}H{}-{}d{}W{}-{}".format(*c[:6], str(c[6])[6:]))
def test_decode_qh_small(case):
    L, B, Hq, Hkv, hd, W, dt = case
    log(f"decode_qh case {case}")
    d = _decode_inputs(L, B, Hq, Hkv, hd, W, seed=L * 100 + Hq + W, dtype=dt)
    d["pos"] = torch.tensor([0, 1, W - 1, W, 5000][:B], dtype=torch.int32)
    for od in (torch.float32, torch.bfloat16):
        _decode_check(d, od)


def test_decode_qh_workload_7b_28_layers():
    """7B-shaped decode step (28 layers x 256 sequences, 28/4 heads, d 128, bf16), S per query head."""
    log("decode_qh 7B-shaped 28 layers")
    d = _decode_inputs(28, 256, 28, 4, 128, 16, seed=1003)
    _decode_check(d, torch.float32)


def test_decode_qh_continues_a_gpu_prefill_qh():
    """prefill_qh(n) then decode_qh steps == prefill_qh(n + steps) (oracle, per query head)."""
    B, Hq, Hkv, hd, W, n, m = 2, 8, 2, 128, 16, 40, 5
    log("decode_qh after prefill_qh")
    d = _prefill_inputs(B, n + m, Hq, Hkv, hd, seed=17)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W, s_per_query=True)
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    _, rk, rv, st = sfa.prefill(c["q"][:, :n].contiguous(), c["k"][:, :n].contiguous(),
                                c["v"][:, :n].contiguous(), c["gamma"], c["alpha"], window=W,
                                gamma_per_query_head=True)
    outs = []
    for i in range(m):
        t = n + i
        o = sfa.decode_step(c["q"][None, :, t].contiguous(), c["k"][None, :, t].contiguous(),
                            c["v"][None, :, t].contiguous(), rk[None], rv[None], st[None],
                            torch.full((B,), t, dtype=torch.int32, device="cuda"),
                            c["gamma"][None], c["alpha"][None], out_dtype=torch.float32,
                            gamma_per_query_head=True)
        outs.append(o[0])
    torch.cuda.synchronize()
    check_output(torch.stack(outs, 1), ref[0][:, n:], True, "decode out")
    check_state(st, ref[3])


def test_decode_qh_negative_position_skips_the_sequence():
    """Per query head: a negative pos entry leaves that sequence untouched."""
    from tests.test_gpu_decode import _skip_case
    L, B, Hq, Hkv, hd = 2, 5, 14, 2, 128
    log("decode_qh skip case")
    d = inputs.decode_inputs(L, B, Hq, Hkv, hd, seed=41)
    d["state"] = inputs.normal((L, B, Hq, hd), 4242, 1.0, torch.float32)
    d["gamma"] = inputs.uniform((L, Hq), 0.90, 0.99, 4343)
    d["pos"] = torch.tensor([5, 100, 16, 3, 31], dtype=torch.int32)
    _skip_case(d, 1, True)
