"""GPU parity of sfa_decode_step against the CPU fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import windowed_ewma_state_amd as sfa
from windowed_ewma_state_amd import inputs
from tests.parity import check_exact, check_output, check_state, log

pytestmark = pytest.mark.gpu


def _run(d, out_dtype, device="cuda"):
    """Run the GPU step on copies; return (out, ring_k, ring_v, state) on the GPU."""
    rk = d["ring_k"].to(device).clone()
    rv = d["ring_v"].to(device).clone()
    st = d["state"].to(device).clone()
    out = sfa.decode_step(d["q"].to(device), d["k_new"].to(device), d["v_new"].to(device), rk, rv,
                          st, d["pos"].to(device), d["gamma"].to(device), d["alpha"].to(device),
                          out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, rk, rv, st


def _oracle(d):
    return oracle.decode_step(d["q"], d["k_new"], d["v_new"], d["ring_k"], d["ring_v"], d["state"],
                              d["pos"], d["gamma"], d["alpha"])


CASES = [  # (L, B, Hq, Hkv, hd, W, in_dtype)
    (2, 5, 8, 2, 64, 16, torch.bfloat16),
    (2, 5, 8, 2, 128, 16, torch.bfloat16),
    (1, 5, 4, 4, 128, 4, torch.bfloat16),
    (3, 5, 6, 1, 64, 1, torch.bfloat16),
    (2, 5, 36, 2, 128, 16, torch.bfloat16),  # 18 query heads per KV head: two head tiles
    (2, 5, 24, 2, 128, 16, torch.bfloat16),  # 12 query heads per KV head: 16-row query tiles (d 128)
    (2, 5, 32, 2, 64, 16, torch.bfloat16),  # 16 query heads per KV head: 16-row query tiles (d 64)
    (2, 5, 8, 2, 128, 16, torch.float32),
    (1, 5, 3, 3, 64, 7, torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "L{}B{}H{}-{}d{}W{}-{}".format(*c[:6], str(c[6])[6:]))
def test_decode_small(case):
    L, B, Hq, Hkv, hd, W, dt = case
    log(f"decode case {case}")
    d = inputs.decode_inputs(L, B, Hq, Hkv, hd, seed=77 + Hq + W, W=W, dtype=dt)
    d["pos"] = torch.tensor([0, W - 1, W, 3 * W + 2, 1000][:B], dtype=torch.int32)
    ref = _oracle(d)
    for od in (torch.float32, torch.bfloat16):
        out, rk, rv, st = _run(d, od)
        check_output(out, ref[0], dt == torch.bfloat16, f"out[{od}]")
        check_exact(rk, ref[1], "ring_k")
        check_exact(rv, ref[2], "ring_v")
        check_state(st, ref[3])


def test_decode_workload_7b_28_layers():
    """7B-shaped decode step over 28 layers (256 sequences, GQA 28/4, d 128, bf16)."""
    d = inputs.workload(3)
    log("decode 7B-shaped workload, 28 layers x 256 sequences")
    ref = _oracle(d)
    for od in (torch.float32, torch.bfloat16):
        out, rk, rv, st = _run(d, od)
        check_output(out, ref[0], True, f"out[{od}]")
        check_exact(rk, ref[1], "ring_k")
        check_exact(rv, ref[2], "ring_v")
        check_state(st, ref[3])


def test_decode_evicted_slot_identified_on_gpu():
    """S_new - γ S_old = (1-γ) k_evicted names slot pos mod W (random keys)."""
    L, B, Hq, Hkv, hd, W = 1, 4, 4, 2, 128, 16
    d = inputs.decode_inputs(L, B, Hq, Hkv, hd, seed=5, W=W, dtype=torch.float32)
    d["pos"] = torch.tensor([16, 21, 47, 1000], dtype=torch.int32)
    _, _, _, st = _run(d, torch.float32)
    S_new = st.cpu().double().numpy()
    S_old = d["state"].double().numpy()
    g = d["gamma"].double().numpy()
    rk = d["ring_k"].double().numpy()
    for b, p in enumerate(d["pos"].tolist()):
        for G in range(Hkv):
            delta = S_new[0, b, G] - g[0, G] * S_old[0, b, G]
            resid = [np.abs(delta - (1 - g[0, G]) * rk[0, b, G, j]).max() for j in range(W)]
            assert int(np.argmin(resid)) == p % W and resid[p % W] < 1e-5


def test_decode_steps_continue_a_gpu_prefill():
    """P7 on the GPU: prefill(n) then m decode steps == oracle prefill(n+m)."""
    B, Hq, Hkv, hd, W, n, m = 2, 8, 2, 128, 16, 40, 6
    N = n + m
    d = inputs.prefill_inputs(B, N, Hq, Hkv, hd, seed=11, std=0.5)
    full, frk, frv, fst = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W)
    cu = {k_: v_.cuda() for k_, v_ in d.items() if isinstance(v_, torch.Tensor)}
    _, rk, rv, st = sfa.prefill(cu["q"][:, :n].contiguous(), cu["k"][:, :n].contiguous(),
                                cu["v"][:, :n].contiguous(), cu["gamma"], cu["alpha"], window=W,
                                out_dtype=torch.float32)
    rk, rv, st = rk[None], rv[None], st[None]
    for i in range(m):
        t = n + i
        o = sfa.decode_step(cu["q"][None, :, t].contiguous(), cu["k"][None, :, t].contiguous(),
                            cu["v"][None, :, t].contiguous(), rk, rv, st,
                            torch.full((B,), t, dtype=torch.int32, device="cuda"),
                            cu["gamma"][None], cu["alpha"][None], out_dtype=torch.float32)
        check_output(o[0], full[:, t], True, f"step {t}")
    check_exact(rk[0], frk, "ring_k")
    check_exact(rv[0], frv, "ring_v")
    check_state(st[0], fst)


def _skip_case(d, skip, qh):
    """Run with pos[skip] = -1; check the skipped sequence is untouched (bit for
    bit) and the others match the oracle run on the batch without it."""
    keep = [b for b in range(d["pos"].numel()) if b != skip]
    pos = d["pos"].clone()
    pos[skip] = -1
    sentinel = torch.full(d["q"].shape, 7.25, dtype=torch.float32)
    out = sentinel.cuda()
    rk, rv, st = d["ring_k"].cuda(), d["ring_v"].cuda(), d["state"].cuda()
    sfa.decode_step(d["q"].cuda(), d["k_new"].cuda(), d["v_new"].cuda(), rk, rv, st, pos.cuda(),
                    d["gamma"].cuda(), d["alpha"].cuda(), out=out, gamma_per_query_head=qh)
    torch.cuda.synchronize()
    assert torch.equal(out[:, skip].cpu(), sentinel[:, skip]), "skipped sequence: out written"
    assert torch.equal(rk[:, skip].cpu(), d["ring_k"][:, skip]), "skipped sequence: ring_k written"
    assert torch.equal(rv[:, skip].cpu(), d["ring_v"][:, skip]), "skipped sequence: ring_v written"
    assert torch.equal(st[:, skip].cpu(), d["state"][:, skip]), "skipped sequence: state written"
    sub = {k_: (v_[:, keep].contiguous() if k_ not in ("gamma", "alpha", "pos", "window") else v_)
           for k_, v_ in d.items()}
    sub["pos"] = d["pos"][keep].contiguous()
    ref = oracle.decode_step(sub["q"], sub["k_new"], sub["v_new"], sub["ring_k"], sub["ring_v"],
                             sub["state"], sub["pos"], sub["gamma"], sub["alpha"], s_per_query=qh)
    check_output(out[:, keep], ref[0], d["q"].dtype == torch.bfloat16, "out (kept sequences)")
    check_exact(rk[:, keep], ref[1], "ring_k")
    check_exact(rv[:, keep], ref[2], "ring_v")
    check_state(st[:, keep], ref[3])


@pytest.mark.parametrize("hd", [64, 128])
def test_decode_negative_position_skips_the_sequence(hd):
    """A negative pos entry leaves that sequence's out, ring and S untouched."""
    L, B, Hq, Hkv = 3, 6, 8, 2
    log(f"decode skip case hd {hd}")
    d = inputs.decode_inputs(L, B, Hq, Hkv, hd, seed=31 + hd)
    d["pos"] = torch.tensor([3, 40, 16, 15, 200, 7], dtype=torch.int32)
    _skip_case(d, 2, False)


def test_decode_per_layer_launches_equal_one_launch_7b():
    """The 7B-shaped step (28 layers x 256 sequences, 28/4 heads, d 128, bf16)
    as 28 single-layer launches (the form bench.py replays per layer: one unit
    per wave) equals the one launch over all layers bit for bit: out, both
    rings and S.  (The one launch is checked against the oracle at this shape.)"""
    log("decode 7B: 28 per-layer launches vs one launch")
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inputs.workload(3).items()}
    L = d["q"].shape[0]
    one = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    per = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    o1 = sfa.decode_step(one["q"], one["k_new"], one["v_new"], one["ring_k"], one["ring_v"], one["state"],
                         one["pos"], one["gamma"], one["alpha"], out_dtype=torch.bfloat16)
    o2 = torch.empty_like(o1)
    for l in range(L):
        sl = slice(l, l + 1)
        sfa.decode_step(per["q"][sl], per["k_new"][sl], per["v_new"][sl], per["ring_k"][sl], per["ring_v"][sl],
                        per["state"][sl], per["pos"], per["gamma"][sl], per["alpha"][sl], out=o2[sl])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "out"
    for key in ("ring_k", "ring_v", "state"):
        assert torch.equal(one[key], per[key]), key
