"""GPU parity of a prefill and a decode step whose tensors pass 2^31 elements
and 2^32 bytes.

Two sequences of 2^20 + 37 tokens with 9 query heads over one KV head (d 128,
bf16 in, fp32 out): the second sequence's queries start past 2^30 elements and
cross 2^31 about 815K tokens in, and all of its fp32 outputs lie past 2^32
bytes.  The sequences are independent, so the oracle runs the second one alone
(fp64 over its whole length: its state at every token) and the test compares
the outputs around the 2^31-element crossing, at both ends, the final state and
the ring.  The inputs are drawn by the seeded generator on the GPU and copied
to the host for the oracle.

The decode step covers 28 layers x 9,400 sequences with 28/4 heads (d 128,
W 16): its K and V rings hold 2.16e9 elements each (4.3 GB), so the units of
the last layers sit past 2^31 elements.  Every (layer, sequence) is
independent, so the oracle runs the last layer's last sequences alone.

The enhancement covers 24 layers x 32,768 tokens x hidden 4,096 (3.2e9
elements of bf16 input, per-layer pools, a carried ring and field): the last
layer starts past 2^31 elements.  Layers are independent apart from α_l, so
the oracle runs the last layer alone at its layer index.
"""
import numpy as np
import pytest
import torch

import oracle
import windowed_ewma_state_amd as sfa
from windowed_ewma_state_amd import inputs
from tests.parity import check_exact, check_output, check_state, log

pytestmark = pytest.mark.gpu


def test_prefill_past_2_31_elements():
    B, n, Hq, Hkv, hd, W = 2, (1 << 20) + 37, 9, 1, 128, 16
    log(f"prefill large: B {B} n {n} Hq {Hq} Hkv {Hkv} d {hd}")
    d = inputs.prefill_inputs(B, n, Hq, Hkv, hd, seed=2031, device="cuda")
    assert d["q"].numel() > 2 ** 31
    out, rk, rv, st = sfa.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], window=W,
                                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert out.numel() * out.element_size() > 2 ** 33
    b = 1
    ref = oracle.prefill(d["q"][b:b + 1].cpu(), d["k"][b:b + 1].cpu(), d["v"][b:b + 1].cpu(),
                         d["gamma"].cpu(), d["alpha"].cpu(), W)
    t_cross = -(-(2 ** 31) // (Hq * hd)) - b * n  # first token of sequence b past 2^31 query elements
    assert 0 < t_cross < n
    for lo, hi in [(0, 4096), (t_cross - 4096, t_cross + 4096), (n - 4096, n)]:
        check_output(out[b, lo:hi], ref[0][0, lo:hi], True, f"out[{b}, {lo}:{hi}]")
    check_exact(rk[b], ref[1][0], "ring_k")
    check_exact(rv[b], ref[2][0], "ring_v")
    check_state(st[b], ref[3][0])


def test_decode_past_2_31_elements():
    L, B, Hq, Hkv, hd, W = 28, 9400, 28, 4, 128, 16
    log(f"decode large: L {L} B {B} Hq {Hq} Hkv {Hkv} d {hd} W {W}")
    d = inputs.decode_inputs(L, B, Hq, Hkv, hd, seed=2032, W=W, device="cuda")
    assert d["ring_k"].numel() > 2 ** 31
    rk, rv, st = d["ring_k"].clone(), d["ring_v"].clone(), d["state"].clone()
    out = sfa.decode_step(d["q"], d["k_new"], d["v_new"], rk, rv, st, d["pos"], d["gamma"], d["alpha"],
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    ls, bs = slice(L - 1, L), slice(B - 8, B)  # units (27·B + b)·Hkv + G: past 2^31 ring elements
    assert ((L - 1) * B + B - 8) * Hkv * W * hd > 2 ** 31
    sub = {k: d[k][ls, bs].cpu() for k in ("q", "k_new", "v_new", "ring_k", "ring_v", "state")}
    ref = oracle.decode_step(sub["q"], sub["k_new"], sub["v_new"], sub["ring_k"], sub["ring_v"], sub["state"],
                             d["pos"][bs].cpu(), d["gamma"][ls].cpu(), d["alpha"][ls].cpu())
    check_output(out[ls, bs], ref[0], True, "out")
    check_exact(rk[ls, bs], ref[1], "ring_k")
    check_exact(rv[ls, bs], ref[2], "ring_v")
    check_state(st[ls, bs], ref[3])


def test_enhance_past_2_31_elements():
    L, T, H, R = 24, 32768, 4096, 16
    log(f"enhance large: L {L} T {T} H {H}")
    d = inputs.enhance_inputs(L, T, H, seed=2033, device="cuda")
    assert d["attn"].numel() > 2 ** 31 and (L - 1) * T * H > 2 ** 31
    ring = inputs.normal((L, R, H), 2034, 1.0, torch.float32, "cuda")
    field = inputs.normal((L, H), 2035, 1.0, torch.float32, "cuda")
    kw = dict(alpha_base=0.7, cross_decay=0.9, ema_gamma=0.95, temperature=0.07, clip=0.5)
    ring0, field0 = ring[L - 1].cpu().numpy()[None], field[L - 1].cpu().numpy()[None]
    out, _ = sfa.enhance(d["attn"], d["pool"], ring, field, t0=100, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    ref = oracle.enhance(d["attn"][L - 1:].cpu(), d["pool"][L - 1:].cpu(), ring0, field0, t0=100,
                         layer0=L - 1, n_layers=L, **kw)
    check_output(out[L - 1:], ref[0], True, "out")
    check_exact(ring[L - 1:], ref[2], "ring")
    rf = float(np.linalg.norm((field[L - 1:].cpu().double().numpy() - ref[3]).ravel()) / np.linalg.norm(ref[3].ravel()))
    log(f"  field rel-L2 {rf:.3e}")
    assert rf <= 1e-5
