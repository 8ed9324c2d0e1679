"""Pins for the CPU fp64 oracle: things the pages and the mathematics fix.

Each test checks the oracle against something other than itself:
  * hand-computed worked examples (tests/golden/hand_examples.json);
  * special cases that reduce to a library routine (torch SDPA in fp64);
  * closed forms of the EWMA far field (explicit power sums, not the recurrence);
  * invariants (prefill/decode consistency, GQA == repeated-KV MHA, bit-exact ring);
  * brute force on tiny inputs written in a different form (masked dense
    attention + explicit power sum).

Sources: [P1] "Signal Field Attention (SFA)：8KB代码实现4.16倍推理加速与248倍内存压缩"
section 2.1 (near field, far field, fusion) and 2.2 (k = 16 ring);
[P3] "Dalin Soma SFA基于信号场注意力机制的神经网络推理加速框架" sections 2.1, 2.2,
2.4; [P2] "Signal Field Attention (SFA)" project page (SFA_Config, cross-layer decay).
"""
import json
import math
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))
RNG = np.random.default_rng(20261203)


def _rand(shape, std=1.0):
    return (RNG.standard_normal(shape) * std).astype(np.float32)


def _sdpa(q, k, v, mask, scale):
    """Reference attention via torch SDPA in fp64.  q [B,n,Hq,d], k/v [B,n,Hkv,d]."""
    g = q.shape[2] // k.shape[2]
    Q = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
    K = torch.from_numpy(k.astype(np.float64)).repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    V = torch.from_numpy(v.astype(np.float64)).repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, attn_mask=torch.from_numpy(mask), scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def _band(n, W):
    t = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return (j <= t) & (j > t - W)


def _ewma_closed_form(k, gamma, W):
    """S_t = (1-γ) Σ_{j=0}^{t-W} γ^{t-W-j} k_j for t >= W, 0 before.  k [n,d]."""
    n = k.shape[0]
    S = np.zeros((n, k.shape[1]))
    for t in range(W, n):
        m = t - W
        w = (1.0 - gamma) * gamma ** (m - np.arange(m + 1))
        S[t] = w @ k[: m + 1].astype(np.float64)
    return S


def _far_field_trajectory(q, k, v, gamma, W, scale=0.0):
    """S_t per (b, query head) recovered as O(α=1) - O(α=0)."""
    B, n, Hq, d = q.shape
    o1, *_ = oracle.prefill(q, k, v, gamma, np.ones(Hq), W, scale)
    o0, *_ = oracle.prefill(q, k, v, gamma, np.zeros(Hq), W, scale)
    return o1 - o0


# --------------------------------------------------------------------------
# hand-computed worked examples
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["prefill_ewma_w1", "prefill_softmax_two_keys",
                                  "prefill_eviction_order"])
def test_golden_prefill(name):
    g = GOLD[name]
    n = len(g["q"])
    sh = (1, n, 1, 1)
    out, rk, rv, st = oracle.prefill(np.array(g["q"]).reshape(sh), np.array(g["k"]).reshape(sh),
                                     np.array(g["v"]).reshape(sh), g["gamma"], g["alpha"],
                                     g["W"], g["scale"])
    np.testing.assert_allclose(out.ravel(), g["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(st.ravel(), [g["state"]], rtol=0, atol=1e-12)
    assert rk.ravel().tolist() == g["ring_k"]
    assert rv.ravel().tolist() == g["ring_v"]


def test_golden_decode():
    g = GOLD["decode_step"]
    W = g["W"]
    out, rk, rv, st = oracle.decode_step(
        np.full((1, 1, 1, 1), g["q"]), np.full((1, 1, 1, 1), g["k_new"]),
        np.full((1, 1, 1, 1), g["v_new"]), np.array(g["ring_k_in"]).reshape(1, 1, 1, W, 1),
        np.array(g["ring_v_in"]).reshape(1, 1, 1, W, 1), np.full((1, 1, 1, 1), g["state_in"]),
        np.array([g["pos"]]), np.full((1, 1), g["gamma"]), np.full((1, 1), g["alpha"]),
        g["scale"])
    assert out.item() == g["out"]
    assert st.item() == g["state"]
    assert rk.ravel().tolist() == g["ring_k"]
    assert rv.ravel().tolist() == g["ring_v"]


def test_golden_enhance():
    g = GOLD["enhance_two_tokens"]
    attn = np.array(g["attn"], dtype=np.float32).reshape(1, -1, 1)
    pool = np.array(g["pool"], dtype=np.float32).reshape(1, 1, 1)
    out, enh, R, F = oracle.enhance(attn, pool, alpha_base=g["alpha_base"],
                                    cross_decay=g["cross_decay"], ema_gamma=g["ema_gamma"],
                                    temperature=g["temperature"], clip=g["clip"],
                                    ring_size=g["ring_size"])
    np.testing.assert_allclose(out.ravel(), g["out"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(enh.ravel(), g["enhancement"], rtol=0, atol=1e-15)
    assert R.ravel().tolist() == g["ring"]
    assert F.item() == g["field"]


def test_golden_alpha_layer():
    g = GOLD["alpha_layer_quickstart"]
    for layer, want in zip(g["layers"], g["alpha"]):
        got = oracle.alpha_layer(g["alpha_base"], g["cross_decay"], layer, g["n_layers"])
        assert got == pytest.approx(want, rel=1e-14)
    # a single-layer model uses ratio 0
    assert oracle.alpha_layer(0.1, 0.8, 0, 1) == pytest.approx(0.03, rel=1e-15)


# --------------------------------------------------------------------------
# P1 / P2: library special cases (torch SDPA in fp64)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("B,n,Hq,Hkv,d,W", [(1, 12, 1, 1, 8, 16), (2, 16, 4, 2, 8, 16),
                                             (1, 5, 3, 1, 4, 7), (2, 9, 6, 3, 16, 9)])
def test_full_causal_when_window_covers_sequence(B, n, Hq, Hkv, d, W):
    """P1: W >= n -> nothing leaves the window, S stays 0, O is causal softmax attention."""
    q, k, v = _rand((B, n, Hq, d)), _rand((B, n, Hkv, d)), _rand((B, n, Hkv, d))
    alpha = RNG.uniform(0, 1, Hq)  # α is irrelevant while S = 0
    out, rk, rv, st = oracle.prefill(q, k, v, RNG.uniform(0.5, 0.99, Hkv), alpha, W)
    ref = _sdpa(q, k, v, np.tril(np.ones((n, n), dtype=bool)), 1.0 / math.sqrt(d))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert np.all(st == 0.0)


@pytest.mark.parametrize("B,n,Hq,Hkv,d,W", [(1, 40, 2, 1, 8, 16), (2, 33, 4, 4, 16, 5),
                                             (1, 20, 7, 1, 8, 1), (1, 64, 2, 2, 4, 3)])
def test_band_attention_when_alpha_zero(B, n, Hq, Hkv, d, W):
    """P2: α = 0 -> O is band-masked softmax attention (t-W < j <= t)."""
    q, k, v = _rand((B, n, Hq, d)), _rand((B, n, Hkv, d)), _rand((B, n, Hkv, d))
    scale = 0.3
    out, *_ = oracle.prefill(q, k, v, RNG.uniform(0.5, 0.99, Hkv), np.zeros(Hq), W, scale)
    ref = _sdpa(q, k, v, _band(n, W), scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# P3 - P6: closed forms of the far field
# --------------------------------------------------------------------------
@pytest.mark.parametrize("W", [1, 2, 16])
def test_gamma_zero_state_is_last_evicted_key(W):
    """P3: γ = 0 -> S_t = k_{t-W} for t >= W, 0 before; final state = k_{n-1-W}."""
    n, d = 40, 8
    q, k, v = _rand((1, n, 2, d)), _rand((1, n, 1, d)), _rand((1, n, 1, d))
    S = _far_field_trajectory(q, k, v, 0.0, W)
    for h in range(2):
        np.testing.assert_allclose(S[0, W:, h], k[0, : n - W, 0], rtol=0, atol=1e-12)
        assert np.all(np.abs(S[0, :W, h]) <= 1e-12)
    _, _, _, st = oracle.prefill(q, k, v, 0.0, 0.0, W)
    assert np.array_equal(st[0, 0], k[0, n - 1 - W, 0].astype(np.float64))


@pytest.mark.parametrize("gamma,W", [(0.9, 16), (0.5, 3), (0.99, 1), (0.3, 7)])
def test_state_matches_power_sum(gamma, W):
    """P4: S_t = (1-γ) Σ_{j<=t-W} γ^{t-W-j} k_j, per KV head, for every t."""
    n, d, Hkv, Hq = 50, 8, 2, 4
    q, k, v = _rand((1, n, Hq, d)), _rand((1, n, Hkv, d)), _rand((1, n, Hkv, d))
    gam = np.array([gamma, gamma * 0.9])
    S = _far_field_trajectory(q, k, v, gam, W)
    for h in range(Hq):
        G = h // (Hq // Hkv)
        ref = _ewma_closed_form(k[0, :, G], gam[G], W)
        np.testing.assert_allclose(S[0, :, h], ref, rtol=1e-10, atol=1e-12)
    _, _, _, st = oracle.prefill(q, k, v, gam, 0.0, W)
    for G in range(Hkv):
        ref = _ewma_closed_form(k[0, :, G], gam[G], W)[-1]
        np.testing.assert_allclose(st[0, G], ref, rtol=1e-12, atol=1e-14)


def test_constant_keys_state():
    """P5: constant key k -> S_t = k (1 - γ^m), m = t - W + 1."""
    n, d, W, gamma = 60, 4, 16, 0.93
    kc = _rand((d,))
    k = np.broadcast_to(kc, (1, n, 1, d)).copy()
    q, v = _rand((1, n, 1, d)), _rand((1, n, 1, d))
    S = _far_field_trajectory(q, k, v, gamma, W)
    for t in range(n):
        m = t - W + 1
        ref = kc.astype(np.float64) * (1.0 - gamma ** m) if m > 0 else np.zeros(d)
        np.testing.assert_allclose(S[0, t, 0], ref, rtol=1e-12, atol=1e-14)


def test_window_one_is_value_plus_far_field():
    """P6: W = 1 -> O_t = v_t + α S_t with S_t the EWMA of k_0..k_{t-1}."""
    n, d, gamma, alpha = 30, 8, 0.8, 0.37
    q, k, v = _rand((1, n, 1, d)), _rand((1, n, 1, d)), _rand((1, n, 1, d))
    out, *_ = oracle.prefill(q, k, v, gamma, alpha, 1)
    S = _ewma_closed_form(k[0, :, 0], gamma, 1)
    np.testing.assert_allclose(out[0, :, 0], v[0, :, 0] + alpha * S, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# P11: brute force on tiny inputs (masked dense attention + explicit power sum)
# --------------------------------------------------------------------------
def _brute_force(q, k, v, gamma, alpha, W, scale):
    B, n, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    out = np.zeros((B, n, Hq, d))
    for b in range(B):
        for h in range(Hq):
            G = h // g
            K = k[b, :, G].astype(np.float64)
            V = v[b, :, G].astype(np.float64)
            S = _ewma_closed_form(K, gamma[G], W)
            s = scale * (q[b, :, h].astype(np.float64) @ K.T)  # [n, n]
            s = np.where(_band(n, W), s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            out[b, :, h] = p @ V + alpha[h] * S
    return out


@pytest.mark.parametrize("case", range(12))
def test_brute_force_tiny(case):
    r = np.random.default_rng(case)
    W = int(r.integers(1, 17))
    n = int(r.integers(1, 41))
    d = int(r.integers(1, 9))
    Hkv = int(r.integers(1, 3))
    Hq = Hkv * int(r.integers(1, 4))
    B = int(r.integers(1, 3))
    q = r.standard_normal((B, n, Hq, d)).astype(np.float32)
    k = r.standard_normal((B, n, Hkv, d)).astype(np.float32)
    v = r.standard_normal((B, n, Hkv, d)).astype(np.float32)
    gamma = r.uniform(0.0, 0.99, Hkv)
    alpha = r.uniform(-0.5, 0.5, Hq)
    scale = float(r.uniform(0.1, 1.0))
    out, *_ = oracle.prefill(q, k, v, gamma, alpha, W, scale)
    np.testing.assert_allclose(out, _brute_force(q, k, v, gamma, alpha, W, scale),
                               rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# P7 - P9: invariants
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n,m,W", [(20, 5, 16), (3, 20, 16), (0, 9, 4), (16, 1, 16), (15, 2, 16),
                                   (7, 7, 1), (90, 12, 80)])
def test_prefill_then_decode_equals_longer_prefill(n, m, W):
    """P7: prefill(n) followed by m decode steps reproduces prefill(n+m)."""
    B, Hq, Hkv, d = 2, 4, 2, 8
    N = n + m
    q, k, v = _rand((B, N, Hq, d)), _rand((B, N, Hkv, d)), _rand((B, N, Hkv, d))
    gamma, alpha = RNG.uniform(0.5, 0.99, Hkv), RNG.uniform(0, 0.5, Hq)
    full, frk, frv, fst = oracle.prefill(q, k, v, gamma, alpha, W)
    if n > 0:
        _, rk, rv, st = oracle.prefill(q[:, :n], k[:, :n], v[:, :n], gamma, alpha, W)
    else:
        rk, rv, st = np.zeros((B, Hkv, W, d)), np.zeros((B, Hkv, W, d)), np.zeros((B, Hkv, d))
    for i in range(m):
        t = n + i
        o, rk, rv, st = oracle.decode_step(q[None, :, t], k[None, :, t], v[None, :, t],
                                           rk[None], rv[None], st[None],
                                           np.full(B, t, dtype=np.int32), gamma[None],
                                           alpha[None])
        rk, rv, st = rk[0], rv[0], st[0]
        np.testing.assert_allclose(o[0], full[:, t], rtol=1e-12, atol=1e-12)
    # ring slots that were ever written agree bit for bit
    written = min(N, W)
    assert np.array_equal(rk[:, :, :written], frk[:, :, :written])
    assert np.array_equal(rv[:, :, :written], frv[:, :, :written])
    np.testing.assert_allclose(st, fst, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("n1,n2,W", [(20, 13, 16), (5, 30, 16), (40, 3, 4), (9, 9, 1)])
def test_prefill_continuation_equals_single_prefill(n1, n2, W):
    """Chunked prefill: prefill(n1) then prefill(n2, from the carried ring/state)."""
    B, Hq, Hkv, d = 2, 6, 3, 8
    N = n1 + n2
    q, k, v = _rand((B, N, Hq, d)), _rand((B, N, Hkv, d)), _rand((B, N, Hkv, d))
    gamma, alpha = RNG.uniform(0.5, 0.99, Hkv), RNG.uniform(0, 0.5, Hq)
    full, frk, frv, fst = oracle.prefill(q, k, v, gamma, alpha, W)
    o1, rk, rv, st = oracle.prefill(q[:, :n1], k[:, :n1], v[:, :n1], gamma, alpha, W)
    o2, rk, rv, st = oracle.prefill(q[:, n1:], k[:, n1:], v[:, n1:], gamma, alpha, W,
                                    ring_k=rk, ring_v=rv, state=st,
                                    pos0=np.full(B, n1, dtype=np.int32))
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), full, rtol=1e-12, atol=1e-12)
    assert np.array_equal(rk, frk) and np.array_equal(rv, frv)
    np.testing.assert_allclose(st, fst, rtol=1e-12, atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv():
    """P8: GQA == MHA with each KV head (and its γ) repeated g times."""
    B, n, Hq, Hkv, d, W = 2, 37, 6, 2, 8, 5
    g = Hq // Hkv
    q, k, v = _rand((B, n, Hq, d)), _rand((B, n, Hkv, d)), _rand((B, n, Hkv, d))
    gamma, alpha = RNG.uniform(0.5, 0.99, Hkv), RNG.uniform(0, 0.5, Hq)
    o_gqa, *_ = oracle.prefill(q, k, v, gamma, alpha, W)
    o_mha, *_ = oracle.prefill(q, np.repeat(k, g, axis=2), np.repeat(v, g, axis=2),
                               np.repeat(gamma, g), alpha, W)
    np.testing.assert_array_equal(o_gqa, o_mha)


@pytest.mark.parametrize("W", [1, 4, 16])
def test_decode_ring_update_is_exact(W):
    """P9: slot pos mod W takes k_new/v_new, others are unchanged, and
    S_new - γ S_old = (1-γ) k_evicted names the evicted slot."""
    L, B, Hq, Hkv, d = 2, 5, 4, 2, 8
    ring_k, ring_v = _rand((L, B, Hkv, W, d)), _rand((L, B, Hkv, W, d))
    state = _rand((L, B, Hkv, d))
    kn, vn, q = _rand((L, B, Hkv, d)), _rand((L, B, Hkv, d)), _rand((L, B, Hq, d))
    pos = np.array([0, W - 1, W, 3 * W + 2, 1000], dtype=np.int32)[:B]
    gamma, alpha = RNG.uniform(0.5, 0.99, (L, Hkv)), RNG.uniform(0, 0.5, (L, Hq))
    out, rk, rv, st = oracle.decode_step(q, kn, vn, ring_k, ring_v, state, pos, gamma, alpha)
    for b, p in enumerate(pos):
        s = p % W
        for j in range(W):
            want_k = kn[:, b] if j == s else ring_k[:, b, :, j]
            want_v = vn[:, b] if j == s else ring_v[:, b, :, j]
            assert np.array_equal(rk[:, b, :, j], want_k.astype(np.float64))
            assert np.array_equal(rv[:, b, :, j], want_v.astype(np.float64))
        for l in range(L):
            for G in range(Hkv):
                delta = st[l, b, G] - gamma[l, G] * state[l, b, G]
                if p >= W:
                    resid = [np.abs(delta - (1 - gamma[l, G]) * ring_k[l, b, G, j]).max()
                             for j in range(W)]
                    assert int(np.argmin(resid)) == s and resid[s] < 1e-12
                else:
                    np.testing.assert_array_equal(st[l, b, G], state[l, b, G])


def test_decode_partial_ring_uses_only_valid_slots():
    """pos < W-1: softmax over slots 0..pos only (slot contents above pos are ignored)."""
    L, B, Hq, Hkv, d, W = 1, 1, 2, 1, 8, 16
    p = 5
    ring_k, ring_v = _rand((L, B, Hkv, W, d)), _rand((L, B, Hkv, W, d))
    kn, vn, q = _rand((L, B, Hkv, d)), _rand((L, B, Hkv, d)), _rand((L, B, Hq, d))
    state = np.zeros((L, B, Hkv, d))
    out1, *_ = oracle.decode_step(q, kn, vn, ring_k, ring_v, state, [p], 0.9, 0.3)
    junk_k, junk_v = ring_k.copy(), ring_v.copy()
    junk_k[..., p + 1:, :] = 1e6
    junk_v[..., p + 1:, :] = -1e6
    out2, *_ = oracle.decode_step(q, kn, vn, junk_k, junk_v, state, [p], 0.9, 0.3)
    np.testing.assert_array_equal(out1, out2)
    # and equals band attention over positions 0..p with positions taken from the slots
    K = np.concatenate([ring_k[0, 0, 0, :p], kn[0, 0]], axis=0)[None, :, None]
    V = np.concatenate([ring_v[0, 0, 0, :p], vn[0, 0]], axis=0)[None, :, None]
    ref = _sdpa(np.repeat(q[0, 0][None, None], p + 1, axis=1), K, V,
                np.tril(np.ones((p + 1, p + 1), dtype=bool)), 1 / math.sqrt(d))
    np.testing.assert_allclose(out1[0, 0], ref[0, p], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# P10: triple-channel enhancement closed forms
# --------------------------------------------------------------------------
def _enh_inputs(L, T, H, S, seed):
    r = np.random.default_rng(seed)
    attn = r.standard_normal((L, T, H)).astype(np.float32)
    pool = r.standard_normal((L, S, H))
    pool = (pool / np.linalg.norm(pool, axis=-1, keepdims=True)).astype(np.float32)
    return attn, pool


def test_enhance_alpha_zero_is_identity():
    attn, pool = _enh_inputs(3, 20, 16, 8, 1)
    out, enh, *_ = oracle.enhance(attn, pool, alpha_base=0.0)
    assert np.array_equal(out, attn.astype(np.float64))
    assert np.all(enh == 0.0)


def test_enhance_is_bounded_by_clip_times_alpha():
    attn, pool = _enh_inputs(4, 30, 16, 8, 2)
    out, enh, *_ = oracle.enhance(attn, pool, alpha_base=0.7, cross_decay=0.9, clip=0.5)
    for l in range(4):
        al = oracle.alpha_layer(0.7, 0.9, l, 4)
        assert np.abs(out[l] - attn[l]).max() <= 0.5 * al * (1 + 1e-12)
        assert np.abs(enh[l]).max() == pytest.approx(0.5 * al)  # N(0,1) inputs saturate


def test_enhance_constant_input_closed_form():
    """Constant a, one-slot pool (sem = s_0), no clipping:
    e_t = a·min(t+1,R)/R + 0.5·a(1-γ^{t+1}) + 0.5·s_0."""
    L, T, H, R, gam = 2, 40, 8, 16, 0.9
    r = np.random.default_rng(3)
    a = r.standard_normal(H).astype(np.float32)
    attn = np.broadcast_to(a, (L, T, H)).copy()
    s0 = r.standard_normal((L, 1, H))
    s0 = (s0 / np.linalg.norm(s0, axis=-1, keepdims=True)).astype(np.float32)
    out, enh, Rf, Ff = oracle.enhance(attn, s0, alpha_base=0.2, cross_decay=0.8, ema_gamma=gam,
                                      clip=1e9, ring_size=R)
    for l in range(L):
        al = oracle.alpha_layer(0.2, 0.8, l, L)
        for t in range(T):
            a64, s64 = a.astype(np.float64), s0[l, 0].astype(np.float64)
            e = a64 * min(t + 1, R) / R + 0.5 * a64 * (1 - gam ** (t + 1)) + 0.5 * s64
            np.testing.assert_allclose(enh[l, t], al * e, rtol=1e-12, atol=1e-15)


def test_enhance_gamma_zero_field_is_current_token():
    """γ_e = 0 -> F = a_t; ring of 1 -> rm = a_t; so e = 1.5 a_t + 0.5 sem."""
    attn, pool = _enh_inputs(1, 10, 8, 1, 4)
    out, enh, *_ = oracle.enhance(attn, pool, alpha_base=1.0, ema_gamma=0.0, clip=1e9,
                                  ring_size=1)
    al = oracle.alpha_layer(1.0, 0.8, 0, 1)
    e = 1.5 * attn[0].astype(np.float64) + 0.5 * pool[0, 0].astype(np.float64)
    np.testing.assert_allclose(enh[0], al * e, rtol=1e-12, atol=1e-15)


def test_enhance_semantic_softmax_closed_form():
    """Orthonormal slots e1, e2 and a = r(0.6, 0.8): cosines (0.6, 0.8),
    w = softmax((0.6, 0.8)/T), sem = (w1, w2)."""
    T = 0.07
    attn = np.array([[[0.6 * 3, 0.8 * 3]]], dtype=np.float32)  # |a| = 3
    pool = np.array([[[1.0, 0.0], [0.0, 1.0]]], dtype=np.float32)
    out, enh, *_ = oracle.enhance(attn, pool, alpha_base=1.0, ema_gamma=0.0, clip=1e9,
                                  ring_size=1, temperature=T)
    a64 = attn[0, 0].astype(np.float64)
    c = a64 / math.hypot(*a64)  # cosines with e1, e2 are the unit vector's coordinates
    w = np.exp(c / T) / np.exp(c / T).sum()
    e = 1.5 * attn[0, 0].astype(np.float64) + 0.5 * w
    np.testing.assert_allclose(enh[0, 0], 0.3 * e, rtol=1e-12)


def test_enhance_state_carry_and_ring_contents():
    """Ring holds the last R tokens at slot (t0+t) mod R, bit-exact; the field
    equals γ^T F_0 + (1-γ) Σ γ^{T-1-t} a_t; and two calls equal one."""
    L, T, H, S, R, gam = 2, 37, 8, 4, 16, 0.95
    attn, pool = _enh_inputs(L, T, H, S, 5)
    out, enh, Rf, Ff = oracle.enhance(attn, pool, ema_gamma=gam, ring_size=R)
    for t in range(T - R, T):
        assert np.array_equal(Rf[:, t % R], attn[:, t].astype(np.float64))
    wts = (1 - gam) * gam ** (T - 1 - np.arange(T))
    np.testing.assert_allclose(Ff, np.einsum("t,lth->lh", wts, attn.astype(np.float64)),
                               rtol=1e-12, atol=1e-14)
    T1 = 11
    o1, e1, R1, F1 = oracle.enhance(attn[:, :T1], pool, ema_gamma=gam, ring_size=R)
    o2, e2, R2, F2 = oracle.enhance(attn[:, T1:], pool, R1, F1, ema_gamma=gam, ring_size=R,
                                    t0=T1)
    np.testing.assert_allclose(np.concatenate([o1, o2], 1), out, rtol=1e-13, atol=1e-14)
    assert np.array_equal(R2, Rf)
    np.testing.assert_allclose(F2, Ff, rtol=1e-13, atol=1e-15)


def test_enhance_layer_offset_and_shared_pool():
    L, T, H, S = 4, 9, 8, 5
    attn, pool = _enh_inputs(L, T, H, S, 6)
    full, *_ = oracle.enhance(attn, pool)
    part, *_ = oracle.enhance(attn[2:], pool[2:], layer0=2, n_layers=4)
    np.testing.assert_array_equal(part, full[2:])
    shared, *_ = oracle.enhance(attn, pool[0], shared_pool=True)
    rep, *_ = oracle.enhance(attn, np.broadcast_to(pool[0], (L, S, H)).copy())
    np.testing.assert_array_equal(shared, rep)


def test_enhance_brute_force_tiny():
    """Each output rebuilt from scratch: ring mean from the explicit last-R window
    (zeros before the start), field as a power sum, cosine softmax with numpy."""
    L, T, H, S, R, gam, Tmp, clip = 2, 25, 6, 3, 4, 0.7, 0.5, 0.4
    attn, pool = _enh_inputs(L, T, H, S, 7)
    out, enh, *_ = oracle.enhance(attn, pool, alpha_base=0.5, cross_decay=0.6, ema_gamma=gam,
                                  temperature=Tmp, clip=clip, ring_size=R)
    A = attn.astype(np.float64)
    P = pool.astype(np.float64)
    for l in range(L):
        al = 0.5 * (0.3 + 0.7 * l / (L - 1)) * 0.6 ** l
        for t in range(T):
            rm = A[l, max(0, t - R + 1): t + 1].sum(0) / R
            F = ((1 - gam) * gam ** (t - np.arange(t + 1))) @ A[l, : t + 1]
            a = A[l, t]
            c = (P[l] @ a) / (np.linalg.norm(a) * np.linalg.norm(P[l], axis=1))
            w = np.exp(c / Tmp - (c / Tmp).max())
            w /= w.sum()
            e = np.clip(rm + 0.5 * F + 0.5 * (w @ P[l]), -clip, clip)
            np.testing.assert_allclose(out[l, t], a + al * e, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# P12: the other reading of "per-head γ" (γ and S per query head)
# --------------------------------------------------------------------------
def _brute_force_per_query(q, k, v, gamma_q, alpha, W, scale):
    """Masked dense attention plus, per query head h, the power sum of its KV
    head's evicted keys with γ_h."""
    B, n, Hq, d = q.shape
    g = Hq // k.shape[2]
    out = np.zeros((B, n, Hq, d))
    for b in range(B):
        for h in range(Hq):
            K = k[b, :, h // g].astype(np.float64)
            V = v[b, :, h // g].astype(np.float64)
            S = _ewma_closed_form(K, gamma_q[h], W)
            s = scale * (q[b, :, h].astype(np.float64) @ K.T)
            s = np.where(_band(n, W), s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            out[b, :, h] = p @ V + alpha[h] * S
    return out


@pytest.mark.parametrize("case", range(8))
def test_per_query_gamma_brute_force_tiny(case):
    r = np.random.default_rng(100 + case)
    W = int(r.integers(1, 17))
    n = int(r.integers(1, 41))
    d = int(r.integers(1, 9))
    Hkv = int(r.integers(1, 3))
    Hq = Hkv * int(r.integers(2, 4))
    B = int(r.integers(1, 3))
    q = r.standard_normal((B, n, Hq, d)).astype(np.float32)
    k = r.standard_normal((B, n, Hkv, d)).astype(np.float32)
    v = r.standard_normal((B, n, Hkv, d)).astype(np.float32)
    gamma_q = r.uniform(0.0, 0.99, Hq)
    alpha = r.uniform(-0.5, 0.5, Hq)
    scale = float(r.uniform(0.1, 1.0))
    out, _, _, st = oracle.prefill(q, k, v, gamma_q, alpha, W, scale, s_per_query=True)
    np.testing.assert_allclose(out, _brute_force_per_query(q, k, v, gamma_q, alpha, W, scale),
                               rtol=1e-11, atol=1e-12)
    # the final state of every query head is its power sum at the last token
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            K = k[b, :, h // g].astype(np.float64)
            last = _ewma_closed_form(K, gamma_q[h], W)[n - 1]
            np.testing.assert_allclose(st[b, h], last, rtol=1e-11, atol=1e-12)


def test_per_query_gamma_equal_within_group_is_kv_mode():
    """γ_h equal to γ_G for every query head of group G: the same outputs, and
    every query head's S equal to its KV head's S (prefill and decode)."""
    B, n, Hq, Hkv, d, W = 2, 45, 6, 2, 8, 16
    g = Hq // Hkv
    q, k, v = _rand((B, n, Hq, d)), _rand((B, n, Hkv, d)), _rand((B, n, Hkv, d))
    gamma, alpha = RNG.uniform(0.5, 0.99, Hkv), RNG.uniform(0, 0.5, Hq)
    a = oracle.prefill(q, k, v, gamma, alpha, W)
    b_ = oracle.prefill(q, k, v, np.repeat(gamma, g), alpha, W, s_per_query=True)
    np.testing.assert_array_equal(a[0], b_[0])
    np.testing.assert_array_equal(np.repeat(a[3], g, axis=1), b_[3])
    L = 2
    dq, dk, dv = _rand((L, B, Hq, d)), _rand((L, B, Hkv, d)), _rand((L, B, Hkv, d))
    rk, rv, st = _rand((L, B, Hkv, W, d)), _rand((L, B, Hkv, W, d)), _rand((L, B, Hkv, d))
    pos = np.array([3, 40], dtype=np.int32)
    gl, al = RNG.uniform(0.5, 0.99, (L, Hkv)), RNG.uniform(0, 0.5, (L, Hq))
    x = oracle.decode_step(dq, dk, dv, rk, rv, st, pos, gl, al)
    y = oracle.decode_step(dq, dk, dv, rk, rv, np.repeat(st, g, axis=2), pos, np.repeat(gl, g, axis=1),
                           al, s_per_query=True)
    np.testing.assert_array_equal(x[0], y[0])
    np.testing.assert_array_equal(np.repeat(x[3], g, axis=2), y[3])
    assert np.array_equal(x[1], y[1]) and np.array_equal(x[2], y[2])


@pytest.mark.parametrize("n,m,W", [(20, 5, 16), (0, 9, 4), (15, 2, 16), (7, 7, 1)])
def test_per_query_prefill_then_decode_equals_longer_prefill(n, m, W):
    """P7 with γ and S per query head."""
    B, Hq, Hkv, d = 2, 6, 2, 8
    N = n + m
    q, k, v = _rand((B, N, Hq, d)), _rand((B, N, Hkv, d)), _rand((B, N, Hkv, d))
    gamma, alpha = RNG.uniform(0.3, 0.99, Hq), RNG.uniform(0, 0.5, Hq)
    full, frk, frv, fst = oracle.prefill(q, k, v, gamma, alpha, W, s_per_query=True)
    if n > 0:
        _, rk, rv, st = oracle.prefill(q[:, :n], k[:, :n], v[:, :n], gamma, alpha, W, s_per_query=True)
    else:
        rk, rv, st = np.zeros((B, Hkv, W, d)), np.zeros((B, Hkv, W, d)), np.zeros((B, Hq, d))
    for i in range(m):
        t = n + i
        o, rk, rv, st = oracle.decode_step(q[None, :, t], k[None, :, t], v[None, :, t],
                                           rk[None], rv[None], st[None],
                                           np.full(B, t, dtype=np.int32), gamma[None],
                                           alpha[None], s_per_query=True)
        rk, rv, st = rk[0], rv[0], st[0]
        np.testing.assert_allclose(o[0], full[:, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st, fst, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("n1,n2,W", [(20, 13, 16), (40, 3, 4)])
def test_per_query_continuation_equals_single_prefill(n1, n2, W):
    B, Hq, Hkv, d = 2, 4, 2, 8
    N = n1 + n2
    q, k, v = _rand((B, N, Hq, d)), _rand((B, N, Hkv, d)), _rand((B, N, Hkv, d))
    gamma, alpha = RNG.uniform(0.3, 0.99, Hq), RNG.uniform(0, 0.5, Hq)
    full, frk, frv, fst = oracle.prefill(q, k, v, gamma, alpha, W, s_per_query=True)
    o1, rk, rv, st = oracle.prefill(q[:, :n1], k[:, :n1], v[:, :n1], gamma, alpha, W, s_per_query=True)
    o2, rk, rv, st = oracle.prefill(q[:, n1:], k[:, n1:], v[:, n1:], gamma, alpha, W,
                                    ring_k=rk, ring_v=rv, state=st,
                                    pos0=np.full(B, n1, dtype=np.int32), s_per_query=True)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), full, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st, fst, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# P13: the other reading of "mean(K_hist)" ([P1] §2.1 far-field equation): the
# EWMA input at position t >= W is the mean of every key that has left the
# window, positions 0..t-W, not only the key leaving at t
# --------------------------------------------------------------------------
def _running_mean_closed_form(k, gamma, W):
    """S_t = (1-γ) Σ_{s=W}^{t} γ^{t-s} M_s with M_s = mean(k_0 .. k_{s-W}),
    each mean taken directly (np.mean), each S as an explicit power sum.
    Returns (S [n,d], M [n,d]); both 0 before t = W."""
    n, d = k.shape
    K = k.astype(np.float64)
    M = np.zeros((n, d))
    for s in range(W, n):
        M[s] = K[: s - W + 1].mean(axis=0)
    S = np.zeros((n, d))
    for t in range(W, n):
        s = np.arange(W, t + 1)
        S[t] = ((1.0 - gamma) * gamma ** (t - s)) @ M[W: t + 1]
    return S, M


def _brute_force_running_mean(q, k, v, gamma, alpha, W, scale):
    B, n, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    out = np.zeros((B, n, Hq, d))
    state = np.zeros((B, Hkv, 2, d))
    for b in range(B):
        for G in range(Hkv):
            K = k[b, :, G].astype(np.float64)
            V = v[b, :, G].astype(np.float64)
            S, M = _running_mean_closed_form(K, gamma[G], W)
            state[b, G, 0], state[b, G, 1] = S[n - 1], M[n - 1]
            for h in range(G * g, (G + 1) * g):
                s = scale * (q[b, :, h].astype(np.float64) @ K.T)
                s = np.where(_band(n, W), s, -np.inf)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                out[b, :, h] = p @ V + alpha[h] * S
    return out, state


@pytest.mark.parametrize("case", range(8))
def test_running_mean_brute_force_tiny(case):
    r = np.random.default_rng(300 + case)
    W = int(r.integers(1, 17))
    n = int(r.integers(1, 41))
    d = int(r.integers(1, 9))
    Hkv = int(r.integers(1, 3))
    Hq = Hkv * int(r.integers(1, 4))
    B = int(r.integers(1, 3))
    q = r.standard_normal((B, n, Hq, d)).astype(np.float32)
    k = r.standard_normal((B, n, Hkv, d)).astype(np.float32)
    v = r.standard_normal((B, n, Hkv, d)).astype(np.float32)
    gamma = r.uniform(0.0, 0.99, Hkv)
    alpha = r.uniform(-0.5, 0.5, Hq)
    scale = float(r.uniform(0.1, 1.0))
    out, _, _, st = oracle.prefill(q, k, v, gamma, alpha, W, scale, running_mean=True)
    ref, ref_st = _brute_force_running_mean(q, k, v, gamma, alpha, W, scale)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(st, ref_st, rtol=1e-11, atol=1e-12)


def test_running_mean_gamma_zero_is_the_mean_of_the_left_keys():
    """γ = 0: S_t is exactly the running mean of keys 0..t-W (a textbook mean)."""
    B, n, H, d, W = 1, 50, 1, 5, 7
    q, k, v = _rand((B, n, H, d)), _rand((B, n, H, d)), _rand((B, n, H, d))
    o1, *_ = oracle.prefill(q, k, v, 0.0, 1.0, W, running_mean=True)
    o0, *_ = oracle.prefill(q, k, v, 0.0, 0.0, W, running_mean=True)
    S = (o1 - o0)[0, :, 0]
    for t in range(n):
        ref = k[0, : t - W + 1, 0].astype(np.float64).mean(axis=0) if t >= W else np.zeros(d)
        np.testing.assert_allclose(S[t], ref, rtol=1e-12, atol=1e-13)


def test_running_mean_constant_keys():
    """Constant keys c: every mean is c, so S_t = (1 - γ^{t-W+1}) c."""
    B, n, H, d, W, gamma = 1, 60, 1, 3, 16, 0.9
    c = np.array([0.5, -2.0, 3.0], dtype=np.float32)
    k = np.broadcast_to(c, (B, n, H, d)).copy()
    q, v = _rand((B, n, H, d)), _rand((B, n, H, d))
    o1, *_ = oracle.prefill(q, k, v, gamma, 1.0, W, running_mean=True)
    o0, *_ = oracle.prefill(q, k, v, gamma, 0.0, W, running_mean=True)
    for t in range(n):
        ref = (1.0 - gamma ** (t - W + 1)) * c.astype(np.float64) if t >= W else np.zeros(d)
        np.testing.assert_allclose((o1 - o0)[0, t, 0], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n,m,W", [(20, 5, 16), (0, 9, 4), (15, 3, 16), (7, 7, 1)])
def test_running_mean_prefill_then_decode_equals_longer_prefill(n, m, W):
    """P7 for the running mean: decode steps after a prefill carry (S, M)."""
    B, Hq, Hkv, d = 2, 4, 2, 8
    N = n + m
    q, k, v = _rand((B, N, Hq, d)), _rand((B, N, Hkv, d)), _rand((B, N, Hkv, d))
    gamma, alpha = RNG.uniform(0.3, 0.99, Hkv), RNG.uniform(0, 0.5, Hq)
    full, frk, frv, fst = oracle.prefill(q, k, v, gamma, alpha, W, running_mean=True)
    if n > 0:
        _, rk, rv, st = oracle.prefill(q[:, :n], k[:, :n], v[:, :n], gamma, alpha, W, running_mean=True)
    else:
        rk, rv, st = np.zeros((B, Hkv, W, d)), np.zeros((B, Hkv, W, d)), np.zeros((B, Hkv, 2, d))
    for i in range(m):
        t = n + i
        o, rk, rv, st = oracle.decode_step(q[None, :, t], k[None, :, t], v[None, :, t],
                                           rk[None], rv[None], st[None],
                                           np.full(B, t, dtype=np.int32), gamma[None],
                                           alpha[None], running_mean=True)
        rk, rv, st = rk[0], rv[0], st[0]
        np.testing.assert_allclose(o[0], full[:, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st, fst, rtol=1e-12, atol=1e-13)
    assert np.array_equal(rk, frk) and np.array_equal(rv, frv)


@pytest.mark.parametrize("n1,n2,W", [(20, 13, 16), (40, 3, 4), (5, 30, 16)])
def test_running_mean_continuation_equals_single_prefill(n1, n2, W):
    B, Hq, Hkv, d = 2, 4, 2, 8
    N = n1 + n2
    q, k, v = _rand((B, N, Hq, d)), _rand((B, N, Hkv, d)), _rand((B, N, Hkv, d))
    gamma, alpha = RNG.uniform(0.3, 0.99, Hkv), RNG.uniform(0, 0.5, Hq)
    full, frk, frv, fst = oracle.prefill(q, k, v, gamma, alpha, W, running_mean=True)
    o1, rk, rv, st = oracle.prefill(q[:, :n1], k[:, :n1], v[:, :n1], gamma, alpha, W, running_mean=True)
    o2, rk, rv, st = oracle.prefill(q[:, n1:], k[:, n1:], v[:, n1:], gamma, alpha, W,
                                    ring_k=rk, ring_v=rv, state=st,
                                    pos0=np.full(B, n1, dtype=np.int32), running_mean=True)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), full, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st, fst, rtol=1e-12, atol=1e-13)


def test_decode_negative_position_skips_the_sequence():
    """R21: a negative pos entry leaves that sequence's ring and S untouched and
    its outputs unwritten; the other sequences are unaffected."""
    L, B, Hq, Hkv, d, W = 2, 3, 4, 2, 8, 16
    dq, dk, dv = _rand((L, B, Hq, d)), _rand((L, B, Hkv, d)), _rand((L, B, Hkv, d))
    rk, rv, st = _rand((L, B, Hkv, W, d)), _rand((L, B, Hkv, W, d)), _rand((L, B, Hkv, d))
    gl, al = RNG.uniform(0.5, 0.99, (L, Hkv)), RNG.uniform(0, 0.5, (L, Hq))
    pos = np.array([20, -1, 5], dtype=np.int32)
    out, rk2, rv2, st2 = oracle.decode_step(dq, dk, dv, rk, rv, st, pos, gl, al)
    assert np.array_equal(rk2[:, 1], rk[:, 1]) and np.array_equal(rv2[:, 1], rv[:, 1])
    assert np.array_equal(st2[:, 1], st[:, 1])
    keep = [0, 2]
    ref = oracle.decode_step(dq[:, keep], dk[:, keep], dv[:, keep], rk[:, keep], rv[:, keep], st[:, keep],
                             pos[keep], gl, al)
    np.testing.assert_array_equal(out[:, keep], ref[0])
    np.testing.assert_array_equal(st2[:, keep], ref[3])


def test_invalid_window_is_rejected_loudly():
    """A window of zero slots is rejected by the wrapper, and the C library
    itself aborts with a message instead of returning an unwritten result."""
    q = _rand((1, 4, 1, 8))
    with pytest.raises(ValueError):
        oracle.prefill(q, q, q, 0.9, 0.1, 0)
    with pytest.raises(ValueError):
        oracle.decode_step(q[None, :, 0], q[None, :, 0], q[None, :, 0], np.zeros((1, 1, 1, 0, 8)),
                           np.zeros((1, 1, 1, 0, 8)), np.zeros((1, 1, 1, 8)), np.zeros(1, np.int32),
                           np.full((1, 1), 0.9), np.full((1, 1), 0.1))
    code = ("import ctypes, numpy as np, oracle; L = oracle._load(); "
            "z = np.zeros(64); "
            "L.oracle_prefill(*[z.ctypes.data_as(ctypes.c_void_p)] * 9, None, "
            "1, 4, 1, 1, 8, 0, 0.0, 0, 0)")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0 and "invalid argument" in r.stderr


@pytest.mark.parametrize("rbf16", [True, False], ids=["bf16-row", "fp32-row"])
def test_decode_step_enhance_equals_prefill_then_stream_enhance(rbf16):
    """A prefill of n tokens followed by m fused decode-and-enhance steps gives,
    token by token, what a prefill of n + m tokens followed by one enhancement
    of the whole token stream gives (ring slot = stream position mod R, the
    layer's α at global layer layer0 + l, both sequences independent)."""
    B, Hq, Hkv, d, W, R, S, n, m = 2, 4, 2, 8, 4, 3, 5, 6, 5
    H, N = Hq * d, n + m
    q, k, v = _rand((B, N, Hq, d)), _rand((B, N, Hkv, d)), _rand((B, N, Hkv, d))
    gamma, alpha = RNG.uniform(0.5, 0.99, Hkv), RNG.uniform(0, 0.5, Hq)
    pool = _rand((S, H))
    pool /= np.linalg.norm(pool, axis=1, keepdims=True)
    kw = dict(alpha_base=0.8, cross_decay=0.9, ema_gamma=0.7, temperature=0.2, clip=0.6)

    def rnd(x):
        x = np.ascontiguousarray(x)
        return torch.from_numpy(x).to(torch.bfloat16).double().numpy() if rbf16 else x.astype(np.float32)

    full, *_ = oracle.prefill(q, k, v, gamma, alpha, W)
    ref = [oracle.enhance(rnd(full[b].reshape(1, N, H)), pool, layer0=2, n_layers=5, ring_size=R,
                          shared_pool=True, **kw)[0][0] for b in range(B)]
    o, rk, rv, st = oracle.prefill(q[:, :n], k[:, :n], v[:, :n], gamma, alpha, W)
    er = np.zeros((1, B, R, H))
    fd = np.zeros((1, B, H))
    for b in range(B):
        _, _, rb, fb = oracle.enhance(rnd(o[b].reshape(1, n, H)), pool, layer0=2, n_layers=5, ring_size=R,
                                      shared_pool=True, **kw)
        er[0, b], fd[0, b] = rb[0], fb[0]
    rk, rv, st = rk[None], rv[None], st[None]
    for i in range(m):
        t = n + i
        out, _, rk, rv, st, er, fd = oracle.decode_step_enhance(
            q[None, :, t], k[None, :, t], v[None, :, t], rk, rv, st, np.full(B, t, dtype=np.int32),
            gamma[None], alpha[None], pool, er, fd, layer0=2, n_layers=5, shared_pool=True,
            round_bf16=rbf16, **kw)
        for b in range(B):
            np.testing.assert_allclose(out[0, b], ref[b][t], rtol=1e-12, atol=1e-12)
