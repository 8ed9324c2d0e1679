"""GPU parity at the far field's degenerate parameters, for prefill and decode in
the three far-field modes (S per KV head, γ and S per query head, running mean).

Page "Signal Field Attention (SFA)：8KB代码实现4.16倍推理加速与248倍内存压缩",
section 2.1 (S_t = γ·S_{t-1} + (1-γ)·k_evicted, O = O_near + α·S):
* γ = 0: S is the key that left the window last.  The update is then one
  multiply by 0 and one by 1, so the kernels must return that key exactly
  (its fp32 value), not merely within the tolerance;
* γ = 1: S keeps its value from before the call exactly (0 for a fresh prompt),
  and the output is the near field plus α times that value;
* α = 0: the output is the near-field softmax alone.
Every case is also compared with the oracle at the usual bars.
"""
import pytest
import torch

import oracle
import windowed_ewma_state_amd as sfa
from windowed_ewma_state_amd import inputs
from tests.parity import check_exact, check_output, check_state, log

pytestmark = pytest.mark.gpu

MODES = ["kv", "qh", "rm"]
PREFILL = [  # (B, n, Hq, Hkv, hd, W, dtype): several tiles and a ragged tail
    (2, 300, 4, 2, 128, 16, torch.bfloat16),
    (1, 200, 7, 1, 64, 5, torch.float32),
]
PARAMS = [(0.0, None), (1.0, None), (None, 0.0)]  # (γ, α); None = the generator's values


def _params_id(p):
    g, a = p
    return f"gamma{g:g}" if g is not None else f"alpha{a:g}"


def _flags(mode):
    return dict(gamma_per_query_head=mode == "qh", running_mean=mode == "rm")


def _oracle_flags(mode):
    return dict(s_per_query=mode == "qh", running_mean=mode == "rm")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("params", PARAMS, ids=_params_id)
@pytest.mark.parametrize("case", PREFILL, ids=lambda c: "B{}n{}H{}-{}d{}W{}-{}".format(*c[:6], str(c[6])[6:]))
def test_prefill_degenerate(case, params, mode):
    B, n, Hq, Hkv, hd, W, dt = case
    g, a = params
    log(f"prefill degenerate {case} gamma {g} alpha {a} mode {mode}")
    d = inputs.prefill_inputs(B, n, Hq, Hkv, hd, seed=n + 7 * Hq + W, dtype=dt)
    Hs = Hq if mode == "qh" else Hkv
    if mode == "qh":
        d["gamma"] = inputs.uniform((Hq,), 0.90, 0.99, n + 3)
    if g is not None:
        d["gamma"] = torch.full((Hs,), g, dtype=torch.float32)
    if a is not None:
        d["alpha"] = torch.full_like(d["alpha"], a)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W, **_oracle_flags(mode))
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    out, rk, rv, st = sfa.prefill(c["q"], c["k"], c["v"], c["gamma"], c["alpha"], window=W,
                                  out_dtype=torch.float32, **_flags(mode))
    torch.cuda.synchronize()
    check_output(out, ref[0], dt == torch.bfloat16, "out")
    check_exact(rk[:, :, :W], ref[1][:, :, :W], "ring_k")
    check_state(st, ref[3])
    S = (st[:, :, 0] if mode == "rm" else st).cpu()  # [B, Hs, d]
    if g == 0.0 and mode != "rm":
        # the last key to leave the window: position n-1-W, through its KV head
        kv = torch.arange(Hs) // (Hs // Hkv)
        check_exact(S, d["k"][:, n - 1 - W][:, kv].float(), "S = last evicted key")
    if g == 1.0:
        check_exact(S, torch.zeros_like(S), "S stays 0")


DECODE = [  # (L, B, Hq, Hkv, hd, W, dtype)
    (2, 5, 8, 2, 128, 16, torch.bfloat16),
    (1, 5, 6, 2, 64, 7, torch.float32),
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("params", PARAMS, ids=_params_id)
@pytest.mark.parametrize("case", DECODE, ids=lambda c: "L{}B{}H{}-{}d{}W{}-{}".format(*c[:6], str(c[6])[6:]))
def test_decode_degenerate(case, params, mode):
    L, B, Hq, Hkv, hd, W, dt = case
    g, a = params
    log(f"decode degenerate {case} gamma {g} alpha {a} mode {mode}")
    seed = 31 * L + Hq + W
    d = inputs.decode_inputs(L, B, Hq, Hkv, hd, seed=seed, W=W, dtype=dt)
    Hs = Hq if mode == "qh" else Hkv
    if mode == "qh":
        d["state"] = inputs.normal((L, B, Hq, hd), seed + 1, 1.0, torch.float32)
        d["gamma"] = inputs.uniform((L, Hq), 0.90, 0.99, seed + 2)
    if mode == "rm":
        d["state"] = inputs.normal((L, B, Hkv, 2, hd), seed + 3, 1.0, torch.float32)
    if g is not None:
        d["gamma"] = torch.full((L, Hs), g, dtype=torch.float32)
    if a is not None:
        d["alpha"] = torch.full_like(d["alpha"], a)
    pos = [0, W - 1, W, 3 * W + 2, 1000][:B]
    d["pos"] = torch.tensor(pos, dtype=torch.int32)
    ref = oracle.decode_step(d["q"], d["k_new"], d["v_new"], d["ring_k"], d["ring_v"], d["state"],
                             d["pos"], d["gamma"], d["alpha"], **_oracle_flags(mode))
    rk, rv, st = d["ring_k"].cuda().clone(), d["ring_v"].cuda().clone(), d["state"].cuda().clone()
    out = sfa.decode_step(d["q"].cuda(), d["k_new"].cuda(), d["v_new"].cuda(), rk, rv, st,
                          d["pos"].cuda(), d["gamma"].cuda(), d["alpha"].cuda(), out_dtype=torch.float32,
                          **_flags(mode))
    torch.cuda.synchronize()
    check_output(out, ref[0], dt == torch.bfloat16, "out")
    check_exact(rk, ref[1], "ring_k")
    check_exact(rv, ref[2], "ring_v")
    check_state(st, ref[3])
    S_old = d["state"][:, :, :, 0] if mode == "rm" else d["state"]  # [L, B, Hs, d]
    S_new = (st[:, :, :, 0] if mode == "rm" else st).cpu()
    kv = torch.arange(Hs) // (Hs // Hkv)
    for b, p in enumerate(pos):
        if g == 1.0 or p < W:  # S does not move
            check_exact(S_new[:, b], S_old[:, b], f"S of sequence {b} unchanged")
        elif g == 0.0 and mode != "rm":  # the key in ring slot p mod W leaves the window
            check_exact(S_new[:, b], d["ring_k"][:, b][:, kv, p % W].float(), f"S of sequence {b} = evicted key")
