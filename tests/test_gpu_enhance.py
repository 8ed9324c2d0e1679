"""GPU parity of sfa_enhance against the CPU fp64 oracle (through the C ABI).

Besides `out` (checked with the common tolerances), the fp32 `enhancement`
tensor alpha_l*clip(e) is checked on its own: its rel-L2 error must stay below
2e-4 for bf16 inputs.  Derivation: the cosine scores use the bf16-rounded pool
(relative error 2^-9 per element, ~3e-5 on a cosine of unit vectors in 1024
dimensions), which moves the softmax logits c/T by ~5e-4 and the semantic
vector by ~3e-5 absolute; e then moves by ~1.5e-5 against a typical |e| of
~0.3, i.e. ~5e-5 relative.  fp32 inputs split every operand into bf16 hi+lo,
so their enhancement must meet the fp32 bar of 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
import windowed_ewma_state_amd as sfa
from windowed_ewma_state_amd import inputs
from tests.parity import check_exact, check_output, log, rel_l2

pytestmark = pytest.mark.gpu


def _run(attn, pool, ring, field, out_dtype, shared_pool=False, **kw):
    kw.pop("ring_size", None)  # carried by the ring's shape
    g_ring = torch.as_tensor(ring, dtype=torch.float32).cuda().contiguous()
    g_field = torch.as_tensor(field, dtype=torch.float32).cuda().contiguous()
    L, T, H = attn.shape
    enh = torch.empty((L, T, H), dtype=torch.float32, device="cuda")
    out, _ = sfa.enhance(attn.cuda(), pool.cuda(), g_ring, g_field, out_dtype=out_dtype,
                         enhancement=enh, shared_pool=shared_pool, **kw)
    torch.cuda.synchronize()
    return out, enh, g_ring, g_field


def _check(attn, pool, ref, out_dtypes=(torch.float32, torch.bfloat16), ring=None, field=None,
           shared_pool=False, **kw):
    L, T, H = attn.shape
    R = kw.get("ring_size", 16)
    ring0 = np.zeros((L, R, H)) if ring is None else ring
    field0 = np.zeros((L, H)) if field is None else field
    bf = attn.dtype == torch.bfloat16
    for od in out_dtypes:
        out, enh, g_ring, g_field = _run(attn, pool, ring0, field0, od, shared_pool, **kw)
        check_output(out, ref[0], bf, f"out[{od}]")
        r = rel_l2(enh, ref[1])
        log(f"  enhancement rel-L2 {r:.3e}")
        assert r <= (2e-4 if bf else 1e-5)
        check_exact(g_ring, ref[2], "ring")
        rf = rel_l2(g_field, ref[3])
        log(f"  field rel-L2 {rf:.3e}")
        assert rf <= 1e-5


def _kw(d):
    return {k: d[k] for k in ("alpha_base", "cross_decay", "ema_gamma", "temperature", "clip",
                              "ring_size", "t0")}


def test_enhance_workload_24_layers():
    """24 layers, hidden 1024, 4096 tokens, 64 slots, SFA_Config defaults."""
    d = inputs.workload(5)
    log("enhance triple-channel workload")
    ref = oracle.enhance(d["attn"], d["pool"], **_kw(d))
    _check(d["attn"], d["pool"], ref, **_kw(d))


SMALL = [  # (L, T, H, n_slots, R, dtype)
    (1, 1, 64, 64, 16, torch.bfloat16), (2, 15, 128, 7, 16, torch.bfloat16),
    (2, 64, 64, 64, 1, torch.bfloat16), (3, 100, 128, 1, 4, torch.bfloat16),
    (1, 300, 1024, 64, 16, torch.bfloat16), (2, 257, 896, 33, 16, torch.bfloat16),
    (2, 70, 128, 64, 16, torch.float32), (1, 130, 64, 5, 3, torch.float32),
    # the largest hidden size whose tile aggregates the slot-weight pass forms
    # itself, and one above it (the separate aggregate pass)
    (1, 70, 8192, 64, 16, torch.bfloat16), (1, 33, 8256, 64, 16, torch.bfloat16),
    (1, 20, 8256, 64, 5, torch.float32),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "L{}T{}H{}S{}R{}-{}".format(*c[:5], str(c[5])[6:]))
def test_enhance_small(case):
    L, T, H, S, R, dt = case
    log(f"enhance case {case}")
    d = inputs.enhance_inputs(L, T, H, seed=T + H + S, n_slots=S, dtype=dt)
    kw = dict(alpha_base=0.7, cross_decay=0.9, ema_gamma=0.95, temperature=0.07, clip=0.5,
              ring_size=R, t0=0)
    ref = oracle.enhance(d["attn"], d["pool"], **kw)
    _check(d["attn"], d["pool"], ref, **kw)


def test_enhance_continued_stream_and_layer_offset():
    """Carried ring/field (t0 > 0), global layer index offset, shared pool."""
    L, T, H, S, R = 3, 90, 128, 16, 16
    d0 = inputs.enhance_inputs(L, 37, H, seed=1, n_slots=S)
    d = inputs.enhance_inputs(L, T, H, seed=2, n_slots=S)
    pool = d["pool"][0].contiguous()
    kw = dict(alpha_base=2.0, cross_decay=0.95, ema_gamma=0.9, temperature=0.1, clip=0.5,
              ring_size=R, layer0=5, n_layers=12)
    _, _, ring, field = oracle.enhance(d0["attn"], pool, shared_pool=True, **kw)
    ref = oracle.enhance(d["attn"], pool, ring, field, shared_pool=True, t0=37, **kw)
    _check(d["attn"], pool, ref, ring=ring, field=field, shared_pool=True, t0=37, **kw)


def test_enhance_alpha_zero_is_identity_on_gpu():
    d = inputs.enhance_inputs(2, 50, 128, seed=3)
    L, T, H = d["attn"].shape
    out, enh, _, _ = _run(d["attn"], d["pool"], np.zeros((L, 16, H)), np.zeros((L, H)),
                          torch.bfloat16, alpha_base=0.0)
    assert torch.equal(out.cpu(), d["attn"])
    assert torch.all(enh == 0)
