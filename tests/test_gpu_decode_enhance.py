"""GPU parity of sfa_decode_step_enhance (the decode step fused with the
triple-channel enhancement) against the oracle's composition of decode_step
and the per-sequence enhancement (oracle.decode_step_enhance).

Bars (tests/parity.py, and the enhancement's own from test_gpu_enhance.py):
  * out: the output-dtype bar (fp32: max-abs 2e-3, rel-L2 1e-3; bf16: one
    bf16 ulp + 2e-5);
  * the enhancement tensor: |enh - ref| <= 2e-4·α_l element-wise;
  * the KV ring: bit-exact; S and the EMA field: rel-L2 <= 1e-5;
  * the enhancement ring: slots other than pos mod R untouched (bit-exact);
    the new slot holds the attention row a as the output dtype stores it.
With bf16 outputs a is itself a bf16 rounding, of the GPU's fp32 row here and
of the oracle's fp64 row there: where the row lies within the fp32 error of a
bf16 tie (~5e-4 of the elements) the two round apart by one ulp of a, which
the smaller enhanced output can exceed.  So the bf16 case is checked in its
two stages: the GPU's a (read back from its ring slot) against the oracle's
attention row with the bf16 output bar, then the enhancement of that same a
against the oracle's enhancement of it.
"""
import numpy as np
import pytest
import torch

import oracle
import windowed_ewma_state_amd as sfa
from windowed_ewma_state_amd import inputs
from tests.parity import check_exact, check_output, check_state, log, rel_l2, to64
from tests.test_gpu_enhance import _check_elementwise

pytestmark = pytest.mark.gpu

KW = dict(alpha_base=0.6, cross_decay=0.9, ema_gamma=0.9, temperature=0.07, clip=0.5)


def _inputs(L, B, Hq, Hkv, hd, W, R, S, seed, shared, pos):
    d = inputs.decode_inputs(L, B, Hq, Hkv, hd, seed=seed, W=W)
    H = Hq * hd
    d["pos"] = torch.tensor(pos, dtype=torch.int32)
    d["e_ring"] = inputs.normal((L, B, R, H), seed * 16 + 12, 0.5, torch.float32)
    d["field"] = inputs.normal((L, B, H), seed * 16 + 13, 0.3, torch.float32)
    pool = inputs.normal((1 if shared else L, S, H), seed * 16 + 14, 1.0, torch.float32)
    pool = pool / pool.norm(dim=-1, keepdim=True)
    d["pool"] = pool[0].contiguous() if shared else pool.contiguous()
    return d


def _run(d, out_dtype, shared, layer0=0, n_layers=None, prep=None):
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    for key in ("ring_k", "ring_v", "state", "e_ring", "field"):
        c[key] = c[key].clone()
    if prep is None:
        prep = sfa.enhance_prepare_pool(c["pool"], shared_pool=shared)
    L, B, Hq, hd = d["q"].shape
    enh = torch.empty((L, B, Hq * hd), device="cuda")
    out = sfa.decode_step_enhance(c["q"], c["k_new"], c["v_new"], c["ring_k"], c["ring_v"], c["state"],
                                  c["pos"], c["gamma"], c["alpha"], c["e_ring"], c["field"], prep,
                                  layer0=layer0, n_layers=n_layers, out_dtype=out_dtype, enhancement=enh,
                                  **KW)
    torch.cuda.synchronize()
    return out, enh, c


def _stage_ref(d, a_rows, shared, layer0, nl):
    """The oracle's enhancement of the given attention rows a [L,B,H] (per
    sequence, at its position): (out, enhancement, e_ring, field)."""
    L, B, H = a_rows.shape
    out, enh = np.zeros((L, B, H)), np.zeros((L, B, H))
    er, fd = to64(d["e_ring"]).copy(), to64(d["field"]).copy()
    for b, p in enumerate(d["pos"].tolist()):
        if p < 0:
            continue
        ob, eb, rb, fb = oracle.enhance(a_rows[:, b:b + 1], d["pool"], er[:, b], fd[:, b], layer0=layer0,
                                        n_layers=nl, t0=p, ring_size=er.shape[2], shared_pool=shared, **KW)
        out[:, b], enh[:, b], er[:, b], fd[:, b] = ob[:, 0], eb[:, 0], rb, fb
    return out, enh, er, fd


def _check(d, out_dtype, shared, layer0=0, n_layers=None):
    out, enh, c = _run(d, out_dtype, shared, layer0, n_layers)
    _check_result(d, out, enh, c, out_dtype, shared, layer0, n_layers)


def _check_result(d, out, enh, c, out_dtype, shared, layer0=0, n_layers=None):
    """The GPU results (out, enhancement, updated state `c`) of inputs `d`
    against the oracle."""
    nl = (layer0 + d["q"].shape[0]) if n_layers is None else n_layers
    ref = oracle.decode_step_enhance(d["q"], d["k_new"], d["v_new"], d["ring_k"], d["ring_v"], d["state"],
                                     d["pos"], d["gamma"], d["alpha"], d["pool"], d["e_ring"], d["field"],
                                     layer0=layer0, n_layers=nl, shared_pool=shared,
                                     round_bf16=out_dtype == torch.bfloat16, **KW)
    live = [b for b, p in enumerate(d["pos"].tolist()) if p >= 0]
    L, B, Hq, hd = d["q"].shape
    R = d["e_ring"].shape[2]
    if out_dtype == torch.bfloat16:
        # stage 1: the attention row the GPU rounded, against the oracle's
        o_ref = oracle.decode_step(d["q"], d["k_new"], d["v_new"], d["ring_k"], d["ring_v"], d["state"],
                                   d["pos"], d["gamma"], d["alpha"])[0].reshape(L, B, Hq * hd)
        a_gpu = torch.stack([c["e_ring"][:, b, p % R] if p >= 0 else torch.zeros_like(c["e_ring"][:, b, 0])
                             for b, p in enumerate(d["pos"].tolist())], 1)
        check_output(a_gpu[:, live].to(torch.bfloat16), o_ref[:, live], True, "attention row a")
        # stage 2: the enhancement of that row
        st2 = _stage_ref(d, a_gpu.cpu().float().numpy(), shared, layer0, nl)
        ref = (st2[0], st2[1]) + ref[2:5] + (st2[2], st2[3])
    check_output(out[:, live], ref[0][:, live], True, f"out[{out_dtype}]")
    _check_elementwise(enh[:, live], ref[1][:, live], dict(layer0=layer0, n_layers=nl, **KW))
    check_exact(c["ring_k"], ref[2], "ring_k")
    check_exact(c["ring_v"], ref[3], "ring_v")
    check_state(c["state"], ref[4])
    er = to64(c["e_ring"])
    for b, p in enumerate(d["pos"].tolist()):
        if p < 0:
            assert np.array_equal(er[:, b], to64(d["e_ring"])[:, b])
            continue
        keep = [j for j in range(R) if j != p % R]
        assert np.array_equal(er[:, b][:, keep], ref[5][:, b][:, keep]), "untouched ring slots"
    r = rel_l2(c["e_ring"], ref[5])
    log(f"  enhancement ring rel-L2 {r:.3e}")
    assert r <= 1e-3
    check_state(c["field"][:, live], ref[6][:, live], "field")


CASES = [  # (L, B, Hq, Hkv, hd, W, R, n_slots, shared)
    (2, 5, 8, 2, 64, 16, 16, 64, False),
    (3, 3, 14, 2, 64, 16, 16, 64, True),     # the 0.5B row (hidden 896)
    (2, 4, 28, 4, 128, 16, 16, 64, False),   # the 7B row (hidden 3584)
    (1, 5, 32, 2, 64, 16, 16, 40, False),    # 16 query heads per KV head
    (2, 3, 4, 4, 128, 4, 5, 7, True),
    (1, 2, 18, 3, 64, 1, 1, 1, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "L{}B{}H{}-{}d{}W{}R{}S{}{}".format(
    *c[:8], "-shared" if c[8] else ""))
def test_decode_step_enhance_small(case):
    L, B, Hq, Hkv, hd, W, R, S, shared = case
    log(f"decode+enhance case {case}")
    pos = [0, 1, W - 1, W, 5000][:B]
    d = _inputs(L, B, Hq, Hkv, hd, W, R, S, seed=L * 7 + Hq + R, shared=shared, pos=pos)
    for od in (torch.float32, torch.bfloat16):
        _check(d, od, shared)


def test_decode_step_enhance_engine_shape_7b():
    """One sequence through all 28 layers of the 7B shape (hidden 3584), per-layer
    pools, the call starting at global layer 0 of 28."""
    log("decode+enhance 7B engine shape, 28 layers x 1 sequence")
    d = _inputs(28, 1, 28, 4, 128, 16, 16, 64, seed=1031, shared=False, pos=[777])
    for od in (torch.bfloat16, torch.float32):
        _check(d, od, False)


def test_decode_step_enhance_layer_offset_and_skip():
    """A call over layers 3..5 of 9 (α of the global layers), a skipped sequence."""
    log("decode+enhance layer offset and skipped sequence")
    L, B, Hq, Hkv, hd = 3, 4, 14, 2, 64
    d = _inputs(L, B, Hq, Hkv, hd, 16, 16, 64, seed=77, shared=False, pos=[40, -3, 16, 2])
    sentinel = torch.full((L, B, Hq * hd), 9.5)
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    out = sentinel.cuda()
    prep = sfa.enhance_prepare_pool(c["pool"])
    sfa.decode_step_enhance(c["q"], c["k_new"], c["v_new"], c["ring_k"], c["ring_v"], c["state"], c["pos"],
                            c["gamma"], c["alpha"], c["e_ring"], c["field"], prep, layer0=3, n_layers=9,
                            out=out, **KW)
    torch.cuda.synchronize()
    assert torch.equal(out[:, 1].cpu(), sentinel[:, 1])
    assert torch.equal(c["e_ring"][:, 1].cpu(), d["e_ring"][:, 1])
    assert torch.equal(c["field"][:, 1].cpu(), d["field"][:, 1])
    assert torch.equal(c["state"][:, 1].cpu(), d["state"][:, 1])
    _check(d, torch.float32, False, layer0=3, n_layers=9)


def test_decode_step_enhance_steps_follow_a_gpu_prefill():
    """GPU prefill of 40 tokens and GPU enhancement of their rows, then 6 fused
    steps, against the oracle in the two stages: every attention row the GPU
    produced (the prompt's bf16 output, each step's row from its ring slot)
    against the oracle's prefill of 46 tokens, then the GPU's 6 enhanced
    outputs against the oracle's enhancement of that whole stream of rows."""
    B, Hq, Hkv, hd, W, n, m, R = 2, 8, 2, 128, 16, 40, 6, 16
    H = Hq * hd
    log("decode+enhance after a GPU prefill")
    d = inputs.prefill_inputs(B, n + m, Hq, Hkv, hd, seed=91)
    pool = inputs.normal((64, H), 92, 1.0, torch.float32)
    pool = (pool / pool.norm(dim=-1, keepdim=True)).contiguous()
    kw = dict(layer0=1, n_layers=4, **KW)
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    o, rk, rv, st = sfa.prefill(c["q"][:, :n].contiguous(), c["k"][:, :n].contiguous(),
                                c["v"][:, :n].contiguous(), c["gamma"], c["alpha"], window=W)
    prep = sfa.enhance_prepare_pool(pool.cuda(), shared_pool=True)
    er = torch.zeros((1, B, R, H), device="cuda")
    fd = torch.zeros((1, B, H), device="cuda")
    for b in range(B):  # the prompt's rows through the stream enhancement
        ring_b, field_b = er[:, b].contiguous(), fd[:, b].contiguous()
        sfa.enhance_prepared(o[b].reshape(1, n, H), prep, ring_b, field_b, **kw)
        er[:, b], fd[:, b] = ring_b, field_b
    rows = [o.reshape(B, n, H).float().cpu()]
    outs = []
    for i in range(m):
        t = n + i
        out = sfa.decode_step_enhance(c["q"][None, :, t].contiguous(), c["k"][None, :, t].contiguous(),
                                      c["v"][None, :, t].contiguous(), rk[None], rv[None], st[None],
                                      torch.full((B,), t, dtype=torch.int32, device="cuda"), c["gamma"][None],
                                      c["alpha"][None], er, fd, prep, out_dtype=torch.bfloat16, **kw)
        torch.cuda.synchronize()
        rows.append(er[0, :, t % R][:, None].cpu())
        outs.append(out[0])
    rows = torch.cat(rows, 1)  # [B, n + m, H], the rows as the GPU holds them
    full, *_ = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W)
    check_output(rows.to(torch.bfloat16), full.reshape(B, n + m, H), True, "attention rows")
    got = torch.stack(outs, 1)  # [B, m, H]
    for b in range(B):
        ref = oracle.enhance(rows[b][None], pool, shared_pool=True, ring_size=R, **kw)[0][0]
        check_output(got[b], ref[n:], True, f"enhanced outputs, sequence {b}")


def test_decode_step_enhance_batch_256_sampled():
    """The bench's 256-sequence fused step (28 layers, 28/4 heads, d 128, hidden
    3,584, a 64-slot pool per layer, bf16 out).  Every (layer, sequence) is
    independent, so the whole batch runs on the GPU and five sampled sequences
    are checked against the oracle on those sequences alone, with the bars of
    _check; every output of the batch must be finite."""
    L, B, Hq, Hkv, hd, W, R, S = 28, 256, 28, 4, 128, 16, 16, 64
    pos = [128 + (b * 997) % 8064 for b in range(B)]
    log("decode + enhance, 256 sequences (sampled check)")
    d = _inputs(L, B, Hq, Hkv, hd, W, R, S, seed=61, shared=False, pos=pos)
    out, enh, c = _run(d, torch.bfloat16, False)
    assert torch.isfinite(out.float()).all() and torch.isfinite(enh).all()
    sb = [0, 1, 77, 200, 255]
    idx = torch.tensor(sb)
    batch_dim = {"q": 1, "k_new": 1, "v_new": 1, "ring_k": 1, "ring_v": 1, "state": 1, "pos": 0, "e_ring": 1,
                 "field": 1}
    sub = {k: (v.index_select(batch_dim[k], idx).contiguous() if k in batch_dim else v) for k, v in d.items()}
    csub = {k: (v.cpu().index_select(batch_dim[k], idx).contiguous() if k in batch_dim else v) for k, v in c.items()}
    csub = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in csub.items()}
    _check_result(sub, out.cpu()[:, idx].contiguous().cuda(), enh.cpu()[:, idx].contiguous().cuda(), csub,
                  torch.bfloat16, False)
