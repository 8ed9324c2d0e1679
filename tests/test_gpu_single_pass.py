"""GPU parity of the single-pass prefill (sfa_prefill_part with
SFA_PREFILL_SINGLE_PASS): the far-field scan folded into the attention kernel,
each 64-token chunk's aggregate published and folded by the chunks after it.

Checked against the oracle with the tolerances of tests/parity.py, for ragged
lengths up to the 64-chunk limit, both head sizes, 8 and fewer sequence-head
chains (the two workgroup orders), continuations from per-sequence positions,
the 0.5B-shaped workload, and bit for bit against a second call (the result
does not depend on the order in which the workgroups publish).
"""
import numpy as np
import pytest
import torch

import oracle
import windowed_ewma_state_amd as sfa
from windowed_ewma_state_amd import _lib, inputs
from tests.parity import check_exact, check_output, check_state, log

pytestmark = pytest.mark.gpu

SP = _lib.SFA_PREFILL_SINGLE_PASS

CASES = [  # (B, n, Hq, Hkv, hd, W)
    (1, 1, 2, 1, 64, 16), (2, 17, 4, 2, 128, 16), (1, 64, 7, 1, 128, 16), (3, 65, 6, 3, 64, 1),
    (2, 300, 8, 2, 128, 3), (1, 1000, 7, 1, 128, 16), (2, 4096, 8, 4, 64, 16), (1, 4033, 28, 4, 128, 16),
    (4, 777, 16, 2, 64, 5),
]


def _gpu(d, out_dtype, W, **kw):
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    out, rk, rv, st = sfa.prefill(c["q"], c["k"], c["v"], c["gamma"], c["alpha"], window=W, out_dtype=out_dtype,
                                  parts=SP, **kw)
    torch.cuda.synchronize()
    return out, rk, rv, st


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}n{}H{}-{}d{}W{}".format(*c))
def test_single_pass_small(case):
    B, n, Hq, Hkv, hd, W = case
    log(f"single pass case {case}")
    d = inputs.prefill_inputs(B, n, Hq, Hkv, hd, seed=n * 3 + Hq + W)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W)
    for od in (torch.float32, torch.bfloat16):
        out, rk, rv, st = _gpu(d, od, W)
        check_output(out, ref[0], True, f"out[{od}]")
        w = min(n, W)
        check_exact(rk[:, :, :w], ref[1][:, :, :w], "ring_k")
        check_exact(rv[:, :, :w], ref[2][:, :, :w], "ring_v")
        check_state(st, ref[3])


def test_single_pass_workload_05b_and_repeatable():
    """0.5B-shaped prefill (B 4, n 4096, 14/2 heads, d 64): 8 chains, 64 chunks
    each, every chunk of the launch resident at once; two calls agree bit for bit."""
    log("single pass 0.5B-shaped workload")
    d = inputs.workload(2)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], 16)
    o1, _, _, s1 = _gpu(d, torch.float32, 16)
    check_output(o1, ref[0], True, "out")
    check_state(s1, ref[3])
    o2, _, _, s2 = _gpu(d, torch.float32, 16)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_single_pass_continuation_per_sequence_positions():
    B, Hq, Hkv, hd, W, n2 = 4, 6, 2, 128, 16, 2500
    hist = [0, 5, 16, 9000]
    log(f"single pass continuation from {hist}")
    d = inputs.prefill_inputs(B, n2, Hq, Hkv, hd, seed=61)
    rk = np.zeros((B, Hkv, W, hd))
    rv = np.zeros((B, Hkv, W, hd))
    st = np.zeros((B, Hkv, hd))
    for b, h in enumerate(hist):
        if h == 0:
            continue
        hb = inputs.prefill_inputs(1, h, Hq, Hkv, hd, seed=300 + b)
        _, rk1, rv1, st1 = oracle.prefill(hb["q"], hb["k"], hb["v"], d["gamma"], d["alpha"], W)
        rk[b], rv[b], st[b] = rk1[0], rv1[0], st1[0]
    rk = torch.from_numpy(rk).to(torch.bfloat16)
    rv = torch.from_numpy(rv).to(torch.bfloat16)
    st = torch.from_numpy(st).float()
    pos0 = torch.tensor(hist, dtype=torch.int32)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W, ring_k=rk, ring_v=rv, state=st,
                         pos0=pos0)
    g_rk, g_rv, g_st = rk.cuda(), rv.cuda(), st.cuda()
    out, *_ = _gpu(d, torch.float32, W, ring_k=g_rk, ring_v=g_rv, state=g_st, pos0=pos0.cuda())
    check_output(out, ref[0], True, "out")
    check_exact(g_rk, ref[1], "ring_k")
    check_exact(g_rv, ref[2], "ring_v")
    check_state(g_st, ref[3])


def test_single_pass_limits_are_reported():
    """Past 64 chunks, fp32 inputs: SFA_ERR_UNSUPPORTED, nothing written."""
    d = inputs.prefill_inputs(1, 64 * 64 + 1, 4, 2, 64, seed=5, device="cuda")
    out = torch.full((1, 64 * 64 + 1, 4, 64), 2.5, device="cuda")
    with pytest.raises(sfa.SFAError, match="UNSUPPORTED"):
        sfa.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], out=out, parts=SP)
    f = inputs.prefill_inputs(1, 100, 4, 2, 64, seed=6, dtype=torch.float32, device="cuda")
    with pytest.raises(sfa.SFAError, match="UNSUPPORTED"):
        sfa.prefill(f["q"], f["k"], f["v"], f["gamma"], f["alpha"], parts=SP)
    torch.cuda.synchronize()
    assert torch.all(out == 2.5)
