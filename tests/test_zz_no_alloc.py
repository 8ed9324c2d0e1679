"""sfa_prefill_noalloc (through the C ABI) against sfa_prefill.

The no-allocation entry point runs the same kernels with the library's static
scratch as the workspace, so its results must equal sfa_prefill's bit for bit.
Two calls in a row, the second smaller, then a continued call (the ring
hand-off path); an oversized call is rejected with nothing written; and the
call replays correctly from a HIP graph with eager work between replays.
"""
import pytest
import torch

import oracle
import windowed_ewma_state_amd as sfa
from windowed_ewma_state_amd import _lib, inputs
from tests.parity import check_output, check_state, log

pytestmark = pytest.mark.gpu


def _buffers(d, out_dtype, W=16):
    B, n, Hq, hd = d["q"].shape
    Hkv = d["k"].shape[2]
    return dict(out=torch.empty((B, n, Hq, hd), dtype=out_dtype, device="cuda"),
                ring_k=torch.zeros((B, Hkv, W, hd), dtype=d["q"].dtype, device="cuda"),
                ring_v=torch.zeros((B, Hkv, W, hd), dtype=d["q"].dtype, device="cuda"),
                state=torch.zeros((B, Hkv, hd), dtype=torch.float32, device="cuda"))


def _both(d, out_dtype, **cont):
    """(no-allocation result, sfa_prefill result), each (out, ring_k, ring_v, state)."""
    a = _buffers(d, out_dtype)
    b = _buffers(d, out_dtype)
    if cont:
        for key in ("ring_k", "ring_v", "state"):
            a[key].copy_(cont[key])
            b[key].copy_(cont[key])
    pos0 = cont.get("pos0")
    r1 = sfa.prefill_noalloc(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], pos0=pos0, **a)
    r2 = sfa.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], pos0=pos0, **b)
    torch.cuda.synchronize()
    return r1, r2


def _equal(r1, r2):
    for x, y, name in zip(r1, r2, ("out", "ring_k", "ring_v", "state")):
        assert torch.equal(x, y), f"{name} differs from sfa_prefill"


def test_noalloc_two_calls_then_a_continuation():
    log("noalloc call 1: 7B-shaped 64K layer, bf16 out")
    d1 = inputs.workload(4, device="cuda", layer=3)
    r1, r2 = _both(d1, torch.bfloat16)
    _equal(r1, r2)
    del d1, r1, r2
    torch.cuda.empty_cache()

    log("noalloc call 2: B 2, n 3017, 14/2 heads, d 64, fp32 out")
    d2 = inputs.prefill_inputs(2, 3017, 14, 2, 64, seed=71, device="cuda")
    r1, r2 = _both(d2, torch.float32)
    _equal(r1, r2)
    ref = oracle.prefill(d2["q"].cpu(), d2["k"].cpu(), d2["v"].cpu(), d2["gamma"].cpu(),
                         d2["alpha"].cpu(), 16)
    check_output(r1[0], ref[0], True, "out vs oracle")
    check_state(r1[3], ref[3])

    log("noalloc call 3: continuation of call 2 by 500 tokens")
    d3 = inputs.prefill_inputs(2, 500, 14, 2, 64, seed=72, device="cuda")
    d3["gamma"], d3["alpha"] = d2["gamma"], d2["alpha"]
    pos0 = torch.full((2,), 3017, dtype=torch.int32, device="cuda")
    c1, c2 = _both(d3, torch.float32, ring_k=r1[1], ring_v=r1[2], state=r1[3], pos0=pos0)
    _equal(c1, c2)


def test_noalloc_rejects_an_oversized_call_without_writing():
    log("noalloc oversized call")
    B, n, Hq, Hkv, hd = 4, 65536, 28, 4, 128  # 50 MB of scan scratch > 16 MiB
    assert sfa.prefill_workspace_size(B, n, Hkv, hd) > _lib.SFA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, 64, Hq, hd), dtype=torch.bfloat16, device="cuda")  # never read
    out = torch.full((16,), 3.5, device="cuda")
    st = _lib.lib().sfa_prefill_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), out.data_ptr(),
                                        out.data_ptr(), out.data_ptr(), q.data_ptr(), q.data_ptr(),
                                        out.data_ptr(), None, B, n, Hq, Hkv, hd, 16, 0.0,
                                        _lib.SFA_BF16, _lib.SFA_F32, None)
    torch.cuda.synchronize()
    assert st == _lib.SFA_ERR_TOO_LARGE
    assert torch.all(out == 3.5)


def test_noalloc_replays_from_a_graph():
    log("noalloc in a HIP graph")
    d = inputs.prefill_inputs(1, 2000, 8, 2, 128, seed=73, device="cuda")
    buf = _buffers(d, torch.float32)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sfa.prefill_noalloc(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], **buf)
    torch.cuda.current_stream().wait_stream(side)
    eager = [t.clone() for t in (buf["out"], buf["ring_k"], buf["ring_v"], buf["state"])]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sfa.prefill_noalloc(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], **buf)
    other = inputs.prefill_inputs(1, 700, 8, 2, 128, seed=74, device="cuda")
    for rep in range(3):
        buf["out"].fill_(float("nan"))
        buf["state"].fill_(float("nan"))
        g.replay()
        # eager work between replays, itself using the same scratch
        o2 = _buffers(other, torch.float32)
        sfa.prefill_noalloc(other["q"], other["k"], other["v"], other["gamma"], other["alpha"], **o2)
        torch.cuda.synchronize()
        for x, y, name in zip((buf["out"], buf["ring_k"], buf["ring_v"], buf["state"]), eager,
                              ("out", "ring_k", "ring_v", "state")):
            assert torch.equal(x, y), f"replay {rep}: {name} differs from the eager call"
