"""Calls on a stream other than the current one, with temporaries the binding
allocates itself (default workspace, scalar γ/α broadcast to device vectors).

The side stream is held back by a bounded spin kernel, so the SFA kernels run
well after the Python call has returned and freed its temporaries; meanwhile
the current stream allocates blocks of the same sizes and fills them with NaN.
If a temporary were handed to those allocations, the SFA kernels would read
NaN.  The result must equal, bit for bit, the same call made on the current
stream (the kernels are deterministic).
"""
import pytest
import torch

import windowed_ewma_state_amd as sfa
from windowed_ewma_state_amd import inputs
from tests.parity import log

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 20_000_000  # bounded busy-wait on the side stream


def _hold(stream):
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)


def _scribble(sizes):
    """Allocate blocks of these byte sizes on the current stream and fill them with NaN."""
    return [torch.full((max(1, n // 4),), float("nan"), device="cuda") for n in sizes]


@pytest.mark.skipif(not hasattr(torch.cuda, "_sleep"), reason="torch.cuda._sleep not available")
def test_prefill_on_side_stream_with_binding_temporaries():
    B, n, Hq, Hkv, hd = 1, 3000, 8, 2, 128
    log("prefill on a held side stream")
    d = inputs.prefill_inputs(B, n, Hq, Hkv, hd, seed=12, device="cuda")
    ref, *_ = sfa.prefill(d["q"], d["k"], d["v"], 0.95, 0.1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    out = torch.empty_like(ref)
    side.wait_stream(torch.cuda.current_stream())
    _hold(side)
    sfa.prefill(d["q"], d["k"], d["v"], 0.95, 0.1, out=out, stream=side)
    junk = _scribble([sfa.prefill_workspace_size(B, n, Hkv, hd), Hkv * 4, Hq * 4] * 4)
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(out, ref)


@pytest.mark.skipif(not hasattr(torch.cuda, "_sleep"), reason="torch.cuda._sleep not available")
def test_decode_on_side_stream_with_binding_temporaries():
    L, B, Hq, Hkv, hd = 2, 6, 8, 2, 128
    log("decode on a held side stream")
    d = inputs.decode_inputs(L, B, Hq, Hkv, hd, seed=13, device="cuda")
    st = d["state"].clone()
    rk, rv = d["ring_k"].clone(), d["ring_v"].clone()
    ref = sfa.decode_step(d["q"], d["k_new"], d["v_new"], rk, rv, st, d["pos"], 0.93, 0.12,
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    st2 = d["state"].clone()
    rk2, rv2 = d["ring_k"].clone(), d["ring_v"].clone()
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    _hold(side)
    sfa.decode_step(d["q"], d["k_new"], d["v_new"], rk2, rv2, st2, d["pos"], 0.93, 0.12, out=out,
                    stream=side)
    junk = _scribble([L * Hkv * 4, L * Hq * 4] * 4)
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(out, ref) and torch.equal(st2, st) and torch.equal(rk2, rk)


@pytest.mark.skipif(not hasattr(torch.cuda, "_sleep"), reason="torch.cuda._sleep not available")
def test_enhance_on_side_stream_with_binding_temporaries():
    L, T, H = 2, 200, 256
    log("enhance on a held side stream")
    d = inputs.enhance_inputs(L, T, H, seed=14, device="cuda")
    ring, field = torch.zeros((L, 16, H), device="cuda"), torch.zeros((L, H), device="cuda")
    ref, _ = sfa.enhance(d["attn"], d["pool"], ring, field, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ring2, field2 = torch.zeros_like(ring), torch.zeros_like(field)
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    _hold(side)
    sfa.enhance(d["attn"], d["pool"], ring2, field2, out=out, stream=side)
    junk = _scribble([sfa.enhance_workspace_size(L, T, H)] * 4)
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(out, ref) and torch.equal(ring2, ring) and torch.equal(field2, field)
