"""The entry points under HIP graph capture: a captured sequence of calls,
replayed several times with eager work and synchronisation in between, gives
exactly the eager results every time (the kernels are deterministic and record
no memset nodes)."""
import pytest
import torch

import windowed_ewma_state_amd as sfa
from windowed_ewma_state_amd import inputs
from tests.parity import log

pytestmark = pytest.mark.gpu


def _clone(d):
    return {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def _replays_match(run, state, n_replays=3):
    """run(bufs) enqueues the calls on the current stream and returns the output
    tensors; state holds the pristine in/out buffers."""
    eager = _clone(state)
    ref = [t.clone() for t in run(eager)]
    torch.cuda.synchronize()
    work = _clone(state)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(work)  # first calls outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run(work)
    for r in range(n_replays):
        for k, v in state.items():  # eager reset of the in/out buffers between replays
            if isinstance(v, torch.Tensor):
                work[k].copy_(v)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, ref)):
            assert torch.equal(o, e), f"replay {r}: output {i} differs from the eager result"
        torch.cuda.synchronize()


def test_graph_decode_per_layer():
    """Three per-layer decode launches captured in one graph."""
    log("graph: decode L3 B8 per-layer")
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v)
         for k, v in inputs.decode_inputs(3, 8, 14, 2, 128, seed=11).items()}
    d["out"] = torch.empty((3, 8, 14, 128), dtype=torch.bfloat16, device="cuda")

    def run(b):
        for l in range(3):
            sl = slice(l, l + 1)
            sfa.decode_step(b["q"][sl], b["k_new"][sl], b["v_new"][sl], b["ring_k"][sl], b["ring_v"][sl],
                            b["state"][sl], b["pos"], b["gamma"][sl], b["alpha"][sl], out=b["out"][sl])
        return [b["out"], b["ring_k"], b["ring_v"], b["state"]]

    _replays_match(run, d)


def test_graph_prefill():
    """One prefill (scan and attention parts, ring hand-off) captured in a graph."""
    log("graph: prefill B2 n700 14/2 d64")
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v)
         for k, v in inputs.prefill_inputs(2, 700, 14, 2, 64, seed=12).items()}
    d.update(out=torch.empty((2, 700, 14, 64), dtype=torch.float32, device="cuda"),
             ring_k=torch.zeros((2, 2, 16, 64), dtype=torch.bfloat16, device="cuda"),
             ring_v=torch.zeros((2, 2, 16, 64), dtype=torch.bfloat16, device="cuda"),
             state=torch.zeros((2, 2, 64), dtype=torch.float32, device="cuda"),
             ws=torch.empty(sfa.prefill_workspace_size(2, 700, 2, 64), dtype=torch.uint8, device="cuda"))

    def run(b):
        sfa.prefill(b["q"], b["k"], b["v"], b["gamma"], b["alpha"], window=16, out=b["out"],
                    ring_k=b["ring_k"], ring_v=b["ring_v"], state=b["state"], workspace=b["ws"])
        return [b["out"], b["ring_k"], b["ring_v"], b["state"]]

    _replays_match(run, d)


def test_graph_enhance():
    """Two enhancement calls on one stream (the second continues the first's
    ring and field) captured in a graph."""
    log("graph: enhance L2 T200 H256")
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v)
         for k, v in inputs.enhance_inputs(2, 200, 256, seed=13).items()}
    d.update(ring=torch.zeros((2, 16, 256), device="cuda"), field=torch.zeros((2, 256), device="cuda"),
             out=torch.empty((2, 200, 256), dtype=torch.bfloat16, device="cuda"),
             out2=torch.empty((2, 200, 256), dtype=torch.bfloat16, device="cuda"),
             ws=torch.empty(sfa.enhance_workspace_size(2, 200, 256), dtype=torch.uint8, device="cuda"))

    def run(b):
        sfa.enhance(b["attn"], b["pool"], b["ring"], b["field"], out=b["out"], workspace=b["ws"])
        sfa.enhance(b["attn"], b["pool"], b["ring"], b["field"], out=b["out2"], t0=200, workspace=b["ws"])
        return [b["out"], b["out2"], b["ring"], b["field"]]

    _replays_match(run, d)
