"""GPU parity of sfa_prefill against the CPU fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import windowed_ewma_state_amd as sfa
from windowed_ewma_state_amd import inputs
from tests.parity import check_exact, check_output, check_state, log

pytestmark = pytest.mark.gpu


def _gpu(d, out_dtype, window, **kw):
    cu = lambda x: x.cuda() if isinstance(x, torch.Tensor) else x  # noqa: E731
    out, rk, rv, st = sfa.prefill(cu(d["q"]), cu(d["k"]), cu(d["v"]), cu(d["gamma"]), cu(d["alpha"]),
                                  window=window, out_dtype=out_dtype,
                                  **{k: cu(v) for k, v in kw.items()})
    torch.cuda.synchronize()
    return out, rk, rv, st


def _check_all(d, window, ref, in_bf16, out_dtypes=(torch.float32, torch.bfloat16)):
    n = d["q"].shape[1]
    for od in out_dtypes:
        out, rk, rv, st = _gpu(d, od, window)
        check_output(out, ref[0], in_bf16, f"out[{od}]")
        w = min(n, window)  # slots written by a fresh prompt
        check_exact(rk[:, :, :w], ref[1][:, :, :w], "ring_k")
        check_exact(rv[:, :, :w], ref[2][:, :, :w], "ring_v")
        check_state(st, ref[3])


def test_prefill_tiny_fp32():
    """Tiny fp32 prefill: B 1, one head, d 64, n 256, W 16, γ 0.9, α 0.1."""
    d = inputs.workload(1)
    log("prefill tiny fp32 workload")
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], 16)
    _check_all(d, 16, ref, False, (torch.float32,))


def test_prefill_workload_05b():
    """0.5B-shaped prefill: B 4, n 4096, GQA 14/2, d 64, bf16, per-head γ and α."""
    d = inputs.workload(2)
    log("prefill 0.5B-shaped workload")
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], 16)
    _check_all(d, 16, ref, True)


def test_prefill_workload_7b_64k_one_layer():
    """Long-context 7B-shaped prefill, one full layer: n 65536, GQA 28/4, d 128,
    in the launch configuration the bench times (bf16 in, bf16 out), plus fp32 out."""
    d = inputs.workload(4, device="cuda", layer=0)
    log("prefill 7B-shaped 64K workload (layer 0)")
    cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    ref = oracle.prefill(cpu["q"], cpu["k"], cpu["v"], cpu["gamma"], cpu["alpha"], 16)
    _check_all(d, 16, ref, True)


SMALL = [  # (B, n, Hq, Hkv, hd, W)
    (1, 1, 1, 1, 64, 16), (2, 7, 3, 1, 64, 16), (1, 16, 2, 2, 128, 16), (1, 17, 7, 1, 128, 16),
    (2, 63, 4, 2, 64, 5), (1, 64, 7, 1, 128, 16), (3, 65, 6, 3, 64, 1), (1, 130, 14, 2, 64, 16),
    (2, 300, 8, 2, 128, 3), (1, 1000, 7, 1, 128, 16), (1, 200, 20, 1, 64, 16),
    # more group sizes (3, 2, 8, 5, 1) on grids of a multiple of 8 tiles
    (2, 256, 6, 2, 64, 16), (1, 512, 2, 1, 128, 16), (4, 100, 16, 2, 128, 16), (1, 500, 5, 1, 64, 7),
    (8, 64, 1, 1, 64, 16),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}n{}H{}-{}d{}W{}".format(*c))
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_prefill_small(case, dt):
    B, n, Hq, Hkv, hd, W = case
    log(f"prefill case {case} {dt}")
    d = inputs.prefill_inputs(B, n, Hq, Hkv, hd, seed=n * 31 + Hq + W, dtype=dt)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W)
    _check_all(d, W, ref, dt == torch.bfloat16)


def test_prefill_custom_scale_and_alpha_sign():
    B, n, Hq, Hkv, hd, W = 1, 150, 4, 2, 64, 16
    d = inputs.prefill_inputs(B, n, Hq, Hkv, hd, seed=3, alpha=(-0.5, 0.5))
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W, scale=0.37)
    out, *_ = sfa.prefill(d["q"].cuda(), d["k"].cuda(), d["v"].cuda(), d["gamma"].cuda(),
                          d["alpha"].cuda(), window=W, scale=0.37, out_dtype=torch.float32)
    check_output(out, ref[0], True, "out")


def test_prefill_short_prompt_leaves_other_slots_untouched():
    """n < W: slots >= n keep their previous contents (sentinel), slots < n hold positions."""
    B, n, Hq, Hkv, hd, W = 2, 5, 4, 2, 128, 16
    d = inputs.prefill_inputs(B, n, Hq, Hkv, hd, seed=9)
    rk = torch.full((B, Hkv, W, hd), 7.0, dtype=torch.bfloat16, device="cuda")
    rv = torch.full((B, Hkv, W, hd), -3.0, dtype=torch.bfloat16, device="cuda")
    st = torch.full((B, Hkv, hd), 5.0, dtype=torch.float32, device="cuda")
    sfa.prefill(d["q"].cuda(), d["k"].cuda(), d["v"].cuda(), d["gamma"].cuda(), d["alpha"].cuda(),
                window=W, ring_k=rk, ring_v=rv, state=st)
    torch.cuda.synchronize()
    assert torch.all(rk[:, :, n:] == 7.0) and torch.all(rv[:, :, n:] == -3.0)
    check_exact(rk[:, :, :n], d["k"].permute(0, 2, 1, 3).double().numpy(), "ring_k")
    check_exact(rv[:, :, :n], d["v"].permute(0, 2, 1, 3).double().numpy(), "ring_v")
    assert torch.all(st == 0.0)  # nothing left the window: fresh S is zero


@pytest.mark.parametrize("hd", [64, 128])
def test_prefill_continuation_per_sequence_positions(hd):
    """Chunked prefill: each sequence continues from its own position (0, < W, >= W)."""
    B, Hq, Hkv, W, n2 = 4, 6, 2, 16, 90
    hist = [0, 5, 16, 203]
    d = inputs.prefill_inputs(B, n2, Hq, Hkv, hd, seed=21)
    rk = np.zeros((B, Hkv, W, hd))
    rv = np.zeros((B, Hkv, W, hd))
    st = np.zeros((B, Hkv, hd))
    for b, h in enumerate(hist):
        if h == 0:
            continue
        hb = inputs.prefill_inputs(1, h, Hq, Hkv, hd, seed=100 + b)
        _, rk1, rv1, st1 = oracle.prefill(hb["q"], hb["k"], hb["v"], d["gamma"], d["alpha"], W)
        rk[b], rv[b], st[b] = rk1[0], rv1[0], st1[0]
    pos0 = torch.tensor(hist, dtype=torch.int32)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W, ring_k=rk, ring_v=rv,
                         state=st, pos0=pos0)
    g_rk = torch.from_numpy(rk).to(torch.bfloat16).cuda()
    g_rv = torch.from_numpy(rv).to(torch.bfloat16).cuda()
    g_st = torch.from_numpy(st).float().cuda()
    out, *_ = sfa.prefill(d["q"].cuda(), d["k"].cuda(), d["v"].cuda(), d["gamma"].cuda(),
                          d["alpha"].cuda(), window=W, out_dtype=torch.float32, ring_k=g_rk,
                          ring_v=g_rv, state=g_st, pos0=pos0.cuda())
    torch.cuda.synchronize()
    check_output(out, ref[0], True, "out")
    check_exact(g_rk, ref[1], "ring_k")
    check_exact(g_rv, ref[2], "ring_v")
    check_state(g_st, ref[3])


def test_prefill_two_chunks_equal_one():
    """GPU prefill(n1) then GPU prefill(n2, continued) == oracle prefill(n1 + n2)."""
    B, Hq, Hkv, hd, W, n1, n2 = 2, 7, 1, 128, 16, 100, 77
    d = inputs.prefill_inputs(B, n1 + n2, Hq, Hkv, hd, seed=4)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W)
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    o1, rk, rv, st = sfa.prefill(c["q"][:, :n1].contiguous(), c["k"][:, :n1].contiguous(),
                                 c["v"][:, :n1].contiguous(), c["gamma"], c["alpha"], window=W,
                                 out_dtype=torch.float32)
    o2, rk, rv, st = sfa.prefill(c["q"][:, n1:].contiguous(), c["k"][:, n1:].contiguous(),
                                 c["v"][:, n1:].contiguous(), c["gamma"], c["alpha"], window=W,
                                 out_dtype=torch.float32, ring_k=rk, ring_v=rv, state=st,
                                 pos0=torch.full((B,), n1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    check_output(torch.cat([o1, o2], 1), ref[0], True, "out")
    check_exact(rk, ref[1], "ring_k")
    check_exact(rv, ref[2], "ring_v")
    check_state(st, ref[3])


@pytest.mark.parametrize("n", [1000, 4096, 4096 + 29], ids=["n1000", "n4096", "n4125"])
def test_prefill_parts_in_two_calls_equal_one(n):
    """sfa_prefill_part: SCAN, then ATTEND in a second call on the same
    workspace, equals one SCAN | ATTEND call bit for bit (out, ring, final S),
    fresh and continued (per-sequence positions), on both sides of the 64-chunk
    limit of the folded carries; and against the oracle."""
    B, Hq, Hkv, hd, W = 2, 6, 2, 64, 16
    d = inputs.prefill_inputs(B, n, Hq, Hkv, hd, seed=n + 7)
    hist = [0, 37]
    rk0 = inputs.normal((B, Hkv, W, hd), 901, 1.0, torch.bfloat16)
    rv0 = inputs.normal((B, Hkv, W, hd), 902, 1.0, torch.bfloat16)
    st0 = inputs.normal((B, Hkv, hd), 903, 1.0, torch.float32)
    c = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    ws = torch.empty(sfa.prefill_workspace_size(B, n, Hkv, hd), dtype=torch.uint8, device="cuda")
    for cont in (False, True):
        log(f"prefill parts in two calls, n={n}, continued={cont}")
        res = []
        for split in (False, True):
            kw = dict(window=W, out_dtype=torch.float32, workspace=ws)
            if cont:
                kw.update(ring_k=rk0.cuda(), ring_v=rv0.cuda(), state=st0.cuda(),
                          pos0=torch.tensor(hist, dtype=torch.int32, device="cuda"))
            else:
                kw.update(ring_k=torch.zeros_like(rk0).cuda(), ring_v=torch.zeros_like(rv0).cuda(),
                          state=torch.zeros_like(st0).cuda())
            if split:
                out = torch.empty((B, n, Hq, hd), dtype=torch.float32, device="cuda")
                sfa.prefill(c["q"], c["k"], c["v"], c["gamma"], c["alpha"], out=out, parts=1, **kw)
                r = sfa.prefill(c["q"], c["k"], c["v"], c["gamma"], c["alpha"], out=out, parts=2, **kw)
            else:
                r = sfa.prefill(c["q"], c["k"], c["v"], c["gamma"], c["alpha"], **kw)
            torch.cuda.synchronize()
            res.append([t.clone() for t in r])
        for a_, b_, name in zip(res[0], res[1], ("out", "ring_k", "ring_v", "state")):
            assert torch.equal(a_, b_), name
        if cont:
            ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W, ring_k=rk0.float().numpy(),
                                 ring_v=rv0.float().numpy(), state=st0.double().numpy(),
                                 pos0=torch.tensor(hist, dtype=torch.int32))
        else:
            ref = oracle.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], W)
        check_output(res[0][0], ref[0], True, "out")
        check_exact(res[0][1], ref[1], "ring_k")
        check_exact(res[0][2], ref[2], "ring_v")
        check_state(res[0][3], ref[3])
