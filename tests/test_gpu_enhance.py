"""GPU parity of sfa_enhance against the CPU fp64 oracle (through the C ABI).

Besides `out` (checked with the common tolerances), the fp32 `enhancement`
tensor α_l·clip(e) is checked on its own, element by element and as a whole.

Element-wise bar: |enh - ref| <= 2e-4·α_l in every layer l (α_l > 0).  clip is
1-Lipschitz, so the error is at most α_l·|δe|, e = rm + 0.5·F + 0.5·sem.  The
kernels feed the MFMAs exact bf16 attention values (fp32 inputs: split into
bf16 hi + lo, ~2^-17 relative) and the pool, slot weights and band/field
coefficients as bf16 hi + lo pairs (relative error ~2^-17 = 7.6e-6):
  * rm and F are weighted sums of |a| <= ~6 with weights summing to at most 1
    (rm) and 0.5 (the field term): |δ| <= 6·2^-17·1.5 ~ 7e-5;
  * the cosines c_j move by at most ~2^-17 from the operand split plus the
    fp32 accumulation over H terms (~sqrt(H)·2^-24), ~1e-5, so the logits c/T
    move by ~1.5e-4 at T = 0.07 and Σ|δw_j| <= 2·1.5e-4; with |s_jx| <= ~0.2
    (unit slots) the semantic term 0.5·sem moves by <= ~3e-5, plus 2^-16·0.2
    from the w and s splits;
so |δe| <= ~1e-4, and 2e-4 leaves a factor of two.  Against |enh| <= clip·α_l
this bar rejects any element more than 0.04% of the clip range off.

Single-bf16 semantic operands.  With bf16 inputs, a layer whose
α_l·0.5·(2^-8 + 2^-18)·max|s| is at most 1e-5 takes the pool and the slot
weights as bf16 hi alone (the library's stated rule; max over the layer's
pool entries): each product w_s·s_sx is then off by at most
(2^-8 + 2^-18)·w_s·|s_sx|, the weights sum to one, so 0.5·sem moves by at most
0.5·(2^-8 + 2^-18)·max|s| more.  For such a layer the element-wise bar is
α_l·(2e-4 + 0.5·(2^-8 + 2^-18)·max|s|), i.e. at most 2e-4·α_l + 1e-5: the
outputs' own bars (one bf16 ulp + 2e-5; 2e-3 for fp32 outputs) are unchanged.
Whole-tensor bar: rel-L2 <= 2e-4 (bf16 inputs), 1e-5 (fp32 inputs).
"""
import numpy as np
import pytest
import torch

import oracle
import windowed_ewma_state_amd as sfa
from windowed_ewma_state_amd import inputs
from tests.parity import check_exact, check_output, log, rel_l2, to64

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


SEM_SINGLE_ERR = 0.5 * (2.0 ** -8 + 2.0 ** -18)
SEM_SINGLE_BOUND = 1e-5


def sem_single_extra(pool, kw, L, shared_pool, bf16):
    """Per layer of the call: the extra element-wise allowance / α_l of the
    single-bf16 semantic operands (0 where the layer keeps hi + lo)."""
    extra = np.zeros(L)
    if not bf16:
        return extra
    p = np.abs(np.asarray(pool, dtype=np.float64))
    layer0 = kw.get("layer0", 0)
    n_layers = kw.get("n_layers", layer0 + L)
    for i in range(L):
        m = p.max() if shared_pool else p[i].max()
        al = oracle.alpha_layer(kw.get("alpha_base", 0.1), kw.get("cross_decay", 0.8), layer0 + i, n_layers)
        if abs(al) * SEM_SINGLE_ERR * m <= SEM_SINGLE_BOUND:
            extra[i] = SEM_SINGLE_ERR * m
    return extra


def _check(attn, pool, ref, out_dtypes=(torch.float32, torch.bfloat16), ring=None, field=None,
           shared_pool=False, enh_rel_l2=True, **kw):
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
        assert r <= (2e-4 if bf else 1e-5) or not enh_rel_l2
        _check_elementwise(enh, ref[1], kw, sem_single_extra(pool, kw, L, shared_pool, bf))
        check_exact(g_ring, ref[2], "ring")
        rf = rel_l2(g_field, ref[3])
        log(f"  field rel-L2 {rf:.3e}")
        assert rf <= 1e-5


def _check_elementwise(enh, ref, kw, extra=None):
    """max |enh - ref| <= (2e-4 + extra_l)·α_l per layer (derivation in the
    module docstring); returns the largest |err| / α_l."""
    L = ref.shape[0]
    layer0 = kw.get("layer0", 0)
    n_layers = kw.get("n_layers", layer0 + L)
    extra = np.zeros(L) if extra is None else extra
    err = np.abs(to64(enh) - ref).reshape(L, -1).max(axis=1) if ref.size else np.zeros(L)
    worst = 0.0
    for i in range(L):
        al = oracle.alpha_layer(kw.get("alpha_base", 0.1), kw.get("cross_decay", 0.8), layer0 + i,
                                n_layers)
        if al > 0:
            worst = max(worst, err[i] / al)
            assert err[i] <= (2e-4 + extra[i]) * al, f"layer {i}: enhancement element error {err[i] / al}·α_l"
        else:
            assert err[i] == 0.0
    log(f"  enhancement max |err| / α_l = {worst:.3e} (single-operand layers: {int((extra > 0).sum())} of {L})")
    return worst


def _kw(d):
    return {k: d[k] for k in ("alpha_base", "cross_decay", "ema_gamma", "temperature", "clip",
                              "ring_size", "t0")}


def test_enhance_workload_24_layers():
    """24 layers, hidden 1024, 4096 tokens, 64 slots, SFA_Config defaults;
    and the form bench.py times (sfa_enhance_prepared on the pool prepared
    once, bf16 out) bit for bit equal to sfa_enhance on the same inputs."""
    d = inputs.workload(5)
    log("enhance triple-channel workload")
    ref = oracle.enhance(d["attn"], d["pool"], **_kw(d))
    _check(d["attn"], d["pool"], ref, **_kw(d))
    L, T, H = d["attn"].shape
    attn, pool = d["attn"].cuda(), d["pool"].cuda()
    prep = sfa.enhance_prepare_pool(pool)
    res = []
    for fn in ("per-call", "prepared"):
        ring = torch.zeros((L, 16, H), device="cuda")
        field = torch.zeros((L, H), device="cuda")
        kw = {k: v for k, v in _kw(d).items() if k != "ring_size"}
        if fn == "per-call":
            o, _ = sfa.enhance(attn, pool, ring, field, out_dtype=torch.bfloat16, **kw)
        else:
            o, _ = sfa.enhance_prepared(attn, prep, ring, field, out_dtype=torch.bfloat16, **kw)
        torch.cuda.synchronize()
        res.append((o, ring, field))
    for x, y, name in zip(res[0], res[1], ("out", "ring", "field")):
        assert torch.equal(x, y), name


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


DEGENERATE = [  # (ema_gamma, clip, temperature): the field's decay at both ends; a clip that saturates
    (0.0, 0.5, 0.07), (1.0, 0.5, 0.07), (0.95, 1e-3, 0.07), (0.95, 0.5, 10.0),
]


@pytest.mark.parametrize("eg,clip,temp", DEGENERATE, ids=lambda v: f"{v:g}")
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_enhance_degenerate_parameters(eg, clip, temp, dt):
    """ema_gamma 0 (the field is the current token) and 1 (the field keeps its
    carried value), a clip far below |e| (almost every element at ±clip) and a
    high temperature (near-uniform slot weights), with a carried ring and field
    over several tiles and a ragged tail, against the oracle.

    With the clip at 1e-3 the enhancement's norm shrinks to about α·clip per
    element while the error of an unclipped element is still that of e (an
    absolute quantity), so its rel-L2 bar, derived for |enh| ~ α·|e|, does not
    carry over: there the element-wise bar (absolute, per layer) is the check."""
    L, T, H, S, R = 2, 150, 256, 64, 16
    log(f"enhance degenerate ema_gamma {eg} clip {clip} temperature {temp} {dt}")
    d0 = inputs.enhance_inputs(L, 20, H, seed=41, n_slots=S, dtype=dt)
    d = inputs.enhance_inputs(L, T, H, seed=42, n_slots=S, dtype=dt)
    kw = dict(alpha_base=0.7, cross_decay=0.9, ema_gamma=eg, temperature=temp, clip=clip, ring_size=R)
    _, _, ring, field = oracle.enhance(d0["attn"], d["pool"], **kw)
    ref = oracle.enhance(d["attn"], d["pool"], ring, field, t0=20, **kw)
    _check(d["attn"], d["pool"], ref, ring=ring, field=field, t0=20, enh_rel_l2=clip >= 0.5, **kw)


def test_enhance_alpha_zero_is_identity_on_gpu():
    d = inputs.enhance_inputs(2, 50, 128, seed=3)
    L, T, H = d["attn"].shape
    out, enh, _, _ = _run(d["attn"], d["pool"], np.zeros((L, 16, H)), np.zeros((L, H)),
                          torch.bfloat16, alpha_base=0.0)
    assert torch.equal(out.cpu(), d["attn"])
    assert torch.all(enh == 0)


def test_enhance_semantic_operand_switch():
    """The per-layer choice of single-bf16 or hi + lo semantic operands, on the
    same inputs (shared 64-slot pool, hidden 1024): α_base set so that every
    layer, no layer, or only the first layer is at least 17% inside the
    single-operand bound; each call against the oracle with the bars of the
    module docstring.  The single-operand call must show the larger error
    (the switch engaged)."""
    L, T, H = 4, 200, 1024
    d = inputs.enhance_inputs(L, T, H, seed=404, n_slots=64)
    pool = d["pool"][0].contiguous()
    m = float(np.abs(pool.double().numpy()).max())
    thr = SEM_SINGLE_BOUND / (SEM_SINGLE_ERR * m)  # largest α_l of a single-operand layer
    ratios = [oracle.alpha_layer(1.0, 0.8, l, L) for l in range(L)]  # 0.3 .. 0.512
    worst = {}
    for name, ab, want in (("single", 0.5 * thr / max(ratios), L), ("hi+lo", 2.0 * thr / min(ratios), 0),
                           ("mixed", thr / 0.36, 1)):
        kw = dict(alpha_base=ab, cross_decay=0.8, ema_gamma=0.95, temperature=0.07, clip=0.5,
                  ring_size=16, t0=0)
        extra = sem_single_extra(pool, kw, L, True, True)
        assert int((extra > 0).sum()) == want
        for i, r in enumerate(ratios):  # no layer near the bound
            assert abs(ab * r / thr - 1.0) > 0.15
        log(f"enhance semantic operands: {name}, α_base {ab:.4g}")
        ref = oracle.enhance(d["attn"], pool, shared_pool=True, **kw)
        ring0 = np.zeros((L, 16, H))
        field0 = np.zeros((L, H))
        for od in (torch.float32, torch.bfloat16):
            out, enh, g_ring, g_field = _run(d["attn"], pool, ring0, field0, od, True, **kw)
            check_output(out, ref[0], True, f"out[{od}]")
            assert rel_l2(enh, ref[1]) <= 2e-4
            worst[name] = _check_elementwise(enh, ref[1], kw, extra)
            check_exact(g_ring, ref[2], "ring")
            assert rel_l2(g_field, ref[3]) <= 1e-5
    assert worst["single"] > 3.0 * worst["hi+lo"], worst


@pytest.mark.parametrize("shared", [False, True], ids=["per-layer", "shared"])
def test_enhance_prepared_pool_equals_per_call(shared):
    """sfa_enhance_prepared on a pool prepared once == sfa_enhance (bit for bit),
    two calls in a row continuing the stream, the second starting at global
    layer 2 of 5 (records from layer 2 on); and both against the oracle."""
    L, T, H, S = 3, 150, 256, 64
    log(f"enhance prepared pool, shared={shared}")
    d = inputs.enhance_inputs(5, T, H, seed=88, n_slots=S)
    pool_all = d["pool"][0].contiguous() if shared else d["pool"].contiguous()
    prep = sfa.enhance_prepare_pool(pool_all.cuda(), shared_pool=shared)
    kw = dict(alpha_base=0.5, cross_decay=0.9, ema_gamma=0.95, temperature=0.07, clip=0.5)
    attn = d["attn"][2:2 + L].contiguous()
    pool = pool_all if shared else pool_all[2:2 + L].contiguous()
    ring0 = torch.zeros((L, 16, H), device="cuda")
    field0 = torch.zeros((L, H), device="cuda")
    g1, g2 = (ring0.clone(), field0.clone()), (ring0.clone(), field0.clone())
    outs = []
    for t0, sl in ((0, slice(0, 100)), (100, slice(100, T))):
        a = attn[:, sl].contiguous().cuda()
        e1 = torch.empty(a.shape, device="cuda")
        e2 = torch.empty(a.shape, device="cuda")
        o1, _ = sfa.enhance(a, pool.cuda(), *g1, layer0=2, n_layers=5, t0=t0, shared_pool=shared,
                            out_dtype=torch.float32, enhancement=e1, **kw)
        o2, _ = sfa.enhance_prepared(a, prep.layer_offset(2), *g2, layer0=2, n_layers=5, t0=t0,
                                     out_dtype=torch.float32, enhancement=e2, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(e1, e2)
        assert torch.equal(g1[0], g2[0]) and torch.equal(g1[1], g2[1])
        outs.append((o2, e2))
    ref = oracle.enhance(attn, pool, shared_pool=shared, layer0=2, n_layers=5, ring_size=16, **kw)
    check_output(torch.cat([o for o, _ in outs], 1), ref[0], True, "out")
    _check_elementwise(torch.cat([e for _, e in outs], 1), ref[1], dict(layer0=2, n_layers=5, **kw),
                       sem_single_extra(pool, dict(layer0=2, n_layers=5, **kw), L, shared, True))
    check_exact(g2[0], ref[2], "ring")


# The one-pass form (bf16 inputs, hidden 256, 512, 768 or 1024): one workgroup
# per (layer, 64-token tile) takes the field before its tile from the tiles
# before it, up to 7 aggregates ahead of a published field-after, so these
# cases span 1 .. 16 tiles, ragged tails, ring sizes below and above the tail,
# layer counts that are not a multiple of 8 and both semantic operand forms
# (α_base 0.7 keeps the pairs; 0.004 takes single operands in every layer).
ONE_PASS = [  # (L, T, H, n_slots, R, alpha_base)
    (1, 1, 256, 64, 16, 0.7), (3, 15, 512, 7, 16, 0.7), (9, 130, 256, 33, 4, 0.7),
    (2, 1000, 768, 64, 16, 0.7), (1, 577, 1024, 64, 1, 0.7), (2, 64, 1024, 16, 16, 0.7),
    (5, 520, 512, 64, 16, 0.004), (1, 1030, 256, 64, 13, 0.004),
]


@pytest.mark.parametrize("case", ONE_PASS, ids=lambda c: "L{}T{}H{}S{}R{}a{}".format(*c))
def test_enhance_one_pass(case):
    L, T, H, S, R, ab = case
    log(f"enhance one-pass case {case}")
    d = inputs.enhance_inputs(L, T, H, seed=3 * T + H + S, n_slots=S)
    kw = dict(alpha_base=ab, cross_decay=0.9, ema_gamma=0.95, temperature=0.07, clip=0.5,
              ring_size=R, t0=0)
    ref = oracle.enhance(d["attn"], d["pool"], **kw)
    _check(d["attn"], d["pool"], ref, **kw)


@pytest.mark.parametrize("H", [256, 1024])
def test_enhance_one_pass_continued_and_repeatable(H):
    """A stream in three calls (t0 = 0, 300, 347; the middle call shorter than
    the ring) against the oracle over the whole stream, with a non-zero carried
    ring and field at the start; then the same three calls again, bit for bit."""
    L, S, R = 3, 64, 16
    d = inputs.enhance_inputs(L, 700, H, seed=H + 7, n_slots=S)
    kw = dict(alpha_base=0.7, cross_decay=0.9, ema_gamma=0.97, temperature=0.07, clip=0.5,
              ring_size=R, layer0=1, n_layers=6)
    rng = np.random.default_rng(H)
    # fp32 values, as the library holds them
    ring0 = (rng.standard_normal((L, R, H)) * 0.5).astype(np.float32).astype(np.float64)
    field0 = (rng.standard_normal((L, H)) * 0.5).astype(np.float32).astype(np.float64)
    ref = oracle.enhance(d["attn"], d["pool"], ring0, field0, t0=11, **kw)
    runs = []
    for rep in range(2):
        g_ring = torch.as_tensor(ring0, dtype=torch.float32).cuda().contiguous()
        g_field = torch.as_tensor(field0, dtype=torch.float32).cuda().contiguous()
        pool = d["pool"].cuda()
        outs, enhs = [], []
        for a0, a1 in ((0, 300), (300, 347), (347, 700)):
            a = d["attn"][:, a0:a1].contiguous().cuda()
            e = torch.empty(a.shape, dtype=torch.float32, device="cuda")
            o, _ = sfa.enhance(a, pool, g_ring, g_field, out_dtype=torch.bfloat16, enhancement=e,
                               t0=11 + a0, **{k: v for k, v in kw.items() if k != "ring_size"})
            outs.append(o)
            enhs.append(e)
        torch.cuda.synchronize()
        runs.append((torch.cat(outs, 1), torch.cat(enhs, 1), g_ring, g_field))
    out, enh, g_ring, g_field = runs[0]
    check_output(out, ref[0], True, "out")
    assert rel_l2(enh, ref[1]) <= 2e-4
    _check_elementwise(enh, ref[1], kw)
    check_exact(g_ring, ref[2], "ring")
    assert rel_l2(g_field, ref[3]) <= 1e-5
    for x, y, name in zip(runs[0], runs[1], ("out", "enhancement", "ring", "field")):
        assert torch.equal(x, y), f"repeat differs: {name}"
