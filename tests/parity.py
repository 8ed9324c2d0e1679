"""Comparison helpers for GPU-vs-oracle parity.

Tolerances (stated once, used by every GPU test):
  * bf16 inputs, fp32 outputs: max-abs <= 2e-3 and rel-L2 <= 1e-3;
  * fp32 inputs, fp32 outputs: rel-L2 <= 1e-5;
  * bf16 outputs: every element within one bf16 ulp of the oracle value
    rounded to bf16, plus 2e-5 absolute (rounding the output alone costs up to
    half an ulp, which at |O| in [1, 2) is 3.9e-3, already above the
    fp32-output bar; the absolute term is the fp32 computation's own error
    before rounding, ~1e-6 measured, which exceeds an ulp only for outputs
    within ~1e-3 of zero);
  * ring contents and evicted slots: bit-exact;
  * far-field state S (fp32): rel-L2 <= 1e-5.
"""
import sys

import numpy as np
import torch


BF16_OUT_ABS = 2e-5


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def rel_l2(got, ref):
    got, ref = to64(got), to64(ref)
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((got - ref).ravel()) / (den if den > 0 else 1.0))


def max_abs(got, ref):
    return float(np.max(np.abs(to64(got) - to64(ref)))) if np.size(ref) else 0.0


def bf16_round(ref):
    return torch.from_numpy(np.ascontiguousarray(to64(ref))).to(torch.bfloat16).double().numpy()


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    e = np.floor(np.log2(ax))
    return np.exp2(e - 7)


def check_output(got, ref, in_bf16, name=""):
    """Apply the stated tolerance for this output dtype / input dtype."""
    got64, ref = to64(got), to64(ref)
    assert got64.shape == ref.shape, (got64.shape, ref.shape)
    assert np.all(np.isfinite(got64)), f"{name}: non-finite output"
    if isinstance(got, torch.Tensor) and got.dtype == torch.bfloat16:
        rb = bf16_round(ref)
        err = np.abs(got64 - rb)
        ulp = bf16_ulp(rb)
        excess = float(np.max(err - ulp)) if err.size else 0.0
        worst = float(np.max(err / ulp)) if err.size else 0.0
        log(f"  {name}: bf16 out, worst |got - bf16(ref)| = {worst:.1f} ulp, "
            f"max excess over 1 ulp {max(excess, 0.0):.2e}, rel-L2 vs fp64 {rel_l2(got64, ref):.3e}")
        assert excess <= BF16_OUT_ABS, f"{name}: {excess} beyond one bf16 ulp"
        return
    r, m = rel_l2(got64, ref), max_abs(got64, ref)
    log(f"  {name}: rel-L2 {r:.3e}, max-abs {m:.3e}")
    if in_bf16:
        assert m <= 2e-3 and r <= 1e-3, f"{name}: max-abs {m}, rel-L2 {r}"
    else:
        assert r <= 1e-5, f"{name}: rel-L2 {r}"


def check_state(got, ref, name="state"):
    r = rel_l2(got, ref)
    log(f"  {name}: rel-L2 {r:.3e}")
    assert r <= 1e-5, f"{name}: rel-L2 {r}"


def check_exact(got, ref, name="ring"):
    got64, ref = to64(got), to64(ref)
    bad = int(np.sum(got64 != ref))
    assert bad == 0, f"{name}: {bad} elements differ"
