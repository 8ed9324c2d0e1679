"""CPU fp64 oracle for Signal Field Attention (SFA) -- test infrastructure.

Only the test suite, the package smoke check and the bench's CPU-baseline leg
import this module.  The GPU product path never imports it and shares no code
with it.  The arithmetic lives in ``sfa_oracle.c`` (plain C, fp64, one token at
a time); this module only marshals numpy/torch-CPU arrays into it.

Pages cited:
  [P1] "Signal Field Attention (SFA)：8KB代码实现4.16倍推理加速与248倍内存压缩",
       section 2.1 (near-field, far-field and fusion equations), section 2.2.
  [P2] "Signal Field Attention (SFA)" project page: SFA_Config defaults,
       cross-layer decay formula, triple-channel diagram.
  [P3] "Dalin Soma SFA基于信号场注意力机制的神经网络推理加速框架", sections
       2.1, 2.2 and 2.4.

Every function here is pinned by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sfa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_sfa.so")
# a test may point the wrapper at another build of the oracle (planted mistakes)
_LIB_OVERRIDE = os.environ.get("SFA_ORACLE_LIB")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        lib.oracle_prefill.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, D, I, I]
        lib.oracle_prefill.restype = None
        lib.oracle_decode_step.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, D, I, I]
        lib.oracle_decode_step.restype = None
        lib.oracle_enhance.argtypes = [P, P, P, P, P, ctypes.c_long, P,
                                       I, I, I, I, I, I, D, D, D, D, D, I, I]
        lib.oracle_enhance.restype = None
        lib.oracle_alpha_layer.argtypes = [D, D, I, I]
        lib.oracle_alpha_layer.restype = D
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = I
        _lib = lib
    return _lib


def _np(x, dtype):
    """Contiguous numpy copy/view of ``x`` (numpy array or torch CPU tensor)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: upcast exactly (bf16/fp32 -> float)
        x = x.detach().cpu()
        x = x.double() if dtype == np.float64 else x.float()
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=dtype))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def alpha_layer(alpha_base: float, cross_decay: float, layer: int, n_layers: int) -> float:
    """Per-layer enhancement factor ([P3] section 2.2, [P2] cross-layer formula)."""
    return float(_load().oracle_alpha_layer(alpha_base, cross_decay, layer, n_layers))


def prefill(q, k, v, gamma, alpha, window: int, scale: float = 0.0,
            ring_k=None, ring_v=None, state=None, pos0=None, s_per_query: bool = False,
            running_mean: bool = False):
    """Windowed softmax attention plus EWMA far field over one prompt ([P1] 2.1).

    q [B,n,Hq,d]; k, v [B,n,Hkv,d]; gamma [Hkv]; alpha [Hq].
    Optional continuation: ring_k/ring_v [B,Hkv,W,d], state [B,Hkv,d] and
    pos0 [B] (positions of the first token); absent means a fresh sequence.
    s_per_query: γ [Hq] and S [B,Hq,d] per query head instead of per KV head.
    running_mean: the EWMA input is the mean of all keys that have left the
    window (the other reading of "mean(K_hist)"); state [B,Hs,2,d] = (S, M).
    Returns (out [B,n,Hq,d], ring_k, ring_v, state), all float64.
    """
    q = _np(q, np.float32)
    k = _np(k, np.float32)
    v = _np(v, np.float32)
    B, n, Hq, d = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, n, Hkv, d) and v.shape == k.shape and Hq % Hkv == 0
    W = int(window)
    if W < 1:
        raise ValueError(f"window must be >= 1, got {W}")
    Hs = Hq if s_per_query else Hkv
    gamma = _np(np.broadcast_to(_np(gamma, np.float64), (Hs,)), np.float64)
    alpha = _np(np.broadcast_to(_np(alpha, np.float64), (Hq,)), np.float64)
    rk = np.zeros((B, Hkv, W, d)) if ring_k is None else _np(ring_k, np.float64).copy()
    rv = np.zeros((B, Hkv, W, d)) if ring_v is None else _np(ring_v, np.float64).copy()
    sshape = (B, Hs, 2, d) if running_mean else (B, Hs, d)
    st = np.zeros(sshape) if state is None else _np(state, np.float64).copy()
    assert st.shape == sshape
    p0 = None if pos0 is None else _np(pos0, np.int32)
    out = np.empty((B, n, Hq, d), dtype=np.float64)
    _load().oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(alpha),
                           _ptr(out), _ptr(rk), _ptr(rv), _ptr(st), _ptr(p0),
                           B, n, Hq, Hkv, d, W, float(scale), int(bool(s_per_query)),
                           int(bool(running_mean)))
    return out, rk, rv, st


def decode_step(q, k_new, v_new, ring_k, ring_v, state, pos, gamma, alpha,
                scale: float = 0.0, s_per_query: bool = False, running_mean: bool = False):
    """One decode step over L layers with the W-slot ring ([P1] 2.1, 2.2).

    q [L,B,Hq,d]; k_new, v_new [L,B,Hkv,d]; ring_k, ring_v [L,B,Hkv,W,d];
    state [L,B,Hkv,d]; pos [B]; gamma [L,Hkv]; alpha [L,Hq].
    s_per_query: γ [L,Hq] and S [L,B,Hq,d] per query head.
    running_mean: state [L,B,Hs,2,d] = (S, M), see prefill.
    A negative pos[b] skips sequence b (nothing of it is written).
    Returns (out [L,B,Hq,d], ring_k, ring_v, state) as new float64 arrays.
    """
    q = _np(q, np.float32)
    kn = _np(k_new, np.float32)
    vn = _np(v_new, np.float32)
    L, B, Hq, d = q.shape
    Hkv = kn.shape[2]
    rk = _np(ring_k, np.float64).copy()
    rv = _np(ring_v, np.float64).copy()
    W = rk.shape[3]
    if W < 1:
        raise ValueError(f"the ring needs at least one slot, got {W}")
    assert rk.shape == (L, B, Hkv, W, d) and rv.shape == rk.shape
    Hs = Hq if s_per_query else Hkv
    st = _np(state, np.float64).copy()
    assert st.shape == ((L, B, Hs, 2, d) if running_mean else (L, B, Hs, d))
    pos = _np(pos, np.int32)
    gamma = _np(np.broadcast_to(_np(gamma, np.float64), (L, Hs)), np.float64)
    alpha = _np(np.broadcast_to(_np(alpha, np.float64), (L, Hq)), np.float64)
    out = np.empty((L, B, Hq, d), dtype=np.float64)
    _load().oracle_decode_step(_ptr(q), _ptr(kn), _ptr(vn), _ptr(rk), _ptr(rv), _ptr(st),
                               _ptr(pos), _ptr(gamma), _ptr(alpha), _ptr(out),
                               L, B, Hq, Hkv, d, W, float(scale), int(bool(s_per_query)),
                               int(bool(running_mean)))
    return out, rk, rv, st


def enhance(attn, pool, ring=None, field=None, *, layer0: int = 0, n_layers: int | None = None,
            t0: int = 0, alpha_base: float = 0.1, cross_decay: float = 0.8,
            ema_gamma: float = 0.98, temperature: float = 0.07, clip: float = 0.5,
            ring_size: int = 16, shared_pool: bool = False):
    """Triple-channel enhancement ([P3] 2.1-2.2; defaults from [P2] SFA_Config).

    attn [L,T,H]; pool [L,n_slots,H] (or [n_slots,H] with shared_pool=True);
    ring [L,ring_size,H] and field [L,H] carried state (zeros when absent).
    Returns (out, enhancement, ring, field), float64.
    """
    a = _np(attn, np.float32)
    L, T, H = a.shape
    p = _np(pool, np.float32)
    if shared_pool:
        n_slots = p.shape[0]
        stride = 0
    else:
        assert p.shape[0] == L
        n_slots = p.shape[1]
        stride = n_slots * H
    assert p.shape[-1] == H
    R = np.zeros((L, ring_size, H)) if ring is None else _np(ring, np.float64).copy()
    F = np.zeros((L, H)) if field is None else _np(field, np.float64).copy()
    out = np.empty((L, T, H))
    enh = np.empty((L, T, H))
    nl = L + layer0 if n_layers is None else n_layers
    _load().oracle_enhance(_ptr(a), _ptr(out), _ptr(R), _ptr(F), _ptr(p), stride, _ptr(enh),
                           L, layer0, nl, T, H, t0, alpha_base, cross_decay, ema_gamma,
                           temperature, clip, ring_size, n_slots)
    return out, enh, R, F


def decode_step_enhance(q, k_new, v_new, ring_k, ring_v, state, pos, gamma, alpha, pool, e_ring, field, *,
                        layer0: int = 0, n_layers: int | None = None, alpha_base: float = 0.1,
                        cross_decay: float = 0.8, ema_gamma: float = 0.98, temperature: float = 0.07,
                        clip: float = 0.5, shared_pool: bool = False, round_bf16: bool = True,
                        scale: float = 0.0):
    """The decode step followed, per sequence, by the triple-channel enhancement
    of its new token ([P1] 2.1-2.2 for the step; [P3] 2.1-2.2, 2.4 for the
    enhancement, applied per layer to each token's attention output as the
    engine of [P2] does).  A composition of decode_step and enhance: no
    arithmetic of its own beyond rounding the attention row to the step's
    output dtype (bf16 with round_bf16, else fp32, as enhance reads it).

    q [L,B,Hq,d] ... as decode_step (S per KV head); pool as enhance;
    e_ring [L,B,R,H], field [L,B,H] each sequence's enhancement state, the new
    token at stream position pos[b] (ring slot pos[b] mod R).  A negative
    pos[b] leaves the sequence untouched.
    Returns (out [L,B,H], enhancement [L,B,H], ring_k, ring_v, state, e_ring,
    field) as float64 arrays.
    """
    o, rk, rv, st = decode_step(q, k_new, v_new, ring_k, ring_v, state, pos, gamma, alpha, scale=scale)
    L, B, Hq, d = o.shape
    H = Hq * d
    a = o.reshape(L, B, H)
    if round_bf16:
        import torch
        a = torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).double().numpy()
    er = _np(e_ring, np.float64).copy()
    fd = _np(field, np.float64).copy()
    out = np.zeros((L, B, H))
    enh = np.zeros((L, B, H))
    p = _np(pos, np.int32)
    nl = layer0 + L if n_layers is None else n_layers
    for b in range(B):
        if p[b] < 0:
            continue
        ob, eb, rb, fb = enhance(a[:, b:b + 1], pool, er[:, b], fd[:, b], layer0=layer0,
                                 n_layers=nl, t0=int(p[b]), alpha_base=alpha_base, cross_decay=cross_decay,
                                 ema_gamma=ema_gamma, temperature=temperature, clip=clip,
                                 ring_size=er.shape[2], shared_pool=shared_pool)
        out[:, b], enh[:, b], er[:, b], fd[:, b] = ob[:, 0], eb[:, 0], rb, fb
    return out, enh, rk, rv, st, er, fd
