"""Thin Python binding of libsfa.so: torch tensors in, the C ABI underneath.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind include/sfa.h; PyTorch provides device memory and the current
stream.  Names and argument meanings follow the C entry points: prefill
(sfa_prefill, sfa_prefill_part, sfa_prefill_qh, sfa_prefill_rm), prefill_noalloc,
decode_step (sfa_decode_step, _qh, _rm), decode_step_enhance, enhance,
enhance_prepare_pool and enhance_prepared, and the workspace and record sizes.
"""
from __future__ import annotations

import functools

import torch

from . import _lib

_DT = {torch.float32: _lib.SFA_F32, torch.bfloat16: _lib.SFA_BF16}


def _dtype_code(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"{name}: dtype {t.dtype} not supported (float32 or bfloat16)")
    return _DT[t.dtype]


def _dev(t, name, dtype=None, shape=None, device=None):
    """Validate a device tensor and return its pointer (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.data_ptr()


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _on_call_stream(fn):
    """Run an entry point with its stream (`stream=`, else the current one)
    current.  The temporaries it allocates (a default workspace, γ/α converted
    or broadcast to device vectors, default outputs and state) then belong to
    that stream in the caching allocator: freed on return, they are not handed
    to an allocation on another stream before the kernels enqueued on this one
    have run."""
    @functools.wraps(fn)
    def wrapper(x, *args, stream=None, **kw):
        if not isinstance(x, torch.Tensor) or not x.is_cuda:
            raise TypeError(f"{fn.__name__}: the first argument must be a GPU tensor")
        s = torch.cuda.current_stream(x.device) if stream is None else stream
        with torch.cuda.stream(s):
            return fn(x, *args, stream=s, **kw)
    return wrapper


def _vec(x, n, device, name):
    """Per-head parameter as an fp32 device vector of length n (scalars broadcast)."""
    if isinstance(x, torch.Tensor):
        x = x.to(device=device, dtype=torch.float32)
        if x.numel() == 1:
            x = x.reshape(1).expand(n)
        x = x.contiguous()
        if tuple(x.shape) != (n,) and x.numel() == n:
            x = x.reshape(n)
        if x.numel() != n:
            raise ValueError(f"{name} must have {n} elements")
        return x
    return torch.full((n,), float(x), dtype=torch.float32, device=device)


def prefill_workspace_size(B: int, n: int, Hkv: int, d: int) -> int:
    return int(_lib.lib().sfa_prefill_workspace_size(B, n, Hkv, d))


@_on_call_stream
def prefill(q, k, v, gamma, alpha, *, window: int = 16, scale: float = 0.0, out=None,
            out_dtype=None, ring_k=None, ring_v=None, state=None, pos0=None, workspace=None,
            stream=None, parts: int | None = None, gamma_per_query_head: bool = False,
            running_mean: bool = False):
    """sfa_prefill: q [B,n,Hq,d], k/v [B,n,Hkv,d] (BNHD, bf16 or fp32).

    gamma: [Hkv] (or scalar) decay per KV head; alpha: [Hq] (or scalar).
    Returns (out, ring_k, ring_v, state).  ring_k/ring_v [B,Hkv,W,d] and
    state [B,Hkv,d] fp32 are allocated when not given; pass them (and pos0 [B]
    int32) to continue an existing cache.  `parts` (SFA_PREFILL_SCAN = 1,
    SFA_PREFILL_ATTEND = 2, or SFA_PREFILL_SINGLE_PASS = 4) selects
    sfa_prefill_part; the two parts must share every argument, including the
    workspace.  gamma_per_query_head=True calls
    sfa_prefill_qh: gamma [Hq] and state [B,Hq,d].  running_mean=True calls
    sfa_prefill_rm: state [B,Hkv,2,d] (S, then the mean of the keys that have
    left the window).
    """
    B, n, Hq, d = q.shape
    Hkv = k.shape[2]
    if (gamma_per_query_head or running_mean) and parts is not None:
        raise ValueError("sfa_prefill_qh / sfa_prefill_rm run both parts")
    if gamma_per_query_head and running_mean:
        raise ValueError("gamma_per_query_head and running_mean are separate entry points")
    Hs = Hq if gamma_per_query_head else Hkv
    sshape = (B, Hkv, 2, d) if running_mean else (B, Hs, d)
    dev = q.device
    W = int(window)
    in_code = _dtype_code(q, "q")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, n, Hq, d), dtype=out_dtype, device=dev)
    out_code = _dtype_code(out, "out")
    if ring_k is None and pos0 is None:
        ring_k = torch.zeros((B, Hkv, W, d), dtype=q.dtype, device=dev)
        ring_v = torch.zeros((B, Hkv, W, d), dtype=q.dtype, device=dev)
    if state is None and pos0 is None:
        state = torch.zeros(sshape, dtype=torch.float32, device=dev)
    g = _vec(gamma, Hs, dev, "gamma")
    a = _vec(alpha, Hq, dev, "alpha")
    need = prefill_workspace_size(B, n, 3 * Hkv if running_mean else Hs, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    L = _lib.lib()
    if gamma_per_query_head:
        fn = L.sfa_prefill_qh
    elif running_mean:
        fn = L.sfa_prefill_rm
    else:
        fn = L.sfa_prefill if parts is None else (lambda *a_: L.sfa_prefill_part(int(parts), *a_))
    st = fn(
        _dev(q, "q", q.dtype, (B, n, Hq, d), dev), _dev(k, "k", q.dtype, (B, n, Hkv, d), dev),
        _dev(v, "v", q.dtype, (B, n, Hkv, d), dev), _dev(g, "gamma"), _dev(a, "alpha"),
        _dev(out, "out", None, (B, n, Hq, d), dev),
        _dev(ring_k, "ring_k", q.dtype, (B, Hkv, W, d), dev),
        _dev(ring_v, "ring_v", q.dtype, (B, Hkv, W, d), dev),
        _dev(state, "state", torch.float32, sshape, dev),
        _dev(pos0, "pos0", torch.int32, (B,), dev),
        B, n, Hq, Hkv, d, W, float(scale), in_code, out_code,
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream, dev))
    _lib.check(st, "sfa_prefill_qh" if gamma_per_query_head else "sfa_prefill_rm" if running_mean else
               "sfa_prefill" if parts is None else "sfa_prefill_part")
    return out, ring_k, ring_v, state


@_on_call_stream
def prefill_noalloc(q, k, v, gamma, alpha, *, out, ring_k, ring_v, state, pos0=None, window: int = 16,
                    scale: float = 0.0, stream=None):
    """sfa_prefill_noalloc: sfa_prefill with the library's static scratch as the
    workspace, for callers that cannot allocate.  Nothing is allocated here
    either: every buffer is the caller's (gamma [Hkv] and alpha [Hq] as fp32
    device tensors, out [B,n,Hq,d], ring_k/ring_v [B,Hkv,W,d], state [B,Hkv,d]
    fp32, pos0 [B] int32 or None).  Calls that overlap on one GPU race."""
    B, n, Hq, d = q.shape
    Hkv = k.shape[2]
    dev = q.device
    W = int(window)
    for t, name in ((out, "out"), (ring_k, "ring_k"), (ring_v, "ring_v"), (state, "state")):
        if t is None:
            raise ValueError(f"sfa_prefill_noalloc allocates nothing: pass {name}")
    st = _lib.lib().sfa_prefill_noalloc(
        _dev(q, "q", q.dtype, (B, n, Hq, d), dev), _dev(k, "k", q.dtype, (B, n, Hkv, d), dev),
        _dev(v, "v", q.dtype, (B, n, Hkv, d), dev), _dev(gamma, "gamma", torch.float32, (Hkv,), dev),
        _dev(alpha, "alpha", torch.float32, (Hq,), dev), _dev(out, "out", None, (B, n, Hq, d), dev),
        _dev(ring_k, "ring_k", q.dtype, (B, Hkv, W, d), dev),
        _dev(ring_v, "ring_v", q.dtype, (B, Hkv, W, d), dev),
        _dev(state, "state", torch.float32, (B, Hkv, d), dev),
        _dev(pos0, "pos0", torch.int32, (B,), dev),
        B, n, Hq, Hkv, d, W, float(scale), _dtype_code(q, "q"), _dtype_code(out, "out"),
        _stream(stream, dev))
    _lib.check(st, "sfa_prefill_noalloc")
    return out, ring_k, ring_v, state


@_on_call_stream
def decode_step(q, k_new, v_new, ring_k, ring_v, state, pos, gamma, alpha, *, scale: float = 0.0,
                out=None, out_dtype=None, stream=None, gamma_per_query_head: bool = False,
                running_mean: bool = False):
    """sfa_decode_step over L layers: q [L,B,Hq,d], k_new/v_new [L,B,Hkv,d],
    ring_k/ring_v [L,B,Hkv,W,d] and state [L,B,Hkv,d] fp32 updated in place,
    pos [B] int32, gamma [L,Hkv], alpha [L,Hq].  Returns out [L,B,Hq,d].
    gamma_per_query_head=True calls sfa_decode_step_qh: gamma [L,Hq] and
    state [L,B,Hq,d].  running_mean=True calls sfa_decode_step_rm: state
    [L,B,Hkv,2,d]."""
    L, B, Hq, d = q.shape
    Hkv = k_new.shape[2]
    if gamma_per_query_head and running_mean:
        raise ValueError("gamma_per_query_head and running_mean are separate entry points")
    Hs = Hq if gamma_per_query_head else Hkv
    sshape = (L, B, Hkv, 2, d) if running_mean else (L, B, Hs, d)
    W = ring_k.shape[3]
    dev = q.device
    in_code = _dtype_code(q, "q")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((L, B, Hq, d), dtype=out_dtype, device=dev)
    out_code = _dtype_code(out, "out")
    g = _vec(gamma, L * Hs, dev, "gamma")
    a = _vec(alpha, L * Hq, dev, "alpha")
    name = ("sfa_decode_step_qh" if gamma_per_query_head else "sfa_decode_step_rm" if running_mean
            else "sfa_decode_step")
    fn = getattr(_lib.lib(), name)
    st = fn(
        _dev(q, "q", q.dtype, (L, B, Hq, d), dev), _dev(k_new, "k_new", q.dtype, (L, B, Hkv, d), dev),
        _dev(v_new, "v_new", q.dtype, (L, B, Hkv, d), dev),
        _dev(ring_k, "ring_k", q.dtype, (L, B, Hkv, W, d), dev),
        _dev(ring_v, "ring_v", q.dtype, (L, B, Hkv, W, d), dev),
        _dev(state, "state", torch.float32, sshape, dev),
        _dev(pos, "pos", torch.int32, (B,), dev), _dev(g, "gamma"), _dev(a, "alpha"),
        _dev(out, "out", None, (L, B, Hq, d), dev),
        L, B, Hq, Hkv, d, W, float(scale), in_code, out_code, _stream(stream, dev))
    _lib.check(st, name)
    return out


def enhance_workspace_size(L: int, T: int, H: int) -> int:
    return int(_lib.lib().sfa_enhance_workspace_size(L, T, H))


@_on_call_stream
def enhance(attn, pool, ring, field, *, layer0: int = 0, n_layers: int | None = None, t0: int = 0,
            alpha_base: float = 0.1, cross_decay: float = 0.8, ema_gamma: float = 0.98,
            temperature: float = 0.07, clip: float = 0.5, shared_pool: bool = False, out=None,
            out_dtype=None, enhancement=None, workspace=None, stream=None):
    """sfa_enhance: attn [L,T,H]; pool [L,n_slots,H] fp32 (or [n_slots,H] with
    shared_pool=True); ring [L,R,H] and field [L,H] fp32 updated in place.
    Returns (out, enhancement) -- enhancement is None unless a buffer is given."""
    L, T, H = attn.shape
    R = ring.shape[1]
    dev = attn.device
    in_code = _dtype_code(attn, "attn")
    out_dtype = attn.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((L, T, H), dtype=out_dtype, device=dev)
    out_code = _dtype_code(out, "out")
    if shared_pool:
        n_slots = pool.shape[0]
        stride = 0
        pshape = (n_slots, H)
    else:
        n_slots = pool.shape[1]
        stride = n_slots * H
        pshape = (L, n_slots, H)
    nl = layer0 + L if n_layers is None else n_layers
    need = enhance_workspace_size(L, T, H)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = _lib.lib().sfa_enhance(
        _dev(attn, "attn", None, (L, T, H), dev), _dev(out, "out", None, (L, T, H), dev),
        _dev(ring, "ring", torch.float32, (L, R, H), dev), _dev(field, "field", torch.float32, (L, H), dev),
        _dev(pool, "pool", torch.float32, pshape, dev), stride,
        _dev(enhancement, "enhancement", torch.float32, (L, T, H), dev),
        L, layer0, nl, T, H, t0, float(alpha_base), float(cross_decay), float(ema_gamma),
        float(temperature), float(clip), R, n_slots, in_code, out_code,
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream, dev))
    _lib.check(st, "sfa_enhance")
    return out, enhancement


class PreparedPool:
    """The MFMA-operand form of a read-only semantic pool (sfa_enhance_prepare_pool):
    `buf` is a uint8 device tensor of sfa_enhance_pool_bytes(n_layers, H) bytes."""

    def __init__(self, buf, n_layers: int, n_slots: int, H: int, shared: bool):
        self.buf, self.n_layers, self.n_slots, self.H, self.shared = buf, n_layers, n_slots, H, shared

    def layer_offset(self, layer0: int) -> "PreparedPool":
        """The records from pool layer `layer0` on (a call that starts at that global layer)."""
        if self.shared:
            return self
        rec = int(_lib.lib().sfa_enhance_pool_bytes(1, self.H))
        return PreparedPool(self.buf[layer0 * rec:], self.n_layers - layer0, self.n_slots, self.H, False)


def enhance_pool_bytes(n_pool_layers: int, H: int) -> int:
    return int(_lib.lib().sfa_enhance_pool_bytes(n_pool_layers, H))


@_on_call_stream
def enhance_prepare_pool(pool, *, shared_pool: bool = False, stream=None) -> PreparedPool:
    """sfa_enhance_prepare_pool: pool [L,n_slots,H] fp32 (or [n_slots,H] with
    shared_pool=True) -> its prepared form, kept by the caller for later calls
    of enhance_prepared."""
    dev = pool.device
    if shared_pool:
        n_layers, (n_slots, H) = 1, pool.shape
        stride = 0
    else:
        n_layers, n_slots, H = pool.shape
        stride = n_slots * H
    nbytes = enhance_pool_bytes(n_layers, H)
    buf = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = _lib.lib().sfa_enhance_prepare_pool(
        _dev(pool, "pool", torch.float32, tuple(pool.shape), dev), stride, n_layers, n_slots, H,
        _dev(buf, "prepared"), buf.numel(), _stream(stream, dev))
    _lib.check(st, "sfa_enhance_prepare_pool")
    return PreparedPool(buf, n_layers, n_slots, H, shared_pool)


@_on_call_stream
def enhance_prepared(attn, prepared: PreparedPool, ring, field, *, layer0: int = 0,
                     n_layers: int | None = None, t0: int = 0, alpha_base: float = 0.1,
                     cross_decay: float = 0.8, ema_gamma: float = 0.98, temperature: float = 0.07,
                     clip: float = 0.5, out=None, out_dtype=None, enhancement=None, workspace=None,
                     stream=None):
    """sfa_enhance_prepared: enhance() with the pool in prepared form.  Layer i of
    the call uses record i of `prepared` (record 0 for a shared pool): pass
    prepared.layer_offset(layer0) for a call that starts at global layer layer0."""
    L, T, H = attn.shape
    R = ring.shape[1]
    dev = attn.device
    if prepared.H != H:
        raise ValueError(f"pool prepared for hidden size {prepared.H}, attention has {H}")
    if not prepared.shared and prepared.n_layers < L:
        raise ValueError(f"{prepared.n_layers} prepared pool layers for a call over {L} layers")
    in_code = _dtype_code(attn, "attn")
    out_dtype = attn.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((L, T, H), dtype=out_dtype, device=dev)
    out_code = _dtype_code(out, "out")
    nl = layer0 + L if n_layers is None else n_layers
    if workspace is None:
        workspace = torch.empty(max(enhance_workspace_size(L, T, H), 1), dtype=torch.uint8, device=dev)
    st = _lib.lib().sfa_enhance_prepared(
        _dev(attn, "attn", None, (L, T, H), dev), _dev(out, "out", None, (L, T, H), dev),
        _dev(ring, "ring", torch.float32, (L, R, H), dev), _dev(field, "field", torch.float32, (L, H), dev),
        _dev(prepared.buf, "prepared"), int(prepared.shared),
        _dev(enhancement, "enhancement", torch.float32, (L, T, H), dev),
        L, layer0, nl, T, H, t0, float(alpha_base), float(cross_decay), float(ema_gamma),
        float(temperature), float(clip), R, prepared.n_slots, in_code, out_code,
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream, dev))
    _lib.check(st, "sfa_enhance_prepared")
    return out, enhancement


@_on_call_stream
def decode_step_enhance(q, k_new, v_new, ring_k, ring_v, state, pos, gamma, alpha, e_ring, field,
                        prepared: PreparedPool, *, layer0: int = 0, n_layers: int | None = None,
                        alpha_base: float = 0.1, cross_decay: float = 0.8, ema_gamma: float = 0.98,
                        temperature: float = 0.07, clip: float = 0.5, scale: float = 0.0, out=None,
                        out_dtype=None, enhancement=None, stream=None):
    """sfa_decode_step_enhance: the decode step of decode_step (S per KV head)
    with each (layer, sequence)'s attention row enhanced on chip.  e_ring
    [L,B,R,H] and field [L,B,H] fp32 (the enhancement state of every
    sequence, updated in place), prepared: enhance_prepare_pool of the pool
    (record l for layer l of the call, or a shared one).  Returns out [L,B,H]."""
    L, B, Hq, d = q.shape
    Hkv = k_new.shape[2]
    H = Hq * d
    W = ring_k.shape[3]
    R = e_ring.shape[2]
    dev = q.device
    if prepared.H != H:
        raise ValueError(f"pool prepared for hidden size {prepared.H}, the attention row has {H}")
    if not prepared.shared and prepared.n_layers < L:
        raise ValueError(f"{prepared.n_layers} prepared pool layers for a call over {L} layers")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((L, B, H), dtype=out_dtype, device=dev)
    g = _vec(gamma, L * Hkv, dev, "gamma")
    a = _vec(alpha, L * Hq, dev, "alpha")
    nl = layer0 + L if n_layers is None else n_layers
    st = _lib.lib().sfa_decode_step_enhance(
        _dev(q, "q", q.dtype, (L, B, Hq, d), dev), _dev(k_new, "k_new", q.dtype, (L, B, Hkv, d), dev),
        _dev(v_new, "v_new", q.dtype, (L, B, Hkv, d), dev),
        _dev(ring_k, "ring_k", q.dtype, (L, B, Hkv, W, d), dev),
        _dev(ring_v, "ring_v", q.dtype, (L, B, Hkv, W, d), dev),
        _dev(state, "state", torch.float32, (L, B, Hkv, d), dev),
        _dev(pos, "pos", torch.int32, (B,), dev), _dev(g, "gamma"), _dev(a, "alpha"),
        _dev(out, "out", None, (L, B, H), dev),
        _dev(e_ring, "e_ring", torch.float32, (L, B, R, H), dev), _dev(field, "field", torch.float32, (L, B, H), dev),
        _dev(prepared.buf, "prepared"), int(prepared.shared),
        _dev(enhancement, "enhancement", torch.float32, (L, B, H), dev),
        L, B, Hq, Hkv, d, W, float(scale), layer0, nl, float(alpha_base), float(cross_decay),
        float(ema_gamma), float(temperature), float(clip), R, prepared.n_slots, _dtype_code(q, "q"),
        _dtype_code(out, "out"), _stream(stream, dev))
    _lib.check(st, "sfa_decode_step_enhance")
    return out
