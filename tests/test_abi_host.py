"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

The library must load, export every entry point include/sfa.h declares, and
reject bad arguments before it touches any memory or launches anything.
"""
import ctypes
import os
import re

import pytest

from windowed_ewma_state_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sfa.h")

P = 4096  # a fake, 16-byte aligned, non-null "device pointer": never dereferenced here


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sfa_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    names = _declared()
    assert names, "no declarations parsed from include/sfa.h"
    for name in names:
        assert hasattr(lib, name), f"{name} declared in sfa.h but not exported"
    assert set(names) == set(_lib.EXPORTS)


def test_status_strings_and_version():
    lib = _lib.lib()
    assert lib.sfa_abi_version() == 2
    for code in range(5):
        assert lib.sfa_status_string(code).startswith(b"SFA")
    assert b"unknown" in lib.sfa_status_string(99)


def test_workspace_sizes():
    lib = _lib.lib()
    # 6 fp32 arrays of B*Hkv*ceil(n/64)*d (16-token block and 64-token tile aggregates, carries)
    assert lib.sfa_prefill_workspace_size(1, 65536, 4, 128) == 4 * 1024 * 128 * 4 * 6
    assert lib.sfa_prefill_workspace_size(4, 4095, 2, 64) == 4 * 2 * 64 * 64 * 4 * 6
    assert lib.sfa_prefill_workspace_size(0, 10, 1, 64) == 0
    assert lib.sfa_enhance_workspace_size(24, 4096, 1024) > 0
    assert lib.sfa_enhance_workspace_size(1, 0, 1024) == 0
    # tile counts in 64-bit arithmetic up to the largest int
    assert lib.sfa_prefill_workspace_size(1, 2**31 - 1, 1, 64) == 2**25 * 64 * 4 * 6


def _prefill(**kw):
    args = dict(q=P, k=P, v=P, gamma=P, alpha=P, out=P, ring_k=P, ring_v=P, state=P, pos0=None,
                B=1, n=8, Hq=2, Hkv=1, d=64, window=16, scale=0.0, in_dtype=1, out_dtype=0,
                ws=P, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return _lib.lib().sfa_prefill(*args.values())


def _decode(**kw):
    args = dict(q=P, k_new=P, v_new=P, ring_k=P, ring_v=P, state=P, pos=P, gamma=P, alpha=P, out=P,
                L=1, B=1, Hq=2, Hkv=1, d=64, window=16, scale=0.0, in_dtype=1, out_dtype=0,
                stream=None)
    args.update(kw)
    return _lib.lib().sfa_decode_step(*args.values())


def _enhance(**kw):
    args = dict(attn=P, out=P, ring=P, field=P, pool=P, stride=0, enh=None, L=1, layer0=0,
                n_layers=1, T=8, H=64, t0=0, alpha_base=0.1, cross_decay=0.8, ema_gamma=0.98,
                temperature=0.07, clip=0.5, ring_size=16, n_slots=64, in_dtype=1, out_dtype=1,
                ws=P, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return _lib.lib().sfa_enhance(*args.values())


INV, UNS, OK = _lib.SFA_ERR_INVALID_ARG, _lib.SFA_ERR_UNSUPPORTED, _lib.SFA_OK


@pytest.mark.parametrize("kw,want", [
    (dict(window=0), INV), (dict(window=17), INV), (dict(Hq=3, Hkv=2), INV), (dict(Hkv=0), INV),
    (dict(n=-1), INV), (dict(d=96), UNS), (dict(in_dtype=7), UNS), (dict(out_dtype=-1), UNS),
    (dict(q=None), INV), (dict(alpha=None), INV), (dict(ws=None), INV), (dict(ws_bytes=16), INV),
    (dict(q=P + 2), INV), (dict(ring_v=None), INV), (dict(pos0=P, state=None), INV),
    (dict(pos0=P, ring_k=None, ring_v=None), INV),
    (dict(B=0, q=None, k=None, v=None), OK), (dict(n=0, q=None), OK),
    # past the 32-bit tile numbering (with a workspace large enough not to be the reason)
    (dict(n=2**31 - 10, ws_bytes=1 << 62), INV),
    (dict(B=1 << 16, n=1 << 20, ws_bytes=1 << 62), INV),
])
def test_prefill_rejects_before_launch(kw, want):
    assert _prefill(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(parts=3), OK), (dict(parts=0), INV), (dict(parts=5), INV), (dict(parts=8), INV),
    (dict(parts=4, in_dtype=0), UNS), (dict(parts=4, n=64 * 64 + 1), UNS),
    (dict(parts=4, n=64 * 64, q=None), INV), (dict(parts=4, B=0, q=None), OK),
])
def test_prefill_part_modes(kw, want):
    args = dict(parts=3, q=P, k=P, v=P, gamma=P, alpha=P, out=P, ring_k=P, ring_v=P, state=P, pos0=None,
                B=1, n=8, Hq=2, Hkv=1, d=64, window=16, scale=0.0, in_dtype=1, out_dtype=0,
                ws=P, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    if want == OK and args["B"] != 0:
        return  # a valid call would launch: not on the host
    assert _lib.lib().sfa_prefill_part(*args.values()) == want


@pytest.mark.parametrize("kw,want", [
    (dict(window=0), INV), (dict(Hq=5, Hkv=2), INV), (dict(d=32), UNS), (dict(in_dtype=3), UNS),
    (dict(pos=None), INV), (dict(state=None), INV), (dict(ring_k=P + 8), INV),
    (dict(L=0, q=None), OK), (dict(B=0, pos=None), OK),
    (dict(L=1 << 13, B=1 << 12), INV),  # 64·L·B·Hkv reaches 2^31
    (dict(L=1 << 12, B=1 << 11, Hq=2), INV),  # 128·L·B·Hq reaches 2^31 (64·L·B·Hkv is 2^29)
])
def test_decode_rejects_before_launch(kw, want):
    assert _decode(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(ring_size=0), INV), (dict(ring_size=17), INV), (dict(n_slots=65), INV),
    (dict(n_slots=0), INV), (dict(temperature=0.0), INV), (dict(clip=-1.0), INV),
    (dict(H=96), UNS), (dict(n_layers=0), INV), (dict(layer0=1, n_layers=1), INV),
    (dict(stride=8), INV), (dict(pool=None), INV), (dict(ws_bytes=100), INV),
    (dict(T=0, attn=None), OK), (dict(L=0, attn=None), OK),
    (dict(T=2**31 - 10, ws_bytes=1 << 62), INV),
    (dict(L=1 << 13, n_layers=1 << 13, T=1 << 20, H=2048, ws_bytes=1 << 62), INV),
])
def test_enhance_rejects_before_launch(kw, want):
    assert _enhance(**kw) == want


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError, match="no CPU fallback"):
        _lib.lib()


def _prefill_noalloc(**kw):
    args = dict(q=P, k=P, v=P, gamma=P, alpha=P, out=P, ring_k=P, ring_v=P, state=P, pos0=None,
                B=1, n=8, Hq=2, Hkv=1, d=64, window=16, scale=0.0, in_dtype=1, out_dtype=0,
                stream=None)
    args.update(kw)
    return _lib.lib().sfa_prefill_noalloc(*args.values())


@pytest.mark.parametrize("kw,want", [
    (dict(window=0), INV), (dict(Hq=3, Hkv=2), INV), (dict(d=96), UNS), (dict(q=None), INV),
    (dict(q=P + 2), INV), (dict(pos0=P, state=None), INV), (dict(B=0, q=None), OK),
    # one 65,536-token layer with 4 KV heads at d 128 needs 12.6 MB: it fits;
    # 4 of them need 50 MB: past the 16 MiB static scratch
    (dict(B=4, n=65536, Hq=28, Hkv=4, d=128), _lib.SFA_ERR_TOO_LARGE),
    (dict(B=1, n=200000, Hq=28, Hkv=4, d=128), _lib.SFA_ERR_TOO_LARGE),
])
def test_prefill_noalloc_rejects_before_launch(kw, want):
    assert _prefill_noalloc(**kw) == want


def test_prefill_noalloc_scratch_holds_the_64k_layer():
    lib = _lib.lib()
    assert lib.sfa_prefill_workspace_size(1, 65536, 4, 128) <= _lib.SFA_NOALLOC_SCRATCH_BYTES
    assert b"TOO_LARGE" in lib.sfa_status_string(_lib.SFA_ERR_TOO_LARGE)


def _prepare_pool(**kw):
    args = dict(pool=P, stride=0, n_pool_layers=1, n_slots=64, H=64, prepared=P, prepared_bytes=1 << 20,
                stream=None)
    args.update(kw)
    return _lib.lib().sfa_enhance_prepare_pool(*args.values())


def _enhance_prepared(**kw):
    args = dict(attn=P, out=P, ring=P, field=P, prepared=P, shared=1, enh=None, L=1, layer0=0,
                n_layers=1, T=8, H=64, t0=0, alpha_base=0.1, cross_decay=0.8, ema_gamma=0.98,
                temperature=0.07, clip=0.5, ring_size=16, n_slots=64, in_dtype=1, out_dtype=1,
                ws=P, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return _lib.lib().sfa_enhance_prepared(*args.values())


@pytest.mark.parametrize("kw,want", [
    (dict(n_slots=0), INV), (dict(n_slots=65), INV), (dict(H=96), UNS), (dict(pool=None), INV),
    (dict(prepared=None), INV), (dict(prepared=P + 16), INV), (dict(prepared_bytes=100), INV),
    (dict(n_pool_layers=2, stride=64), INV), (dict(stride=-4), INV), (dict(n_pool_layers=0, pool=None), OK),
])
def test_enhance_prepare_pool_rejects_before_launch(kw, want):
    assert _prepare_pool(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(ring_size=0), INV), (dict(n_slots=65), INV), (dict(H=96), UNS), (dict(prepared=None), INV),
    (dict(prepared=P + 16), INV), (dict(ws=None), INV), (dict(ws_bytes=100), INV),
    (dict(layer0=1, n_layers=1), INV), (dict(T=0, attn=None), OK),
])
def test_enhance_prepared_rejects_before_launch(kw, want):
    assert _enhance_prepared(**kw) == want


def test_enhance_pool_bytes():
    lib = _lib.lib()
    rec = lib.sfa_enhance_pool_bytes(1, 1024)
    assert rec % 256 == 0 and rec >= 1024 * 64 * 4 * 2  # both operand orders, bf16 hi + lo
    assert lib.sfa_enhance_pool_bytes(24, 1024) == 24 * rec
    assert lib.sfa_enhance_pool_bytes(0, 1024) == 0


def _decode_enhance(**kw):
    args = dict(q=P, k_new=P, v_new=P, ring_k=P, ring_v=P, state=P, pos=P, gamma=P, alpha=P, out=P,
                e_ring=P, field=P, prepared=P, shared=1, enh=None, L=1, B=1, Hq=2, Hkv=1, d=64, window=16,
                scale=0.0, layer0=0, n_layers=1, alpha_base=0.1, cross_decay=0.8, ema_gamma=0.98,
                temperature=0.07, clip=0.5, ring_size=16, n_slots=64, in_dtype=1, out_dtype=1, stream=None)
    args.update(kw)
    return _lib.lib().sfa_decode_step_enhance(*args.values())


@pytest.mark.parametrize("kw,want", [
    (dict(window=0), INV), (dict(ring_size=17), INV), (dict(n_slots=0), INV), (dict(temperature=0.0), INV),
    (dict(layer0=1), INV), (dict(d=96), UNS), (dict(in_dtype=0), UNS), (dict(Hq=34, Hkv=2), UNS),
    (dict(Hq=33, Hkv=1, d=128), UNS), (dict(prepared=None), INV), (dict(prepared=P + 16), INV),
    (dict(e_ring=None), INV), (dict(field=P + 4), INV), (dict(L=0, q=None), OK), (dict(B=0, pos=None), OK),
])
def test_decode_step_enhance_rejects_before_launch(kw, want):
    assert _decode_enhance(**kw) == want
