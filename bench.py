#!/usr/bin/env python3
"""SFA benchmark on one MI355X.

Headline step: the long-context 7B-shaped prefill -- batch 1, 65,536 tokens,
28 query / 4 KV heads, head_dim 128, bf16 in and out, window 16, γ 0.98,
α 0.1 -- over 28 stacked layers, each layer with its own seeded inputs (one
call of sfa_prefill per layer, run back to back; the inputs are resident in HBM
before timing starts).  A step is the 28 calls; value = tokens·heads/s =
65,536 · 28 heads · 28 layers / step time.

The roofline object covers the dominant kernel, the windowed-attention pass
(SFA_PREFILL_ATTEND): its average duration comes from HIP events recorded on
the launch stream around that part of every seventh layer's call in the timed
region (4 of the 28 per step; a timing event idles the GPU for a few
microseconds, so it is not put around every call), and its
algorithmic bytes are one read of Q, K, V, one write of O and the ring
hand-off.  The EWMA scan part (SFA_PREFILL_SCAN) runs just before it in every
call and is part of the step time.

Also reported in the same line: the 0.5B-shaped prefill, the 28-layer batched
decode step (256 sequences), the 24-layer triple-channel enhancement, the decode
step fused with the enhancement and the far-field variants, each with its own
achieved HBM bandwidth, and the CPU fp64 oracle timed on this host.  The
shorter calls (the 0.5B-shaped prefill, the decode steps, the enhancement) are
timed as HIP-graph replays of back-to-back calls over rotating input sets, with
events only around the whole replay; the decode step and the enhancement also
report the per-call HIP-event figure (`events_us_*`).

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import windowed_ewma_state_amd as sfa  # noqa: E402
from windowed_ewma_state_amd import _lib, inputs  # noqa: E402

PEAK_HBM = 8.0e12  # MI355X HBM3E, bytes/s
METRIC = "SFA tokens·heads/s (prefill, decode) + achieved HBM GB/s vs MI355X peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_window_attn_prefill_7b_64k_traffic.json")
PREFILL_SRC = os.path.join(ROOT, "windowed_ewma_state_amd", "csrc", "prefill.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def src_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


# ----------------------------------------------------------------------------
# prefill, 7B-shaped, 64K tokens, stacked layers
# ----------------------------------------------------------------------------
B, N, HQ, HKV, HD, WIN = 1, 65536, 28, 4, 128, 16
EVENT_STRIDE = 7  # layers per timed attention launch (4 of the 28 layers per step)


def prefill_bytes_per_launch():
    """Algorithmic HBM bytes of one attention pass: Q, K, V read once, O written
    once (bf16), plus the ring hand-off (last W keys/values)."""
    q = B * N * HQ * HD * 2
    kv = 2 * B * N * HKV * HD * 2
    o = B * N * HQ * HD * 2
    ring = 2 * B * HKV * WIN * HD * 2
    return q + kv + o + ring


def run_prefill(args):
    dev = torch.device("cuda:0")
    L = args.layers
    log(f"prefill: generating {L} layers of seeded inputs on the GPU")
    layers = []
    for l in range(L):
        d = inputs.workload(4, device=dev, layer=l)
        layers.append(dict(
            q=d["q"], k=d["k"], v=d["v"], gamma=d["gamma"], alpha=d["alpha"],
            out=torch.empty((B, N, HQ, HD), dtype=torch.bfloat16, device=dev),
            ring_k=torch.zeros((B, HKV, WIN, HD), dtype=torch.bfloat16, device=dev),
            ring_v=torch.zeros((B, HKV, WIN, HD), dtype=torch.bfloat16, device=dev),
            state=torch.zeros((B, HKV, HD), dtype=torch.float32, device=dev)))
    ws = torch.empty(sfa.prefill_workspace_size(B, N, HKV, HD), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    # HIP events bracket the attention part of every EVENT_STRIDE-th layer in
    # the timed steps: each timing event leaves the GPU idle for a few
    # microseconds between kernels, so sampling keeps that cost out of most
    # of the step while still timing the kernel live, on its own stream
    timed = {l: i for i, l in enumerate(l for l in range(L) if l % EVENT_STRIDE == min(EVENT_STRIDE // 2, L - 1))}

    def step(evs=None):
        for l, x in enumerate(layers):
            kw = dict(window=WIN, out=x["out"], ring_k=x["ring_k"], ring_v=x["ring_v"],
                      state=x["state"], workspace=ws, stream=stream)
            sfa.prefill(x["q"], x["k"], x["v"], x["gamma"], x["alpha"], parts=_lib.SFA_PREFILL_SCAN, **kw)
            ev = evs[timed[l]] if evs is not None and l in timed else None
            if ev:
                ev[0].record(stream)
            sfa.prefill(x["q"], x["k"], x["v"], x["gamma"], x["alpha"], parts=_lib.SFA_PREFILL_ATTEND, **kw)
            if ev:
                ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in timed] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_ms = [e[0].elapsed_time(e[1]) for st in evs for e in st]
    return dict(layers=layers, wall=wall, attn_ms=sum(attn_ms) / len(attn_ms))


# ----------------------------------------------------------------------------
# secondary: the Qwen2.5-0.5B-shaped prefill (B 4, n 4096, 14/2 heads, d 64)
# ----------------------------------------------------------------------------
C2 = dict(B=4, N=4096, HQ=14, HKV=2, HD=64)


def c2_bytes():
    """Algorithmic bytes of one 0.5B-shaped call: Q, K, V read once, O written
    once (bf16), the ring hand-off and the final S (fp32)."""
    B_, N_, HQ_, HKV_, HD_ = C2["B"], C2["N"], C2["HQ"], C2["HKV"], C2["HD"]
    return (2 * B_ * N_ * HQ_ * HD_ * 2 + 2 * B_ * N_ * HKV_ * HD_ * 2
            + 2 * B_ * HKV_ * WIN * HD_ * 2 + B_ * HKV_ * HD_ * 4)


def c2_attn_bytes():
    """Algorithmic bytes of the attention launch alone (the final S is written by the scan)."""
    B_, HKV_, HD_ = C2["B"], C2["HKV"], C2["HD"]
    return c2_bytes() - B_ * HKV_ * HD_ * 4


def run_c2(reps=40, sets=6):
    """The 0.5B-shaped prefill call on `sets` rotating input sets of 67 MB
    each, more than the 256 MB MALL holds, so every call streams from HBM.  A
    call's GPU time (~20-30 us) is about what the Python binding takes to issue
    it, so the calls are captured once in HIP graphs and replayed: `sets` whole
    calls per replay (the single pass), the same as separate scan and attention
    parts (the two-pass form), and the attention parts alone.  HIP events on
    the replay stream bracket `reps` back-to-back replays."""
    dev = torch.device("cuda:0")
    B_, N_, HQ_, HKV_, HD_ = C2["B"], C2["N"], C2["HQ"], C2["HKV"], C2["HD"]
    bufs = []
    for i in range(sets):
        d = inputs.workload(2, device=dev) if i == 0 else inputs.prefill_inputs(
            B_, N_, HQ_, HKV_, HD_, seed=5000 + i, device=dev)
        d["out"] = torch.empty((B_, N_, HQ_, HD_), dtype=torch.bfloat16, device=dev)
        d["ring_k"] = torch.zeros((B_, HKV_, WIN, HD_), dtype=torch.bfloat16, device=dev)
        d["ring_v"] = torch.zeros_like(d["ring_k"])
        d["state"] = torch.zeros((B_, HKV_, HD_), dtype=torch.float32, device=dev)
        d["ws"] = torch.empty(sfa.prefill_workspace_size(B_, N_, HKV_, HD_), dtype=torch.uint8, device=dev)
        bufs.append(d)

    def call(d, part):
        sfa.prefill(d["q"], d["k"], d["v"], d["gamma"], d["alpha"], window=WIN, out=d["out"],
                    ring_k=d["ring_k"], ring_v=d["ring_v"], state=d["state"], workspace=d["ws"],
                    parts=part)

    both = _lib.SFA_PREFILL_SCAN | _lib.SFA_PREFILL_ATTEND

    def graph_of(part):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for d in bufs:  # first calls outside the capture
                call(d, both)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for d in bufs:
                for p in (part if isinstance(part, tuple) else (part,)):
                    call(d, p)
        return g

    def per_call_ms(g):
        stream = torch.cuda.current_stream(dev)
        for _ in range(3):
            g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * sets)

    # sfa_prefill (scan launches, then attention), its attention part alone,
    # and the single pass (the scan folded into the attention kernel)
    ms = per_call_ms(graph_of(both))
    ms_attn = per_call_ms(graph_of(_lib.SFA_PREFILL_ATTEND))
    ms_one = per_call_ms(graph_of(_lib.SFA_PREFILL_SINGLE_PASS))
    byts, abyts = c2_bytes(), c2_attn_bytes()
    return {"workload": "Qwen2.5-0.5B-shaped prefill, batch 4 x 4096 tokens, 14/2 heads, d 64, bf16 in/out, "
                        f"{sets} rotating input sets, HIP-graph replays",
            "value": B_ * N_ * HQ_ / (ms * 1e-3), "unit": "tokens·heads/s", "us_per_call": ms * 1e3,
            "roofline": {"bound": "hbm", "achieved": byts / (ms * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9,
                         "unit": "GB/s", "frac": byts / (ms * 1e-3) / PEAK_HBM, "bytes_per_call": byts},
            "attention": {"kernel": "k_window_attn (d 64, carries folded from the tile aggregates)",
                          "avg_launch_us": ms_attn * 1e3,
                          "achieved": abyts / (ms_attn * 1e-3) / 1e9, "frac": abyts / (ms_attn * 1e-3) / PEAK_HBM,
                          "bytes_per_launch": abyts},
            "single_pass": {"us_per_call": ms_one * 1e3, "frac": byts / (ms_one * 1e-3) / PEAK_HBM,
                            "launches": "k_fused_init, k_window_attn with the scan folded in"}}


# ----------------------------------------------------------------------------
# secondary: decode step (28 layers x 256 sequences) and enhancement (24 layers)
# ----------------------------------------------------------------------------
def decode_bytes(L=28, Bd=256, Hq=28, Hkv=4, d=128, W=16):
    """Per step: q, k_new, v_new, 16 ring keys + 15 ring values (the evicted
    value is never read), one ring slot written (K and V), S read and written
    (fp32), O written (bf16), pos."""
    per = (Hq * d * 2 + 2 * Hkv * d * 2 + Hkv * W * d * 2 + Hkv * (W - 1) * d * 2
           + 2 * Hkv * d * 2 + 2 * Hkv * d * 4 + Hq * d * 2)
    return L * Bd * per + Bd * 4


def replay_ms(call, bufs, reps):
    """Per-call time of `call` over the rotating input sets `bufs`: one call per
    set, in order, captured once in a HIP graph; HIP events on the replay stream
    bracket `reps` back-to-back replays, so no timing event sits between two
    calls (each one idles the GPU for a few microseconds)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for d in bufs:  # first calls outside the capture
            call(d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for d in bufs:
            call(d)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        g.replay()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * len(bufs))


def run_decode(steps=40, warmup=5, sets=3):
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    bufs = []
    for i in range(sets):  # rotate input sets so the 256 MB MALL cannot hold them
        d = inputs.workload(3, device=dev) if i == 0 else inputs.decode_inputs(
            28, 256, 28, 4, 128, seed=2000 + i, device=dev)
        d["out"] = torch.empty((28, 256, 28, 128), dtype=torch.bfloat16, device=dev)
        bufs.append(d)

    def call(d):
        sfa.decode_step(d["q"], d["k_new"], d["v_new"], d["ring_k"], d["ring_v"], d["state"], d["pos"],
                        d["gamma"], d["alpha"], out=d["out"], stream=stream)

    for i in range(warmup):
        call(bufs[i % sets])
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        call(bufs[i % sets])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms_ev = sum(a.elapsed_time(b) for a, b in ev) / steps
    ms = replay_ms(lambda d: sfa.decode_step(d["q"], d["k_new"], d["v_new"], d["ring_k"], d["ring_v"], d["state"],
                                             d["pos"], d["gamma"], d["alpha"], out=d["out"]),
                   bufs, steps // sets + 1)
    ms_graph = decode_per_layer_graph(bufs, steps)
    byts = decode_bytes()
    return {"workload": "7B-shaped decode step, 28 layers x 256 sequences, 28/4 heads, d 128, bf16",
            "value": 28 * 256 * 28 / (ms * 1e-3), "unit": "tokens·heads/s (sequence, query head, layer)",
            "us_per_step": ms * 1e3, "timing": f"HIP-graph replays of {sets} rotating input sets",
            "events_us_per_step": ms_ev * 1e3, "kernel": "k_decode_mfma",
            "per_layer_launches_graph_us_per_step": ms_graph * 1e3,
            "roofline": {"bound": "hbm", "achieved": byts / (ms * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9,
                         "unit": "GB/s", "frac": byts / (ms * 1e-3) / PEAK_HBM, "bytes_per_step": byts}}


def decode_per_layer_graph(bufs, steps):
    """The same decode step as 28 launches of one layer each, captured once per
    input set in a HIP graph and replayed (the alternative to one launch that
    covers all layers)."""
    graphs = []
    for d in bufs:
        L = d["q"].shape[0]

        def layers(d=d, L=L):
            for l in range(L):
                sl = slice(l, l + 1)
                sfa.decode_step(d["q"][sl], d["k_new"][sl], d["v_new"][sl], d["ring_k"][sl], d["ring_v"][sl],
                                d["state"][sl], d["pos"], d["gamma"][sl], d["alpha"][sl], out=d["out"][sl])

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            layers()  # first calls outside the capture (the library caches its launch geometry)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layers()
        graphs.append(g)
    stream = torch.cuda.current_stream()
    for i in range(3):
        graphs[i % len(graphs)].replay()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        graphs[i % len(graphs)].replay()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / steps


def run_variants(steps=10, warmup=2):
    """The far-field variants: γ and S per query head (sfa_prefill_qh,
    sfa_decode_step_qh) and the running mean of the keys that have left the
    window (sfa_prefill_rm, sfa_decode_step_rm), each on one 64K-token 7B-shaped
    prefill layer and the 28-layer decode step."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    res = {}
    # prefill: three layers of the 64K workload in turn, so that no layer's
    # K and V (134 MB) can stay in the 256 MB MALL from one call to its next
    layers = [inputs.workload(4, device=dev, layer=i) for i in range(3)]

    def prefill_ms(gammas, **kw):
        # calls back to back, as the headline step runs its layers: events on
        # the launch stream around all `reps` of them
        reps = 3 * steps
        for i in range(warmup):
            d = layers[i % 3]
            sfa.prefill(d["q"], d["k"], d["v"], gammas[i % 3], d["alpha"], **kw)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(reps):
            d = layers[i % 3]
            sfa.prefill(d["q"], d["k"], d["v"], gammas[i % 3], d["alpha"], **kw)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    # one decay per query head
    gq = [inputs.uniform((HQ,), 0.90, 0.99, 77 + i, device=dev) for i in range(3)]
    kw = dict(window=WIN, out=torch.empty((B, N, HQ, HD), dtype=torch.bfloat16, device=dev),
              ring_k=torch.zeros((B, HKV, WIN, HD), dtype=torch.bfloat16, device=dev),
              ring_v=torch.zeros((B, HKV, WIN, HD), dtype=torch.bfloat16, device=dev),
              state=torch.zeros((B, HQ, HD), dtype=torch.float32, device=dev),
              workspace=torch.empty(sfa.prefill_workspace_size(B, N, HQ, HD), dtype=torch.uint8, device=dev),
              stream=stream, gamma_per_query_head=True)
    ms = prefill_ms(gq, **kw)
    byts = prefill_bytes_per_launch() + B * HQ * HD * 4
    res["prefill_qh"] = {"workload": "7B-shaped 64K-token prefill layer, γ and S per query head",
                         "us_per_call": ms * 1e3, "value": B * N * HQ / (ms * 1e-3),
                         "unit": "tokens·heads/s", "timing": "back-to-back calls over three layers in turn, events around all",
                         "roofline": {"bound": "hbm", "achieved": byts / (ms * 1e-3) / 1e9,
                                      "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                                      "frac": byts / (ms * 1e-3) / PEAK_HBM, "bytes_per_call": byts}}
    # decode: the 28-layer step with S [L,B,Hq,d] and γ [L,Hq]
    L, Bd, Hq, Hkv, hd = 28, 256, 28, 4, 128
    sets = []
    for i in range(3):
        dd = inputs.decode_inputs(L, Bd, Hq, Hkv, hd, seed=4000 + i, device=dev)
        dd["state"] = inputs.normal((L, Bd, Hq, hd), 4100 + i, 1.0, torch.float32, dev)
        dd["gamma"] = inputs.uniform((L, Hq), 0.90, 0.99, 4200 + i, dev)
        dd["out"] = torch.empty((L, Bd, Hq, hd), dtype=torch.bfloat16, device=dev)
        sets.append(dd)

    ms = replay_ms(lambda dd: sfa.decode_step(dd["q"], dd["k_new"], dd["v_new"], dd["ring_k"], dd["ring_v"],
                                              dd["state"], dd["pos"], dd["gamma"], dd["alpha"], out=dd["out"],
                                              gamma_per_query_head=True), sets, 4 * steps // 3 + 1)
    byts = decode_bytes() + L * Bd * (Hq - Hkv) * hd * 4 * 2
    res["decode_qh"] = {"workload": "7B-shaped decode step, 28 layers x 256 sequences, γ and S per query head",
                        "us_per_step": ms * 1e3, "value": L * Bd * Hq / (ms * 1e-3),
                        "unit": "tokens·heads/s (sequence, query head, layer)",
                        "roofline": {"bound": "hbm", "achieved": byts / (ms * 1e-3) / 1e9,
                                     "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                                     "frac": byts / (ms * 1e-3) / PEAK_HBM, "bytes_per_step": byts}}
    del sets
    torch.cuda.empty_cache()
    # running mean of the keys that have left the window (state carries S and M)
    kw = dict(window=WIN, out=kw["out"],
              ring_k=torch.zeros((B, HKV, WIN, HD), dtype=torch.bfloat16, device=dev),
              ring_v=torch.zeros((B, HKV, WIN, HD), dtype=torch.bfloat16, device=dev),
              state=torch.zeros((B, HKV, 2, HD), dtype=torch.float32, device=dev),
              workspace=torch.empty(sfa.prefill_workspace_size(B, N, 3 * HKV, HD), dtype=torch.uint8,
                                    device=dev),
              stream=stream, running_mean=True)
    ms = prefill_ms([d["gamma"] for d in layers], **kw)
    byts = prefill_bytes_per_launch() + B * HKV * HD * 4
    res["prefill_rm"] = {"workload": "7B-shaped 64K-token prefill layer, running mean of the keys that left the window",
                         "us_per_call": ms * 1e3, "value": B * N * HQ / (ms * 1e-3),
                         "unit": "tokens·heads/s", "timing": "back-to-back calls over three layers in turn, events around all",
                         "roofline": {"bound": "hbm", "achieved": byts / (ms * 1e-3) / 1e9,
                                      "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                                      "frac": byts / (ms * 1e-3) / PEAK_HBM, "bytes_per_call": byts}}
    del layers, kw
    torch.cuda.empty_cache()
    sets = []
    for i in range(3):
        dd = inputs.decode_inputs(L, Bd, Hq, Hkv, hd, seed=4300 + i, device=dev)
        dd["state"] = inputs.normal((L, Bd, Hkv, 2, hd), 4400 + i, 1.0, torch.float32, dev)
        dd["out"] = torch.empty((L, Bd, Hq, hd), dtype=torch.bfloat16, device=dev)
        sets.append(dd)

    ms = replay_ms(lambda dd: sfa.decode_step(dd["q"], dd["k_new"], dd["v_new"], dd["ring_k"], dd["ring_v"],
                                              dd["state"], dd["pos"], dd["gamma"], dd["alpha"], out=dd["out"],
                                              running_mean=True), sets, 4 * steps // 3 + 1)
    byts = decode_bytes() + L * Bd * Hkv * hd * 4 * 2
    res["decode_rm"] = {"workload": "7B-shaped decode step, 28 layers x 256 sequences, running mean",
                        "us_per_step": ms * 1e3, "value": L * Bd * Hq / (ms * 1e-3),
                        "unit": "tokens·heads/s (sequence, query head, layer)",
                        "roofline": {"bound": "hbm", "achieved": byts / (ms * 1e-3) / 1e9,
                                     "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                                     "frac": byts / (ms * 1e-3) / PEAK_HBM, "bytes_per_step": byts}}
    del sets
    torch.cuda.empty_cache()
    return res


def run_decode_enhance(reps=50, sets=4):
    """The decode step fused with the triple-channel enhancement
    (sfa_decode_step_enhance) on the 7B shape (28 layers, 28/4 heads, d 128,
    hidden 3584, a 64-slot pool per layer, bf16 out): one sequence (the
    engine's shape: every layer of one token), against the same work unfused
    (sfa_decode_step, then sfa_enhance_prepared on its one-token rows), both
    replayed from HIP graphs over `sets` rotating input sets; and a batch of 256
    sequences through the fused form (each workgroup reads its layer's pool)."""
    dev = torch.device("cuda:0")
    L, Hq, Hkv, hd, R = 28, 28, 4, 128, 16
    H = Hq * hd

    def make(Bs, seed):
        d = inputs.decode_inputs(L, Bs, Hq, Hkv, hd, seed=seed, device=dev)
        pool = inputs.normal((L, 64, H), seed * 16 + 14, 1.0, torch.float32, dev)
        d["prep"] = sfa.enhance_prepare_pool((pool / pool.norm(dim=-1, keepdim=True)).contiguous())
        d["e_ring"] = torch.zeros((L, Bs, R, H), device=dev)
        d["field"] = torch.zeros((L, Bs, H), device=dev)
        d["out"] = torch.empty((L, Bs, H), dtype=torch.bfloat16, device=dev)
        d["o"] = torch.empty((L, Bs, Hq, hd), dtype=torch.bfloat16, device=dev)
        d["ws"] = torch.empty(sfa.enhance_workspace_size(L, 1, H), dtype=torch.uint8, device=dev)
        return d

    def fused(d):
        sfa.decode_step_enhance(d["q"], d["k_new"], d["v_new"], d["ring_k"], d["ring_v"], d["state"], d["pos"],
                                d["gamma"], d["alpha"], d["e_ring"], d["field"], d["prep"], out=d["out"])

    def unfused(d):  # one sequence: its enhancement stream starts at its position
        sfa.decode_step(d["q"], d["k_new"], d["v_new"], d["ring_k"], d["ring_v"], d["state"], d["pos"],
                        d["gamma"], d["alpha"], out=d["o"])
        sfa.enhance_prepared(d["o"].view(L, 1, H), d["prep"], d["e_ring"][:, 0], d["field"][:, 0],
                             t0=int(d["pos0"]), out=d["out"].view(L, 1, H), workspace=d["ws"])

    def per_call_us(fn, bufs):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for d in bufs:
                fn(d)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for d in bufs:
                fn(d)
        for _ in range(3):
            g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        stream = torch.cuda.current_stream(dev)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * len(bufs))

    one = []
    for i in range(sets):
        d = make(1, 6000 + i)
        d["pos0"] = int(d["pos"][0])
        one.append(d)
    us_fused = per_call_us(fused, one)
    us_unfused = per_call_us(unfused, one)
    del one
    torch.cuda.empty_cache()
    big = [make(256, 6100)]
    us_big = per_call_us(fused, big)
    del big
    torch.cuda.empty_cache()
    return {"workload": "7B-shaped decode step fused with the triple-channel enhancement, 28 layers, "
                        "hidden 3584, 64-slot pool per layer, bf16",
            "one_sequence": {"fused_us_per_step": us_fused, "unfused_us_per_step": us_unfused,
                             "unfused": "sfa_decode_step + sfa_enhance_prepared (T = 1)"},
            "batch_256_fused_us_per_step": us_big}


def enhance_bytes(L=24, T=4096, H=1024, S=64, R=16):
    return L * T * H * 2 * 2 + L * S * H * 4 + 2 * L * R * H * 4 + 2 * L * H * 4


def run_enhance(steps=20, warmup=3, sets=3):
    """The 24-layer enhancement on `sets` rotating input sets (each larger than
    the 256 MB MALL).  The main figure uses the pool in prepared form
    (sfa_enhance_prepare_pool once per input set, outside the timed region: the
    pool is read-only); `per_call_prepare_us` is sfa_enhance, which derives the
    pool operands on every call."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    L, T, H = 24, 4096, 1024
    bufs = []
    for i in range(sets):
        d = inputs.workload(5, device=dev) if i == 0 else inputs.enhance_inputs(L, T, H, seed=3000 + i,
                                                                                device=dev)
        d["ring"] = torch.zeros((L, 16, H), device=dev)
        d["field"] = torch.zeros((L, H), device=dev)
        d["out"] = torch.empty((L, T, H), dtype=torch.bfloat16, device=dev)
        d["prepared"] = sfa.enhance_prepare_pool(d["pool"])
        bufs.append(d)
    ws = torch.empty(sfa.enhance_workspace_size(L, T, H), dtype=torch.uint8, device=dev)

    def call_prepared(d):
        sfa.enhance_prepared(d["attn"], d["prepared"], d["ring"], d["field"], out=d["out"], workspace=ws,
                             stream=stream)

    def timed(fn):
        for i in range(warmup):
            fn(bufs[i % sets])
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            ev[i][0].record(stream)
            fn(bufs[i % sets])
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / steps

    ms_ev = timed(call_prepared)
    reps = steps // sets + 1
    ms = replay_ms(lambda d: sfa.enhance_prepared(d["attn"], d["prepared"], d["ring"], d["field"], out=d["out"],
                                                  workspace=ws), bufs, reps)
    ms_pc = replay_ms(lambda d: sfa.enhance(d["attn"], d["pool"], d["ring"], d["field"], out=d["out"],
                                            workspace=ws), bufs, reps)
    byts = enhance_bytes()
    return {"workload": "triple-channel enhancement, 24 layers x 4096 tokens, hidden 1024, 64 slots, bf16",
            "value": L * T / (ms * 1e-3), "unit": "tokens·layers/s", "us_per_call": ms * 1e3,
            "timing": f"HIP-graph replays of {sets} rotating input sets",
            "events_us_per_call": ms_ev * 1e3,
            "kernel": "sfa_enhance_prepared (3 launches: k_sem, k_field_carry, k_cols)",
            "per_call_prepare_us": ms_pc * 1e3,
            "roofline": {"bound": "hbm", "achieved": byts / (ms * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9,
                         "unit": "GB/s", "frac": byts / (ms * 1e-3) / PEAK_HBM, "bytes_per_call": byts}}


# ----------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on whole layers of the same workload
# ----------------------------------------------------------------------------
def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(n_layers, budget_s=10.0):
    import numpy as np

    import oracle
    done, t_cpu = 0, 0.0
    for l in range(n_layers):
        x = inputs.workload(4, device="cuda", layer=l)  # the same seeded inputs as the GPU run
        q = np.ascontiguousarray(x["q"].float().cpu().numpy())
        k = np.ascontiguousarray(x["k"].float().cpu().numpy())
        v = np.ascontiguousarray(x["v"].float().cpu().numpy())
        g, a = x["gamma"].cpu(), x["alpha"].cpu()
        t0 = time.perf_counter()
        oracle.prefill(q, k, v, g, a, WIN)
        t_cpu += time.perf_counter() - t0
        done += 1
        log(f"cpu baseline: oracle layer {done} done, {t_cpu:.1f} s")
        if t_cpu >= budget_s:
            break
    return {"value": done * B * N * HQ / t_cpu, "unit": "tokens·heads/s", "cores": oracle.num_threads(),
            "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": t_cpu,
            "sample": f"{done} of the 28 layers of the same 64K-token prefill workload, fp64 C oracle "
                      f"(OpenMP over heads), wall time of the oracle call only"}


def copy_ceiling(nbytes=1 << 30, reps=5):
    """Device-to-device copy of 1 GiB (the runtime's copy kernel), timed with HIP
    events: read + write bytes per second, the practical ceiling that a
    streaming kernel with equal read and write traffic can be compared with."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
    torch.cuda.synchronize()
    ms = min(a.elapsed_time(b) for a, b in ev)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


def traffic():
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source; else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("prefill_src_sha256_16") != src_hash(PREFILL_SRC):
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=28, help="stacked prefill layers per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--only", choices=["c2", "decode", "enhance", "decode_enhance", "variants"], default=None,
                    help="run only this secondary measurement (for profiling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every kernel here runs on a single MI355X and "
              "there is no multi-GPU path to time; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.only:
        run = {"c2": run_c2, "decode": run_decode, "enhance": run_enhance, "decode_enhance": run_decode_enhance,
               "variants": run_variants}[args.only]
        print(json.dumps(run()), flush=True)
        return

    pre = run_prefill(args)
    ms_step = pre["wall"] * 1e3 / args.steps
    value = B * N * HQ * args.layers / (pre["wall"] / args.steps)
    byts = prefill_bytes_per_launch()
    achieved = byts / (pre["attn_ms"] * 1e-3)
    tr = traffic()
    res = {
        "metric": METRIC, "value": value, "unit": "tokens·heads/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "7B-shaped long-context SFA prefill, 28 stacked layers",
                   "batch": B, "seq_len": N, "q_heads": HQ, "kv_heads": HKV, "head_dim": HD,
                   "window": WIN, "layers": args.layers, "gamma": 0.98, "alpha": 0.1},
        "roofline": {"bound": "hbm", "kernel": "k_window_attn", "achieved": achieved / 1e9,
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": achieved / PEAK_HBM,
                     "traffic": tr, "algorithmic_bytes_per_launch": byts,
                     "avg_launch_us": pre["attn_ms"] * 1e3},
        "prefill_step_gbps": byts * args.layers / (ms_step * 1e-3) / 1e9,
    }
    del pre["layers"]
    torch.cuda.empty_cache()
    if not args.no_secondary:
        res["c2"] = run_c2()
        res["decode"] = run_decode()
        res["enhance"] = run_enhance()
        res["decode_enhance"] = run_decode_enhance()
        res["variants"] = run_variants()
        res["copy_ceiling_gbps"] = copy_ceiling()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.layers)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
