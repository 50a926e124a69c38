"""Benchmark: MASW draft decode attention vs the full-KV draft baseline on one MI355X.

Workload: Llama-3.2-3B-shaped draft attention stack (28 layers, 24 query heads, 8 KV
heads, head_dim 128, bf16), batch 8, S=4 sinks, W=2048 local window, r=64 slot
interval; seeded synthetic N(0,1) K/V/q, slots pre-materialized as the bf16 projection
of seeded hidden states through seeded mirrored weights.

One step = one decode position for all 8 sequences through all 28 layers: per layer
raw append (with eviction), slot materialization when the step is a slot boundary
(mirrored projection + structured-mask slot query + slot append), and the draft
attention over sink ++ window ++ slots.  The headline value is MASW steps/s at prefix
32768; the same line carries the prefix sweep 1K..32K for MASW and for the full-KV
baseline (same kernel over the whole cache), the roofline of the decode attention
kernel and the fp64 oracle timed on the host cores.

Steps are captured once into HIP graphs (one for ordinary steps, one for boundary
steps) and replayed; the host picks the graph from its own position counter, so no
device value is read inside the timed region.

    python bench.py [--gpus 1] [--steps 256] [--warmup 16]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import draft_kv_attention_amd as M   # noqa: E402
import seeded_inputs as SI           # noqa: E402

METRIC = "draft attn steps/s + HBM GB/s (% peak) vs prefix 1K-32K, MASW vs full-KV"
# Counter summary of the dominant kernel (two rocprofv3 --pmc passes of --traffic-probe)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_b8_prefix32768_hbm_traffic.md")
DECODE_SOURCES = ("decode_attn.hip", "decode_args.hpp", "masw_device.hpp", "masw_internal.hpp", "project_mfma.hpp")
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak (no sparsity)
SHAPE = SI.SWEEP_3B
T_HEAD = 32768


def n_slots_at(t, S, W, r):
    return max(0, t - S - W) // r if r else 0   # r = 0: no slot chain


def keys_at(t, S, W, r):
    return min(t, S) + min(max(t - S, 0), W) + n_slots_at(t, S, W, r)


def is_boundary(t, S, W, r):
    d = t - S - W
    return r > 0 and d >= r and d % r == 0


class Stack:
    """28 layers of MASW memory plus the full caches, inputs and graphs."""

    def __init__(self, shape, t_max, dev, seed=0, with_full=True):
        self.shape = shape
        S, W, r = shape.sink, shape.window, shape.interval
        self.S, self.W, self.r = S, W, r
        self.L = shape.layers
        self.dev = dev
        self.max_slots = n_slots_at(t_max, S, W, r) + 2
        self.d = M.Dims(batch=shape.batch, n_q_heads=shape.n_q_heads, n_kv_heads=shape.n_kv_heads,
                        head_dim=shape.head_dim, sink=S, window=W, interval=r,
                        max_slots=self.max_slots, dtype=shape.dtype)
        B, Hq, Hkv, D, hid = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.hidden
        g = torch.Generator(device=dev)
        g.manual_seed(seed)

        def rnd(*s, std=1.0):
            return (torch.randn(*s, generator=g, device=dev, dtype=torch.float32) * std).to(shape.dtype)

        self.layers, self.wk, self.wv = [], [], []
        for _ in range(self.L):
            lay = M.alloc_layer(self.d, dev, fill=None)
            kvs = shape.kv_std
            lay.k_sink.copy_(rnd(*lay.k_sink.shape, std=kvs)); lay.v_sink.copy_(rnd(*lay.v_sink.shape, std=kvs))
            lay.k_ring.copy_(rnd(*lay.k_ring.shape, std=kvs)); lay.v_ring.copy_(rnd(*lay.v_ring.shape, std=kvs))
            wk, wv = rnd(hid, Hkv * D, std=shape.w_std), rnd(hid, Hkv * D, std=shape.w_std)
            hs = rnd(B * self.max_slots, hid)
            lay.k_slot.copy_((hs @ wk).view(B, self.max_slots, Hkv, D).permute(0, 2, 1, 3))
            lay.v_slot.copy_((hs @ wv).view(B, self.max_slots, Hkv, D).permute(0, 2, 1, 3))
            self.layers.append(lay)
            self.wk.append(wk)
            self.wv.append(wv)
        self.seq = M.alloc_seq(B, dev)
        self.ws = M.workspace(self.d, M.OP_MATERIALIZE, device=dev)
        self.k_new = [rnd(B, 1, Hkv, D, std=shape.kv_std) for _ in range(self.L)]
        self.v_new = [rnd(B, 1, Hkv, D, std=shape.kv_std) for _ in range(self.L)]
        self.q = [rnd(B, Hq, D) for _ in range(self.L)]
        self.out = [torch.empty(B, Hq, D, dtype=shape.dtype, device=dev) for _ in range(self.L)]
        self.h = [rnd(B, hid) for _ in range(self.L)]
        self.qg = [rnd(B, Hq, D) for _ in range(self.L)]
        self.og = [torch.empty(B, Hq, D, dtype=shape.dtype, device=dev) for _ in range(self.L)]
        self.full_len = t_max + 8
        self.kf, self.vf = [], []
        if with_full:
            for _ in range(self.L):
                self.kf.append(rnd(B, Hkv, self.full_len, D, std=shape.kv_std))
                self.vf.append(rnd(B, Hkv, self.full_len, D, std=shape.kv_std))
            self.fd = M.Dims(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, dtype=shape.dtype)
            self.seq_full = torch.zeros(B, dtype=torch.int32, device=dev)
            self.err_full = torch.zeros(1, dtype=torch.int32, device=dev)
            self.ws_full = M.workspace(self.fd, M.OP_FULLKV_DECODE, max_keys=self.full_len, device=dev)
        self.graphs = {}

    # -- state -------------------------------------------------------------
    def set_position(self, t):
        self.seq.seq_len.fill_(t)
        n = n_slots_at(t, self.S, self.W, self.r)
        for lay in self.layers:
            lay.n_slots.fill_(n)
        if self.kf:
            self.seq_full.fill_(t)
        self.t = t

    def mirror_full_into_masw(self, t):
        """Make the MASW memory hold the full cache's own raw rows at position t: sinks
        1..S and the ring cells of positions t-C+1..t (cell (i-S-1) mod C); slots keep
        their projected values."""
        S, C = self.S, self.d.ring
        lo = max(S + 1, t - C + 1)
        pos = torch.arange(lo, t + 1, device=self.dev)
        cells = (pos - S - 1) % C
        for lay, kf, vf in zip(self.layers, self.kf, self.vf):
            lay.k_sink.copy_(kf[:, :, :S]); lay.v_sink.copy_(vf[:, :, :S])
            lay.k_ring[:, :, cells] = kf[:, :, pos - 1]
            lay.v_ring[:, :, cells] = vf[:, :, pos - 1]

    # -- one step ----------------------------------------------------------
    def masw_step(self, boundary):
        """One decode position: per layer, the slot materialization when the step is a
        boundary (it reads only older tokens, so it may precede the append), then the
        fused raw append + draft attention."""
        self.seq.seq_len.add_(1)
        for l in range(self.L):
            lay = self.layers[l]
            if boundary:
                M.masw_materialize_slot(self.d, lay, self.seq, self.h[l], self.wk[l], self.wv[l],
                                        self.qg[l], self.og[l], self.ws)
            M.masw_decode_step(self.d, lay, self.seq, self.k_new[l], self.v_new[l], self.q[l],
                               self.out[l], self.ws)

    def full_step(self):
        self.seq_full.add_(1)
        for l in range(self.L):
            M.fullkv_decode_step(self.fd, self.kf[l], self.vf[l], self.seq_full, self.err_full,
                                 self.k_new[l], self.v_new[l], self.q[l], self.out[l], self.ws_full)

    def capture(self):
        """Capture the three step variants; each capture advances nothing (state is reset)."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for name, fn in (("masw", lambda: self.masw_step(False)),
                             ("masw_boundary", (lambda: self.masw_step(True)) if self.r else None),
                             ("full", self.full_step if self.kf else None)):
                if fn is None:
                    continue
                fn()   # warm once eagerly on the side stream
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    fn()
                self.graphs[name] = g
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()

    def replay_masw(self):
        nxt = self.t + 1
        self.graphs["masw_boundary" if is_boundary(nxt, self.S, self.W, self.r) else "masw"].replay()
        self.t = nxt

    def replay_full(self):
        self.graphs["full"].replay()
        self.t += 1

    # -- algorithmic bytes ---------------------------------------------------
    def kv_row_bytes(self):
        sh = self.shape
        return sh.n_kv_heads * sh.head_dim * 2 * 2          # K and V, bf16

    def attn_bytes(self, keys):
        sh = self.shape
        return sh.batch * (keys * self.kv_row_bytes() + 2 * sh.n_q_heads * sh.head_dim * 2)

    def masw_step_bytes(self, t):
        sh = self.shape
        b = self.L * (self.attn_bytes(keys_at(t, self.S, self.W, self.r)) + sh.batch * self.kv_row_bytes())
        if is_boundary(t, self.S, self.W, self.r):
            m = (t - self.S - self.W) // self.r
            proj = 2 * sh.hidden * sh.n_kv_heads * sh.head_dim * 2 + sh.batch * sh.hidden * 2
            b += self.L * (proj + self.attn_bytes(self.S + self.W + m - 1) + sh.batch * self.kv_row_bytes())
        return b

    def full_step_bytes(self, t):
        return self.L * (self.attn_bytes(t) + self.shape.batch * self.kv_row_bytes())


def first_boundary_after(t, S, W, r):
    """The first slot-boundary position > t (r = 0: none)."""
    if not r:
        return None
    d = max(t + 1 - S - W, r)
    return S + W + -(-d // r) * r


def time_steps(stack, which, t_start, warmup, steps, quantiles=False):
    """Replay `steps` graph steps from position t_start after `warmup` untimed ones.
    Returns (mean ms per step, mean algorithmic bytes per step) and, with quantiles,
    also (p10, p50, p90) of the per-step durations from an event before every replay."""
    stack.set_position(t_start)
    rep = stack.replay_masw if which == "masw" else stack.replay_full
    for _ in range(warmup):
        rep()
    t0 = stack.t
    stack.timed_positions = (t0 + 1, t0 + steps)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        rep()
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / steps
    bytes_fn = stack.masw_step_bytes if which == "masw" else stack.full_step_bytes
    avg_bytes = sum(bytes_fn(t) for t in range(t0 + 1, t0 + steps + 1)) / steps
    if not quantiles:
        return ms, avg_bytes
    d = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
    return ms, avg_bytes, tuple(round(float(np.percentile(d, p)), 4) for p in (10, 50, 90))


def linear_fit(xs, ys):
    """Least-squares ys = a + b xs; returns (a, b, R^2)."""
    x, y = np.asarray(xs, dtype=np.float64), np.asarray(ys, dtype=np.float64)
    b, a = np.polyfit(x, y, 1)
    res = y - (a + b * x)
    r2 = 1.0 - float(res @ res) / float(((y - y.mean()) ** 2).sum())
    return float(a), float(b), r2


def stream_read_leg(dev, launch_bytes, reps=5):
    """Measured HBM read rate of a plain streaming kernel (masw_stream_read): over one
    4 GiB buffer (sustained), and at the decode launch's size, 28 distinct buffers
    rotated in a HIP graph as the attention layers are."""
    total = torch.zeros(M.STREAM_SUMS, dtype=torch.int32, device=dev)
    big = torch.ones(1 << 28, dtype=torch.int32, device=dev)     # 1 GiB
    big = torch.cat([big, big, big, big])                        # 4 GiB
    nb = big.numel() * 4
    M.stream_read(big, total)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        M.stream_read(big, total)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    us_big = float(np.median(ts))
    del big
    n16 = launch_bytes // 16 * 16
    bufs = [torch.ones(n16 // 4, dtype=torch.int32, device=dev) for _ in range(28)]
    us_small = graph_per_call_us(lambda i: M.stream_read(bufs[i % 28], total), 56)
    del bufs
    torch.cuda.empty_cache()
    return dict(kernel="masw_stream_read (2048 work-groups, 8 x 16 B loads in flight per lane)",
                sustained_4gib_gbs=round(nb / us_big / 1e3, 1),
                sustained_pct_peak=round(100 * nb / us_big / 1e3 / HBM_PEAK_GBS, 1),
                launch_size_bytes=int(n16), launch_size_us=round(us_small, 2),
                launch_size_gbs=round(n16 / us_small / 1e3, 1),
                launch_size_pct_peak=round(100 * n16 / us_small / 1e3 / HBM_PEAK_GBS, 1))


SECOND_WORKLOADS = (("paper_w128_s128_r4", 128, 128, 4), ("paper_w128_s128_r8", 128, 128, 8),
                    ("swa_w1024", 0, 1024, 0), ("sink4_window2048", 4, 2048, 0))


def second_workload_leg(dev, prefixes=(8192, 16384, 32768), steps=32, warmup=4):
    """The paper's own memory geometry (W = S = 128, r = 4 / 8 raw tokens per slot) and
    memories without a slot chain (a 1,024-token sliding window, sinks + window) through
    the same kernels, at the 3B draft shapes, B = 8: graph-replayed 28-layer steps with
    boundary steps (slot materialization) where the geometry has them."""
    out = []
    for name, S, W, r in SECOND_WORKLOADS:
        shape = dataclasses.replace(SHAPE, sink=S, window=W, interval=r)
        st = Stack(shape, max(prefixes) + steps + warmup + 8, dev, seed=3, with_full=False)
        st.capture()
        for t in prefixes:
            ms, nb = time_steps(st, "masw", t, warmup, steps)
            out.append(dict(workload=name, sink=S, window=W, interval=r, prefix=t,
                            keys=keys_at(t, S, W, r), ms=round(ms, 4), steps_per_s=round(1e3 / ms, 2),
                            gbs=round(nb / (ms * 1e-3) / 1e9, 1),
                            pct_peak=round(100 * nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)))
        assert int(st.seq.err.item()) == 0, name
        del st
        torch.cuda.empty_cache()
    return out


def rollback_leg(dev, reps=4):
    """masw_rollback per layer at the bench shape (B = 8, rollback rows 16, the paper's
    retained window): truncating n_slots after a rejected speculation, graph-replayed
    over 28 layers; the raw tokens need no data movement."""
    sh = SHAPE
    d = M.Dims(batch=sh.batch, n_q_heads=sh.n_q_heads, n_kv_heads=sh.n_kv_heads, head_dim=sh.head_dim,
               sink=sh.sink, window=sh.window, interval=sh.interval, max_slots=8, dtype=sh.dtype, rollback=16)
    layers = [M.alloc_layer(d, dev, fill=None) for _ in range(sh.layers)]
    seq = M.alloc_seq(sh.batch, dev)
    seq.seq_len.fill_(sh.sink + sh.window + 5 * sh.interval)
    t_spec = seq.seq_len + 5
    for lay in layers:
        lay.n_slots.fill_(6)
    us = graph_per_call_us(lambda i: M.masw_rollback(d, layers[i % sh.layers], seq, t_spec), sh.layers * reps)
    ok = int(seq.err.item()) == 0 and all(int(l.n_slots[0].item()) == 5 for l in layers)
    return dict(op="masw_rollback", us_per_layer=round(us, 2), rollback_rows=16, batch=sh.batch, checked=ok)


def read_floor_us(dev, nbytes, n_bufs, reps=3):
    """Per-launch time of the plain streaming-read kernel (masw_stream_read) at `nbytes`
    per launch over `n_bufs` distinct buffers replayed in a graph, the fastest of 256 to
    2048 work-groups: what a kernel that only reads can do at this launch size."""
    total = torch.zeros(M.STREAM_SUMS, dtype=torch.int32, device=dev)
    n16 = nbytes // 16 * 16
    bufs = [torch.ones(n16 // 4, dtype=torch.int32, device=dev) for _ in range(n_bufs)]
    us = min(graph_per_call_us(lambda i: M.stream_read(bufs[i % n_bufs], total, work_groups=wgs), 2 * n_bufs)
             for wgs in (256, 512, 1024, 2048) for _ in range(reps))
    del bufs
    torch.cuda.empty_cache()
    return round(us, 2), int(n16)


def single_sequence_leg(dev, steps=32, warmup=6):
    """The batch-1 workload: one sequence at prefix 8192, K,V ~ 0.5 N(0,1), the MASW
    memory holding the full cache's own raw rows; MASW and full-KV graph steps.

    Two sets of the 28 layers are allocated and every graph replay runs both in turn (56
    distinct layers: 492 MB of MASW memory, 1.9 GB of full cache), so nothing is served
    from the 256 MB last-level cache; the figures are per 28-layer step.  Next to them,
    the streaming-read floor at each launch's size over the same number of buffers."""
    sh, t = SI.DRAFT_3B, SI.DRAFT_3B_PREFIX
    sets = 2
    st = Stack(dataclasses.replace(sh, layers=sets * sh.layers), t + steps + warmup + 16, dev, seed=1)
    st.capture()                   # its eager warm-up steps append into both caches
    st.mirror_full_into_masw(t)
    out = dict(workload="masw vs full-KV, 28 layers, batch 1, prefix 8192", prefix=t, batch=1,
               keys_masw=keys_at(t, sh.sink, sh.window, sh.interval), keys_full=t,
               layer_sets=sets, distinct_layers=st.L)
    for which in ("masw", "full"):
        ms, nb, q = time_steps(st, which, t, warmup, steps, quantiles=True)
        ms, nb, q = ms / sets, nb / sets, tuple(round(x / sets, 4) for x in q)
        out[f"{which}_ms"] = round(ms, 4)
        out[f"{which}_ms_p10_p50_p90"] = q
        out[f"{which}_steps_per_s"] = round(1e3 / ms, 2)
        out[f"{which}_gbs"] = round(nb / (ms * 1e-3) / 1e9, 1)
        out[f"{which}_pct_peak"] = round(100 * nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)
        layer_bytes = nb / sh.layers
        floor_us, floor_bytes = read_floor_us(dev, int(layer_bytes), st.L)
        out[f"{which}_us_per_layer"] = round(ms * 1e3 / sh.layers, 2)
        out[f"{which}_read_floor_us_per_layer"] = floor_us
        out[f"{which}_over_read_floor"] = round(ms * 1e3 / sh.layers / floor_us, 2)
    out["full_over_masw_latency"] = round(out["full_ms"] / out["masw_ms"], 3)
    out["device_err_bits"] = int(st.seq.err.item()) | int(st.err_full.item())
    del st
    torch.cuda.empty_cache()
    return out


def mfma_reference_leg(dev, iters=20000):
    """Matrix-core rate this device sustains (`masw_mfma_rate`: four independent
    32x32x16 bf16 MFMA chains per wave, register operands) with one and with two waves
    per SIMD, and the shader clock under that load (s_memtime ticks per 100 MHz
    s_memrealtime tick): the measured reference next to the nominal 2.5 PFLOP/s."""
    res = {}
    for label, wgs in (("one_wave_per_simd", 256), ("two_waves_per_simd", 512)):
        out = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
        clocks = torch.zeros(2, dtype=torch.int64, device=dev)
        M.mfma_rate(wgs, 100, out, clocks)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        M.mfma_rate(wgs, iters, out, clocks)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        c = clocks.cpu().tolist()
        flops = wgs * 4 * iters * 4 * 2 * 32 * 32 * 16
        res[label] = dict(pflops=round(flops / (ms * 1e-3) / 1e15, 3),
                          pct_of_nominal=round(100 * flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 1),
                          shader_ghz=round(c[0] / (c[1] / 100e6) / 1e9, 3) if c[1] else None,
                          cycles_per_mfma=round(c[0] / (4 * iters), 2))
    return res


def prefill_flops(P, S, W, r, Hq, D, hidden=0, n_kv=0):
    """Algorithmic flops of a prefill: 4 D Hq per (query, visible key) for S = QK^T and
    O = PV, over every raw query i (keylist(i)) and slot query m (keylist(t_m - r)), plus
    2 x 2 hidden (Hkv D) per projected slot."""
    att = sum(keys_at(i, S, W, r) for i in range(1, P + 1))
    n = n_slots_at(P, S, W, r)
    att += sum(keys_at(S + W + (m - 1) * r, S, W, r) for m in range(1, n + 1))
    return 4 * D * Hq * att + 4 * hidden * n_kv * D * n


def prefill_leg(dev, reps=10):
    """Draft prefill of one layer at the 3B draft shape, B = 1, a 32768-token prefix
    (479 slots): masw_prefill (slot projection, memory load, attention of every raw and
    slot query); the same call without a slot chain (sinks + window only); and the same
    attention kernel as a full causal prefill (every token a sink).  Matrix-core
    roofline: algorithmic flops / time vs the dense bf16 peak."""
    sh, P = SI.PREFILL_3B, SI.PREFILL_LEN
    S, W, r = sh.sink, sh.window, sh.interval
    n = n_slots_at(P, S, W, r)
    k, v, q, h, qs = SI.prefill_inputs(sh, 17, 0, P, n, device=dev)
    wk, wv = SI.mirrored_weights(sh, 17, device=dev)
    out = torch.empty_like(q)
    o_slot = torch.empty_like(qs)
    seq = M.alloc_seq(1, dev)
    seq.seq_len.fill_(P)
    res = dict(workload="draft prefill, 3B draft shapes, batch 1, prefix 32768, one layer", prefix=P, slots=n)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    d = M.Dims(batch=1, n_q_heads=sh.n_q_heads, n_kv_heads=sh.n_kv_heads, head_dim=sh.head_dim, sink=S,
               window=W, interval=r, max_slots=n, dtype=sh.dtype)
    layer = M.alloc_layer(d, dev, fill=None)
    layer.n_slots.zero_()
    ms = timed(lambda: M.masw_prefill(d, layer, seq, k, v, q, out, h, wk, wv, qs, o_slot))
    fl = prefill_flops(P, S, W, r, sh.n_q_heads, sh.head_dim, sh.hidden, sh.n_kv_heads)
    res.update(masw_ms=round(ms, 4), masw_tokens_per_s=round(P / (ms * 1e-3), 1),
               masw_tflops=round(fl / (ms * 1e-3) / 1e12, 1),
               masw_pct_bf16_peak=round(100 * fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 1))
    # without materialization: the same sinks and window, no slot chain (the comparison
    # the pages' Table 2 draws for prefill cost)
    d0 = M.Dims(batch=1, n_q_heads=sh.n_q_heads, n_kv_heads=sh.n_kv_heads, head_dim=sh.head_dim, sink=S,
                window=W, interval=0, max_slots=0, dtype=sh.dtype)
    l0 = M.alloc_layer(d0, dev, fill=None)
    l0.n_slots.zero_()
    ms0 = timed(lambda: M.masw_prefill(d0, l0, seq, k, v, q, out))
    fl0 = prefill_flops(P, S, W, 0, sh.n_q_heads, sh.head_dim)
    res.update(no_slots_ms=round(ms0, 4), no_slots_pct_bf16_peak=round(100 * fl0 / (ms0 * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 1),
               masw_over_no_slots=round(ms / ms0, 2))
    # the same kernels as a full causal prefill: S = P, no window beyond it, no slots
    dfull = M.Dims(batch=1, n_q_heads=sh.n_q_heads, n_kv_heads=sh.n_kv_heads, head_dim=sh.head_dim, sink=P,
                   window=1, interval=0, max_slots=0, dtype=sh.dtype)
    lfull = M.alloc_layer(dfull, dev, fill=None)
    lfull.n_slots.zero_()
    msf = timed(lambda: M.masw_prefill(dfull, lfull, seq, k, v, q, out))
    flf = 4 * sh.head_dim * sh.n_q_heads * P * (P + 1) // 2
    res.update(full_causal_ms=round(msf, 4), full_causal_tflops=round(flf / (msf * 1e-3) / 1e12, 1),
               full_causal_pct_bf16_peak=round(100 * flf / (msf * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 1),
               full_over_masw=round(msf / ms, 2), algorithmic_flops_masw=fl, algorithmic_flops_full=flf,
               device_err_bits=int(seq.err.item()))
    del layer, lfull, l0
    torch.cuda.empty_cache()
    return res


def graph_per_call_us(fn, calls, replays=5):
    """Average duration of one call inside a captured graph of `calls` back-to-back calls."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(calls):
            fn(i)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(calls):
                fn(i)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * calls)


def decode_source_hash():
    """sha256 over the sources the decode kernel is built from."""
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "draft_kv_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter summary, or
    None when there is none or the kernel sources changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    src = re.search(r"source_sha256:\s*([0-9a-f]+)", text)
    tot = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    if not src or not tot or src.group(1) != decode_source_hash():
        return None
    return int(tot.group(1))


def kernel_roofline(stack, t, reps=4):
    """The dominant kernel of the MASW step: the fused append + draft attention launch.

    Average launch duration from HIP events around graph replays of 28 layers x reps
    back-to-back launches at prefix t (distinct per-layer buffers, 2.3 GB per pass, so
    nothing is served from the 256 MB last-level cache).  Algorithmic bytes per launch:
    the working set's K and V read once, q read, out written, the new token read from
    the caller and written into the ring.
    """
    stack.set_position(t)
    L = stack.L
    us = graph_per_call_us(lambda i: M.masw_decode_step(stack.d, stack.layers[i % L], stack.seq,
                                                        stack.k_new[i % L], stack.v_new[i % L],
                                                        stack.q[i % L], stack.out[i % L], stack.ws),
                           L * reps)
    sh = stack.shape
    nbytes = stack.attn_bytes(keys_at(t, stack.S, stack.W, stack.r)) + 2 * sh.batch * stack.kv_row_bytes()
    achieved = nbytes / (us * 1e-6) / 1e9
    return dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4), traffic=measured_traffic(),
                kernel="decode_kernel<bf16,128,3> (masw_decode_step)", avg_us=round(us, 2),
                bytes_per_launch=int(nbytes), prefix=t, launches_timed=L * reps * 5)


def verify_leg(dev, prefix=32768, n_q=6, batch=4):
    """Verifier attention, one GPU's share of an 8B / 70B layer (8 KV heads)."""
    out = []
    t = prefix + n_q
    for Hq in (32, 64):
        vd = M.Dims(batch=batch, n_q_heads=Hq, n_kv_heads=8, head_dim=128, dtype=torch.bfloat16)
        g = torch.Generator(device=dev)
        g.manual_seed(7)
        kv = [torch.randn(batch, 8, t + 8, 128, device=dev, dtype=torch.bfloat16, generator=g) for _ in range(2)]
        vv = [torch.randn(batch, 8, t + 8, 128, device=dev, dtype=torch.bfloat16, generator=g) for _ in range(2)]
        qv = torch.randn(batch, n_q, Hq, 128, device=dev, dtype=torch.bfloat16, generator=g)
        ov = torch.empty_like(qv)
        sv = torch.full((batch,), t, dtype=torch.int32, device=dev)
        ev = torch.zeros(1, dtype=torch.int32, device=dev)
        wsv = M.workspace(vd, M.OP_FULLKV_VERIFY, max_keys=t + 8, n_q=n_q, device=dev)
        us = graph_per_call_us(lambda i: M.fullkv_verify_attn(vd, kv[i % 2], vv[i % 2], sv, ev, qv, ov, wsv), 8)
        nbytes = batch * (t * 8 * 128 * 2 * 2 + 2 * n_q * Hq * 128 * 2)
        flops = 4.0 * batch * n_q * Hq * 128 * t
        out.append(dict(shape=f"{Hq}q/8kv heads, prefix {prefix}+{n_q}, batch {batch}", us_per_layer=round(us, 2),
                        gbs=round(nbytes / us / 1e3, 1), pct_peak=round(100 * nbytes / us / 1e3 / HBM_PEAK_GBS, 1),
                        tflops=round(flops / us / 1e6, 1),
                        mfma_pct_bf16_peak=round(100 * flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 1),
                        err_bits=int(ev.item())))
        del kv, vv
        torch.cuda.empty_cache()
    return out


def materialize_leg(stack, t_boundary, replays=5, dims=None, ws=None):
    """One slot boundary across the 28 layers (projection + structured-mask slot query).

    Each replay first resets every layer's n_slots to m-1 (so the boundary is pending
    again); a graph holding only those resets is timed separately and subtracted.
    `dims` overrides the stack's (e.g. to rotate the slot keys, or a smaller batch: the
    first sequences of every tensor), `ws` the workspace (one per plan).
    """
    L = stack.L
    d = dims if dims is not None else stack.d
    ws = ws if ws is not None else stack.ws
    B = d.batch

    def sub(x):
        return x if B == stack.shape.batch else x[:B]

    layers = [M.Layer(**{f.name: sub(getattr(lay, f.name)) for f in dataclasses.fields(lay)})
              for lay in stack.layers]
    seq = M.Seq(seq_len=sub(stack.seq.seq_len), err=stack.seq.err)
    stack.set_position(t_boundary)
    m = (t_boundary - stack.S - stack.W) // stack.r

    def resets():
        for lay in stack.layers:
            lay.n_slots.fill_(m - 1)

    def boundary():
        resets()
        for i in range(L):
            M.masw_materialize_slot(d, layers[i], seq, sub(stack.h[i]), stack.wk[i], stack.wv[i],
                                    sub(stack.qg[i]), sub(stack.og[i]), ws)

    times = {}
    for name, fn in (("resets", resets), ("boundary", boundary)):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                fn()
        torch.cuda.current_stream().wait_stream(s)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) * 1e3 / replays
    per_layer = (times["boundary"] - times["resets"]) / L
    sh = stack.shape
    keys = stack.S + stack.W + m - 1
    nbytes = (2 * sh.hidden * sh.n_kv_heads * sh.head_dim * 2 + B * sh.hidden * 2
              + stack.attn_bytes(keys) * B // sh.batch + B * stack.kv_row_bytes())
    return dict(batch=B, slot_index=m, us_per_layer=round(per_layer, 2), bytes_per_layer=int(nbytes),
                gbs=round(nbytes / per_layer / 1e3, 1), pct_peak=round(100 * nbytes / per_layer / 1e3 / HBM_PEAK_GBS, 1),
                boundaries_per_s=round(1e6 / (per_layer * L), 1), per_decode_step_us=round(per_layer * L / stack.r, 2),
                slots_after=int(stack.layers[0].n_slots[0].item()), device_err_bits=int(seq.err.item()))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_sample(seed):
    """Seeded memory of one (layer, sequence) unit at prefix 32768: its K/V rows gathered
    into the key order of the MASW memory (and of the full cache), and queries."""
    from oracle import masw_oracle as O
    sh = SHAPE
    S, W, r, Hq, Hkv, D = sh.sink, sh.window, sh.interval, sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    t = T_HEAD
    rng = np.random.default_rng(seed)
    n = O.visible_slot_count(t, S, W, r)
    raw_k = rng.standard_normal((t + 1, Hkv, D), dtype=np.float32)
    raw_v = rng.standard_normal((t + 1, Hkv, D), dtype=np.float32)
    slot_k = rng.standard_normal((n + 1, Hkv, D), dtype=np.float32)
    slot_v = rng.standard_normal((n + 1, Hkv, D), dtype=np.float32)
    keys = O.keylist(t, S, W, r)
    g0 = time.perf_counter()
    ks = np.stack([raw_k[i] if kind == "raw" else slot_k[i] for kind, i in keys], axis=1).astype(np.float64)
    vs = np.stack([raw_v[i] if kind == "raw" else slot_v[i] for kind, i in keys], axis=1).astype(np.float64)
    gather_s = time.perf_counter() - g0
    return dict(ks=ks, vs=vs, raw_k=raw_k, raw_v=raw_v, qs=rng.standard_normal((64, Hq, D)),
                scale=O.default_scale(D), keys=len(keys), gather_s=gather_s)


def _oracle_time(seed, seconds):
    """(units, seconds) of the oracle's gqa_attend on one unit's gathered rows, repeated
    for about `seconds`, BLAS on one thread."""
    from threadpoolctl import threadpool_limits
    from oracle import masw_oracle as O
    smp = _oracle_sample(seed)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < seconds:
            O.gqa_attend(smp["qs"][done % 64], smp["ks"], smp["vs"], smp["scale"])
            done += 1
        return done, time.perf_counter() - t0


def cpu_baseline(seconds=3.0, full_units=2):
    """The fp64 oracle's decode on the host cores, on the same memory shapes.

    Sample: (layer, sequence) units of the 3B-shaped MASW decode at prefix 32768 - one
    query per q head, the oracle's own gqa_attend on key/value rows gathered beforehand
    (the gather is timed separately) - on one core for `seconds`, then on `procs` cores
    at once (one process per core, forked before the GPU is touched, each with its own
    seeded memory, seconds / 2 each).  Scaled to steps/s of the 28-layer, 8-sequence
    step.  The full-KV baseline (32768 keys per unit) is timed on `full_units` units on
    one core and scaled the same way (an extrapolation: ~90 GFLOP per step).
    """
    import multiprocessing
    from threadpoolctl import threadpool_limits
    from oracle import masw_oracle as O
    sh = SHAPE
    units_per_step = sh.layers * sh.batch
    procs = max(1, min(16, len(os.sched_getaffinity(0))))
    single, el1 = _oracle_time(0, seconds)
    with multiprocessing.get_context("fork").Pool(procs) as pool:
        parts = pool.starmap(_oracle_time, [(1 + i, seconds / 2) for i in range(procs)])
    multi = sum(p[0] for p in parts)
    eln = max(p[1] for p in parts)
    smp = _oracle_sample(0)
    kf = smp["raw_k"][1:T_HEAD + 1].transpose(1, 0, 2).astype(np.float64)
    vf = smp["raw_v"][1:T_HEAD + 1].transpose(1, 0, 2).astype(np.float64)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for i in range(full_units):
            O.gqa_attend(smp["qs"][i], kf, vf, smp["scale"])
        elf = time.perf_counter() - t0
    per_step_1 = el1 / single * units_per_step
    per_step_n = eln / multi * units_per_step
    per_step_full = elf / full_units * units_per_step
    return dict(value=round(1.0 / per_step_n, 5), unit="steps/s", cores=procs, kind="oracle",
                sample=f"{multi} (layer, sequence) MASW decode units at prefix {T_HEAD} ({smp['keys']} keys, "
                       f"{sh.n_q_heads} q heads) on {procs} cores in {eln:.1f} s, scaled x{units_per_step} to one "
                       f"28-layer batch-8 step; key/value rows gathered beforehand",
                cpu_model=_cpu_model(), host_cpus=os.cpu_count(),
                single_core=dict(value=round(1.0 / per_step_1, 5), units=single, seconds=round(el1, 2)),
                gather_s_per_unit=round(smp["gather_s"], 4),
                fullkv=dict(value=round(1.0 / per_step_full, 6), unit="steps/s", cores=1, units=full_units,
                            seconds=round(elf, 2), keys=T_HEAD, extrapolated=True,
                            note=f"{full_units} full-KV units timed on one core, scaled x{units_per_step}"))


def profile_modes(args, dev):
    """Runs the dominant kernel alone, at the configuration of kernel_roofline."""
    stack = Stack(SHAPE, T_HEAD + 64, dev, with_full=args.traffic_probe)
    if args.roofline_only:
        roof = kernel_roofline(stack, T_HEAD)
        print(json.dumps({"roofline": roof, "source_sha256": decode_source_hash()}), flush=True)
        return
    counter_probe(stack, dev)


def counter_probe(stack, dev):
    """--traffic-probe: eager launches of every leg's kernels in a fixed order, for
    rocprofv3 --pmc runs (FETCH_SIZE / WRITE_SIZE / matrix-core counters per dispatch).

    Calibration first: 4 launches of a plain elementwise copy over 256 MiB (torch.mul by 1
    into another buffer), whose FETCH_SIZE / WRITE_SIZE give the counters' scale, and 4
    launches of masw_mfma_rate (register-operand MFMA chains) whose matrix-core busy
    counter gives the busy figure of a saturated matrix core.  Then the legs, each a run
    of `launches` dispatches of the kernel named in the printed manifest, in manifest
    order; dispatches of other kernels (fills, input generation) come in between."""
    sh = SHAPE
    L = stack.L
    legs = []
    copy_bytes = 256 << 20
    src = torch.ones(copy_bytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    mfma_wgs, mfma_iters = 256, 20000
    mout = torch.empty(mfma_wgs * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    for _ in range(4):
        M.mfma_rate(mfma_wgs, mfma_iters, mout, clocks)
    torch.cuda.synchronize()
    legs.append(dict(leg="mfma_rate", kernel="mfma_rate", launches=4,
                     flops_per_launch=mfma_wgs * 4 * mfma_iters * 4 * 2 * 32 * 32 * 16))

    # the dominant kernel: fused append + MASW attention, B=8, prefix 32768
    stack.set_position(T_HEAD)
    for i in range(2 * L):
        M.masw_decode_step(stack.d, stack.layers[i % L], stack.seq, stack.k_new[i % L], stack.v_new[i % L],
                           stack.q[i % L], stack.out[i % L], stack.ws)
    torch.cuda.synchronize()
    nbytes = stack.attn_bytes(keys_at(T_HEAD, stack.S, stack.W, stack.r)) + 2 * sh.batch * stack.kv_row_bytes()
    legs.append(dict(leg="masw_decode_b8_t32768", kernel="decode_kernel", launches=2 * L,
                     bytes_per_launch=int(nbytes)))

    # full-KV fused append + attention at the same prefix (default plan)
    stack.seq_full.fill_(T_HEAD)
    for i in range(L):
        M.fullkv_decode_step(stack.fd, stack.kf[i], stack.vf[i], stack.seq_full, stack.err_full,
                             stack.k_new[i], stack.v_new[i], stack.q[i], stack.out[i], stack.ws_full)
    torch.cuda.synchronize()
    legs.append(dict(leg="fullkv_decode_b8_t32768", kernel="decode_kernel", launches=L,
                     bytes_per_launch=int(stack.attn_bytes(T_HEAD) + 2 * sh.batch * stack.kv_row_bytes())))

    # a slot boundary (projection + slot query in one launch) at B=8 and at B=4
    t_b = first_boundary_after(T_HEAD + 64, stack.S, stack.W, stack.r)
    m = (t_b - stack.S - stack.W) // stack.r
    stack.set_position(t_b)
    proj_bytes = 2 * sh.hidden * sh.n_kv_heads * sh.head_dim * 2
    for B in (sh.batch, sh.batch // 2):
        d = dataclasses.replace(stack.d, batch=B)
        ws = M.workspace(d, M.OP_MATERIALIZE, device=dev)
        seq = M.Seq(seq_len=stack.seq.seq_len[:B], err=stack.seq.err)
        for i in range(L):
            lay = stack.layers[i]
            lay.n_slots.fill_(m - 1)
            lb = M.Layer(**{f.name: getattr(lay, f.name)[:B] for f in dataclasses.fields(lay)})
            M.masw_materialize_slot(d, lb, seq, stack.h[i][:B], stack.wk[i], stack.wv[i],
                                    stack.qg[i][:B], stack.og[i][:B], ws)
        torch.cuda.synchronize()
        keys = stack.S + stack.W + m - 1
        legs.append(dict(leg=f"boundary_b{B}_slot{m}", kernel="boundary_kernel", launches=L,
                         bytes_per_launch=int(proj_bytes + B * sh.hidden * 2 + stack.attn_bytes(keys) * B // sh.batch
                                              + B * stack.kv_row_bytes()),
                         flops_per_launch=2 * B * sh.hidden * 2 * sh.n_kv_heads * sh.head_dim,
                         mfma_rows_per_launch=-(-B // 16) * 16))
        del ws
    del stack
    torch.cuda.empty_cache()

    # the batch-1 workload at prefix 8192 (one layer set)
    sh1, t1 = SI.DRAFT_3B, SI.DRAFT_3B_PREFIX
    st = Stack(sh1, t1 + 64, dev, seed=1)
    st.mirror_full_into_masw(t1)
    st.set_position(t1)
    for i in range(st.L):
        M.masw_decode_step(st.d, st.layers[i], st.seq, st.k_new[i], st.v_new[i], st.q[i], st.out[i], st.ws)
    for i in range(st.L):
        M.fullkv_decode_step(st.fd, st.kf[i], st.vf[i], st.seq_full, st.err_full,
                             st.k_new[i], st.v_new[i], st.q[i], st.out[i], st.ws_full)
    torch.cuda.synchronize()
    legs.append(dict(leg="masw_decode_b1_t8192", kernel="decode_kernel", launches=st.L,
                     bytes_per_launch=int(st.attn_bytes(keys_at(t1, st.S, st.W, st.r)) + 2 * st.kv_row_bytes())))
    legs.append(dict(leg="fullkv_decode_b1_t8192", kernel="decode_kernel", launches=st.L,
                     bytes_per_launch=int(st.attn_bytes(t1) + 2 * st.kv_row_bytes())))
    err = int(st.seq.err.item()) | int(st.err_full.item())
    del st
    torch.cuda.empty_cache()

    # verifier layers (8B and 70B shapes, one GPU's 8 KV heads, batch 4, prefix 32768 + 6)
    batch, n_q, t = 4, 6, 32768 + 6
    for Hq in (32, 64):
        vd = M.Dims(batch=batch, n_q_heads=Hq, n_kv_heads=8, head_dim=128, dtype=torch.bfloat16)
        g = torch.Generator(device=dev)
        g.manual_seed(7)
        kv = [torch.randn(batch, 8, t + 8, 128, device=dev, dtype=torch.bfloat16, generator=g) for _ in range(4)]
        vv = [torch.randn(batch, 8, t + 8, 128, device=dev, dtype=torch.bfloat16, generator=g) for _ in range(4)]
        qv = torch.randn(batch, n_q, Hq, 128, device=dev, dtype=torch.bfloat16, generator=g)
        ov = torch.empty_like(qv)
        sv = torch.full((batch,), t, dtype=torch.int32, device=dev)
        ev = torch.zeros(1, dtype=torch.int32, device=dev)
        wsv = M.workspace(vd, M.OP_FULLKV_VERIFY, max_keys=t + 8, n_q=n_q, device=dev)
        for i in range(8):
            M.fullkv_verify_attn(vd, kv[i % 4], vv[i % 4], sv, ev, qv, ov, wsv)
        torch.cuda.synchronize()
        err |= int(ev.item())
        legs.append(dict(leg=f"verify_{Hq}q8kv_b4_t32774", kernel="verify_stream", launches=8,
                         bytes_per_launch=batch * (t * 8 * 128 * 2 * 2 + 2 * n_q * Hq * 128 * 2),
                         flops_per_launch=4 * batch * n_q * Hq * 128 * t))
        del kv, vv
        torch.cuda.empty_cache()
    print(json.dumps({"copy_bytes_per_launch": copy_bytes, "copy_launches": 4, "legs": legs,
                      "source_sha256": decode_source_hash(), "err": err}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--sweep-steps", type=int, default=48)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the dominant-kernel roofline leg (for rocprofv3 --kernel-trace --stats)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the draft prefill leg (for rocprofv3 --kernel-trace --stats)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="eager launches of every leg's kernels after copy and matrix-core "
                         "calibration kernels (for rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the draft path shards by sequence or KV head "
              "without communication, so a multi-GPU figure is not produced", file=sys.stderr)
        sys.exit(2)
    sh = SHAPE
    plain = not (args.roofline_only or args.traffic_probe or args.prefill_only)
    cpu = None
    if plain and not args.no_cpu:
        # first, before anything touches the GPU: the oracle's worker processes are forked
        cpu = cpu_baseline()
        print(f"[bench] cpu baseline {cpu}", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    M.lib()
    if args.roofline_only or args.traffic_probe:
        profile_modes(args, dev)
        return
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_leg(dev), "mfma_reference": mfma_reference_leg(dev)}), flush=True)
        return
    t_max = T_HEAD + args.warmup + args.steps + 8
    if not args.no_sweep:
        t_max = max(t_max, max(SI.SWEEP_PREFIXES) + args.sweep_steps + 40)
    print(f"[bench] allocating 28-layer stack, prefix up to {t_max}", file=sys.stderr, flush=True)
    stack = Stack(sh, t_max, dev)
    stack.capture()
    print("[bench] graphs captured", file=sys.stderr, flush=True)

    # headline: MASW at prefix 32768.  The timed window starts on the first slot boundary
    # after the prefix (the warm-up steps end just before it), so it holds
    # ceil(steps / r) boundary steps: the materialization cost is inside the headline
    # at least at its steady-state rate (exactly, when steps is a multiple of r).
    b0 = first_boundary_after(T_HEAD, sh.sink, sh.window, sh.interval)
    head_start = b0 - 1 - args.warmup
    ms, nbytes, head_q = time_steps(stack, "masw", head_start, args.warmup, args.steps, quantiles=True)
    lo, hi = stack.timed_positions
    n_bound = sum(1 for t in range(lo, hi + 1) if is_boundary(t, sh.sink, sh.window, sh.interval))
    value = 1e3 / ms
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(f"[bench] MASW prefix {T_HEAD}: positions {lo}..{hi} ({n_bound} boundary steps): "
          f"{ms:.3f} ms/step {gbs:.0f} GB/s", file=sys.stderr, flush=True)

    sweep = []
    if not args.no_sweep:
        for t in SI.SWEEP_PREFIXES:
            row = dict(prefix=t, keys_masw=keys_at(t, sh.sink, sh.window, sh.interval), keys_full=t)
            for which in ("masw", "full"):
                m_s, b_s = time_steps(stack, which, t, 4, args.sweep_steps)
                row[f"{which}_ms"] = round(m_s, 4)
                row[f"{which}_steps_per_s"] = round(1e3 / m_s, 2)
                row[f"{which}_gbs"] = round(b_s / (m_s * 1e-3) / 1e9, 1)
                row[f"{which}_pct_peak"] = round(100 * b_s / (m_s * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)
            sweep.append(row)
            print(f"[bench] sweep t={t}: masw {row['masw_ms']} ms ({row['masw_gbs']} GB/s), "
                  f"full {row['full_ms']} ms ({row['full_gbs']} GB/s)", file=sys.stderr, flush=True)

    fits = None
    if sweep:
        fits = {}
        for which in ("masw", "full"):
            a, b, r2 = linear_fit([r[f"keys_{which}"] for r in sweep], [r[f"{which}_ms"] for r in sweep])
            lat = {r["prefix"]: r[f"{which}_ms"] for r in sweep}
            fits[which] = dict(a_ms=round(a, 5), b_us_per_key=round(b * 1e3, 6), r2=round(r2, 4),
                               latency_ratio_32k_over_4k=round(lat[32768] / lat[4096], 3))
        print(f"[bench] eq.3 fits {fits}", file=sys.stderr, flush=True)

    roof = kernel_roofline(stack, T_HEAD)
    print(f"[bench] roofline {roof}", file=sys.stderr, flush=True)
    mat = materialize_leg(stack, 2052 + 480 * 64)
    mat_rope = materialize_leg(stack, 2052 + 480 * 64,
                               dims=dataclasses.replace(stack.d, rope_theta=500000.0, rope_style=M.ROPE_ROTATE_HALF))
    mat["rope_us_per_layer"] = mat_rope["us_per_layer"]
    # trend in the number of prior slots (the slot query's key list grows by one per slot)
    mat["us_per_layer_by_slot"] = {m: materialize_leg(stack, 2052 + m * 64)["us_per_layer"] for m in (1, 128, 256, 480)}
    # the slot-chain workload's own batch of 4 (the first 4 sequences of the stack)
    d4 = dataclasses.replace(stack.d, batch=4)
    ws4 = M.workspace(d4, M.OP_MATERIALIZE, device=dev)
    mat["batch4"] = {m: materialize_leg(stack, 2052 + m * 64, dims=d4, ws=ws4) for m in (1, 480)}
    print(f"[bench] materialization {mat}", file=sys.stderr, flush=True)
    err_bits = int(stack.seq.err.item()) | int(stack.err_full.item())   # every leg on the stack
    del stack
    torch.cuda.empty_cache()
    ver = verify_leg(dev)
    print(f"[bench] verifier {ver}", file=sys.stderr, flush=True)
    single = single_sequence_leg(dev)
    print(f"[bench] batch-1 prefix-8192 {single}", file=sys.stderr, flush=True)
    rb = rollback_leg(dev)
    print(f"[bench] rollback {rb}", file=sys.stderr, flush=True)
    pre = prefill_leg(dev)
    print(f"[bench] prefill {pre}", file=sys.stderr, flush=True)
    second = None if args.no_sweep else second_workload_leg(dev)
    for row in second or ():
        print(f"[bench] second workload {row}", file=sys.stderr, flush=True)
    sread = stream_read_leg(dev, roof["bytes_per_launch"])
    print(f"[bench] streaming read {sread}", file=sys.stderr, flush=True)
    mref = mfma_reference_leg(dev)
    print(f"[bench] matrix-core reference {mref}", file=sys.stderr, flush=True)


    full_head = next((r for r in sweep if r["prefix"] == T_HEAD), None)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "masw_draft_decode_llama3b_28L_b8_prefix32768", "layers": sh.layers,
                   "batch": sh.batch, "prefix": T_HEAD, "q_heads": sh.n_q_heads,
                   "kv_heads": sh.n_kv_heads, "head_dim": sh.head_dim, "sink": sh.sink,
                   "window": sh.window, "interval": sh.interval},
        "ms_per_step_p10_p50_p90": head_q,
        "timed_positions": [lo, hi], "boundary_steps_timed": n_bound,
        "hbm_gbs": round(gbs, 1), "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
        "tokens_per_s": round(value * sh.batch, 1),
        "fullkv_at_prefix": full_head, "sweep": sweep, "eq3_fit": fits, "device_err_bits": err_bits,
        "batch1_prefix8192": single, "second_workloads": second, "rollback": rb, "prefill": pre, "streaming_read": sread, "mfma_reference": mref,
        "materialization": mat, "verifier": ver,
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
