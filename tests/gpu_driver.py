"""Drive one MASW layer through the C ABI and the fp64 oracle side by side.

Both sides consume the same seeded tensors (seeded_inputs); the HIP side gets device
copies, the oracle gets the stored values as numpy arrays.  Nothing flows from the HIP
side into the oracle.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import draft_kv_attention_amd as M
import seeded_inputs as SI
from oracle import masw_oracle as O


def np_in(t: torch.Tensor) -> np.ndarray:
    """Stored input values as a CPU array (fp32 holds bf16 and fp32 inputs exactly)."""
    return t.detach().to("cpu", torch.float32).numpy()


class LayerDriver:
    """One draft layer: device memory + per-sequence oracle memories, same token stream."""

    def __init__(self, shape: SI.DraftShape, max_slots: int, seed: int = 0, device="cuda",
                 num_splits: int = 0, oracle: bool = True, fill: float = float("nan"),
                 copy_init_perturb=None, rope_theta: float = 0.0, rope_style: int = 0):
        self.shape = shape
        self.seed = seed
        self.dev = torch.device(device)
        self.d = M.Dims(batch=shape.batch, n_q_heads=shape.n_q_heads, n_kv_heads=shape.n_kv_heads,
                        head_dim=shape.head_dim, sink=shape.sink, window=shape.window,
                        interval=shape.interval, max_slots=max_slots, dtype=shape.dtype,
                        num_splits=num_splits, rope_theta=rope_theta, rope_style=rope_style)
        # unused cells start as NaN: reading a dead cell would poison the output
        self.layer = M.alloc_layer(self.d, self.dev, fill=fill)
        self.layer.n_slots.zero_()
        self.seq = M.alloc_seq(shape.batch, self.dev)
        self.ws = M.workspace(self.d, M.OP_MATERIALIZE, device=self.dev)
        wk, wv = SI.mirrored_weights(shape, seed, copy_init_perturb=copy_init_perturb)
        self.wk, self.wv = wk.to(self.dev), wv.to(self.dev)
        self.wk_np, self.wv_np = np_in(wk).astype(np.float64), np_in(wv).astype(np.float64)
        self.bf16 = shape.dtype == torch.bfloat16
        self.mems = ([O.DraftMemory(shape.sink, shape.window, shape.interval, shape.n_kv_heads,
                                    shape.head_dim, self.bf16, rope_theta, rope_style)
                      for _ in range(shape.batch)]
                     if oracle else None)
        self.t = 0
        self.tokens_k = {}   # position -> [B][Hkv][D] stored values (for buffer checks)
        self.tokens_v = {}
        self.slot_checks = []

    @property
    def scale(self) -> float:
        return self.d.softmax_scale

    def append(self, n: int):
        k, v = SI.token_kv(self.shape, self.seed, 0, self.t + 1, n)
        self.seq.seq_len.fill_(self.t + n)
        M.masw_evict_append(self.d, self.layer, self.seq, k.to(self.dev), v.to(self.dev))
        kn, vn = np_in(k), np_in(v)
        for j in range(n):
            self.tokens_k[self.t + 1 + j] = kn[:, j]
            self.tokens_v[self.t + 1 + j] = vn[:, j]
        if self.mems is not None:
            for b, mem in enumerate(self.mems):
                mem.append(kn[b], vn[b])
        self.t += n

    def materialize(self, include_self: bool = False, check: bool = True):
        """Call materialize (a device no-op off boundaries); returns (gpu o_g, oracle o_g)."""
        h, qg = SI.slot_inputs(self.shape, self.seed, 0, self.t)
        o = torch.full((self.d.batch, self.d.n_q_heads, self.d.head_dim), float("nan"),
                       dtype=self.d.dtype, device=self.dev)
        M.masw_materialize_slot(self.d, self.layer, self.seq, h.to(self.dev), self.wk, self.wv,
                                qg.to(self.dev), o, self.ws, include_self=include_self)
        ref = None
        if self.mems is not None and check:
            hn, qn = np_in(h).astype(np.float64), np_in(qg).astype(np.float64)
            outs = [mem.materialize(hn[b], self.wk_np, self.wv_np, qn[b], self.scale, include_self)
                    for b, mem in enumerate(self.mems)]
            if outs[0] is not None:
                ref = np.stack(outs)
        return o, ref

    def advance_to(self, t_target: int, include_self: bool = False, on_slot=None):
        """Append up to t_target, materializing at every boundary on the way."""
        S, W, r = self.shape.sink, self.shape.window, self.shape.interval
        if r == 0:                       # no slot chain: nothing to materialize
            if self.t < t_target:
                self.append(t_target - self.t)
            return
        while self.t < t_target:
            if self.t < S + W:
                nxt = S + W + r
            else:
                nxt = self.t + (r - (self.t - S - W) % r)
            self.append(min(nxt, t_target) - self.t)
            if O.is_boundary(self.t, S, W, r):
                o, ref = self.materialize(include_self)
                if on_slot is not None:
                    on_slot(self.t, o, ref)

    def decode(self, step_key: int, out_fill=float("nan")):
        q = SI.decode_query(self.shape, self.seed, 0, step_key)
        out = torch.full((self.d.batch, self.d.n_q_heads, self.d.head_dim), out_fill,
                         dtype=self.d.dtype, device=self.dev)
        M.masw_draft_attn(self.d, self.layer, self.seq, q.to(self.dev), out, self.ws)
        ref = None
        if self.mems is not None:
            qn = np_in(q).astype(np.float64)
            ref = np.stack([mem.decode(qn[b], self.scale) for b, mem in enumerate(self.mems)])
        return q, out, ref

    def err(self) -> int:
        return int(self.seq.err.item())


def shape_of(base: SI.DraftShape, **kw) -> SI.DraftShape:
    return dataclasses.replace(base, **kw)
