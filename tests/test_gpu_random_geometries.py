"""Seeded random geometries through the C ABI against the oracle: group sizes 1-8,
head dims 64 and 128, fp32 and bf16 caches, 0-8 sinks, windows 4-96, slot intervals
0..W, batches 1-3, split plans 1-5, rollback rows and rotated slot keys.  Each case
runs a decode loop across several boundaries (materializing at each), compares every
slot query and decode with the oracle, and for cases with rollback rows undoes a
speculative run of appends and decodes again.  The configurations are drawn once from
a fixed seed; each is printed before it runs."""
import dataclasses
import random

import numpy as np
import pytest
import torch

import draft_kv_attention_amd as M
import seeded_inputs as SI
from oracle import masw_oracle as O
from tests.gpu_driver import LayerDriver
from tests.parity import assert_close

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.lib()


def _configs(n=40, seed=2024):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        G = rng.choice([1, 2, 3, 4, 6, 8])
        Hkv = rng.choice([1, 2])
        dtype = rng.choice([torch.float32, torch.bfloat16])
        D = rng.choice([64, 128])
        S = rng.choice([0, 1, 4, 8])
        W = rng.randint(4, 96)
        r = rng.choice([0, 1, rng.randint(1, W), W])
        B = rng.randint(1, 3)
        splits = rng.randint(1, 5)
        R = rng.choice([0, 0, 3, 9])
        rope = (rng.choice([0.0, 10000.0]), rng.choice([0, 1]))
        out.append(dict(i=i, G=G, Hkv=Hkv, dtype=dtype, D=D, S=S, W=W, r=r, B=B, splits=splits, R=R, rope=rope))
    return out


@pytest.mark.parametrize("cfg", _configs(), ids=lambda c: f"cfg{c['i']}")
def test_random_geometry_decode_loop(cfg):
    print("random geometry:", cfg, flush=True)
    c = cfg
    shape = dataclasses.replace(SI.TINY, name=f"rand{c['i']}", n_q_heads=c["G"] * c["Hkv"], n_kv_heads=c["Hkv"],
                                head_dim=c["D"], hidden=64, sink=c["S"], window=c["W"], interval=c["r"],
                                batch=c["B"], dtype=c["dtype"])
    S, W, r = c["S"], c["W"], c["r"]
    T = S + W + (5 * r if r else 2 * W) + 3
    drv = LayerDriver(shape, max_slots=O.visible_slot_count(T + 20, S, W, r) + 1, seed=100 + c["i"],
                      num_splits=c["splits"], rope_theta=c["rope"][0], rope_style=c["rope"][1])
    if c["R"]:
        # the rollback rows are part of the ring: rebuild the layer with them
        drv.d.rollback = c["R"]
        drv.layer = M.alloc_layer(drv.d, drv.dev, fill=float("nan"))
        drv.layer.n_slots.zero_()

    def on_slot(t, o, ref):
        assert_close(o, ref, shape.dtype, f"slot query t={t}")

    step = max(1, (r or W) // 2 + 1)
    while drv.t < T:
        drv.advance_to(min(T, drv.t + step), on_slot=on_slot)
        _, out, ref = drv.decode(step_key=drv.t)
        assert_close(out, ref, shape.dtype, f"decode t={drv.t}")
    assert drv.err() == 0
    if c["R"]:
        # speculate R - 1 tokens past an accepted point, then roll back and decode there
        t_acc = drv.t
        drv.advance_to(t_acc + c["R"] - 1, on_slot=on_slot)
        t_spec = torch.full((c["B"],), drv.t, dtype=torch.int32, device=drv.dev)
        drv.seq.seq_len.fill_(t_acc)
        M.masw_rollback(drv.d, drv.layer, drv.seq, t_spec)
        for mem in drv.mems:
            mem.rollback(t_acc)
        drv.t = t_acc
        _, out, ref = drv.decode(step_key=t_acc + 1000)
        assert_close(out, ref, shape.dtype, f"decode after rollback to t={t_acc}")
        assert drv.err() == 0
