"""Edge geometries and value distributions through the C ABI against the oracle:
no sinks (sliding window plus slots), one slot per token (r = 1), r = W, a large sink
block, ragged batches, peaky logits, all-zero values, large-magnitude keys, and bf16
and fp32 caches."""
import dataclasses

import numpy as np
import pytest
import torch

import draft_kv_attention_amd as M
import seeded_inputs as SI
from oracle import masw_oracle as O
from tests.gpu_driver import LayerDriver, np_in
from tests.parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.lib()


GEOMS = [(0, 32, 16), (4, 32, 1), (4, 32, 32), (40, 8, 4), (2, 64, 7)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("S,W,r", GEOMS)
def test_geometries_along_a_decode_loop(S, W, r, dtype):
    shape = dataclasses.replace(SI.TINY, sink=S, window=W, interval=r, dtype=dtype, batch=3,
                                n_q_heads=6, n_kv_heads=2, head_dim=128 if dtype == torch.bfloat16 else 64,
                                hidden=128 if dtype == torch.bfloat16 else 64)
    T = S + W + 6 * r + 5
    drv = LayerDriver(shape, max_slots=O.visible_slot_count(T, S, W, r) + 1, seed=61, num_splits=3)
    pts = sorted({1, max(1, S), S + 1, S + W, S + W + 1, S + W + r, S + W + r + 1, T})
    for tc in pts:
        drv.advance_to(tc, on_slot=lambda t, o, ref: assert_close(o, ref, dtype, f"slot t={t}"))
        _, out, ref = drv.decode(tc)
        assert_close(out, ref, dtype, f"decode t={tc} S={S} W={W} r={r}")
    assert drv.err() == 0


@pytest.mark.parametrize("case", ["peaky", "zero_v", "big_keys"])
def test_value_distributions_bf16(case):
    shape = dataclasses.replace(SI.DRAFT_3B, batch=2)
    drv = LayerDriver(shape, max_slots=20, seed=62, oracle=True)
    drv.advance_to(3000)
    if case == "zero_v":
        for buf in (drv.layer.v_sink, drv.layer.v_ring, drv.layer.v_slot):
            buf.zero_()
        for mem in drv.mems:
            for i in list(mem.raw):
                mem.raw[i] = (mem.raw[i][0], np.zeros_like(mem.raw[i][1]))
            for m in list(mem.slots):
                mem.slots[m] = (mem.slots[m][0], np.zeros_like(mem.slots[m][1]))
    if case == "big_keys":
        for buf in (drv.layer.k_sink, drv.layer.k_ring, drv.layer.k_slot):
            buf.mul_(64.0)                     # exact in bf16: a power of two
        for mem in drv.mems:
            for i in list(mem.raw):
                mem.raw[i] = (mem.raw[i][0] * 64.0, mem.raw[i][1])
            for m in list(mem.slots):
                mem.slots[m] = (mem.slots[m][0] * 64.0, mem.slots[m][1])
    q = SI.decode_query(shape, 62, 0, 1)
    if case == "peaky":
        q = (q.float() * 8).to(shape.dtype)
    out = torch.full((2, shape.n_q_heads, shape.head_dim), float("nan"), dtype=shape.dtype, device=DEV)
    M.masw_draft_attn(drv.d, drv.layer, drv.seq, q.to(DEV), out, drv.ws)
    qn = np_in(q).astype(np.float64)
    ref = np.stack([mem.decode(qn[b], drv.scale) for b, mem in enumerate(drv.mems)])
    if case == "zero_v":
        assert bool((out == 0).all())
    else:
        assert_close(out, ref, torch.bfloat16, case)


def test_ragged_batch_different_positions():
    """Sequences at different t in one call: each gets its own key list."""
    shape = dataclasses.replace(SI.DRAFT_3B, batch=1)
    drvs = [LayerDriver(shape, max_slots=40, seed=70 + i) for i in range(3)]
    ts = [5, 2052, 4000]
    for drv, t in zip(drvs, ts):
        drv.advance_to(t)
    d = dataclasses.replace(drvs[0].d, batch=3)
    cat = lambda name: torch.cat([getattr(x.layer, name) for x in drvs])
    layer = M.Layer(*(cat(n) for n in ("k_sink", "v_sink", "k_ring", "v_ring", "k_slot", "v_slot", "n_slots")))
    seq = M.alloc_seq(3, DEV)
    seq.seq_len.copy_(torch.tensor(ts, dtype=torch.int32))
    q = torch.cat([SI.decode_query(shape, 70 + i, 0, 9) for i in range(3)])
    out = torch.empty((3, shape.n_q_heads, shape.head_dim), dtype=shape.dtype, device=DEV)
    M.masw_draft_attn(d, layer, seq, q.to(DEV), out, M.workspace(d, M.OP_DRAFT_ATTN, device=DEV))
    qn = np_in(q).astype(np.float64)
    for i, drv in enumerate(drvs):
        assert_close(out[i], drv.mems[0].decode(qn[i], drv.scale), torch.bfloat16, f"seq {i} t={ts[i]}")
    assert int(seq.err.item()) == 0
