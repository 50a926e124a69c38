"""GPU parity of the rotary embedding of slot keys with the oracle (reading R11:
[TR] §3.2 Algorithm 1 step 6 gives g_m the position id of the raw token right after its
block, S + m*r with 0-based ids; RoFormer's rotation with rotate-half or interleaved
pairs, applied to K_g before the cache rounds it, never to V_g).

Cases: the tiny fp32 layer (D = 64, projection on the vector ALUs) through 12
boundaries with decode steps in between, both pairings; a 3B-shaped bf16 layer (D = 128,
matrix-core projection with hidden splits) through 10 boundaries, both pairings; a single
boundary at slot 500 (id 32004, angles up to 3.2e4 rad); theta = 0 equal bit for bit to
the memory without rotation.  Outputs: fp32 1e-5 / bf16 tolerance of tests/parity.py.
Stored slot K: fp32 within 1e-5; bf16 within one bf16 ulp plus the fp32 dot bound of both
pair components and the fp32 rounding of the turn.
"""
import dataclasses

import numpy as np
import pytest
import torch

import draft_kv_attention_amd as M
import seeded_inputs as SI
from oracle import masw_oracle as O
from tests.gpu_driver import LayerDriver, np_in
from tests.parity import assert_close, assert_slot_close, bf16_ulp, rotated_slot_bound, slot_bound

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.lib()


def _check_slot_rows(drv, m, tol_fp32=1e-5):
    """Stored K/V of slot m against the oracle memories (which hold the rotated K_g)."""
    got_k = drv.layer.k_slot[:, :, m - 1].double().cpu().numpy()
    got_v = drv.layer.v_slot[:, :, m - 1].double().cpu().numpy()
    ref_k = np.stack([mem.slots[m][0] for mem in drv.mems])
    ref_v = np.stack([mem.slots[m][1] for mem in drv.mems])
    if not drv.bf16:
        np.testing.assert_allclose(got_k, ref_k, atol=tol_fp32)
        np.testing.assert_allclose(got_v, ref_v, atol=tol_fp32)
        return
    h, _ = SI.slot_inputs(drv.shape, drv.seed, 0, O.boundary_step(m, drv.shape.sink, drv.shape.window, drv.shape.interval))
    hn = np_in(h).astype(np.float64)
    style = drv.d.rope_style
    kb = rotated_slot_bound(hn, drv.wk_np, drv.d.n_kv_heads, drv.d.head_dim, style, ref_k)
    assert_slot_close(got_k, ref_k, kb, f"rotated slot K m={m}")
    vb = slot_bound(hn, drv.wv_np, drv.d.n_kv_heads, drv.d.head_dim)
    assert_slot_close(got_v, ref_v, vb, f"slot V m={m}")


def _run_chain(shape, max_slots, t_end, style, theta, seed):
    drv = LayerDriver(shape, max_slots=max_slots, seed=seed, rope_theta=theta, rope_style=style)
    print(f"rope chain: {shape.name} style={style} theta={theta} t_end={t_end}", flush=True)
    seen = []

    def on_slot(t, o, ref):
        m = O.is_boundary(t, shape.sink, shape.window, shape.interval)
        assert_close(o, ref, shape.dtype, f"slot query m={m}")
        _check_slot_rows(drv, m)
        seen.append(m)

    S, W, r = shape.sink, shape.window, shape.interval
    step = 0
    while drv.t < t_end:
        drv.advance_to(min(t_end, drv.t + r // 2 + 1), on_slot=on_slot)
        _, out, ref = drv.decode(step_key=drv.t)
        assert_close(out, ref, shape.dtype, f"decode t={drv.t}")
        step += 1
    assert drv.err() == 0
    return drv, seen


@pytest.mark.parametrize("style", [0, 1])
def test_rope_tiny_fp32_chain(style):
    sh = SI.TINY
    drv, seen = _run_chain(sh, max_slots=16, t_end=36 + 12 * 16 + 5, style=style, theta=10000.0, seed=7)
    assert seen == list(range(1, 13))


@pytest.mark.parametrize("style", [0, 1])
def test_rope_bf16_3b_chain(style):
    sh = dataclasses.replace(SI.MATERIALIZE_3B, name="rope3b", batch=2, window=256)
    drv, seen = _run_chain(sh, max_slots=12, t_end=4 + 256 + 10 * 64 + 3, style=style, theta=500000.0, seed=8)
    assert seen == list(range(1, 11))


@pytest.mark.parametrize("style", [0, 1])
def test_rope_large_position_id(style):
    """Slot 500 of the 3B geometry (S=4, W=2048, r=64): id 32004.  The earlier slots are
    taken as present (zero rows), so only the projection of slot 500 is compared."""
    sh = dataclasses.replace(SI.MATERIALIZE_3B, name="rope3b_far", batch=2)
    S, W, r = sh.sink, sh.window, sh.interval
    m = 500
    d = M.Dims(batch=2, n_q_heads=sh.n_q_heads, n_kv_heads=sh.n_kv_heads, head_dim=sh.head_dim, sink=S, window=W,
               interval=r, max_slots=m, dtype=sh.dtype, rope_theta=500000.0, rope_style=style)
    layer = M.alloc_layer(d, DEV, fill=0.0)
    layer.n_slots.fill_(m - 1)
    seq = M.alloc_seq(2, DEV)
    seq.seq_len.fill_(O.boundary_step(m, S, W, r))
    ws = M.workspace(d, M.OP_MATERIALIZE, device=DEV)
    wk, wv = SI.mirrored_weights(sh, 9)
    h, qg = SI.slot_inputs(sh, 9, 0, m)
    o = torch.empty((2, sh.n_q_heads, sh.head_dim), dtype=sh.dtype, device=DEV)
    M.masw_materialize_slot(d, layer, seq, h.to(DEV), wk.to(DEV), wv.to(DEV), qg.to(DEV), o, ws)
    torch.cuda.synchronize()
    assert int(seq.err.item()) == 0 and layer.n_slots.cpu().tolist() == [m, m]
    hn = np_in(h).astype(np.float64)
    wkn, wvn = np_in(wk).astype(np.float64), np_in(wv).astype(np.float64)
    kg, vg = O.project_slot(hn, wkn, wvn, sh.n_kv_heads, sh.head_dim, True, (500000.0, style),
                            O.slot_position_id(m, S, r))
    got_k = layer.k_slot[:, :, m - 1].double().cpu().numpy()
    got_v = layer.v_slot[:, :, m - 1].double().cpu().numpy()
    kb = rotated_slot_bound(hn, wkn, sh.n_kv_heads, sh.head_dim, style, kg)
    assert_slot_close(got_k, kg, kb, "rotated slot K")
    assert_slot_close(got_v, vg, slot_bound(hn, wvn, sh.n_kv_heads, sh.head_dim), "slot V")
    # the rotation matters at this id: the unrotated key is far off
    k0, _ = O.project_slot(hn, wkn, wvn, sh.n_kv_heads, sh.head_dim, True)
    assert np.abs(got_k - k0).max() > 10 * np.abs(got_k - kg).max()


def test_rope_theta_zero_is_no_rotation():
    """theta = 0 leaves the layer bit for bit as a memory without rotation."""
    sh = dataclasses.replace(SI.MATERIALIZE_3B, name="rope_off", batch=2, window=256)
    a = LayerDriver(sh, max_slots=4, seed=10, oracle=False)
    b = LayerDriver(sh, max_slots=4, seed=10, oracle=False, rope_theta=0.0, rope_style=1)
    for drv in (a, b):
        drv.advance_to(4 + 256 + 3 * 64 + 1)
    torch.cuda.synchronize()
    for name in ("k_slot", "v_slot", "k_ring", "v_ring"):
        assert torch.equal(getattr(a.layer, name).view(torch.int16), getattr(b.layer, name).view(torch.int16)), name
