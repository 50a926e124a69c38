"""GPU parity of the MASW decode path through the C ABI against the fp64 oracle.

Covers: the device key resolver (bit-exact), raw append and ring placement (bit-exact),
the tiny fp32 draft layer over a 240-step decode loop crossing slot boundaries, a
Llama-3.2-3B-shaped bf16 layer at edge positions up to t = 8192, the full-KV baseline
(including split plans up to 128 work-groups per sequence and KV head),
bitwise equality MASW == full-KV while t <= S + W, one-hot support, device error bits
and run-to-run determinism.
"""
import dataclasses

import numpy as np
import pytest
import torch

import draft_kv_attention_amd as M
import seeded_inputs as SI
from oracle import masw_oracle as O
from tests.gpu_driver import LayerDriver, np_in, shape_of
from tests.parity import assert_close, assert_slot_close, slot_bound

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.lib()   # fails loudly if the HIP library is missing


def edge_positions(S, W, r):
    return sorted({1, max(1, S), S + 1, S + W - 1, S + W, S + W + 1, S + W + r - 1, S + W + r,
                   S + W + r + 1, S + W + 2 * r, S + W + 2 * r + 1, S + W + 5 * r + 3})


# ---------------------------------------------------------------------------
# key resolver: bit-exact against the oracle's key list and placement
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S,W,r,R", [(4, 32, 16, 0), (0, 5, 2, 0), (3, 4, 4, 0), (2, 6, 1, 0), (7, 8, 5, 0),
                                     (4, 2048, 64, 0), (128, 128, 4, 0), (2, 3, 2, 1), (4, 32, 16, 5),
                                     (0, 5, 2, 3), (4, 2048, 64, 16), (3, 8, 0, 0)])
def test_keylist_bit_exact(S, W, r, R):
    ts = [0] + edge_positions(S, W, max(r, 1)) + [S + W + 37 * max(r, 1) + 11]
    B = len(ts)
    max_slots = O.visible_slot_count(max(ts), S, W, r) + 1
    d = M.Dims(batch=B, n_q_heads=2, n_kv_heads=1, head_dim=64, sink=S, window=W, interval=r,
               max_slots=max_slots, dtype=torch.float32, rollback=R)
    seq = M.alloc_seq(B, DEV)
    seq.seq_len.copy_(torch.tensor(ts, dtype=torch.int32))
    max_keys = S + W + max_slots + 1
    for back in (0, r):
        got = M.masw_debug_keylist(d, seq, back=back, max_keys=max_keys).cpu().numpy()
        for b, t in enumerate(ts):
            tv = t - back
            want = np.array(O.physical_keylist(tv, S, W, r, R) if tv >= 1 else [], dtype=np.int32).reshape(-1, 3)
            n = want.shape[0]
            np.testing.assert_array_equal(got[b, :n], want, err_msg=f"t={t} back={back}")
            assert (got[b, n:] == -1).all()


# ---------------------------------------------------------------------------
# tiny fp32 layer: complete decode loop, prefix 200 then 40 steps
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_tiny_decode_loop(num_splits):
    shape = SI.TINY
    S, W, r = shape.sink, shape.window, shape.interval
    T = SI.TINY_PREFIX + SI.TINY_STEPS
    drv = LayerDriver(shape, max_slots=O.visible_slot_count(T, S, W, r) + 2, seed=1,
                      num_splits=num_splits, copy_init_perturb=0.01)
    worst = 0.0
    boundaries = []
    for t in range(1, T + 1):
        drv.append(1)
        if O.is_boundary(t, S, W, r):
            o, ref = drv.materialize()
            assert ref is not None
            assert_close(o, ref, torch.float32, f"slot query t={t}")
            boundaries.append(t)
        _, out, ref = drv.decode(t)
        s = assert_close(out, ref, torch.float32, f"decode t={t}")
        worst = max(worst, s["max_abs"])
        if t == SI.TINY_PREFIX:
            assert int(drv.layer.n_slots.item()) == 10
    assert [b for b in boundaries if b > SI.TINY_PREFIX] == [212, 228]
    assert drv.err() == 0
    assert int(drv.layer.n_slots.item()) == O.visible_slot_count(T, S, W, r)
    # bookkeeping, bitwise: sink rows, every ring row, every slot row
    ks = drv.layer.k_sink.cpu().numpy()
    for i in range(1, S + 1):
        np.testing.assert_array_equal(ks[0, :, i - 1], drv.tokens_k[i][0])
    ring_k = drv.layer.k_ring.cpu().numpy()
    ring_v = drv.layer.v_ring.cpu().numpy()
    for c, pos in enumerate(O.expected_ring(T, S, W, r)):
        np.testing.assert_array_equal(ring_k[0, :, c], drv.tokens_k[pos][0])
        np.testing.assert_array_equal(ring_v[0, :, c], drv.tokens_v[pos][0])
    slot_k = drv.layer.k_slot.double().cpu().numpy()
    for m, (kg, vg) in drv.mems[0].slots.items():
        np.testing.assert_allclose(slot_k[0, :, m - 1], kg, rtol=1e-5, atol=1e-5)


def test_tiny_include_self():
    shape = SI.TINY
    drv = LayerDriver(shape, max_slots=12, seed=2)
    seen = []

    def on_slot(t, o, ref):
        assert_close(o, ref, torch.float32, f"slot query with self t={t}")
        seen.append(t)

    drv.advance_to(shape.sink + shape.window + 4 * shape.interval, include_self=True, on_slot=on_slot)
    assert len(seen) == 4 and drv.err() == 0


def test_one_hot_support_fp32():
    """V of visible entry j is e_j, every other cell is 0: the output row is the
    probability row, so mass on any excluded or stale cell shows up directly."""
    shape = SI.TINY
    S, W, r, D = shape.sink, shape.window, shape.interval, shape.head_dim
    drv = LayerDriver(shape, max_slots=12, seed=3)
    drv.advance_to(SI.TINY_PREFIX + 7)
    t = drv.t
    keys = O.physical_keylist(t, S, W, r)
    assert len(keys) <= D
    for buf in (drv.layer.v_sink, drv.layer.v_ring, drv.layer.v_slot):
        buf.zero_()
    bufs = {0: drv.layer.v_sink, 1: drv.layer.v_ring, 2: drv.layer.v_slot}
    for j, (seg, row, _) in enumerate(keys):
        bufs[seg][0, 0, row, j] = 1.0
    q, out, _ = drv.decode(9999)
    got = out[0].double().cpu().numpy()
    # oracle probability row over the oracle's own key list and stored keys
    mem = drv.mems[0]
    K, _ = mem.gather(O.keylist(t, S, W, r))
    qn = np_in(q).astype(np.float64)[0]
    for h in range(shape.n_q_heads):
        w = O.softmax_weights(qn[h], K[0], drv.scale)
        np.testing.assert_allclose(got[h, :len(keys)], w, atol=1e-6)
        assert np.abs(got[h, len(keys):]).max() == 0.0
        assert abs(got[h].sum() - 1.0) < 1e-5


# ---------------------------------------------------------------------------
# Llama-3.2-3B-shaped bf16 layer: edge positions up to t = 8192
# ---------------------------------------------------------------------------

def test_3b_layer_bf16_to_8192():
    shape = shape_of(SI.DRAFT_3B, batch=2)
    S, W, r = shape.sink, shape.window, shape.interval
    T = SI.DRAFT_3B_PREFIX
    drv = LayerDriver(shape, max_slots=O.visible_slot_count(T, S, W, r) + 1, seed=4)
    checkpoints = sorted({1, 2, S, S + 1, 1000, S + W - 1, S + W, S + W + 1, S + W + r - 1,
                          S + W + r, S + W + r + 1, S + W + 2 * r, 4096, T - 1, T})
    slot_seen = []

    def on_slot(t, o, ref):
        m = O.is_boundary(t, S, W, r)
        if m in (1, 2, 3, 50, 95):
            assert_close(o, ref, torch.bfloat16, f"slot query m={m}")
            slot_seen.append(m)

    for tc in checkpoints:
        drv.advance_to(tc, on_slot=on_slot)
        _, out, ref = drv.decode(tc)
        assert_close(out, ref, torch.bfloat16, f"decode t={tc}")
    assert slot_seen == [1, 2, 3, 50, 95]
    assert drv.err() == 0
    assert drv.layer.n_slots.cpu().tolist() == [95, 95]
    # stored slot K/V are the bf16 rounding of H W_g: within one bf16 ulp of the oracle's,
    # widened by the fp32 dot-product error bound where the sum cancels
    S, W, r = drv.shape.sink, drv.shape.window, drv.shape.interval
    for which, buf, w in ((0, drv.layer.k_slot, drv.wk_np), (1, drv.layer.v_slot, drv.wv_np)):
        got = buf.double().cpu().numpy()
        for b, mem in enumerate(drv.mems):
            for m in (1, 50, 95):
                ref = mem.slots[m][which]
                h = np_in(SI.slot_inputs(drv.shape, drv.seed, 0, O.boundary_step(m, S, W, r))[0][b])
                assert_slot_close(got[b, :, m - 1], ref, slot_bound(h.astype(np.float64), w, ref.shape[0], ref.shape[1]),
                                  f"slot {'KV'[which]} b={b} m={m}")


# ---------------------------------------------------------------------------
# full-KV baseline, and MASW == full-KV while t <= S + W
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_fullkv_decode(dtype):
    B, Hq, Hkv, D, N = 3, 24, 8, 128, 3000
    ts = [1, 777, N]
    k, v = SI.full_cache(B, Hkv, N, D, seed=5, dtype=dtype)
    q = SI.normal((B, Hq, D), seed=6, dtype=dtype)
    d = M.Dims(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, dtype=dtype)
    seq_len = torch.tensor(ts, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.full((B, Hq, D), float("nan"), dtype=dtype, device=DEV)
    ws = M.workspace(d, M.OP_FULLKV_DECODE, max_keys=N, device=DEV)
    M.fullkv_decode_attn(d, k.to(DEV), v.to(DEV), seq_len, err, q.to(DEV), out, ws)
    kn, vn, qn = np_in(k), np_in(v), np_in(q).astype(np.float64)
    for b, t in enumerate(ts):
        ref = O.fullkv_decode(qn[b], kn[b], vn[b], t, O.default_scale(D))
        assert_close(out[b], ref, dtype, f"full-KV b={b} t={t}")
    assert int(err.item()) == 0


@pytest.mark.parametrize("splits", [9, 16, 40, 128, 256])
@pytest.mark.parametrize("G,D,dtype", [(8, 128, torch.bfloat16), (3, 64, torch.float32), (1, 128, torch.bfloat16)])
def test_fullkv_decode_many_splits(splits, G, D, dtype):
    """Split plans whose last work-group folds more than one batch of eight partials (up to
    the largest plan, 256, where only the first 188 / 136 work-groups hold keys), and
    group sizes where a thread of the merge takes more than one output pair (G = 8)."""
    B, Hkv, N = 2, 2, 6000
    Hq = G * Hkv
    ts = [N, 4321]
    k, v = SI.full_cache(B, Hkv, N, D, seed=15, dtype=dtype)
    q = SI.normal((B, Hq, D), seed=16, dtype=dtype)
    d = M.Dims(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, dtype=dtype, num_splits=splits)
    seq_len = torch.tensor(ts, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.full((B, Hq, D), float("nan"), dtype=dtype, device=DEV)
    ws = M.workspace(d, M.OP_FULLKV_DECODE, max_keys=N, device=DEV)
    kd, vd, qd = k.to(DEV), v.to(DEV), q.to(DEV)
    M.fullkv_decode_attn(d, kd, vd, seq_len, err, qd, out, ws)
    kn, vn, qn = np_in(k), np_in(v), np_in(q).astype(np.float64)
    for b, t in enumerate(ts):
        ref = O.fullkv_decode(qn[b], kn[b], vn[b], t, O.default_scale(D))
        assert_close(out[b], ref, dtype, f"full-KV b={b} t={t} splits={splits}")
    assert int(err.item()) == 0
    # the tickets are back at zero: a second call gives the same bits
    out2 = torch.full_like(out, float("nan"))
    M.fullkv_decode_attn(d, kd, vd, seq_len, err, qd, out2, ws)
    assert torch.equal(out, out2)


@pytest.mark.parametrize("splits", [1, 4, 7])
def test_masw_equals_fullkv_bitwise_before_first_slot(splits):
    """While t <= S + W the memory is the whole prefix in the same order, so with the
    same split plan both paths reduce identically."""
    shape = shape_of(SI.DRAFT_3B, batch=2)
    S, W, r = shape.sink, shape.window, shape.interval
    Hq, Hkv, D = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    for t in (1, S, S + 1, 1500, S + W):
        drv = LayerDriver(shape, max_slots=4, seed=7, num_splits=splits, oracle=False)
        drv.append(t)
        q, out_m, _ = drv.decode(t)
        full_k = torch.zeros((2, Hkv, S + W, D), dtype=shape.dtype, device=DEV)
        full_v = torch.zeros_like(full_k)
        for i in range(1, t + 1):
            full_k[:, :, i - 1] = torch.from_numpy(drv.tokens_k[i]).to(shape.dtype).to(DEV)
            full_v[:, :, i - 1] = torch.from_numpy(drv.tokens_v[i]).to(shape.dtype).to(DEV)
        d = dataclasses.replace(drv.d)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        out_f = torch.full_like(out_m, float("nan"))
        ws = M.workspace(d, M.OP_FULLKV_DECODE, max_keys=S + W, device=DEV)
        M.fullkv_decode_attn(d, full_k, full_v, drv.seq.seq_len, err, q.to(DEV), out_f, ws)
        assert torch.equal(out_m, out_f), f"t={t} splits={splits}"


# ---------------------------------------------------------------------------
# device error bits and suppressed writes
# ---------------------------------------------------------------------------

def test_pending_slot_blocks_append():
    shape = SI.TINY
    S, W, r = shape.sink, shape.window, shape.interval
    drv = LayerDriver(shape, max_slots=4, seed=8, oracle=False)
    drv.append(S + W + r)             # reach the first boundary without materializing
    c = O.ring_cell(S + W + r + 1, S, W, r)
    before = drv.layer.k_ring[0, 0, c].clone()
    drv.append(1)                     # would evict block 1, whose slot is missing
    assert drv.err() & M.DEV_PENDING_SLOT
    assert torch.equal(drv.layer.k_ring[0, 0, c], before)


def test_missing_slot_suppresses_decode():
    shape = SI.TINY
    S, W, r = shape.sink, shape.window, shape.interval
    drv = LayerDriver(shape, max_slots=4, seed=9, oracle=False)
    drv.append(S + W + r)
    _, out, _ = drv.decode(1, out_fill=7.0)
    assert drv.err() & M.DEV_SLOT_MISSING
    assert bool((out == 7.0).all())


def test_slot_capacity():
    shape = SI.TINY
    S, W, r = shape.sink, shape.window, shape.interval
    drv = LayerDriver(shape, max_slots=1, seed=10, oracle=False)
    drv.advance_to(S + W + 2 * r)
    assert drv.err() & M.DEV_SLOT_CAPACITY
    assert int(drv.layer.n_slots.item()) == 1


def test_seq_range_and_host_errors():
    shape = SI.TINY
    drv = LayerDriver(shape, max_slots=2, seed=11, oracle=False)
    drv.seq.seq_len.fill_(0)
    _, out, _ = drv.decode(1, out_fill=3.0)
    assert drv.err() & M.DEV_SEQ_RANGE and bool((out == 3.0).all())
    drv.seq.err.zero_()
    k = torch.zeros((1, 2, 1, 64), device=DEV)
    M.masw_evict_append(drv.d, drv.layer, drv.seq, k, k)    # t = 0 < n_new = 2
    assert drv.err() & M.DEV_SEQ_RANGE
    # same ring size W + r, but r > W: rejected on the host
    bad = dataclasses.replace(drv.d, window=drv.d.interval, interval=drv.d.window)
    with pytest.raises(M.MaswError) as e:
        M.masw_draft_attn(bad, drv.layer, drv.seq, torch.zeros((1, 2, 64), device=DEV),
                          torch.zeros((1, 2, 64), device=DEV), drv.ws)
    assert e.value.status == -1
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(M.MaswError) as e:
        M.masw_materialize_slot(drv.d, drv.layer, drv.seq, torch.zeros((1, 64), device=DEV),
                                drv.wk, drv.wv, torch.zeros((1, 2, 64), device=DEV),
                                torch.zeros((1, 2, 64), device=DEV), small)
    assert e.value.status == -4


def test_determinism_bitwise():
    shape = shape_of(SI.DRAFT_3B, batch=2)
    drv = LayerDriver(shape, max_slots=40, seed=12, oracle=False)
    drv.advance_to(4000)
    q = SI.decode_query(shape, 12, 0, 1).to(DEV)
    outs = []
    for _ in range(3):
        o = torch.empty_like(q)
        M.masw_draft_attn(drv.d, drv.layer, drv.seq, q, o, drv.ws)
        outs.append(o)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
