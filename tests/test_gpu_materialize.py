"""GPU parity of slot materialization along the 512-boundary chain at 3B shapes, and of
the draft attention at the bench's full size and launch configuration (sampled rows).

The chain: batch 4, S=4, W=2048, r=64, one layer; 64 seeded raw tokens appended between
boundaries, the slot hidden state projected through seeded mirrored weights
(3072x1024 bf16 ~ N(0, 0.02)) at every boundary, m = 1..512 (final t = 34820).  The
oracle projects every slot; the slot query and the stored K/V are compared at
m in {1, 2, 64, 256, 512} (0, 1, 63, 255 and 511 prior slots), the decode at the end.
Stored slot K/V: within one bf16 ulp of the oracle's rounded fp64 value, widened by the
fp32 dot-product error bound n 2^-24 sum |h w| (it matters only where the sum cancels).
"""
import numpy as np
import pytest
import torch

import draft_kv_attention_amd as M
import seeded_inputs as SI
from oracle import masw_oracle as O
from tests.gpu_driver import np_in
from tests.parity import assert_close, assert_slot_close, slot_bound

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.lib()


def test_materialize_chain_3b_to_512_slots():
    sh = SI.MATERIALIZE_3B
    S, W, r, B, Hkv, D, hidden = sh.sink, sh.window, sh.interval, sh.batch, sh.n_kv_heads, sh.head_dim, sh.hidden
    n_chain = SI.MATERIALIZE_CHAIN
    d = M.Dims(batch=B, n_q_heads=sh.n_q_heads, n_kv_heads=Hkv, head_dim=D, sink=S, window=W, interval=r,
               max_slots=n_chain, dtype=sh.dtype)
    layer = M.alloc_layer(d, DEV, fill=float("nan"))
    layer.n_slots.zero_()
    seq = M.alloc_seq(B, DEV)
    ws = M.workspace(d, M.OP_MATERIALIZE, device=DEV)
    wk, wv = SI.mirrored_weights(sh, 51)
    wk_d, wv_d = wk.to(DEV), wv.to(DEV)
    wk_n, wv_n = np_in(wk).astype(np.float64), np_in(wv).astype(np.float64)
    mems = [O.DraftMemory(S, W, r, Hkv, D, bf16_cache=True) for _ in range(B)]
    check = {1, 2, 64, 256, 512}
    t = 0
    for m in range(1, n_chain + 1):
        tm = O.boundary_step(m, S, W, r)
        n = tm - t
        k, v = SI.token_kv(sh, 51, 0, t + 1, n)
        t = tm
        seq.seq_len.fill_(t)
        M.masw_evict_append(d, layer, seq, k.to(DEV), v.to(DEV))
        kn, vn = np_in(k), np_in(v)
        for b, mem in enumerate(mems):
            mem.append(kn[b], vn[b])
        h, qg = SI.slot_inputs(sh, 51, 0, m)
        o = torch.full((B, sh.n_q_heads, D), float("nan"), dtype=sh.dtype, device=DEV)
        M.masw_materialize_slot(d, layer, seq, h.to(DEV), wk_d, wv_d, qg.to(DEV), o, ws)
        kg, vg = O.project_slot(np_in(h).astype(np.float64), wk_n, wv_n, Hkv, D, bf16_cache=True)
        for b, mem in enumerate(mems):
            assert mem.pending_boundary() == m
            mem.add_slot(m, kg[b], vg[b])
        if m in check:
            qn = np_in(qg).astype(np.float64)
            ref = np.stack([mem.slot_query(m, qn[b], d.softmax_scale) for b, mem in enumerate(mems)])
            assert_close(o, ref, torch.bfloat16, f"slot query m={m}")
            got_k = layer.k_slot[:, :, m - 1].double().cpu().numpy()
            got_v = layer.v_slot[:, :, m - 1].double().cpu().numpy()
            hn = np_in(h).astype(np.float64)
            assert_slot_close(got_k, kg, slot_bound(hn, wk_n, Hkv, D), f"slot K m={m}")
            assert_slot_close(got_v, vg, slot_bound(hn, wv_n, Hkv, D), f"slot V m={m}")
            # the slot query saw exactly S + W + (m - 1) keys
            assert len(O.slot_query_keylist(m, S, W, r)) == S + W + m - 1
    torch.cuda.synchronize()
    assert int(seq.err.item()) == 0
    assert layer.n_slots.cpu().tolist() == [n_chain] * B
    q = SI.decode_query(sh, 51, 0, t)
    out = torch.empty((B, sh.n_q_heads, D), dtype=sh.dtype, device=DEV)
    M.masw_draft_attn(d, layer, seq, q.to(DEV), out, ws)
    qn = np_in(q).astype(np.float64)
    ref = np.stack([mem.decode(qn[b], d.softmax_scale) for b, mem in enumerate(mems)])
    assert_close(out, ref, torch.bfloat16, "decode after the chain")


def test_bench_launch_configuration_sampled_rows():
    """B=8, prefix 32768, the bench's split plan: sampled (sequence, head) rows of the
    fused append + draft attention against the oracle over the same memory contents."""
    import bench
    sh = SI.SWEEP_3B
    import dataclasses
    shape = dataclasses.replace(sh, layers=2)
    t0 = bench.T_HEAD
    st = bench.Stack(shape, t0 + 64, torch.device(DEV), seed=3, with_full=False)
    st.set_position(t0)
    st.seq.seq_len.fill_(t0 + 1)     # the fused step appends position t0 + 1
    lay = st.layers[1]
    snap = {n: getattr(lay, n).float().cpu().numpy() for n in ("k_sink", "v_sink", "k_ring", "v_ring", "k_slot", "v_slot")}
    M.masw_decode_step(st.d, lay, st.seq, st.k_new[1], st.v_new[1], st.q[1], st.out[1], st.ws)
    torch.cuda.synchronize()
    assert int(st.seq.err.item()) == 0
    S, W, r = sh.sink, sh.window, sh.interval
    t = t0 + 1
    keys = O.physical_keylist(t, S, W, r)
    kn, vn = np_in(st.k_new[1]), np_in(st.v_new[1])
    q = np_in(st.q[1]).astype(np.float64)
    G = sh.group
    got_all, ref_all = [], []
    for b in (0, 3, 7):
        for kvh in (0, 5):
            K = np.empty((len(keys), sh.head_dim))
            V = np.empty_like(K)
            for j, (seg, row, ident) in enumerate(keys):
                if seg != 2 and ident == t:          # the new token, from the caller's buffer
                    K[j], V[j] = kn[b, 0, kvh], vn[b, 0, kvh]
                else:
                    name = ("sink", "ring", "slot")[seg]
                    K[j] = snap["k_" + name][b, kvh, row]
                    V[j] = snap["v_" + name][b, kvh, row]
            for g in range(G):
                h = kvh * G + g
                ref = O.attend(q[b, h], K, V, st.d.softmax_scale)
                assert_close(st.out[1][b, h], ref, torch.bfloat16, f"b={b} h={h}")
                got_all.append(np_in(st.out[1][b, h]).astype(np.float64))
                ref_all.append(ref)
    # Error budget of the bf16 path (P rounded to bf16 for the P.V product, fp32
    # accumulation, a bf16 output): against the rounding of the exact output alone.
    got_all, ref_all = np.concatenate(got_all), np.concatenate(ref_all)
    rel = np.linalg.norm(got_all - ref_all) / np.linalg.norm(ref_all)
    rel_round = np.linalg.norm(O.to_bf16(ref_all) - ref_all) / np.linalg.norm(ref_all)
    print(f"headline decode launch: rel-L2 {rel:.3e} (bf16 rounding of the exact output alone: {rel_round:.3e}), "
          f"max abs {np.abs(got_all - ref_all).max():.3e}")
    assert rel <= 2.0 * rel_round, (rel, rel_round)
    # the new token landed in its ring row
    c = O.ring_cell(t, S, W, r)
    assert torch.equal(lay.k_ring[:, :, c], st.k_new[1][:, 0])


@pytest.mark.parametrize("hidden,B", [(136, 3), (520, 17), (1000, 5), (3072, 17)])
def test_projection_hidden_splits_and_batch_groups(hidden, B):
    """The bf16 projection cuts the hidden dimension into up to 8 slices whose partial
    sums the last-arriving work-group of each column block adds up, and handles
    sequences in groups of 16.  Ragged hidden sizes (the last slice partly empty, one
    slice, five slices) and a batch of 17 (two groups) against the oracle's projection,
    within one bf16 ulp; a second call on fresh memory gives bitwise the same rows."""
    S, W, r, Hkv, D, Hq = 2, 8, 4, 8, 128, 24
    d = M.Dims(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, sink=S, window=W, interval=r,
               max_slots=4, dtype=torch.bfloat16)
    g = torch.Generator().manual_seed(hidden * 100 + B)
    N = Hkv * D
    wk = (torch.randn(hidden, N, generator=g) * 0.02).to(torch.bfloat16)
    wv = (torch.randn(hidden, N, generator=g) * 0.02).to(torch.bfloat16)
    h = torch.randn(B, hidden, generator=g).to(torch.bfloat16)
    qg = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    t1 = S + W + r
    k = torch.randn(B, t1, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, t1, Hkv, D, generator=g).to(torch.bfloat16)
    kg, vg = O.project_slot(np_in(h).astype(np.float64), np_in(wk).astype(np.float64),
                            np_in(wv).astype(np.float64), Hkv, D, bf16_cache=True)
    rows = []
    for _ in range(2):
        layer = M.alloc_layer(d, DEV, fill=float("nan"))
        layer.n_slots.zero_()
        seq = M.alloc_seq(B, DEV)
        ws = M.workspace(d, M.OP_MATERIALIZE, device=DEV)
        seq.seq_len.fill_(t1)
        M.masw_evict_append(d, layer, seq, k.to(DEV), v.to(DEV))
        o = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        M.masw_materialize_slot(d, layer, seq, h.to(DEV), wk.to(DEV), wv.to(DEV), qg.to(DEV), o, ws)
        torch.cuda.synchronize()
        assert int(seq.err.item()) == 0 and layer.n_slots.cpu().tolist() == [1] * B
        got_k = layer.k_slot[:, :, 0].double().cpu().numpy()
        got_v = layer.v_slot[:, :, 0].double().cpu().numpy()
        hn = np_in(h).astype(np.float64)
        assert_slot_close(got_k, kg, slot_bound(hn, np_in(wk).astype(np.float64), Hkv, D), "slot K")
        assert_slot_close(got_v, vg, slot_bound(hn, np_in(wv).astype(np.float64), Hkv, D), "slot V")
        assert torch.isfinite(o.float()).all()
        rows.append((layer.k_slot[:, :, 0].clone(), layer.v_slot[:, :, 0].clone()))
    assert torch.equal(rows[0][0], rows[1][0]) and torch.equal(rows[0][1], rows[1][1])


def test_boundary_launch_graph_replay_matches_eager():
    """The one-launch boundary (projection + gated slot query, bf16) captured in a HIP
    graph and replayed four times, with eager work in between (the layer reset to slot
    m - 1): every replay leaves the same slot rows, outputs and n_slots as the eager
    call, bit for bit, so the launch's tickets are back at zero after every call.
    Sequence 2 already holds slot m and is left untouched."""
    import dataclasses
    import bench
    shape = dataclasses.replace(SI.SWEEP_3B, layers=1, batch=4)
    S, W, r = shape.sink, shape.window, shape.interval
    t_b = bench.first_boundary_after(4000, S, W, r)
    m = (t_b - S - W) // r
    st = bench.Stack(shape, t_b + 64, torch.device(DEV), seed=5, with_full=False)
    st.set_position(t_b)
    lay = st.layers[0]
    have = torch.tensor([m - 1, m - 1, m, m - 1], dtype=torch.int32, device=DEV)
    ks0, vs0 = lay.k_slot.clone(), lay.v_slot.clone()

    def reset():
        lay.n_slots.copy_(have)
        lay.k_slot.copy_(ks0)
        lay.v_slot.copy_(vs0)
        st.og[0].fill_(float("nan"))

    def call():
        M.masw_materialize_slot(st.d, lay, st.seq, st.h[0], st.wk[0], st.wv[0], st.qg[0], st.og[0], st.ws)

    reset()
    call()
    torch.cuda.synchronize()
    assert int(st.seq.err.item()) == 0
    eager = [lay.k_slot.clone(), lay.v_slot.clone(), st.og[0].clone(), lay.n_slots.clone()]
    assert lay.n_slots.tolist() == [m, m, m, m]
    assert torch.equal(lay.k_slot[2], ks0[2]) and torch.isnan(st.og[0][2].float()).all()
    assert not torch.equal(lay.k_slot[0, :, m - 1], ks0[0, :, m - 1])
    reset()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    for i in range(4):
        reset()
        g.replay()
        torch.cuda.synchronize()
        got = [lay.k_slot, lay.v_slot, st.og[0], lay.n_slots]
        for name, a_, b_ in zip(("k_slot", "v_slot", "og", "n_slots"), got, eager):
            assert torch.equal(torch.nan_to_num(a_.float(), 7.0), torch.nan_to_num(b_.float(), 7.0)), f"replay {i} {name}"
    assert int(st.seq.err.item()) == 0


def test_boundary_launch_more_sequences_than_threads():
    """The one-launch boundary (bf16) with 300 sequences, more than a work-group has
    threads: thread b of each work-group takes sequence b's boundary decision at start-up
    and the rest are decided again by the last work-group.  A third of the sequences are
    at their first boundary (projected and queried, n_slots -> 1), a third already hold
    that slot and a third are one step past the boundary (both left untouched: slot rows
    and outputs stay NaN, n_slots unchanged), in every range of sequence indexes."""
    B, Hq, Hkv, D, S, W, r, hidden = 300, 2, 1, 64, 2, 8, 4, 64
    d = M.Dims(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, sink=S, window=W, interval=r,
               max_slots=4, dtype=torch.bfloat16)
    g = torch.Generator().manual_seed(77)
    wk = (torch.randn(hidden, Hkv * D, generator=g) * 0.05).to(torch.bfloat16)
    wv = (torch.randn(hidden, Hkv * D, generator=g) * 0.05).to(torch.bfloat16)
    h = torch.randn(B, hidden, generator=g).to(torch.bfloat16)
    qg = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    t1 = S + W + r
    k = torch.randn(B, t1, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, t1, Hkv, D, generator=g).to(torch.bfloat16)
    layer = M.alloc_layer(d, DEV, fill=float("nan"))
    layer.n_slots.zero_()
    seq = M.alloc_seq(B, DEV)
    ws = M.workspace(d, M.OP_MATERIALIZE, device=DEV)
    seq.seq_len.fill_(t1)
    M.masw_evict_append(d, layer, seq, k.to(DEV), v.to(DEV))
    cls = torch.arange(B) % 3                     # 0: pending, 1: already done, 2: past the boundary
    layer.n_slots.copy_((cls == 1).to(torch.int32).to(DEV))
    seq.seq_len.copy_(torch.where(cls == 2, t1 + 1, t1).to(torch.int32).to(DEV))
    o = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    M.masw_materialize_slot(d, layer, seq, h.to(DEV), wk.to(DEV), wv.to(DEV), qg.to(DEV), o, ws)
    torch.cuda.synchronize()
    assert int(seq.err.item()) == 0
    assert layer.n_slots.cpu().tolist() == [1 if c < 2 else 0 for c in cls.tolist()]
    kg, vg = O.project_slot(np_in(h).astype(np.float64), np_in(wk).astype(np.float64),
                            np_in(wv).astype(np.float64), Hkv, D, bf16_cache=True)
    hn = np_in(h).astype(np.float64)
    on = (cls == 0).numpy()
    got_k = layer.k_slot[:, :, 0].double().cpu().numpy()
    got_v = layer.v_slot[:, :, 0].double().cpu().numpy()
    assert_slot_close(got_k[on], kg[on], slot_bound(hn[on], np_in(wk).astype(np.float64), Hkv, D), "slot K")
    assert_slot_close(got_v[on], vg[on], slot_bound(hn[on], np_in(wv).astype(np.float64), Hkv, D), "slot V")
    assert np.isnan(got_k[~on]).all() and np.isnan(got_v[~on]).all()
    assert torch.isnan(o[torch.from_numpy(~on).to(DEV)].float()).all()
    kn, vn, qn = np_in(k), np_in(v), np_in(qg).astype(np.float64)
    idx = np.flatnonzero(on)
    ref = []
    for b in idx:
        mem = O.DraftMemory(S, W, r, Hkv, D, bf16_cache=True)
        mem.append(kn[b], vn[b])
        ref.append(mem.slot_query(1, qn[b], d.softmax_scale))
    assert_close(o[torch.from_numpy(idx).to(DEV)], np.stack(ref), torch.bfloat16, "slot query, 100 sequences")
