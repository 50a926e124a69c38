"""GPU parity for the second workload family, through the same kernels and C ABI:

* memories without a slot chain (interval 0: sinks ++ the exact window, the structure
  the Technical Review's section 3.1 sink bullet takes from StreamingLLM; with no sinks
  the pure sliding window of section 3's opening and section 4's SWA baseline), checked
  against the oracle along decode loops that wrap the ring several times, with the ring
  contents compared bit for bit;
* the paper's own geometry (section 4: W = S = 128, r = 4 and r = 8 raw tokens per slot)
  at the Llama-3B head shapes, materializing at every boundary.
"""
import dataclasses

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


NO_SLOT = [(4, 32), (0, 64), (0, 1), (7, 5)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("S,W", NO_SLOT)
def test_no_slot_chain_decode_loop(S, W, dtype):
    shape = dataclasses.replace(SI.TINY, sink=S, window=W, interval=0, dtype=dtype, batch=3,
                                n_q_heads=6, n_kv_heads=2, head_dim=128 if dtype == torch.bfloat16 else 64,
                                hidden=64)
    T = S + 4 * W + 7
    drv = LayerDriver(shape, max_slots=0, seed=71, num_splits=3)
    pts = sorted({1, max(1, S), S + 1, S + W, S + W + 1, S + 2 * W + 3, T})
    for tc in pts:
        drv.advance_to(tc)
        _, out, ref = drv.decode(tc)
        assert_close(out, ref, dtype, f"decode t={tc} S={S} W={W}")
    torch.cuda.synchronize()
    assert drv.err() == 0
    # the ring holds exactly the window, cell (i - S - 1) mod W, bit for bit
    ring_k = drv.layer.k_ring.cpu().float().numpy()
    ring_v = drv.layer.v_ring.cpu().float().numpy()
    assert ring_k.shape[2] == W
    for c, pos in enumerate(O.expected_ring(T, S, W, 0)):
        for b in range(shape.batch):
            np.testing.assert_array_equal(ring_k[b, :, c], drv.tokens_k[pos][b])
            np.testing.assert_array_equal(ring_v[b, :, c], drv.tokens_v[pos][b])


def test_no_slot_chain_equals_full_attention_inside_the_window():
    """While t <= S + W a memory without slots holds the whole prefix: same keys, same
    order, same split plan as the full cache, so the outputs are bitwise equal."""
    S, W = 4, 96
    shape = dataclasses.replace(SI.TINY, sink=S, window=W, interval=0, dtype=torch.bfloat16, batch=2,
                                n_q_heads=6, n_kv_heads=2, head_dim=128, hidden=64)
    drv = LayerDriver(shape, max_slots=0, seed=72, num_splits=2)
    fd = M.Dims(batch=2, n_q_heads=6, n_kv_heads=2, head_dim=128, dtype=torch.bfloat16, num_splits=2)
    kf = torch.zeros(2, 2, S + W, 128, dtype=torch.bfloat16, device="cuda")
    vf = torch.zeros_like(kf)
    ws = M.workspace(fd, M.OP_FULLKV_DECODE, max_keys=S + W, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for tc in (1, 17, S + W):
        drv.advance_to(tc)
        for p in range(1, tc + 1):
            kf[:, :, p - 1] = torch.from_numpy(drv.tokens_k[p]).to(torch.bfloat16).cuda()
            vf[:, :, p - 1] = torch.from_numpy(drv.tokens_v[p]).to(torch.bfloat16).cuda()
        q, out, _ = drv.decode(tc)
        out_f = torch.empty_like(out)
        seq = torch.full((2,), tc, dtype=torch.int32, device="cuda")
        M.fullkv_decode_attn(fd, kf, vf, seq, err, q.cuda(), out_f, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, out_f), tc
    assert drv.err() == 0 and int(err.item()) == 0


@pytest.mark.parametrize("r", [4, 8])
def test_paper_geometry_w128_s128(r):
    """W = S = 128 with r = 4 / 8 at the 3B head shapes, bf16, batch 2: every boundary
    materialized on the way to t = 1000 (186 / 93 slots), slot queries checked at the
    first boundaries and late in the chain, decodes at several points."""
    shape = dataclasses.replace(SI.DRAFT_3B, batch=2, sink=128, window=128, interval=r)
    T = 1000
    drv = LayerDriver(shape, max_slots=O.visible_slot_count(T, 128, 128, r) + 1, seed=73 + r)
    checked = []

    def on_slot(t, o, ref):
        m = O.is_boundary(t, 128, 128, r)
        if m in (1, 2, 3, 50) or t > T - 2 * r:
            assert_close(o, ref, torch.bfloat16, f"slot m={m} r={r}")
            checked.append(m)

    for tc in (255, 256, 256 + r, 300, 640, T):
        drv.advance_to(tc, on_slot=on_slot)
        _, out, ref = drv.decode(tc)
        assert_close(out, ref, torch.bfloat16, f"decode t={tc} r={r}")
    torch.cuda.synchronize()
    assert drv.err() == 0
    assert checked[:4] == [1, 2, 3, 50]
    n = O.visible_slot_count(T, 128, 128, r)
    assert drv.layer.n_slots.cpu().tolist() == [n, n]
    assert len(O.keylist(T, 128, 128, r)) == 256 + n


@pytest.mark.parametrize("S,W,r,n_new", [(2, 4, 0, 15), (2, 4, 2, 15), (0, 3, 0, 11), (3, 5, 1, 20)])
def test_append_more_than_the_ring_in_one_call(S, W, r, n_new):
    """One append call with more positions than ring rows must leave the memory as the
    positions appended one by one would: per row the last legal write wins, and writes
    whose evicted token's block has no slot are suppressed and reported."""
    B, Hkv, D = 2, 2, 64
    d = M.Dims(batch=B, n_q_heads=2, n_kv_heads=Hkv, head_dim=D, sink=S, window=W, interval=r,
               max_slots=4, dtype=torch.float32)
    layer = M.alloc_layer(d, "cuda", fill=float("nan"))
    layer.n_slots.zero_()
    seq = M.alloc_seq(B, "cuda")
    seq.seq_len.fill_(n_new)
    g = torch.Generator().manual_seed(S * 100 + W * 10 + r)
    k = torch.randn(B, n_new, Hkv, D, generator=g)
    v = torch.randn(B, n_new, Hkv, D, generator=g)
    M.masw_evict_append(d, layer, seq, k.cuda(), v.cuda())
    torch.cuda.synchronize()
    # sequential reference: positions in order, an eviction needs the victim's slot (none exist)
    C = W + r
    cells = [None] * C
    illegal = False
    for i in range(S + 1, n_new + 1):
        c = (i - S - 1) % C
        victim = cells[c]
        if victim is not None and r > 0 and victim > S:
            illegal = True
            continue
        cells[c] = i
    ring = layer.k_ring.cpu()
    for c, pos in enumerate(cells):
        if pos is None:
            assert torch.isnan(ring[:, :, c]).all()
        else:
            assert torch.equal(ring[:, :, c], k[:, pos - 1]), (c, pos)
    if S:
        assert torch.equal(layer.k_sink.cpu(), k[:, :S].transpose(1, 2))
    assert bool(int(seq.err.item()) & 1) == illegal   # MASW_DEV_PENDING_SLOT
