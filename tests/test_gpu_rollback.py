"""GPU parity of speculative drafting with rollback (Technical Review §3.3, Algorithm 2
steps 4-6): every sequence drafts L_draft tokens (appending, materializing at
boundaries, decoding), accepts its own random prefix, rolls back and appends the
target's correction token.  The oracle mirrors each operation and its rollback is pinned
on the CPU against appending only the accepted tokens.  Decode and slot-query outputs
are compared at every step; at the end the slot counts and the ring rows the accepted
memory needs are compared bit for bit."""
import numpy as np
import pytest
import torch

import draft_kv_attention_amd as M
from oracle import masw_oracle as O
from tests.gpu_driver import np_in
from tests.parity import assert_close

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.lib()


CASES = [
    dict(S=2, W=8, r=4, R=5, L=5, Hq=2, Hkv=1, D=64, dtype=torch.float32, hidden=64, iters=30),
    dict(S=4, W=32, r=8, R=6, L=6, Hq=6, Hkv=2, D=128, dtype=torch.bfloat16, hidden=128, iters=25),
    dict(S=3, W=16, r=0, R=5, L=5, Hq=4, Hkv=2, D=64, dtype=torch.float32, hidden=64, iters=20),
]


@pytest.mark.parametrize("c", CASES, ids=["fp32_r4", "bf16_r8", "fp32_no_slots"])
def test_speculative_drafting_with_rollback(c):
    S, W, r, R, L, B = c["S"], c["W"], c["r"], c["R"], c["L"], 3
    Hq, Hkv, D, dt, hidden = c["Hq"], c["Hkv"], c["D"], c["dtype"], c["hidden"]
    bf16 = dt == torch.bfloat16
    t_max = 1 + c["iters"] * (L + 1)
    max_slots = O.visible_slot_count(t_max + L, S, W, r) + 2
    d = M.Dims(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, sink=S, window=W, interval=r,
               max_slots=max_slots, dtype=dt, rollback=R, num_splits=2)
    layer = M.alloc_layer(d, "cuda", fill=float("nan"))
    layer.n_slots.zero_()
    seq = M.alloc_seq(B, "cuda")
    ws = M.workspace(d, M.OP_MATERIALIZE, device="cuda")
    g = torch.Generator().manual_seed(S * 1000 + W * 10 + r)
    wk = (torch.randn(hidden, Hkv * D, generator=g) * 0.1).to(dt)
    wv = (torch.randn(hidden, Hkv * D, generator=g) * 0.1).to(dt)
    wk_n, wv_n = np_in(wk).astype(np.float64), np_in(wv).astype(np.float64)
    mems = [O.DraftMemory(S, W, r, Hkv, D, bf16) for _ in range(B)]
    scale = d.softmax_scale
    rng = np.random.default_rng(5)

    def step():
        """Append one token to every sequence, materialize where due, decode."""
        seq.seq_len.add_(1)
        k = torch.randn(B, 1, Hkv, D, generator=g).to(dt)
        v = torch.randn(B, 1, Hkv, D, generator=g).to(dt)
        M.masw_evict_append(d, layer, seq, k.cuda(), v.cuda())
        kn, vn = np_in(k), np_in(v)
        for b, mem in enumerate(mems):
            mem.append(kn[b], vn[b])
        if r:
            h = torch.randn(B, hidden, generator=g).to(dt)
            qg = torch.randn(B, Hq, D, generator=g).to(dt)
            og = torch.full((B, Hq, D), float("nan"), dtype=dt, device="cuda")
            M.masw_materialize_slot(d, layer, seq, h.cuda(), wk.cuda(), wv.cuda(), qg.cuda(), og, ws)
            hn, qn = np_in(h).astype(np.float64), np_in(qg).astype(np.float64)
            for b, mem in enumerate(mems):
                ref = mem.materialize(hn[b], wk_n, wv_n, qn[b], scale)
                if ref is not None:
                    assert_close(og[b:b + 1], ref[None], dt, f"slot query b={b} t={mem.t}")
        q = torch.randn(B, Hq, D, generator=g).to(dt)
        out = torch.full((B, Hq, D), float("nan"), dtype=dt, device="cuda")
        M.masw_draft_attn(d, layer, seq, q.cuda(), out, ws)
        qn = np_in(q).astype(np.float64)
        ref = np.stack([mem.decode(qn[b], scale) for b, mem in enumerate(mems)])
        assert_close(out, ref, dt, f"decode t={[m.t for m in mems]}")

    step()                                   # the first accepted token
    for _ in range(c["iters"]):
        t0 = [mem.t for mem in mems]
        for _ in range(L):                   # drafting
            step()
        t_spec = seq.seq_len.clone()
        acc = [int(rng.integers(0, L + 1)) for _ in range(B)]
        seq.seq_len.copy_(torch.tensor([t0[b] + acc[b] for b in range(B)], dtype=torch.int32))
        M.masw_rollback(d, layer, seq, t_spec)
        for b, mem in enumerate(mems):
            mem.rollback(t0[b] + acc[b])
        step()                               # the target's correction token
    torch.cuda.synchronize()
    assert int(seq.err.item()) == 0
    assert layer.n_slots.cpu().tolist() == [len(mem.slots) for mem in mems]
    ring_k = layer.k_ring.cpu().float().numpy()
    for b, mem in enumerate(mems):
        for kind, i in O.keylist(mem.t, S, W, r):
            if kind == "raw" and i > S:
                np.testing.assert_array_equal(ring_k[b, :, O.ring_cell(i, S, W, r, R)], mem.raw[i][0])


def test_rollback_past_the_rollback_rows_is_refused():
    S, W, r, R, B = 2, 8, 4, 3, 2
    d = M.Dims(batch=B, n_q_heads=2, n_kv_heads=1, head_dim=64, sink=S, window=W, interval=r,
               max_slots=8, dtype=torch.float32, rollback=R)
    layer = M.alloc_layer(d, "cuda")
    layer.n_slots.fill_(3)
    seq = M.alloc_seq(B, "cuda")
    seq.seq_len.copy_(torch.tensor([20, 30], dtype=torch.int32))   # n(20) = 2, n(30) = 5
    t_spec = torch.tensor([20 + R, 30 + R + 1], dtype=torch.int32, device="cuda")
    M.masw_rollback(d, layer, seq, t_spec)
    torch.cuda.synchronize()
    # sequence 0: within reach, slots truncated to n(20) = 2; sequence 1: refused, untouched
    assert layer.n_slots.cpu().tolist() == [2, 3]
    assert int(seq.err.item()) == 16   # MASW_DEV_ROLLBACK_RANGE
