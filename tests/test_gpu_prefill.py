"""GPU parity of the draft prefill (masw_prefill) with the oracle.

The oracle side is reading R10 of the Technical Review's §3.3 (Algorithm 2 step 2):
the raw query at position i attends to keylist(i), slot g_m's query to
keylist(t_m - r), the slots projected from their hidden states (oracle.project_slot,
rounded to bf16) and the raw keys taken from the prefix.  Each case checks
  * out and o_slot against oracle.prefill_attend (bf16 tolerance of tests/parity.py);
    rows past a sequence's prefix stay untouched (NaN);
  * the projected slot K/V within one bf16 ulp plus the fp32 dot-product bound;
  * the memory the call leaves: n_slots = n(P), sink rows and the newest C ring rows
    equal to the prefix's K/V bit for bit, the other rows untouched;
  * for the small cases, one decode step after the prefill against the oracle memory
    that holds the same prefix, so the prefill leaves what decoding would.
Shapes: bf16, D = 128, group sizes 1, 3, 4, 6 and 8 (query blocks of 64/G queries, a
ragged last row block for 3 and 6), ragged prefixes that span several query blocks,
no slot chain (r = 0), no sinks, prefixes shorter than the sinks or the window, a
prefix ending on a boundary, rollback rows, and the 3B draft shape at a 32768-token
prefix on sampled rows.
"""
import numpy as np
import pytest
import torch

import draft_kv_attention_amd as M
import seeded_inputs as SI
from oracle import masw_oracle as O
from tests.gpu_driver import np_in
from tests.parity import assert_close, assert_slot_close, bf16_ulp, rotated_slot_bound, slot_bound

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAN = float("nan")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.lib()


def _shape(Hq, Hkv, S, W, r, B, hidden=256):
    return SI.DraftShape(name="prefill_case", layers=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=128,
                         hidden=hidden, sink=S, window=W, interval=r, batch=B, dtype=torch.bfloat16,
                         w_std=0.05)


class Prefill:
    """One masw_prefill call on fresh memory, with the inputs kept for the oracle."""

    def __init__(self, sh, P_list, p_max, ns_max, max_slots, seed, rollback=0, with_slots=True, rope_theta=0.0,
                 rope_style=0):
        self.sh, self.P, self.p_max, self.ns_max = sh, list(P_list), p_max, ns_max
        B = sh.batch
        self.d = M.Dims(batch=B, n_q_heads=sh.n_q_heads, n_kv_heads=sh.n_kv_heads, head_dim=sh.head_dim,
                        sink=sh.sink, window=sh.window, interval=sh.interval, max_slots=max_slots,
                        dtype=sh.dtype, rollback=rollback, rope_theta=rope_theta, rope_style=rope_style)
        self.rope = (rope_theta, rope_style) if rope_theta > 0 else None
        self.layer = M.alloc_layer(self.d, DEV, fill=NAN)
        self.layer.n_slots.zero_()
        self.seq = M.alloc_seq(B, DEV)
        self.seq.seq_len.copy_(torch.tensor(self.P, dtype=torch.int32))
        self.k, self.v, self.q, self.h, self.qs = SI.prefill_inputs(sh, seed, 0, p_max, max(ns_max, 1))
        self.wk, self.wv = SI.mirrored_weights(sh, seed)
        self.out = torch.full(self.q.shape, NAN, dtype=sh.dtype, device=DEV)
        self.o_slot = torch.full(self.qs.shape, NAN, dtype=sh.dtype, device=DEV)
        slots = with_slots and sh.interval > 0 and ns_max > 0
        print(f"prefill case: Hq={sh.n_q_heads} Hkv={sh.n_kv_heads} S={sh.sink} W={sh.window} "
              f"r={sh.interval} R={rollback} P={self.P} p_max={p_max} ns_max={ns_max} seed={seed}", flush=True)
        M.masw_prefill(self.d, self.layer, self.seq, self.k.to(DEV), self.v.to(DEV), self.q.to(DEV), self.out,
                       *( (self.h.to(DEV), self.wk.to(DEV), self.wv.to(DEV), self.qs.to(DEV), self.o_slot)
                          if slots else ()))
        torch.cuda.synchronize()
        self.slots = slots
        self.kn, self.vn, self.qn = np_in(self.k), np_in(self.v), np_in(self.q)
        self.hn, self.qsn = np_in(self.h).astype(np.float64), np_in(self.qs)
        self.wkn, self.wvn = np_in(self.wk).astype(np.float64), np_in(self.wv).astype(np.float64)

    def n(self, b):
        sh = self.sh
        return O.visible_slot_count(self.P[b], sh.sink, sh.window, sh.interval)

    def oracle_slots(self, b):
        sh = self.sh
        n = self.n(b)
        ids = [O.slot_position_id(m, sh.sink, sh.interval) for m in range(1, n + 1)] if self.rope else None
        return O.project_slot(self.hn[b, :n], self.wkn, self.wvn, sh.n_kv_heads, sh.head_dim, True, self.rope, ids)

    def check(self, b, positions=None, slots=None):
        sh = self.sh
        P, n = self.P[b], self.n(b)
        sk, sv = self.oracle_slots(b)
        ref, ref_s = O.prefill_attend(self.kn[b, :P], self.vn[b, :P], sk, sv, self.qn[b, :P], self.qsn[b, :n],
                                      sh.sink, sh.window, sh.interval, self.d.softmax_scale,
                                      positions=positions, slots=slots)
        got = self.out[b].float().cpu().numpy()
        rows = np.arange(P) if positions is None else np.asarray(positions) - 1
        assert_close(got[rows], ref[rows], sh.dtype, f"out b={b}")
        assert np.isnan(got[P:]).all(), "rows past the prefix were written"
        if n:
            gs = self.o_slot[b].float().cpu().numpy()
            srows = np.arange(n) if slots is None else np.asarray(slots) - 1
            assert_close(gs[srows], ref_s[srows], sh.dtype, f"o_slot b={b}")
            if self.ns_max > n:
                assert np.isnan(gs[n:]).all(), "slot rows past n(P) were written"
            # stored slot K/V: [Hkv][max_slots][D] -> [n][Hkv][D]
            for name, ref_kv, w in (("k_slot", sk, self.wkn), ("v_slot", sv, self.wvn)):
                bound = slot_bound(self.hn[b, :n], w, sh.n_kv_heads, sh.head_dim, prefill=True)
                if self.rope and name == "k_slot":
                    bound = rotated_slot_bound(self.hn[b, :n], w, sh.n_kv_heads, sh.head_dim, self.rope[1], ref_kv,
                                               prefill=True)
                got_kv = getattr(self.layer, name)[b, :, :n].float().cpu().numpy().transpose(1, 0, 2)
                assert_slot_close(got_kv, ref_kv, bound, f"{name} b={b}")

    def check_memory(self, b):
        sh, d = self.sh, self.d
        S, W, r, R = sh.sink, sh.window, sh.interval, d.rollback
        P, C = self.P[b], d.ring
        assert int(self.layer.n_slots[b]) == (self.n(b) if self.slots else 0)
        ks = self.layer.k_sink[b].float().cpu().numpy() if S else None
        vs = self.layer.v_sink[b].float().cpu().numpy() if S else None
        kr = self.layer.k_ring[b].float().cpu().numpy()
        vr = self.layer.v_ring[b].float().cpu().numpy()
        for i in range(1, min(S, P) + 1):
            assert np.array_equal(ks[:, i - 1], self.kn[b, i - 1]) and np.array_equal(vs[:, i - 1], self.vn[b, i - 1])
        if S and P < S:
            assert np.isnan(ks[:, P:]).all()
        written = set()
        for i in range(max(S + 1, P - C + 1), P + 1):
            c = O.ring_cell(i, S, W, r, R)
            written.add(c)
            assert np.array_equal(kr[:, c], self.kn[b, i - 1]), (b, i, c)
            assert np.array_equal(vr[:, c], self.vn[b, i - 1]), (b, i, c)
        for c in range(C):
            if c not in written:
                assert np.isnan(kr[:, c]).all() and np.isnan(vr[:, c]).all(), (b, c)

    def decode_next(self, seed):
        """Append position P+1 and decode there; compare with an oracle memory holding
        the prefix (all P equal; P+1 must not be a boundary)."""
        sh, d = self.sh, self.d
        P = self.P[0]
        assert all(p == P for p in self.P) and not O.is_boundary(P + 1, sh.sink, sh.window, sh.interval)
        kx, vx = SI.token_kv(sh, seed, 0, P + 1, 1)
        qx = SI.decode_query(sh, seed, 0, P + 1)
        self.seq.seq_len.fill_(P + 1)
        out = torch.full((d.batch, d.n_q_heads, d.head_dim), NAN, dtype=d.dtype, device=DEV)
        ws = M.workspace(d, M.OP_DRAFT_ATTN, device=DEV)
        M.masw_decode_step(d, self.layer, self.seq, kx.to(DEV), vx.to(DEV), qx.to(DEV), out, ws)
        assert int(self.seq.err.item()) == 0
        refs = []
        for b in range(d.batch):
            mem = O.DraftMemory(sh.sink, sh.window, sh.interval, sh.n_kv_heads, sh.head_dim, True,
                                *(self.rope if self.rope else ()))
            mem.append(self.kn[b, :P], self.vn[b, :P])
            if self.slots:
                sk, sv = self.oracle_slots(b)
                for m in range(1, self.n(b) + 1):
                    mem.add_slot(m, sk[m - 1], sv[m - 1])
            mem.append(np_in(kx)[b], np_in(vx)[b])
            refs.append(mem.decode(np_in(qx)[b].astype(np.float64), d.softmax_scale))
        assert_close(out, np.stack(refs), d.dtype, "decode after prefill")


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (6, 2), (8, 2), (12, 2), (8, 1)])
def test_prefill_group_sizes_ragged(Hq, Hkv):
    sh = _shape(Hq, Hkv, S=4, W=64, r=8, B=2)
    # 517: 62 slots, several query blocks and a ragged last one; 300 ends mid-block
    pf = Prefill(sh, [517, 300], p_max=517, ns_max=62, max_slots=64, seed=Hq * 10 + Hkv)
    assert int(pf.seq.err.item()) == 0
    for b in range(2):
        pf.check(b)
        pf.check_memory(b)


def test_prefill_then_decode_matches_oracle_memory():
    sh = _shape(8, 2, S=4, W=64, r=8, B=2)
    pf = Prefill(sh, [450, 450], p_max=450, ns_max=60, max_slots=60, seed=7)
    assert int(pf.seq.err.item()) == 0
    pf.check(0)
    pf.decode_next(seed=8)


@pytest.mark.parametrize("S,W,r,P,R", [
    (4, 64, 0, 400, 0),      # no slot chain: sinks + exact window
    (0, 64, 16, 400, 0),     # no sinks
    (4, 64, 8, 3, 0),        # prefix inside the sinks
    (4, 64, 8, 50, 0),       # prefix inside the window: no slot yet
    (4, 64, 8, 68 + 5 * 8, 0),   # prefix ends on the boundary of slot 5
    (4, 64, 8, 389, 6),      # rollback rows: a longer ring
    (4, 32, 32, 333, 0),     # r = W
])
def test_prefill_edges(S, W, r, P, R):
    sh = _shape(8, 2, S=S, W=W, r=r, B=1)
    n = O.visible_slot_count(P, S, W, r)
    pf = Prefill(sh, [P], p_max=P + 5, ns_max=n + 1, max_slots=n + 2, seed=P + r, rollback=R)
    assert int(pf.seq.err.item()) == 0
    pf.check(0)
    pf.check_memory(0)
    if not O.is_boundary(P + 1, S, W, r):
        pf.decode_next(seed=P)


def test_prefill_empty_and_errors():
    sh = _shape(8, 2, S=4, W=64, r=8, B=4)
    # b=0 fine, b=1 empty prefix (no-op), b=2 longer than p_max, b=3 more slots than max_slots
    n_ok = O.visible_slot_count(200, 4, 64, 8)
    pf = Prefill(sh, [200, 0, 301, 300], p_max=300, ns_max=40, max_slots=n_ok, seed=3)
    err = int(pf.seq.err.item())
    assert err == (M.DEV_SEQ_RANGE | M.DEV_SLOT_CAPACITY), err
    pf.check(0)
    for b in (1, 2, 3):
        assert torch.isnan(pf.out[b].float()).all(), b
        assert torch.isnan(pf.o_slot[b].float()).all(), b
    # more slots than the caller's slot rows
    pf2 = Prefill(sh, [300, 300, 300, 300], p_max=300, ns_max=10, max_slots=40, seed=4)
    assert int(pf2.seq.err.item()) == M.DEV_SLOT_CAPACITY
    assert torch.isnan(pf2.out.float()).all()


def test_prefill_3b_32k_sampled():
    sh = SI.PREFILL_3B
    P = SI.PREFILL_LEN
    n = O.visible_slot_count(P, sh.sink, sh.window, sh.interval)
    pf = Prefill(sh, [P], p_max=P, ns_max=n, max_slots=n, seed=17)
    assert int(pf.seq.err.item()) == 0
    rng = np.random.default_rng(5)
    S, W, r = sh.sink, sh.window, sh.interval
    fixed = [1, 2, S, S + 1, W, W + 1, S + W, S + W + 1, S + W + r, S + W + r + 1, P - 1, P]
    positions = sorted(set(fixed) | set(int(x) for x in rng.integers(1, P + 1, 36)))
    slots = sorted({1, 2, n // 2, n - 1, n} | set(int(x) for x in rng.integers(1, n + 1, 6)))
    pf.check(0, positions=positions, slots=slots)
    pf.check_memory(0)


@pytest.mark.parametrize("style", [0, 1])
def test_prefill_with_rotated_slot_keys(style):
    """Slot keys rotated to their position ids (reading R11) in the prefill's projection."""
    sh = _shape(8, 2, S=4, W=64, r=8, B=2)
    pf = Prefill(sh, [450, 450], p_max=450, ns_max=60, max_slots=60, seed=12 + style, rope_theta=10000.0,
                 rope_style=style)
    assert int(pf.seq.err.item()) == 0
    for b in range(2):
        pf.check(b)
        pf.check_memory(b)
    pf.decode_next(seed=13)


def test_prefill_graph_replay_matches_eager():
    """masw_prefill captured into a HIP graph: every replay (with eager work and
    synchronizations in between) gives the eager outputs and memory bit for bit."""
    sh = _shape(8, 2, S=4, W=64, r=8, B=2)
    pf = Prefill(sh, [450, 380], p_max=450, ns_max=60, max_slots=60, seed=21)
    names = ("k_ring", "v_ring", "k_slot", "v_slot", "k_sink", "v_sink")
    eager = (pf.out.clone(), pf.o_slot.clone(), {n: getattr(pf.layer, n).clone() for n in names},
             pf.layer.n_slots.clone())
    args = (pf.k.to(DEV), pf.v.to(DEV), pf.q.to(DEV))
    slot_args = (pf.h.to(DEV), pf.wk.to(DEV), pf.wv.to(DEV), pf.qs.to(DEV))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            M.masw_prefill(pf.d, pf.layer, pf.seq, *args, pf.out, *slot_args, pf.o_slot)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: clobber the outputs and the memory
        pf.out.fill_(float("nan"))
        pf.o_slot.fill_(float("nan"))
        pf.layer.k_ring.fill_(0.5 * rep)
        pf.layer.n_slots.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(pf.seq.err.item()) == 0
        assert torch.equal(pf.out.view(torch.int16), eager[0].view(torch.int16)), rep
        assert torch.equal(pf.o_slot.view(torch.int16), eager[1].view(torch.int16)), rep
        assert torch.equal(pf.layer.n_slots, eager[3]), rep
        for n in names:   # both prefixes are longer than the ring, so every cell is refilled
            assert torch.equal(getattr(pf.layer, n).view(torch.int16), eager[2][n].view(torch.int16)), (rep, n)
