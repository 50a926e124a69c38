"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what it pins: a value worked by hand from the pages' definitions, a
workload count, a closed form, a library routine, or a brute-force formulation written
separately from the oracle's key-list code.  A plausible mistake in the oracle (a
dropped sink, an off-by-one window, a wrong slot count, a sign or scale error in the
softmax, a transposed projection, a mis-aligned causal mask) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import masw_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Eq. 2: hand-worked example, closed forms, library routine
# ---------------------------------------------------------------------------

def test_eq2_hand_example():
    g = _load("eq2_hand_example.json")
    q = np.array([math.sqrt(2.0) * math.log(2.0), 0.0])
    K = np.array(g["K"])
    V = np.array(g["V"])
    scale = O.default_scale(g["head_dim"])
    np.testing.assert_allclose(O.softmax_weights(q, K, scale), g["weights"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.attend(q, K, V, scale), g["out"], rtol=0, atol=1e-13)


def test_attend_closed_forms():
    rng = np.random.default_rng(0)
    D = 16
    K = rng.normal(size=(9, D))
    V = rng.normal(size=(9, D))
    q = rng.normal(size=D)
    s = 0.3
    # a single key returns its value exactly
    np.testing.assert_array_equal(O.attend(q, K[:1], V[:1], s), V[0])
    # a zero query averages the values
    np.testing.assert_allclose(O.attend(np.zeros(D), K, V, s), V.mean(axis=0), atol=1e-15)
    # constant values are reproduced
    np.testing.assert_allclose(O.attend(q, K, np.full((9, D), 2.5), s), np.full(D, 2.5), atol=1e-14)
    # weights form a probability row
    w = O.softmax_weights(q, K, s)
    assert abs(w.sum() - 1.0) < 1e-12 and (w > 0).all()
    # a larger score gets a larger weight (sign of the exponent)
    assert np.argmax(w) == np.argmax(K @ q)
    # permuting keys and values together changes nothing
    perm = rng.permutation(9)
    np.testing.assert_allclose(O.attend(q, K[perm], V[perm], s), O.attend(q, K, V, s), atol=1e-14)
    # shifting every key along q shifts every score equally: output unchanged
    K2 = K + 3.0 * q[None, :] / np.dot(q, q)
    np.testing.assert_allclose(O.attend(q, K2, V, s), O.attend(q, K, V, s), atol=1e-13)
    # huge scores do not overflow (max subtraction)
    out = O.attend(q * 1e4, K, V, s)
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out, V[np.argmax(K @ q)], atol=1e-9)


def test_two_key_ratio_closed_form():
    # scores differing by ln 3 give weights 3/4 and 1/4
    D = 4
    scale = O.default_scale(D)
    q = np.array([math.log(3.0) / scale, 0, 0, 0])
    K = np.array([[1.0, 0, 0, 0], [0.0, 1, 0, 0]])
    V = np.array([[4.0, 0, 0, 0], [0.0, 4, 0, 0]])
    np.testing.assert_allclose(O.attend(q, K, V, scale), [3.0, 1.0, 0, 0], atol=1e-14)


def test_gqa_attend_matches_torch_sdpa():
    rng = np.random.default_rng(1)
    Hq, Hkv, n, D = 6, 2, 37, 32
    q = rng.normal(size=(Hq, D))
    K = rng.normal(size=(Hkv, n, D))
    V = rng.normal(size=(Hkv, n, D))
    scale = O.default_scale(D)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :],
        torch.from_numpy(K).repeat_interleave(Hq // Hkv, dim=0),
        torch.from_numpy(V).repeat_interleave(Hq // Hkv, dim=0),
        scale=scale)[:, 0, :].numpy()
    np.testing.assert_allclose(O.gqa_attend(q, K, V, scale), ref, atol=1e-13)
    # the grouping is contiguous: head h reads KV head h // G, not h % Hkv
    wrong = O.gqa_attend(q, K[[1, 0]], V[[1, 0]], scale)
    assert np.abs(wrong - ref).max() > 1e-3


# ---------------------------------------------------------------------------
# Eq. 4: key lists, counts, invariants
# ---------------------------------------------------------------------------

def test_window_hand_example():
    g = _load("window_hand_example.json")
    S, W, r = g["S"], g["W"], g["r"]
    for c in g["cases"]:
        keys = O.keylist(c["t"], S, W, r)
        assert [i for k, i in keys if k == "raw"] == c["raw"], c
        assert [m for k, m in keys if k == "slot"] == c["slots"], c
        # sinks come first, then the window ascending, then slots ascending
        assert keys == [("raw", i) for i in c["raw"]] + [("slot", m) for m in c["slots"]]


def test_physical_keylist_hand_example():
    """Placement of every key (sink row, ring row with and without rollback rows, slot
    row), worked by hand (tests/golden)."""
    g = _load("physical_keylist_hand_example.json")
    for c in g["cases"]:
        got = O.physical_keylist(c["t"], g["S"], g["W"], g["r"], rollback=c["R"])
        assert [list(k) for k in got] == c["keys"], c


def test_no_slot_window_hand_example():
    """Reading R8: without a slot chain the memory is sinks ++ the exact window."""
    g = _load("no_slot_window_hand_example.json")
    for mem in g["memories"]:
        S, W = mem["S"], mem["W"]
        for c in mem["cases"]:
            assert O.keylist(c["t"], S, W, 0) == [("raw", i) for i in c["raw"]], (S, W, c)
            assert O.expected_ring(c["t"], S, W, 0) == c["ring"], (S, W, c)


def test_tiny_workload_counts():
    g = _load("memory_counts.json")["tiny_workload"]
    S, W, r, t = g["S"], g["W"], g["r"], g["t"]
    assert O.visible_slot_count(t, S, W, r) == g["slots"]
    crossed = [u for u in range(t + 1, t + g["next_steps"] + 1) if O.is_boundary(u, S, W, r)]
    assert len(crossed) == g["boundaries_crossed"]
    # a literal floor(t / r) count would give 12 here, a ceiling 11
    assert t // r != g["slots"] and -(-(t - S - W) // r) != g["slots"]


def test_slot_query_count_3b():
    g = _load("memory_counts.json")["slot_query_3b"]
    S, W, r = g["S"], g["W"], g["r"]
    for prior in g["prior_slots"]:
        m = prior + 1
        keys = O.slot_query_keylist(m, S, W, r)
        assert len(keys) == S + W + prior
        assert sum(1 for k, _ in keys if k == "slot") == prior
        # the window of the slot query starts at the first token of the block g_m compresses
        raw = [i for k, i in keys if k == "raw" and i > S]
        assert raw[0] == O.block_positions(m, S, r)[0] and len(raw) == W


def test_worked_example_divergence_is_documented():
    g = _load("memory_counts.json")["worked_example_page"]
    S, W, r, t = g["S"], g["W"], g["r"], g["t"]
    n = O.visible_slot_count(t, S, W, r)
    keys = O.keylist(t, S, W, r)
    assert O.is_boundary(t, S, W, r) == n      # t = 4100 is a boundary under the reading
    assert (n, len(keys)) == (961, 1217)
    assert n != g["page_slots_approx"] and len(keys) != g["page_entries"]
    # the page's 8-token window contradicts Eq. 4 with W = 128
    assert len(O.local_positions(t, S, W)) == W != g["page_local"]


def _invariant_grid():
    for S in (0, 1, 4, 7):
        for W in (1, 3, 8, 32):
            for r in (0, 1, 2, 5, 16, 32):
                if r <= W:
                    yield S, W, r


@pytest.mark.parametrize("S,W,r", list(_invariant_grid()))
def test_keylist_invariants(S, W, r):
    C = O.ring_capacity(W, r)
    for t in range(1, S + W + 6 * max(r, 4) + 3):
        keys = O.keylist(t, S, W, r)
        n = O.visible_slot_count(t, S, W, r)
        raw = [i for k, i in keys if k == "raw"]
        slots = [m for k, m in keys if k == "slot"]
        # I1 exact size; I2 the page's working-set bound (no slot chain: sinks + window)
        assert len(keys) == min(t, S) + min(max(t - S, 0), W) + n
        assert len(keys) <= S + W + (t // r if r else 0)
        if r == 0:
            assert n == 0 and not O.is_boundary(t, S, W, r)
        # I3 local part by enumeration straight from Eq. 4
        local = [i for i in range(1, t + 1) if i > S and max(S + 1, t - W + 1) <= i <= t]
        assert raw == list(range(1, min(S, t) + 1)) + local
        assert len(set(raw)) == len(raw)
        # I4 no slot while t <= S + W: the memory is the whole prefix
        if t <= S + W:
            assert raw == list(range(1, t + 1)) and not slots
        # I7 no visible raw token lies in a block whose slot is visible
        for m in slots:
            assert not set(O.block_positions(m, S, r)) & set(raw)
        # every non-sink raw token older than the window has left it for good:
        # its block's slot is visible, or the block is still waiting (< r steps)
        # (without a slot chain it is simply gone: reading R8)
        for i in range(S + 1, t + 1):
            if i not in raw and r:
                m = -(-(i - S) // r)
                assert m in slots or O.boundary_step(m, S, W, r) > t
                assert O.boundary_step(m, S, W, r) - t < r
        # the ring keeps every visible raw token
        assert t - C < (local[0] if local else t + 1)
    # I6 the slot query sees exactly what the decode query saw r steps before
    for m in range(1, 6 if r else 1):
        assert O.slot_query_keylist(m, S, W, r) == O.keylist(S + W + (m - 1) * r, S, W, r)


@settings(max_examples=200, deadline=None)
@given(S=st.integers(0, 9), W=st.integers(1, 40), r=st.integers(1, 40), t=st.integers(1, 400))
def test_keylist_property(S, W, r, t):
    if r > W:
        return
    keys = O.keylist(t, S, W, r)
    n = O.visible_slot_count(t, S, W, r)
    assert len(keys) == min(t, S) + min(max(t - S, 0), W) + n
    assert len(keys) <= S + W + t // r
    # slots appear exactly at the boundary steps
    assert n == sum(1 for u in range(1, t + 1) if O.is_boundary(u, S, W, r))


# ---------------------------------------------------------------------------
# Ring placement and append legality (bookkeeping behind the key list)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S,W,r", [(0, 1, 1), (4, 32, 16), (2, 3, 2), (7, 8, 5), (1, 5, 5), (4, 8, 0), (0, 5, 0)])
def test_ring_closed_form_vs_fifo_simulation(S, W, r):
    """A literal FIFO of C cells: the next free cell advances by one per non-sink token."""
    C = O.ring_capacity(W, r)
    cells = [None] * C
    nxt = 0
    for t in range(1, S + 4 * C + 3):
        if t > S:
            cells[nxt] = t
            nxt = (nxt + 1) % C
            assert O.ring_cell(t, S, W, r) == (nxt - 1) % C
        assert O.expected_ring(t, S, W, r) == cells
        # every visible raw non-sink token is resident in the ring
        held = set(c for c in cells if c is not None)
        for kind, i in O.keylist(t, S, W, r):
            if kind == "raw" and i > S:
                assert i in held
        # at a boundary the slot query's window is resident as well
        m = O.is_boundary(t, S, W, r)
        if m:
            for kind, i in O.slot_query_keylist(m, S, W, r):
                if kind == "raw" and i > S:
                    assert i in held


@pytest.mark.parametrize("S,W,r", [(4, 32, 16), (0, 3, 3), (2, 3, 2), (5, 9, 4)])
def test_append_legality_schedule(S, W, r):
    """Materializing at every boundary keeps every append legal; skipping one slot makes
    exactly the first append that would overwrite its block illegal, at t_m + 1."""
    n_slots = 0
    for i in range(1, S + W + 8 * r):
        assert O.append_is_legal(i, n_slots, S, W, r)
        if O.is_boundary(i, S, W, r):
            n_slots += 1
    for m in (1, 2, 3):
        tm = O.boundary_step(m, S, W, r)
        assert O.append_is_legal(tm, m - 1, S, W, r)
        assert not O.append_is_legal(tm + 1, m - 1, S, W, r)
        assert O.append_is_legal(tm + 1, m, S, W, r)


@pytest.mark.parametrize("S,W", [(4, 8), (0, 5), (3, 1)])
def test_no_slot_chain_appends_are_always_legal(S, W):
    """Reading R8: without a slot chain no block waits for a slot; the ring keeps W rows
    and the window is exactly what it holds."""
    assert O.ring_capacity(W, 0) == W
    for i in range(1, S + 5 * W + 3):
        assert O.append_is_legal(i, 0, S, W, 0)
        held = set(c for c in O.expected_ring(i, S, W, 0) if c is not None)
        assert held == set(range(max(S + 1, i - W + 1), i + 1))


def test_ring_capacity_is_tight():
    """With one cell fewer than W + r the slot query's window is no longer resident."""
    S, W, r = 4, 32, 16
    C = O.ring_capacity(W, r) - 1
    m = 3
    tm = O.boundary_step(m, S, W, r)
    window = [i for k, i in O.slot_query_keylist(m, S, W, r) if k == "raw" and i > S]
    assert window[0] <= tm - C     # the oldest token would already be overwritten


# ---------------------------------------------------------------------------
# Brute force: dense masks over every entry ever created vs the key-list oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S,W,r", [(4, 32, 16), (0, 5, 2), (3, 4, 4), (2, 6, 1), (1, 8, 3), (4, 8, 0), (0, 6, 0)])
def test_dense_mask_bruteforce(S, W, r):
    rng = np.random.default_rng(7)
    D, Hkv, hidden = 8, 2, 8
    G = 2
    T = S + W + 5 * max(r, 4) + 3
    raw_k = rng.normal(size=(T, Hkv, D))
    raw_v = rng.normal(size=(T, Hkv, D))
    wk = rng.normal(size=(hidden, Hkv * D)) / 3
    wv = rng.normal(size=(hidden, Hkv * D)) / 3
    scale = O.default_scale(D)
    mem = O.DraftMemory(S, W, r, Hkv, D, bf16_cache=False)
    slot_k, slot_v = [], []
    for t in range(1, T + 1):
        mem.append(raw_k[t - 1:t], raw_v[t - 1:t])
        m = mem.pending_boundary()
        if m:
            h = rng.normal(size=hidden)
            qg = rng.normal(size=(Hkv * G, D))
            og = mem.materialize(h, wk, wv, qg, scale)
            kg, vg = mem.slots[m]
            slot_k.append(kg)
            slot_v.append(vg)
            sk, sv = np.stack(slot_k), np.stack(slot_v)
            for hq in range(Hkv * G):
                ref = O.dense_mask_slot_query(qg[hq], raw_k[:t, hq // G], raw_v[:t, hq // G],
                                              sk[:, hq // G], sv[:, hq // G], m, S, W, r, scale)
                np.testing.assert_allclose(og[hq], ref, atol=1e-12)
        q = rng.normal(size=(Hkv * G, D))
        out = mem.decode(q, scale)
        sk = np.stack(slot_k) if slot_k else np.zeros((0, Hkv, D))
        sv = np.stack(slot_v) if slot_v else np.zeros((0, Hkv, D))
        for hq in range(Hkv * G):
            ref = O.dense_mask_decode(q[hq], raw_k[:t, hq // G], raw_v[:t, hq // G],
                                      sk[:, hq // G], sv[:, hq // G], t, S, W, r, scale)
            np.testing.assert_allclose(out[hq], ref, atol=1e-12)
        # I4: full attention while t <= S + W, bitwise (same keys, same order, same fp64 ops)
        if t <= S + W:
            full = O.fullkv_decode(q, raw_k[:t].transpose(1, 0, 2), raw_v[:t].transpose(1, 0, 2), t, scale)
            np.testing.assert_array_equal(out, full)


def test_include_self_bruteforce():
    rng = np.random.default_rng(3)
    S, W, r, D, Hkv, hidden = 2, 6, 3, 8, 1, 8
    T = S + W + 4 * r
    raw_k = rng.normal(size=(T, Hkv, D))
    raw_v = rng.normal(size=(T, Hkv, D))
    wk = rng.normal(size=(hidden, D))
    wv = rng.normal(size=(hidden, D))
    scale = O.default_scale(D)
    mem = O.DraftMemory(S, W, r, Hkv, D, bf16_cache=False)
    sk, sv = [], []
    for t in range(1, T + 1):
        mem.append(raw_k[t - 1:t], raw_v[t - 1:t])
        m = mem.pending_boundary()
        if m:
            qg = rng.normal(size=(1, D))
            og = mem.materialize(rng.normal(size=hidden), wk, wv, qg, scale, include_self=True)
            sk.append(mem.slots[m][0])
            sv.append(mem.slots[m][1])
            ref = O.dense_mask_slot_query(qg[0], raw_k[:t, 0], raw_v[:t, 0], np.stack(sk)[:, 0],
                                          np.stack(sv)[:, 0], m, S, W, r, scale, include_self=True)
            np.testing.assert_allclose(og[0], ref, atol=1e-12)
            assert len(O.slot_query_keylist(m, S, W, r, True)) == len(O.slot_query_keylist(m, S, W, r)) + 1


def test_one_hot_values_expose_the_support():
    """V of entry j = e_j: the output is the probability row, so it shows exactly which
    entries carry mass.  Excluded or evicted entries must carry none."""
    S, W, r, D = 4, 32, 16, 64
    rng = np.random.default_rng(11)
    mem = O.DraftMemory(S, W, r, 1, D, bf16_cache=False)
    T = 200
    K = rng.normal(size=(T, 1, D))
    for t in range(1, T + 1):
        mem.append(K[t - 1:t], np.zeros((1, 1, D)))
        if mem.pending_boundary():
            mem.materialize(rng.normal(size=D), np.eye(D), np.eye(D), rng.normal(size=(1, D)), 0.125)
    keys = O.keylist(T, S, W, r)
    assert len(keys) <= D
    for j, (kind, idx) in enumerate(keys):   # overwrite V of the visible entries by e_j
        e = np.zeros((1, D))
        e[0, j] = 1
        if kind == "raw":
            mem.raw[idx] = (mem.raw[idx][0], e)
        else:
            mem.slots[idx] = (mem.slots[idx][0], e)
    q = rng.normal(size=(1, D))
    out = mem.decode(q, 0.125)[0]
    assert abs(out.sum() - 1.0) < 1e-12
    assert (out[len(keys):] == 0).all()
    np.testing.assert_allclose(out[:len(keys)], mem.decode_weights(q[0], 0, 0.125), atol=1e-15)


# ---------------------------------------------------------------------------
# Mirrored projection and bf16 rounding
# ---------------------------------------------------------------------------

def test_projection_orientation_and_heads():
    rng = np.random.default_rng(5)
    hidden, Hkv, D = 12, 3, 4
    wk = rng.normal(size=(hidden, Hkv * D))
    wv = rng.normal(size=(hidden, Hkv * D))
    for i in range(hidden):
        e = np.zeros(hidden)
        e[i] = 1.0
        kg, vg = O.project_slot(e, wk, wv, Hkv, D, bf16_cache=False)
        # a one-hot hidden state selects row i of the weights; head k is column block k
        np.testing.assert_array_equal(kg, wk[i].reshape(Hkv, D))
        np.testing.assert_array_equal(vg, wv[i].reshape(Hkv, D))
    # copy-initialized mirrored weights reproduce the backbone's own key (library matmul)
    h = rng.normal(size=hidden)
    kg, _ = O.project_slot(h, wk, wv, Hkv, D, bf16_cache=False)
    ref = (torch.from_numpy(h)[None] @ torch.from_numpy(wk))[0].numpy().reshape(Hkv, D)
    np.testing.assert_allclose(kg, ref, atol=1e-12)


def test_to_bf16_matches_torch_and_ties():
    x = torch.randn(20000, dtype=torch.float32) * torch.logspace(-30, 30, 20000)
    ref = x.to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.to_bf16(x.double().numpy()), ref)
    # exact ties round to the even neighbour
    assert O.to_bf16(1.0 + 2.0 ** -8) == 1.0
    assert O.to_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert O.to_bf16(-(1.0 + 2.0 ** -8)) == -1.0
    # just above a tie rounds up; fp64 inputs are rounded once, not through fp32
    assert O.to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    # subnormal range and overflow
    assert O.to_bf16(2.0 ** -133) == 2.0 ** -133
    assert O.to_bf16(1.5 * 2.0 ** -134) == 2.0 ** -133
    assert O.to_bf16(3.0e38) == float(torch.tensor(3.0e38).to(torch.bfloat16))
    assert O.to_bf16(3.4e38) == np.inf and O.to_bf16(0.0) == 0.0


# ---------------------------------------------------------------------------
# Full-KV decode and verifier
# ---------------------------------------------------------------------------

def test_verify_matches_torch_masked_sdpa():
    rng = np.random.default_rng(9)
    n_q, Hq, Hkv, N, D = 6, 8, 2, 50, 16
    t = 45
    q = rng.normal(size=(n_q, Hq, D))
    K = rng.normal(size=(Hkv, N, D))
    V = rng.normal(size=(Hkv, N, D))
    scale = O.default_scale(D)
    out = O.fullkv_verify(q, K, V, t, scale)
    # explicit boolean mask: query j may see key rows 0 .. t - n_q + j (bottom-right aligned)
    mask = np.zeros((n_q, t), dtype=bool)
    for j in range(n_q):
        mask[j, : t - n_q + 1 + j] = True
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq][n_q][D]
    kt = torch.from_numpy(K[:, :t]).repeat_interleave(G, 0)
    vt = torch.from_numpy(V[:, :t]).repeat_interleave(G, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=scale).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, atol=1e-13)
    # the last query sees every key, the first sees n_q - 1 fewer
    np.testing.assert_allclose(out[-1], O.fullkv_decode(q[-1], K, V, t, scale), atol=0)
    np.testing.assert_allclose(out[0], O.fullkv_decode(q[0], K, V, t - n_q + 1, scale), atol=0)


def test_project_slot_batch_rows_are_independent():
    rng = np.random.default_rng(12)
    hidden, Hkv, D = 16, 2, 4
    wk = rng.normal(size=(hidden, Hkv * D))
    wv = rng.normal(size=(hidden, Hkv * D))
    H = rng.normal(size=(3, hidden))
    kb, vb = O.project_slot(H, wk, wv, Hkv, D, bf16_cache=True)
    assert kb.shape == (3, Hkv, D)
    for i in range(3):
        k1, v1 = O.project_slot(H[i], wk, wv, Hkv, D, bf16_cache=True)
        np.testing.assert_array_equal(kb[i], k1)
        np.testing.assert_array_equal(vb[i], v1)


# ---------------------------------------------------------------------------
# Rollback after verification (reading R9, [TR] §3.3 Algorithm 2 step 6)
# ---------------------------------------------------------------------------

def _speculative_run(S, W, r, L_draft, iters, seed):
    """Draft L_draft tokens per iteration (materializing at boundaries), accept a random
    prefix, roll back; returns the memory and the accepted token stream."""
    rng = np.random.default_rng(seed)
    D, Hkv, hidden = 4, 1, 4
    wk, wv = rng.normal(size=(hidden, Hkv * D)), rng.normal(size=(hidden, Hkv * D))
    h_of = {m: rng.normal(size=hidden) for m in range(1, 400)}
    q_of = {m: rng.normal(size=(1, D)) for m in range(1, 400)}
    mem = O.DraftMemory(S, W, r, Hkv, D, bf16_cache=False)
    accepted = []                         # (k, v) per accepted position
    for _ in range(iters):
        t0 = mem.t
        draft = [(rng.normal(size=(Hkv, D)), rng.normal(size=(Hkv, D))) for _ in range(L_draft)]
        for k, v in draft:
            mem.append(k[None], v[None])
            m = mem.pending_boundary()
            if m:
                mem.materialize(h_of[m], wk, wv, q_of[m], 0.5)
        n_acc = int(rng.integers(0, L_draft + 1))
        mem.rollback(t0 + n_acc)
        accepted += draft[:n_acc]
        # the target's correction token is the next accepted one
        k, v = rng.normal(size=(Hkv, D)), rng.normal(size=(Hkv, D))
        mem.append(k[None], v[None])
        m = mem.pending_boundary()
        if m:
            mem.materialize(h_of[m], wk, wv, q_of[m], 0.5)
        accepted.append((k, v))
    return mem, accepted, (wk, wv, h_of, q_of)


@pytest.mark.parametrize("S,W,r,L", [(2, 8, 4, 5), (0, 6, 2, 3), (4, 16, 8, 5), (1, 4, 1, 4), (3, 8, 0, 5)])
def test_rollback_equals_appending_only_accepted_tokens(S, W, r, L):
    mem, accepted, (wk, wv, h_of, q_of) = _speculative_run(S, W, r, L, iters=40, seed=S * 7 + W + r)
    ref = O.DraftMemory(S, W, r, 1, 4, bf16_cache=False)
    for k, v in accepted:
        ref.append(k[None], v[None])
        m = ref.pending_boundary()
        if m:
            ref.materialize(h_of[m], wk, wv, q_of[m], 0.5)
    assert mem.t == ref.t == len(accepted)
    assert sorted(mem.raw) == sorted(ref.raw) and sorted(mem.slots) == sorted(ref.slots)
    for i in ref.raw:
        np.testing.assert_array_equal(mem.raw[i][0], ref.raw[i][0])
    for m in ref.slots:
        np.testing.assert_array_equal(mem.slots[m][0], ref.slots[m][0])
        np.testing.assert_array_equal(mem.slots[m][1], ref.slots[m][1])
    q = np.random.default_rng(1).normal(size=(1, 4))
    np.testing.assert_array_equal(mem.decode(q, 0.5), ref.decode(q, 0.5))


def _ring_run(S, W, r, R, depth, seed=3):
    """Literal FIFO ring of W + r + R cells driven through speculation of `depth`
    positions and rollback; returns False as soon as a token the accepted memory needs
    is not in its cell (or an append is illegal)."""
    rng = np.random.default_rng(seed)
    C = O.ring_capacity(W, r, R)
    cells = [None] * C
    t, n_slots = 0, 0

    def put(i, n):
        if i > S:
            if not O.append_is_legal(i, n, S, W, r, R):
                return False
            cells[O.ring_cell(i, S, W, r, R)] = i
        return True

    def resident(t):
        need = [i for kind, i in O.keylist(t, S, W, r) if kind == "raw" and i > S]
        m = O.is_boundary(t, S, W, r)
        if m:
            need += [i for kind, i in O.slot_query_keylist(m, S, W, r) if kind == "raw" and i > S]
        return all(cells[O.ring_cell(i, S, W, r, R)] == i for i in need)

    for _ in range(60):
        n_spec = n_slots
        for j in range(1, depth + 1):          # speculative appends
            if not put(t + j, n_spec) or not resident(t + j):
                return False
            if O.is_boundary(t + j, S, W, r):
                n_spec += 1
        acc = int(rng.integers(0, depth + 1))
        for j in range(1, acc + 2):            # accepted prefix + correction, re-appended
            if not put(t + j, n_slots) or not resident(t + j):
                return False
            if O.is_boundary(t + j, S, W, r):
                n_slots += 1
        t += acc + 1
    return True


@pytest.mark.parametrize("S,W,r,R", [(2, 8, 4, 5), (0, 6, 2, 3), (4, 16, 8, 16), (1, 4, 1, 4), (3, 8, 0, 5)])
def test_rollback_rows_keep_needed_tokens_resident(S, W, r, R):
    """With W + r + R ring rows any speculation of up to R positions can be undone without
    moving data (R + 1 as well: the next position is always appended before the next
    query reads); R + 2 can lose a token the next query needs (the oldest of a
    boundary's slot-query window, or without a slot chain the oldest of the window)."""
    assert _ring_run(S, W, r, R, depth=R)
    assert _ring_run(S, W, r, R, depth=R + 1)
    assert not all(_ring_run(S, W, r, R, depth=R + 2, seed=sd) for sd in range(8))


# ---------------------------------------------------------------------------
# Draft prefill (reading R10, [TR] §3.3 Algorithm 2 step 2)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S,W,r", [(2, 8, 4), (0, 5, 2), (4, 16, 8), (3, 6, 0)])
def test_prefill_equals_token_by_token_decoding(S, W, r):
    """One pass over the prefix gives exactly what appending and decoding one token at a
    time (materializing at every boundary) gives: same keys, same order, same fp64 ops."""
    rng = np.random.default_rng(S + 10 * W + 100 * r)
    P, Hkv, G, D, hidden = 60, 2, 3, 4, 6
    raw_k, raw_v = rng.normal(size=(P, Hkv, D)), rng.normal(size=(P, Hkv, D))
    q = rng.normal(size=(P, Hkv * G, D))
    n = O.visible_slot_count(P, S, W, r)
    h = rng.normal(size=(max(n, 1), hidden))
    wk, wv = rng.normal(size=(hidden, Hkv * D)), rng.normal(size=(hidden, Hkv * D))
    q_slot = rng.normal(size=(max(n, 1), Hkv * G, D))[:n]
    # one row at a time, as materialize projects (a batched BLAS product rounds differently)
    rows = [O.project_slot(h[m], wk, wv, Hkv, D, bf16_cache=False) for m in range(n)]
    slot_k = np.stack([k for k, _ in rows]) if n else np.zeros((0, Hkv, D))
    slot_v = np.stack([v for _, v in rows]) if n else np.zeros((0, Hkv, D))
    scale = 0.37
    out, o_slot = O.prefill_attend(raw_k, raw_v, slot_k, slot_v, q, q_slot, S, W, r, scale)
    mem = O.DraftMemory(S, W, r, Hkv, D, bf16_cache=False)
    for i in range(1, P + 1):
        mem.append(raw_k[i - 1:i], raw_v[i - 1:i])
        m = mem.pending_boundary()
        if m:
            og = mem.materialize(h[m - 1], wk, wv, q_slot[m - 1], scale)
            np.testing.assert_array_equal(og, o_slot[m - 1])
        np.testing.assert_array_equal(mem.decode(q[i - 1], scale), out[i - 1])
    assert len(mem.slots) == n


def test_prefill_dense_mask_bruteforce():
    """The same prefill from masks over every entry ever created, written separately."""
    S, W, r, P, D = 2, 6, 3, 40, 5
    rng = np.random.default_rng(9)
    raw_k, raw_v = rng.normal(size=(P, 1, D)), rng.normal(size=(P, 1, D))
    n = O.visible_slot_count(P, S, W, r)
    slot_k, slot_v = rng.normal(size=(n, 1, D)), rng.normal(size=(n, 1, D))
    q, q_slot = rng.normal(size=(P, 1, D)), rng.normal(size=(n, 1, D))
    out, o_slot = O.prefill_attend(raw_k, raw_v, slot_k, slot_v, q, q_slot, S, W, r, 0.5)
    for i in range(1, P + 1):
        ref = O.dense_mask_decode(q[i - 1, 0], raw_k[:i, 0], raw_v[:i, 0], slot_k[:, 0], slot_v[:, 0],
                                  i, S, W, r, 0.5)
        np.testing.assert_allclose(out[i - 1, 0], ref, atol=1e-12)
    for m in range(1, n + 1):
        tm = O.boundary_step(m, S, W, r)
        ref = O.dense_mask_slot_query(q_slot[m - 1, 0], raw_k[:tm, 0], raw_v[:tm, 0], slot_k[:m, 0],
                                      slot_v[:m, 0], m, S, W, r, 0.5)
        np.testing.assert_allclose(o_slot[m - 1, 0], ref, atol=1e-12)


def test_prefill_subset_rows_equal_the_full_pass():
    """Restricting the prefill to some queries gives those rows of the full pass exactly
    and leaves the others zero (the GPU tests sample rows at full size this way)."""
    S, W, r, P, D = 2, 6, 3, 40, 5
    rng = np.random.default_rng(11)
    raw_k, raw_v = rng.normal(size=(P, 2, D)), rng.normal(size=(P, 2, D))
    n = O.visible_slot_count(P, S, W, r)
    slot_k, slot_v = rng.normal(size=(n, 2, D)), rng.normal(size=(n, 2, D))
    q, q_slot = rng.normal(size=(P, 4, D)), rng.normal(size=(n, 4, D))
    full, full_s = O.prefill_attend(raw_k, raw_v, slot_k, slot_v, q, q_slot, S, W, r, 0.5)
    pos, sl = [1, 7, 9, 40], [2, n]
    part, part_s = O.prefill_attend(raw_k, raw_v, slot_k, slot_v, q, q_slot, S, W, r, 0.5,
                                    positions=pos, slots=sl)
    for i in range(1, P + 1):
        np.testing.assert_array_equal(part[i - 1], full[i - 1] if i in pos else 0.0)
    for m in range(1, n + 1):
        np.testing.assert_array_equal(part_s[m - 1], full_s[m - 1] if m in sl else 0.0)


# ---------------------------------------------------------------------------
# Rotary position of slot keys (reading R11, [TR] §3.2 Algorithm 1 step 6)
# ---------------------------------------------------------------------------

def test_rope_hand_example():
    """D = 4, theta = 100, id 3, both pairings, worked by hand (tests/golden)."""
    g = json.load(open(os.path.join(GOLDEN, "rope_hand_example.json")))
    x = np.array(g["x"])
    np.testing.assert_allclose(O.rope_rotate(x, g["pos"], g["theta"], O.ROPE_ROTATE_HALF), g["rotate_half"],
                               atol=g["tolerance"])
    np.testing.assert_allclose(O.rope_rotate(x, g["pos"], g["theta"], O.ROPE_INTERLEAVED), g["interleaved"],
                               atol=g["tolerance"])
    for c in g["slot_ids"]:
        assert O.slot_position_id(c["m"], c["S"], c["r"]) == c["id"]


@pytest.mark.parametrize("style", [0, 1])
def test_rope_is_a_complex_phase(style):
    """Written as complex numbers z = x_a + i x_b, the rotation multiplies each pair by
    exp(i pos theta^(-2i/D)) - a formulation independent of the sin/cos lines."""
    rng = np.random.default_rng(3 + style)
    D, theta = 16, 500000.0
    x = rng.normal(size=(3, D))
    for pos in (0, 1, 7, 40000):
        y = O.rope_rotate(x, pos, theta, style)
        if style == O.ROPE_ROTATE_HALF:
            a, b = np.arange(D // 2), np.arange(D // 2) + D // 2
        else:
            a, b = np.arange(0, D, 2), np.arange(1, D, 2)
        z = (x[:, a] + 1j * x[:, b]) * np.exp(1j * pos * theta ** (-2.0 * np.arange(D // 2) / D))
        np.testing.assert_allclose(y[:, a], z.real, atol=1e-12)
        np.testing.assert_allclose(y[:, b], z.imag, atol=1e-12)


@pytest.mark.parametrize("style", [0, 1])
def test_rope_relative_position_and_norm(style):
    """<R(p) q, R(p') k> depends on p - p' only, rotations keep norms, id 0 is the identity."""
    rng = np.random.default_rng(11 + style)
    D, theta = 128, 10000.0
    q, k = rng.normal(size=D), rng.normal(size=D)
    for p, pp in ((5, 2), (3000, 2997), (70, 9)):
        lhs = O.rope_rotate(q, p, theta, style) @ O.rope_rotate(k, pp, theta, style)
        rhs = O.rope_rotate(q, p - pp, theta, style) @ k
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))
        assert abs(np.linalg.norm(O.rope_rotate(q, p, theta, style)) - np.linalg.norm(q)) < 1e-12 * D
    np.testing.assert_array_equal(O.rope_rotate(q, 0, theta, style), q)


def test_rope_pairings_differ_by_a_permutation():
    """Interleaved pairs are the rotate-half pairs after moving component i + D/2 next
    to component i."""
    rng = np.random.default_rng(21)
    D = 8
    x = rng.normal(size=D)
    perm = np.empty(D, dtype=int)
    perm[0::2], perm[1::2] = np.arange(D // 2), np.arange(D // 2) + D // 2   # interleaved slot -> half slot
    y_half = O.rope_rotate(x, 9, 100.0, O.ROPE_ROTATE_HALF)
    y_int = O.rope_rotate(x[perm], 9, 100.0, O.ROPE_INTERLEAVED)
    np.testing.assert_allclose(y_int, y_half[perm], atol=1e-12)


def test_slot_position_id_is_the_next_raw_tokens_id():
    """g_m shares its id with the raw token right after its block (0-based ids: raw
    position i has id i - 1), so it is one past every id in B_m and equals no later raw
    token's id but that one."""
    for S, r in ((0, 1), (4, 64), (3, 5)):
        for m in range(1, 9):
            blk = O.block_positions(m, S, r)
            sid = O.slot_position_id(m, S, r)
            assert sid == (blk[-1] + 1) - 1
            assert all(sid > i - 1 for i in blk)
    with pytest.raises(ValueError):
        O.slot_position_id(1, 4, 0)


@pytest.mark.parametrize("style", [0, 1])
def test_materialize_rotates_slot_keys_only(style):
    """A memory with a rotary base stores R(id(g_m)) K_g and the plain V_g; theta 0 is the
    memory without rotation."""
    rng = np.random.default_rng(31 + style)
    S, W, r, Hkv, G, D, hidden = 2, 6, 3, 2, 2, 8, 5
    wk, wv = rng.normal(size=(hidden, Hkv * D)), rng.normal(size=(hidden, Hkv * D))
    plain = O.DraftMemory(S, W, r, Hkv, D, bf16_cache=False)
    rot = O.DraftMemory(S, W, r, Hkv, D, bf16_cache=False, rope_theta=1000.0, rope_style=style)
    off = O.DraftMemory(S, W, r, Hkv, D, bf16_cache=False, rope_theta=0.0, rope_style=style)
    for t in range(1, 20):
        kv = rng.normal(size=(2, 1, Hkv, D))
        h, qg = rng.normal(size=hidden), rng.normal(size=(Hkv * G, D))
        for mem in (plain, rot, off):
            mem.append(kv[0], kv[1])
            mem.materialize(h, wk, wv, qg, 0.5)
    assert len(rot.slots) == 3   # boundaries 11, 14, 17
    for m, (kg, vg) in plain.slots.items():
        np.testing.assert_array_equal(rot.slots[m][1], vg)
        np.testing.assert_allclose(rot.slots[m][0], O.rope_rotate(kg, O.slot_position_id(m, S, r), 1000.0, style),
                                   atol=1e-12)
        np.testing.assert_array_equal(off.slots[m][0], kg)
