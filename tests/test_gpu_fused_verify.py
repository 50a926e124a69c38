"""GPU parity of the fused decode steps, the verifier attention and graph replay.

* masw_decode_step / fullkv_decode_step (append fused into the attention launch) must
  give outputs and memory contents bitwise equal to the separate calls, and match the
  oracle along a decode loop.
* fullkv_verify_attn against the oracle's verifier: the 8B- and 70B-shaped layers at
  prefix 32768 (sampled sequences), ragged small prefixes, t = n_q, several n_q, the
  vector-ALU fallback shapes, and the out-of-range case.
* A decode step captured in a HIP graph and replayed several times, with eager work in
  between, matches eager execution every time.
"""
import numpy as np
import pytest
import torch

import draft_kv_attention_amd as M
import seeded_inputs as SI
from oracle import masw_oracle as O
from tests.gpu_driver import LayerDriver, np_in, shape_of
from tests.parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.lib()


# ---------------------------------------------------------------------------
# fused decode step == separate append + attention (bitwise), and == oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape,T,splits", [(SI.TINY, 240, 3), (shape_of(SI.DRAFT_3B, batch=2), 2300, 0)])
def test_masw_decode_step_matches_separate_calls(shape, T, splits):
    S, W, r = shape.sink, shape.window, shape.interval
    maxs = O.visible_slot_count(T, S, W, r) + 2
    sep = LayerDriver(shape, max_slots=maxs, seed=21, num_splits=splits, oracle=False)
    fus = LayerDriver(shape, max_slots=maxs, seed=21, num_splits=splits)
    start = S + W - 3
    sep.advance_to(start)
    fus.advance_to(start)
    tol = torch.float32 if shape.dtype == torch.float32 else torch.bfloat16
    for t in range(start + 1, T + 1):
        k, v = SI.token_kv(shape, 21, 0, t, 1)
        q = SI.decode_query(shape, 21, 0, t).to(DEV)
        for drv in (sep, fus):
            drv.seq.seq_len.fill_(t)
            drv.t = t
            drv.tokens_k[t], drv.tokens_v[t] = np_in(k)[:, 0], np_in(v)[:, 0]
        for b, mem in enumerate(fus.mems):
            mem.append(np_in(k)[b], np_in(v)[b])
        M.masw_evict_append(sep.d, sep.layer, sep.seq, k.to(DEV), v.to(DEV))
        if O.is_boundary(t, S, W, r):
            sep.materialize(check=False)
            fus.materialize(check=True)
        out_s = torch.empty_like(q)
        out_f = torch.empty_like(q)
        M.masw_draft_attn(sep.d, sep.layer, sep.seq, q, out_s, sep.ws)
        M.masw_decode_step(fus.d, fus.layer, fus.seq, k.to(DEV), v.to(DEV), q, out_f, fus.ws)
        assert torch.equal(out_s, out_f), f"t={t}"
        if t % 7 == 0 or t == T:
            ref = np.stack([mem.decode(np_in(q).astype(np.float64)[b], fus.scale)
                            for b, mem in enumerate(fus.mems)])
            assert_close(out_f, ref, tol, f"fused decode t={t}")
    for name in ("k_ring", "v_ring", "k_sink", "v_sink", "k_slot", "v_slot", "n_slots"):
        a, b = getattr(sep.layer, name), getattr(fus.layer, name)
        assert torch.equal(torch.nan_to_num(a.float(), 7.0), torch.nan_to_num(b.float(), 7.0)), name
    assert sep.err() == 0 and fus.err() == 0


def test_fullkv_decode_step_matches_separate_calls():
    B, Hq, Hkv, D, N = 3, 24, 8, 128, 2500
    d = M.Dims(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, dtype=torch.bfloat16)
    k0, v0 = SI.full_cache(B, Hkv, N, D, seed=22, dtype=torch.bfloat16)
    ks, vs = k0.to(DEV), v0.to(DEV)
    kf, vf = ks.clone(), vs.clone()
    seq = torch.tensor([5, 1000, 2400], dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = M.workspace(d, M.OP_FULLKV_DECODE, max_keys=N, device=DEV)
    for step in range(40):
        seq += 1
        kn = SI.normal((B, 1, Hkv, D), 100 + step, dtype=torch.bfloat16).to(DEV)
        vn = SI.normal((B, 1, Hkv, D), 200 + step, dtype=torch.bfloat16).to(DEV)
        q = SI.normal((B, Hq, D), 300 + step, dtype=torch.bfloat16).to(DEV)
        o1, o2 = torch.empty_like(q), torch.empty_like(q)
        M.fullkv_append(d, ks, vs, seq, err, kn, vn)
        M.fullkv_decode_attn(d, ks, vs, seq, err, q, o1, ws)
        M.fullkv_decode_step(d, kf, vf, seq, err, kn, vn, q, o2, ws)
        assert torch.equal(o1, o2), step
    assert torch.equal(ks, kf) and torch.equal(vs, vf)
    assert int(err.item()) == 0
    kn_, vn_, qn = np_in(ks), np_in(vs), np_in(q).astype(np.float64)
    for b, t in enumerate(seq.tolist()):
        assert_close(o2[b], O.fullkv_decode(qn[b], kn_[b], vn_[b], t, O.default_scale(D)),
                     torch.bfloat16, f"b={b}")


# ---------------------------------------------------------------------------
# verifier attention
# ---------------------------------------------------------------------------

def _verify_case(B, Hq, Hkv, D, n_q, ts, max_len, dtype, seed, check_b=None, splits=0):
    d = M.Dims(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, dtype=dtype, num_splits=splits)
    k, v = SI.full_cache(B, Hkv, max_len, D, seed=seed, dtype=dtype, device=DEV)
    q = SI.normal((B, n_q, Hq, D), seed + 1, dtype=dtype, device=DEV)
    seq = torch.tensor(ts, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.full_like(q, float("nan"))
    ws = M.workspace(d, M.OP_FULLKV_VERIFY, max_keys=max_len, n_q=n_q, device=DEV)
    M.fullkv_verify_attn(d, k, v, seq, err, q, out, ws)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    scale = O.default_scale(D)
    got_all, ref_all = [], []
    for b in (check_b if check_b is not None else range(B)):
        kn, vn = np_in(k[b]), np_in(v[b])
        ref = O.fullkv_verify(np_in(q[b]).astype(np.float64), kn, vn, ts[b], scale)
        assert_close(out[b], ref, dtype, f"verify b={b} t={ts[b]}")
        got_all.append(np_in(out[b]).astype(np.float64).ravel())
        ref_all.append(np.asarray(ref, np.float64).ravel())
    return out, np.concatenate(got_all), np.concatenate(ref_all)


@pytest.mark.parametrize("Hq", [32, 64])
def test_verify_full_size(Hq):
    """One GPU's share of an 8B / 70B verifier layer: 8 KV heads, prefix 32768 + 6."""
    sh = SI.VERIFY_8B if Hq == 32 else SI.VERIFY_70B
    t = sh.prefix + sh.n_query
    _, got, ref = _verify_case(sh.batch, sh.n_q_heads, sh.n_kv_heads, sh.head_dim, sh.n_query, [t] * sh.batch,
                               t + 10, torch.bfloat16, seed=31, check_b=[0, sh.batch - 1])
    # error budget of the bf16 path (P rounded to bf16 for P.V, fp32 accumulation, a bf16
    # output) against the rounding of the exact output alone
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    rel_round = np.linalg.norm(O.to_bf16(ref) - ref) / np.linalg.norm(ref)
    print(f"verifier {Hq}q: rel-L2 {rel:.3e} (bf16 rounding of the exact output alone: {rel_round:.3e}), "
          f"max abs {np.abs(got - ref).max():.3e}")
    assert rel <= 2.0 * rel_round, (rel, rel_round)


@pytest.mark.parametrize("Hq", [32, 64])
def test_verify_score_growth_restarts(Hq):
    """Keys whose scores pass everything seen before by 200-400 log2 units, in later tiles
    of a wave's range (two of them in one wave): weights taken against a reference max set
    by the first tiles would overflow fp32, so the kernel must raise it on the way (and
    rescale what it has accumulated) to match the oracle."""
    B, Hkv, D, n_q, t, splits = 2, 8, 128, 6, 5000, 16
    G = Hq // Hkv
    k, v = SI.full_cache(B, Hkv, t + 8, D, seed=41, dtype=torch.bfloat16)
    q = SI.normal((B, n_q, Hq, D), 42, dtype=torch.bfloat16)
    scale = O.default_scale(D)
    qh = q[0, 0, 3 * G].double()
    # 16 splits asked for: chunks of 384 keys (96 per wave, tiles of 32), so keys 1876 /
    # 1910 are tiles 1 / 2 of split 4's last wave and 4200 is tile 2 of split 10's
    for pos, target in ((1876, 200.0), (1910, 400.0), (4200, 300.0)):
        kk = qh * (target / (scale * np.log2(np.e)) / float(qh @ qh))
        k[0, 3, pos] = kk.to(torch.bfloat16)
    d = M.Dims(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, dtype=torch.bfloat16, num_splits=splits)
    kd, vd, qd = k.to(DEV), v.to(DEV), q.to(DEV)
    seq = torch.full((B,), t, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.full_like(qd, float("nan"))
    M.fullkv_verify_attn(d, kd, vd, seq, err, qd, out, M.workspace(d, M.OP_FULLKV_VERIFY, max_keys=t + 8, n_q=n_q,
                                                                   device=DEV))
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for b in range(B):
        ref = O.fullkv_verify(np_in(q[b]).astype(np.float64), np_in(k[b]), np_in(v[b]), t, scale)
        assert_close(out[b], ref, torch.bfloat16, f"verify b={b}")
    # the key planted last dominates candidate 0 of head 3G: its output is that value row
    assert torch.allclose(out[0, 0, 3 * G].float().cpu(), v[0, 3, 1910].float(), atol=2e-2)


@pytest.mark.parametrize("Hq,Hkv,n_q", [(24, 8, 6), (32, 8, 6), (64, 8, 6), (8, 8, 1), (32, 8, 16),
                                        (64, 8, 8), (24, 8, 2), (24, 8, 11), (24, 8, 12), (32, 8, 9),
                                        (24, 8, 16)])
def test_verify_ragged_small(Hq, Hkv, n_q):
    """Rows per (sequence, KV head) R = G n_q of 6 to 64: one or two 32-row blocks, or three
    16-row blocks for R in (32, 48] (33, 36 and 36 rows with padded tails, and 48 rows as
    8 heads x 6 candidates or 3 heads x 16)."""
    ts = [n_q, n_q + 1, 31, 33, 100, 1000, 3000]
    _verify_case(len(ts), Hq, Hkv, 128, n_q, ts, 3100, torch.bfloat16, seed=32)


@pytest.mark.parametrize("dtype,D,Hq,n_q", [(torch.float32, 64, 2, 6), (torch.bfloat16, 64, 24, 6),
                                            (torch.bfloat16, 128, 64, 16), (torch.float32, 128, 24, 3)])
def test_verify_vector_alu_shapes(dtype, D, Hq, n_q):
    ts = [n_q, 40, 777]
    _verify_case(len(ts), Hq, 8 if Hq % 8 == 0 else 1, D, n_q, ts, 800, dtype, seed=33)


@pytest.mark.parametrize("splits", [3, 12, 33, 64])
@pytest.mark.parametrize("Hq,n_q", [(32, 6), (64, 6), (64, 8)])
def test_verify_split_plans(splits, Hq, n_q):
    """Split plans whose combine pass folds more than one batch of eight partials (up to
    the MFMA verifier's 64), with causal rows whose last splits see no key."""
    ts = [n_q, 2100, 5000]
    _verify_case(len(ts), Hq, 8, 128, n_q, ts, 5010, torch.bfloat16, seed=36, splits=splits)


def test_verify_out_of_range():
    d = M.Dims(batch=2, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype=torch.bfloat16)
    k, v = SI.full_cache(2, 8, 64, 128, seed=34, dtype=torch.bfloat16, device=DEV)
    q = SI.normal((2, 6, 32, 128), 35, dtype=torch.bfloat16, device=DEV)
    seq = torch.tensor([5, 65], dtype=torch.int32, device=DEV)   # t < n_q, t > max_len
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.full_like(q, 3.0)
    M.fullkv_verify_attn(d, k, v, seq, err, q, out, M.workspace(d, M.OP_FULLKV_VERIFY, 64, 6, device=DEV))
    assert int(err.item()) & M.DEV_SEQ_RANGE
    assert bool((out == 3.0).all())


def test_verify_deterministic_and_counters_reset():
    sh = SI.VERIFY_8B
    d = M.Dims(batch=2, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype=torch.bfloat16)
    k, v = SI.full_cache(2, 8, 9000, 128, seed=36, dtype=torch.bfloat16, device=DEV)
    q = SI.normal((2, 6, 32, 128), 37, dtype=torch.bfloat16, device=DEV)
    seq = torch.tensor([8000, 8999], dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = M.workspace(d, M.OP_FULLKV_VERIFY, 9000, 6, device=DEV)
    outs = []
    for _ in range(3):
        o = torch.empty_like(q)
        M.fullkv_verify_attn(d, k, v, seq, err, q, o, ws)
        outs.append(o)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    # every ticket counter is back at zero (the bytes right after the per-sequence flags)
    assert int(ws[256:256 + 4 * 2 * 8].view(torch.int32).abs().sum().item()) == 0


# ---------------------------------------------------------------------------
# HIP graph replay of a decode step
# ---------------------------------------------------------------------------

def test_graph_replay_matches_eager():
    shape = shape_of(SI.DRAFT_3B, batch=2)
    drv = LayerDriver(shape, max_slots=40, seed=41, oracle=False)
    drv.advance_to(3000)
    q = SI.decode_query(shape, 41, 0, 1).to(DEV)
    out = torch.empty_like(q)
    kn, vn = SI.token_kv(shape, 41, 0, 3001, 1)
    kn, vn = kn.to(DEV), vn.to(DEV)
    drv.seq.seq_len.fill_(3001)
    ring0 = drv.layer.k_ring.clone()
    M.masw_decode_step(drv.d, drv.layer, drv.seq, kn, vn, q, out, drv.ws)
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            M.masw_decode_step(drv.d, drv.layer, drv.seq, kn, vn, q, out, drv.ws)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(4):
        out.fill_(float("nan"))
        drv.layer.k_ring.copy_(ring0)       # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
    assert drv.err() == 0
