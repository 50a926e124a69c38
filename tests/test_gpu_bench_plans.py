"""GPU parity at the benchmark's own launch configurations and default split plans.

- Full-KV decode step (fused append of position t + 1 and attention) at batch 8 and a
  32768-token prefix, the 3B draft layer share (24 query / 8 KV heads, D = 128, bf16):
  the default plan there is 4 splits of 8192 keys per (sequence, KV head).
- The batch-1 workload at prefix 8192 (K, V ~ 0.5 N(0, 1)), built exactly as the bench
  builds it (the MASW memory holds the full cache's own sink and window rows plus
  projected slots): MASW decode step with its default 17 splits, full-KV with 32.

Sampled (sequence, KV head) units are compared with the fp64 oracle's attention over
the same rows; every query head of each sampled unit.  The default plan is pinned by a
second call with that split count given explicitly, which must produce the same bits
(the split count fixes the reduction order).
"""
import dataclasses

import numpy as np
import pytest
import torch

import bench
import draft_kv_attention_amd as M
import seeded_inputs as SI
from oracle import masw_oracle as O
from tests.gpu_driver import np_in
from tests.parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.lib()


def _fullkv_step_check(d, kf, vf, t, k_new, v_new, q, units, splits):
    """One fused full-KV step appending position t; sampled units against the oracle,
    then the same step with num_splits = splits must give the same bits."""
    B, Hq, Hkv, D = d.batch, d.n_q_heads, d.n_kv_heads, d.head_dim
    G = Hq // Hkv
    max_len = kf.shape[2]
    snap = {(b, h): (kf[b, h, :t - 1].float().cpu().numpy(), vf[b, h, :t - 1].float().cpu().numpy()) for b, h in units}
    seq_len = torch.full((B,), t, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    ws = M.workspace(d, M.OP_FULLKV_DECODE, max_keys=max_len, device=DEV)
    M.fullkv_decode_step(d, kf, vf, seq_len, err, k_new, v_new, q, out, ws)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    qn = np_in(q).astype(np.float64)
    kn, vn = np_in(k_new), np_in(v_new)
    for b, kvh in units:
        K = np.concatenate([snap[(b, kvh)][0], kn[b, :, kvh]], axis=0)
        V = np.concatenate([snap[(b, kvh)][1], vn[b, :, kvh]], axis=0)
        assert K.shape[0] == t
        for g in range(G):
            h = kvh * G + g
            ref = O.attend(qn[b, h], K, V, d.softmax_scale)
            assert_close(out[b, h], ref, torch.bfloat16, f"full-KV b={b} h={h} t={t}")
    # the new token landed in row t - 1
    assert torch.equal(kf[:, :, t - 1], k_new[:, 0])
    d2 = dataclasses.replace(d, num_splits=splits)
    out2 = torch.empty_like(out)
    M.fullkv_decode_step(d2, kf, vf, seq_len, err, k_new, v_new, q, out2,
                         M.workspace(d2, M.OP_FULLKV_DECODE, max_keys=max_len, device=DEV))
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(out, out2), f"default plan is not {splits} splits"


def test_fullkv_decode_bench_plan_b8_prefix32768():
    sh = SI.SWEEP_3B
    B, Hq, Hkv, D = sh.batch, sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    t = bench.T_HEAD + 1                       # the headline step appends position 32769
    max_len = bench.T_HEAD + 8
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    kf = torch.randn(B, Hkv, max_len, D, generator=g, device=DEV).to(torch.bfloat16)
    vf = torch.randn(B, Hkv, max_len, D, generator=g, device=DEV).to(torch.bfloat16)
    k_new = torch.randn(B, 1, Hkv, D, generator=g, device=DEV).to(torch.bfloat16)
    v_new = torch.randn(B, 1, Hkv, D, generator=g, device=DEV).to(torch.bfloat16)
    q = torch.randn(B, Hq, D, generator=g, device=DEV).to(torch.bfloat16)
    d = M.Dims(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, dtype=torch.bfloat16)
    _fullkv_step_check(d, kf, vf, t, k_new, v_new, q, units=[(0, 0), (3, 5), (7, 7)], splits=4)


def test_batch1_prefix8192_bench_plans():
    sh, t0 = SI.DRAFT_3B, SI.DRAFT_3B_PREFIX
    st = bench.Stack(sh, t0 + 64, torch.device(DEV), seed=1)
    st.set_position(t0)
    st.mirror_full_into_masw(t0)
    t = t0 + 1                                  # the timed step appends position 8193
    assert not bench.is_boundary(t, sh.sink, sh.window, sh.interval)
    S, W, r = sh.sink, sh.window, sh.interval
    G = sh.group
    lay = st.layers[1]
    # MASW: fused append + draft attention, default plan (17 splits at this size)
    st.seq.seq_len.fill_(t)
    snap = {n: getattr(lay, n).float().cpu().numpy() for n in ("k_sink", "v_sink", "k_ring", "v_ring", "k_slot", "v_slot")}
    M.masw_decode_step(st.d, lay, st.seq, st.k_new[1], st.v_new[1], st.q[1], st.out[1], st.ws)
    torch.cuda.synchronize()
    assert int(st.seq.err.item()) == 0
    keys = O.physical_keylist(t, S, W, r)
    assert len(keys) == S + W + O.visible_slot_count(t, S, W, r) == 2147
    kn, vn = np_in(st.k_new[1]), np_in(st.v_new[1])
    qn = np_in(st.q[1]).astype(np.float64)
    for kvh in range(sh.n_kv_heads):
        K = np.empty((len(keys), sh.head_dim))
        V = np.empty_like(K)
        for j, (seg, row, ident) in enumerate(keys):
            if seg != 2 and ident == t:
                K[j], V[j] = kn[0, 0, kvh], vn[0, 0, kvh]
            else:
                name = ("sink", "ring", "slot")[seg]
                K[j], V[j] = snap["k_" + name][0, kvh, row], snap["v_" + name][0, kvh, row]
        for g in range(G):
            h = kvh * G + g
            ref = O.attend(qn[0, h], K, V, st.d.softmax_scale)
            assert_close(st.out[1][0, h], ref, torch.bfloat16, f"MASW h={h}")
    out_default = st.out[1].clone()
    d17 = dataclasses.replace(st.d, num_splits=17)
    M.masw_decode_step(d17, lay, st.seq, st.k_new[1], st.v_new[1], st.q[1], st.out[1],
                       M.workspace(d17, M.OP_MATERIALIZE, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(out_default, st.out[1]), "default MASW plan is not 17 splits"
    # full-KV over the same cache, default plan (32 splits)
    _fullkv_step_check(st.fd, st.kf[1], st.vf[1], t, st.k_new[1], st.v_new[1], st.q[1],
                       units=[(0, k) for k in range(sh.n_kv_heads)], splits=32)
