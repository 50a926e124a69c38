"""The allocation-free decode step (masw_decode_step_static) against masw_decode_step.

Both run the same kernel with the same split plan; the static entry point keeps its
split partials and tickets in the library's own per-GPU scratch instead of a caller
workspace.  Three calls in a row on the same GPU - the 3B layer share at batch 8
(4 splits), then a smaller input (batch 2, 16 splits: another partial layout in the
same scratch), then batch 8 again - must each give the same output bits and leave the
same memory as masw_decode_step on the same inputs, with no device error.
"""
import pytest
import torch

import draft_kv_attention_amd as M
import seeded_inputs as SI

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.lib()


def _case(batch, t, seed):
    sh = SI.SWEEP_3B
    S, W, r = sh.sink, sh.window, sh.interval
    n = max(0, t - S - W) // r
    d = M.Dims(batch=batch, n_q_heads=sh.n_q_heads, n_kv_heads=sh.n_kv_heads, head_dim=sh.head_dim, sink=S,
               window=W, interval=r, max_slots=n + 2, dtype=sh.dtype)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    lay = M.alloc_layer(d, DEV, fill=None)
    for name in ("k_sink", "v_sink", "k_ring", "v_ring", "k_slot", "v_slot"):
        buf = getattr(lay, name)
        buf.copy_(torch.randn(buf.shape, generator=g, device=DEV).to(buf.dtype))
    lay.n_slots.fill_(n)
    seq = M.alloc_seq(batch, DEV)
    seq.seq_len.fill_(t)
    kn = torch.randn(batch, 1, sh.n_kv_heads, sh.head_dim, generator=g, device=DEV).to(sh.dtype)
    vn = torch.randn(batch, 1, sh.n_kv_heads, sh.head_dim, generator=g, device=DEV).to(sh.dtype)
    q = torch.randn(batch, sh.n_q_heads, sh.head_dim, generator=g, device=DEV).to(sh.dtype)
    return d, lay, seq, kn, vn, q


def _snapshot(lay):
    return {n: getattr(lay, n).clone() for n in ("k_sink", "v_sink", "k_ring", "v_ring", "k_slot", "v_slot", "n_slots")}


@pytest.mark.parametrize("calls", [((8, 32768), (2, 8192), (8, 4096))])
def test_static_scratch_matches_workspace_entry(calls):
    for i, (batch, t) in enumerate(calls):
        d, lay, seq, kn, vn, q = _case(batch, t, seed=100 + i)
        ref = torch.empty_like(q)
        M.masw_decode_step(d, lay, seq, kn, vn, q, ref, M.workspace(d, M.OP_MATERIALIZE, device=DEV))
        torch.cuda.synchronize()
        mem_ref = _snapshot(lay)
        out = torch.full_like(q, float("nan"))
        M.masw_decode_step_static(d, lay, seq, kn, vn, q, out)
        torch.cuda.synchronize()
        assert int(seq.err.item()) == 0, f"call {i}: device error bits"
        assert torch.equal(out, ref), f"call {i} (batch {batch}, t {t}): output differs from masw_decode_step"
        for name, v in _snapshot(lay).items():
            assert torch.equal(v, mem_ref[name]), f"call {i}: {name} differs"
