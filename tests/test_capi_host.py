"""Host-side checks of the C ABI that need no GPU: every symbol include/masw.h declares
is exported by libmasw.so, the ABI version matches, and invalid arguments are rejected
on the host before anything would be enqueued (these calls never reach a kernel)."""
import ctypes
import os
import re

import pytest

import draft_kv_attention_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "masw.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.LIB_PATH):
        from draft_kv_attention_amd import build
        build.build()
    return M.lib()


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"MASW_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_five_entry_points():
    names = set(declared_symbols())
    for n in ("masw_draft_attn", "masw_materialize_slot", "masw_evict_append",
              "fullkv_decode_attn", "fullkv_verify_attn"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert lib.masw_abi_version() == int(re.search(r"MASW_ABI_VERSION (\d+)", open(HEADER).read()).group(1))


def _dims(**kw):
    base = dict(batch=2, n_q_heads=24, n_kv_heads=8, head_dim=128, sink=4, window=2048, interval=64,
                max_slots=100, dtype=M.BF16, scale=0.0, num_splits=0)
    base.update(kw)
    return M._Dims(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(interval=-1), -1), (dict(interval=2049), -1), (dict(rollback=-1), -1), (dict(sink=-1), -1), (dict(max_slots=-1), -1),
    (dict(n_q_heads=20), -3), (dict(head_dim=96), -3), (dict(n_q_heads=40, n_kv_heads=8), -3),
    (dict(dtype=7), -2), (dict(num_splits=257), -1), (dict(batch=0), -3),
    (dict(rope_theta=-1.0), -1), (dict(rope_theta=float("nan")), -1), (dict(rope_theta=float("inf")), -1),
    (dict(rope_theta=10000.0, rope_style=2), -1),
    (dict(window=(1 << 28) + 1), -1), (dict(sink=(1 << 28) + 1), -1), (dict(max_slots=(1 << 28) + 1), -1),
    (dict(batch=65536), -3), (dict(n_q_heads=65536 * 2, n_kv_heads=65536), -3)])
def test_invalid_dims_rejected_on_host(lib, kw, status):
    d = _dims(**kw)
    assert lib.masw_draft_attn(ctypes.byref(d), None, None, None, None, None, 0, None) == status
    assert lib.masw_workspace_bytes(ctypes.byref(d), M.OP_DRAFT_ATTN, 0, 0) == 0


def test_null_arguments_rejected_on_host(lib):
    d = _dims()
    assert lib.masw_draft_attn(None, None, None, None, None, None, 0, None) == -1
    assert lib.masw_draft_attn(ctypes.byref(d), None, None, None, None, None, 0, None) == -1
    layer = M._Layer(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20)
    seq = M._Seq(1 << 20, 1 << 20)
    # workspace missing while the plan splits the key range
    assert lib.masw_draft_attn(ctypes.byref(d), ctypes.byref(layer), ctypes.byref(seq),
                               1 << 20, 1 << 20, None, 0, None) == -4
    # misaligned workspace
    need = lib.masw_workspace_bytes(ctypes.byref(d), M.OP_DRAFT_ATTN, 0, 0)
    assert lib.masw_draft_attn(ctypes.byref(d), ctypes.byref(layer), ctypes.byref(seq),
                               1 << 20, 1 << 20, (1 << 20) + 8, need, None) == -4
    assert lib.masw_evict_append(ctypes.byref(d), ctypes.byref(layer), ctypes.byref(seq),
                                 None, None, -1, None) == -1
    # n_new == 0 is a no-op that enqueues nothing
    assert lib.masw_evict_append(ctypes.byref(d), ctypes.byref(layer), ctypes.byref(seq),
                                 None, None, 0, None) == 0
    assert lib.fullkv_verify_attn(ctypes.byref(d), 1, 1, 10, 1, 1, 0, 1, 1, None, 0, None) == -1
    A = 1 << 20
    assert lib.masw_materialize_slot(ctypes.byref(d), ctypes.byref(layer), ctypes.byref(seq), 3071,
                                     A, A, A, A, A, 0, A, 1 << 30, None) == -3


def test_misaligned_tensors_rejected_on_host(lib):
    """Every tensor pointer must be 16-byte aligned (the kernels move 16-byte pieces of
    rows); a pointer off by 8 or 2 bytes is rejected with MASW_ERR_ARG before anything is
    enqueued, for each entry point that takes tensors."""
    A = 1 << 20
    d = _dims()
    need = lib.masw_workspace_bytes(ctypes.byref(d), M.OP_MATERIALIZE, 0, 0)
    seq = M._Seq(A, A)
    good = M._Layer(A, A, A, A, A, A, A)
    for field in ("k_sink", "v_sink", "k_ring", "v_ring", "k_slot", "v_slot"):
        bad = M._Layer(A, A, A, A, A, A, A)
        setattr(bad, field, A + 8)
        assert lib.masw_draft_attn(ctypes.byref(d), ctypes.byref(bad), ctypes.byref(seq), A, A, A, need, None) == -1, field
        assert lib.masw_evict_append(ctypes.byref(d), ctypes.byref(bad), ctypes.byref(seq), A, A, 1, None) == -1, field
    lay, sq = ctypes.byref(good), ctypes.byref(seq)
    for q, out in ((A + 8, A), (A, A + 2)):
        assert lib.masw_draft_attn(ctypes.byref(d), lay, sq, q, out, A, need, None) == -1
        assert lib.fullkv_decode_attn(ctypes.byref(d), A, A, 4096, A, A, q, out, A, need, None) == -1
        assert lib.fullkv_verify_attn(ctypes.byref(d), A, A, 4096, A, A, 2, q, out, A, need, None) == -1
    for kn, vn in ((A + 8, A), (A, A + 4)):
        assert lib.masw_decode_step(ctypes.byref(d), lay, sq, kn, vn, 1, A, A, A, need, None) == -1
        assert lib.masw_evict_append(ctypes.byref(d), lay, sq, kn, vn, 1, None) == -1
        assert lib.fullkv_append(ctypes.byref(d), A, A, 4096, A, A, kn, vn, 1, None) == -1
    assert lib.fullkv_decode_attn(ctypes.byref(d), A + 8, A, 4096, A, A, A, A, A, need, None) == -1
    for i in range(5):   # h, w_k_g, w_v_g, q_slot, o_slot
        ptrs = [A] * 5
        ptrs[i] = A + 8
        assert lib.masw_materialize_slot(ctypes.byref(d), lay, sq, 3072, *ptrs, 0, A, need, None) == -1, i
        assert lib.masw_prefill(ctypes.byref(d), lay, sq, 100, A, A, A, A, 4, 3072, *ptrs, None) == -1, i
    for i in range(4):   # k, v, q, out of the prefill
        ptrs = [A] * 4
        ptrs[i] = A + 8
        assert lib.masw_prefill(ctypes.byref(d), lay, sq, 100, *ptrs, 4, 3072, A, A, A, A, A, None) == -1, i


def test_stream_read_rejects_bad_sizes_on_host(lib):
    assert lib.masw_stream_read(None, 16, 0, 1 << 20, None) == -1
    assert lib.masw_stream_read(1 << 20, 0, 0, 1 << 20, None) == -1
    assert lib.masw_stream_read(1 << 20, 24, 0, 1 << 20, None) == -1
    assert lib.masw_stream_read((1 << 20) + 4, 32, 0, 1 << 20, None) == -1
    assert lib.masw_stream_read(1 << 20, 32, -1, 1 << 20, None) == -1


def test_no_slot_chain_has_nothing_to_materialize(lib):
    """interval 0 (sinks + window only) is a valid memory, but materialization is not."""
    d = _dims(interval=0, max_slots=0)
    assert lib.masw_workspace_bytes(ctypes.byref(d), M.OP_DRAFT_ATTN, 0, 0) > 0
    layer = M._Layer(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20)
    seq = M._Seq(1 << 20, 1 << 20)
    A = 1 << 20
    assert lib.masw_materialize_slot(ctypes.byref(d), ctypes.byref(layer), ctypes.byref(seq), 3072,
                                     A, A, A, A, A, 0, A, 1 << 30, None) == -1


def test_rollback_rejects_bad_arguments_on_host(lib):
    d = _dims(rollback=16)
    layer = M._Layer(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20)
    seq = M._Seq(1 << 20, 1 << 20)
    assert lib.masw_rollback(ctypes.byref(d), ctypes.byref(layer), ctypes.byref(seq), None, None) == -1
    assert lib.masw_rollback(ctypes.byref(d), None, ctypes.byref(seq), 1 << 20, None) == -1
    bad = _dims(rollback=-3)
    assert lib.masw_rollback(ctypes.byref(bad), ctypes.byref(layer), ctypes.byref(seq), 1 << 20, None) == -1


def test_prefill_rejects_bad_arguments_on_host(lib):
    layer = M._Layer(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20)
    seq = M._Seq(1 << 20, 1 << 20)
    P = 1 << 20

    def call(d, p_max=100, k=P, ns_max=4, hidden=3072, h=P, lay=layer):
        return lib.masw_prefill(ctypes.byref(d), ctypes.byref(lay) if lay else None, ctypes.byref(seq), p_max,
                                k, P, P, P, ns_max, hidden, h, P, P, P, P, None)
    d = _dims()
    assert call(d, p_max=0) == -1
    assert call(d, k=None) == -1
    assert call(d, ns_max=-1) == -1
    assert call(d, h=None) == -1               # a slot chain needs the slot inputs
    assert call(d, hidden=3071) == -3          # hidden % 8
    assert call(d, lay=None) == -1
    assert call(_dims(dtype=M.F32)) == -6      # matrix-core path only
    assert call(_dims(head_dim=64)) == -6
    assert call(_dims(interval=2049)) == -1


def test_mfma_rate_rejects_bad_arguments_on_host(lib):
    assert lib.masw_mfma_rate(0, 10, 1 << 20, 1 << 20, None) == -1
    assert lib.masw_mfma_rate(4, 0, 1 << 20, 1 << 20, None) == -1
    assert lib.masw_mfma_rate(4, 10, None, 1 << 20, None) == -1
    assert lib.masw_mfma_rate(4, 10, 1 << 20, None, None) == -1


def test_workspace_sizes(lib):
    d = _dims(batch=8)
    a = lib.masw_workspace_bytes(ctypes.byref(d), M.OP_DRAFT_ATTN, 0, 0)
    b = lib.masw_workspace_bytes(ctypes.byref(d), M.OP_MATERIALIZE, 0, 0)
    f = lib.masw_workspace_bytes(ctypes.byref(d), M.OP_FULLKV_DECODE, 32768, 0)
    v = lib.masw_workspace_bytes(ctypes.byref(d), M.OP_FULLKV_VERIFY, 32774, 6)
    assert a > 0 and b > a and f > 0 and v > 0   # materialization adds the projection partials
    assert lib.masw_workspace_bytes(ctypes.byref(d), M.OP_FULLKV_DECODE, 0, 0) == 0
    assert all(x % 256 == 0 for x in (a, b, f, v))


def test_status_strings(lib):
    for st in range(-6, 1):
        assert M.status_string(st) not in ("", "unknown status")


def test_static_decode_step_rejects_plans_beyond_its_scratch(lib):
    """masw_decode_step_static keeps its partials in a fixed scratch: a split plan whose
    partials or tickets do not fit returns MASW_ERR_WORKSPACE before anything is
    enqueued (and before the scratch is looked up on a device)."""
    A = 1 << 20
    layer, seq = M._Layer(A, A, A, A, A, A, A), M._Seq(A, A)
    for kw in (dict(batch=64, n_q_heads=64, n_kv_heads=8, num_splits=256),    # partials too big
               dict(batch=4096, n_q_heads=24, n_kv_heads=8, num_splits=2)):   # too many tickets
        d = _dims(**kw)
        assert lib.masw_decode_step_static(ctypes.byref(d), ctypes.byref(layer), ctypes.byref(seq),
                                           A, A, 1, A, A, None) == -4, kw
    d = _dims()
    assert lib.masw_decode_step_static(ctypes.byref(d), ctypes.byref(layer), ctypes.byref(seq),
                                       A + 8, A, 1, A, A, None) == -1
