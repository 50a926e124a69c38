"""Negative controls for the parity tolerance, planted in the oracle on the CPU.

The bf16 tolerance must reject plausible wrong answers at the workloads' real output
magnitudes: an all-zero output, a local window shifted by one position, a dropped sink
segment, dropped slots, and values read from the wrong KV head.  The correct answer
rounded to bf16 must pass.
"""
import numpy as np
import torch

from oracle import masw_oracle as O
from tests.parity import close


def _setup(seed=0, t=8192, S=4, W=2048, r=64, Hq=24, Hkv=8, D=128):
    rng = np.random.default_rng(seed)
    raw_k = rng.standard_normal((t + 2, Hkv, D)).astype(np.float32) * 0.5
    raw_v = rng.standard_normal((t + 2, Hkv, D)).astype(np.float32) * 0.5
    n = O.visible_slot_count(t, S, W, r)
    slot_k = rng.standard_normal((n + 1, Hkv, D)).astype(np.float32)
    slot_v = rng.standard_normal((n + 1, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((Hq, D))
    return raw_k, raw_v, slot_k, slot_v, q


def _attend(keys, raw_k, raw_v, slot_k, slot_v, q, D=128, head_perm=None):
    K = np.stack([raw_k[i] if k == "raw" else slot_k[i] for k, i in keys], axis=1).astype(np.float64)
    V = np.stack([raw_v[i] if k == "raw" else slot_v[i] for k, i in keys], axis=1).astype(np.float64)
    if head_perm is not None:
        V = V[head_perm]
    return O.gqa_attend(q, K, V, O.default_scale(D))


def test_bf16_tolerance_discriminates():
    S, W, r, t = 4, 2048, 64, 8192
    raw_k, raw_v, slot_k, slot_v, q = _setup()
    keys = O.keylist(t, S, W, r)
    ref = _attend(keys, raw_k, raw_v, slot_k, slot_v, q)
    rounded = torch.tensor(ref).to(torch.bfloat16).double().numpy()
    assert close(rounded, ref, torch.bfloat16)
    assert not close(np.zeros_like(ref), ref, torch.bfloat16)
    shifted = [(k, i - 1 if (k == "raw" and i > S) else i) for k, i in keys]
    assert not close(_attend(shifted, raw_k, raw_v, slot_k, slot_v, q), ref, torch.bfloat16)
    no_sink = [(k, i) for k, i in keys if not (k == "raw" and i <= S)]
    assert not close(_attend(no_sink, raw_k, raw_v, slot_k, slot_v, q), ref, torch.bfloat16)
    no_slots = [(k, i) for k, i in keys if k == "raw"]
    assert not close(_attend(no_slots, raw_k, raw_v, slot_k, slot_v, q), ref, torch.bfloat16)
    wrong_head = _attend(keys, raw_k, raw_v, slot_k, slot_v, q, head_perm=[1, 0, 2, 3, 4, 5, 6, 7])
    assert not close(wrong_head, ref, torch.bfloat16)


def test_fp32_tolerance_discriminates():
    S, W, r, t = 4, 32, 16, 240
    raw_k, raw_v, slot_k, slot_v, q = _setup(seed=1, t=t, S=S, W=W, r=r, Hq=2, Hkv=1, D=64)
    keys = O.keylist(t, S, W, r)
    ref = _attend(keys, raw_k, raw_v, slot_k, slot_v, q, D=64)
    assert close(ref.astype(np.float32), ref, torch.float32)
    last_slot_dropped = keys[:-1]
    assert not close(_attend(last_slot_dropped, raw_k, raw_v, slot_k, slot_v, q, D=64), ref, torch.float32)
    assert not close(ref * (1 + 1e-4), ref, torch.float32)
