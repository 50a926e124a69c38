"""Tolerances shared by the parity tests.

Floating-point outputs are compared with the fp64 oracle as:
  * fp32 path: max |gpu - ref| <= 1e-5 and ||gpu - ref||_2 / ||ref||_2 <= 1e-5;
  * bf16 path: max |gpu - ref| <= 2e-2, ||gpu - ref||_2 / ||ref||_2 <= 1e-2 and
    max |gpu - ref| <= 2e-2 * max |ref|.
The absolute bounds are the path's stated tolerance.  The normalised bounds are added
because at the workloads' Gaussian inputs attention outputs are about 0.5/sqrt(n)
(0.003-0.012 for 2K-32K keys), below 2e-2: an all-zero output would pass the absolute
bound alone.  A bf16 output carries one rounding of relative size <= 2^-9, far inside
the normalised bounds; a shifted window or a dropped segment is far outside them (see
test_tolerance_rejects_wrong_answers).
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {
    torch.float32: dict(abs=1e-5, rel_l2=1e-5, rel_max=None),
    torch.bfloat16: dict(abs=2e-2, rel_l2=1e-2, rel_max=2e-2),
}


def as_f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def compare(gpu, ref, dtype) -> dict:
    g, r = as_f64(gpu), as_f64(ref)
    diff = np.abs(g - r)
    rn = float(np.linalg.norm(r))
    return dict(max_abs=float(diff.max()) if diff.size else 0.0,
                rel_l2=float(np.linalg.norm(g - r) / rn) if rn > 0 else float(np.linalg.norm(g - r)),
                ref_max=float(np.abs(r).max()) if r.size else 0.0,
                finite=bool(np.isfinite(g).all()))


def close(gpu, ref, dtype) -> bool:
    s = compare(gpu, ref, dtype)
    t = TOL[dtype]
    ok = s["finite"] and s["max_abs"] <= t["abs"] and s["rel_l2"] <= t["rel_l2"]
    if t["rel_max"] is not None:
        ok = ok and s["max_abs"] <= t["rel_max"] * max(s["ref_max"], 1e-30)
    return ok


def assert_close(gpu, ref, dtype, what=""):
    s = compare(gpu, ref, dtype)
    assert close(gpu, ref, dtype), f"{what}: {s} vs tolerance {TOL[dtype]}"
    return s


def proj_sum_depth(hidden, prefill=False):
    """Longest chain of fp32 additions one product h_k w_kn passes through in the bf16
    slot projection (matrix cores): up to 32 inside the 16x16x32 MFMA that forms it (the
    hardware's own order is not documented, so a sequential chain is assumed), one per
    further MFMA step of its wave's hidden range, 4 for the sum of the work-group's waves
    and one per hidden slice.  A boundary projection cuts the hidden size into at most 8
    slices of a multiple of 128 rows; a prefill projection takes it whole.  Each slice's
    rows are split between 4 waves in steps of 32."""
    if prefill:
        per, splits = -(-hidden // 128) * 128, 1
    else:
        per = -(-(-(-hidden // 8)) // 128) * 128
        splits = -(-hidden // per)
    steps = per // 4 // 32
    return 32 + steps + 4 + splits


def slot_bound(h, w, n_kv_heads, head_dim, prefill=False):
    """Per-element allowance for a stored bf16 slot K/V (the bf16 rounding of an fp32 sum
    H W_g) beyond one bf16 ulp of the oracle's rounded fp64 value: the forward error bound
    of fp32 summation, depth * 2^-24 * sum_k |h_k w_k|, with depth the kernel's longest
    addition chain (proj_sum_depth), shaped [..., Hkv, D].  It matters only where the sum
    cancels."""
    h, w = np.abs(np.asarray(h, np.float64)), np.abs(np.asarray(w, np.float64))
    depth = proj_sum_depth(h.shape[-1], prefill)
    return (depth * 2.0 ** -24 * (h @ w)).reshape(h.shape[:-1] + (n_kv_heads, head_dim))


def assert_slot_close(got, ref, bound, what=""):
    """Stored bf16 slot K/V against the oracle's rounded value: every element within one
    bf16 ulp plus the fp32 summation bound, and at least 99.9% of the elements within one
    ulp outright (both roundings of a sum agree unless it sits near a rounding boundary)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    ulp = bf16_ulp(ref)
    err = np.abs(got - ref)
    ulps = err / ulp
    within1 = float((err <= ulp).mean())
    msg = f"{what}: max {ulps.max():.2f} ulp, {100 * within1:.3f}% within 1 ulp"
    assert (err <= ulp + bound).all(), msg
    assert within1 >= 0.999, msg
    return float(ulps.max())


def bf16_ulp(x):
    """Spacing of bf16 values at |x| (8 significant bits)."""
    return np.ldexp(1.0, np.frexp(np.abs(np.asarray(x, np.float64)))[1] - 8)


def rope_partner(D, style):
    """Index of each head-vector component's rotary pair partner (rotate-half: d ^ D/2,
    interleaved: d ^ 1)."""
    return np.arange(D) ^ (D // 2 if style == 0 else 1)


def rotated_slot_bound(h, w, n_kv_heads, head_dim, style, ref, prefill=False):
    """Allowance for a rotated slot key: the fp32 summation bound of both components of
    its pair (each enters with a weight |cos|, |sin| <= 1) plus the fp32 rounding of the
    turn itself (a few 2^-24 of |x_a| + |x_b|, taken from the reference)."""
    b = slot_bound(h, w, n_kv_heads, head_dim, prefill)
    p = rope_partner(head_dim, style)
    r = np.abs(np.asarray(ref, np.float64))
    return b + b[..., p] + 2.0 ** -21 * (r + r[..., p])
