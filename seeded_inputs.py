"""Seeded synthetic inputs shared by the oracle-side tests, the HIP-side tests and bench.py.

This module holds workload shapes and random-number recipes only. It contains none of
the method's arithmetic (no key lists, no attention, no projection, no ring indexing):
it draws tensors and hands them to whoever asked. Both the CPU oracle and the HIP path
consume the very same tensors produced here.

Workloads (all synthetic, i.i.d. Gaussian; the pages evaluate on long-document
summarization prompts, for which attention cost is data-independent, so seeded
Gaussians of the same shapes stand in for them):

* ``TINY``      - one draft layer, 2 query heads sharing 1 KV head, D=64, fp32,
                  S=4, W=32, r=16, prefix 200 then 40 decode steps.
* ``DRAFT_3B``  - Llama-3.2-3B-shaped draft attention: 28 layers, 24 q heads,
                  8 KV heads, D=128, hidden 3072, bf16; S=4, W=2048, r=64; t=8192, B=1;
                  K,V ~ 0.5*N(0,1), q ~ N(0,1).
* ``SWEEP_3B``  - the same shapes at B=8, t in {1K,2K,4K,8K,16K,24K,32K}; K,V ~ N(0,1).
* ``MATERIALIZE_3B`` - slot materialization chain at 3B shapes, B=4, mirrored
                  projections 3072x1024 bf16 ~ N(0, 0.02), H ~ N(0,1), 512 boundaries.
* ``PREFILL_3B`` - draft prefill at the 3B draft shapes (S=4, W=2048, r=64), B=1, a
                  32768-token prefix with its 479 slots; K,V,q ~ N(0,1), H ~ N(0,1),
                  mirrored projections ~ N(0, 0.02).
* ``VERIFY_8B`` / ``VERIFY_70B`` - verifier attention, 32/64 q heads, 8 KV heads,
                  D=128, bf16, prefix 32768 plus 6 causal query positions, B=4.

"N(0, x)" is read with x as a standard deviation (the usual initializer convention).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import torch


@dataclasses.dataclass(frozen=True)
class DraftShape:
    """Geometry of one draft-attention workload."""
    name: str
    layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    hidden: int
    sink: int
    window: int
    interval: int
    batch: int
    dtype: torch.dtype
    kv_std: float = 1.0
    q_std: float = 1.0
    h_std: float = 1.0
    w_std: float = 0.02

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


TINY = DraftShape(name="tiny_fp32", layers=1, n_q_heads=2, n_kv_heads=1, head_dim=64,
                  hidden=64, sink=4, window=32, interval=16, batch=1,
                  dtype=torch.float32, w_std=1.0 / 64)
TINY_PREFIX = 200
TINY_STEPS = 40

DRAFT_3B = DraftShape(name="draft3b_b1_t8192", layers=28, n_q_heads=24, n_kv_heads=8,
                      head_dim=128, hidden=3072, sink=4, window=2048, interval=64,
                      batch=1, dtype=torch.bfloat16, kv_std=0.5)
DRAFT_3B_PREFIX = 8192

SWEEP_3B = dataclasses.replace(DRAFT_3B, name="draft3b_b8_sweep", batch=8, kv_std=1.0)
SWEEP_PREFIXES = (1024, 2048, 4096, 8192, 16384, 24576, 32768)

MATERIALIZE_3B = dataclasses.replace(DRAFT_3B, name="materialize3b_b4", batch=4, kv_std=1.0)
MATERIALIZE_CHAIN = 512

PREFILL_3B = dataclasses.replace(DRAFT_3B, name="prefill3b_b1_p32768", batch=1, kv_std=1.0)
PREFILL_LEN = 32768


@dataclasses.dataclass(frozen=True)
class VerifyShape:
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    batch: int
    prefix: int
    n_query: int
    dtype: torch.dtype = torch.bfloat16


VERIFY_8B = VerifyShape(name="verify8b_b4_p32768", n_q_heads=32, n_kv_heads=8, head_dim=128,
                        batch=4, prefix=32768, n_query=6)
VERIFY_70B = VerifyShape(name="verify70b_b4_p32768", n_q_heads=64, n_kv_heads=8, head_dim=128,
                         batch=4, prefix=32768, n_query=6)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape: Sequence[int], seed: int, std: float = 1.0, dtype: torch.dtype = torch.float32,
           device="cpu") -> torch.Tensor:
    """i.i.d. N(0, std^2) drawn in fp32 from a seeded generator, then stored in ``dtype``.

    Storing in bf16 rounds each draw once (round-to-nearest-even by torch); the stored
    value *is* the input both sides consume.
    """
    x = torch.randn(tuple(int(s) for s in shape), generator=_gen(seed, device),
                    dtype=torch.float32, device=device)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


def seed_for(base: int, *keys: int) -> int:
    """Deterministic derived seed for a (base, layer, step, ...) tuple."""
    s = int(base) & 0xFFFFFFFF
    for k in keys:
        s = (s * 1000003 + int(k) + 0x9E3779B9) & 0x7FFFFFFFFFFF
    return s


def mirrored_weights(shape: DraftShape, seed: int, device="cpu",
                     copy_init_perturb: Optional[float] = None):
    """Mirrored key/value projection weights [hidden][Hkv*D] for one layer.

    ``copy_init_perturb`` set: the weights are a copy of a backbone projection
    ~N(0, w_std) plus N(0, copy_init_perturb) noise (the tiny workload's recipe);
    otherwise plain N(0, w_std).
    """
    cols = shape.n_kv_heads * shape.head_dim
    out = []
    for which in range(2):
        base = normal((shape.hidden, cols), seed_for(seed, which, 0), std=shape.w_std,
                      dtype=torch.float32, device=device)
        if copy_init_perturb is not None:
            base = base + normal((shape.hidden, cols), seed_for(seed, which, 1),
                                 std=copy_init_perturb, dtype=torch.float32, device=device)
        out.append(base.to(shape.dtype))
    return out[0], out[1]


def token_kv(shape: DraftShape, seed: int, layer: int, first_pos: int, n: int, device="cpu"):
    """Raw K/V for positions first_pos..first_pos+n-1, layout [B][n][Hkv][D]."""
    dims = (shape.batch, n, shape.n_kv_heads, shape.head_dim)
    k = normal(dims, seed_for(seed, 1, layer, first_pos, n), std=shape.kv_std,
               dtype=shape.dtype, device=device)
    v = normal(dims, seed_for(seed, 2, layer, first_pos, n), std=shape.kv_std,
               dtype=shape.dtype, device=device)
    return k, v


def decode_query(shape: DraftShape, seed: int, layer: int, step: int, device="cpu"):
    """Decode query [B][Hq][D] for one (layer, step)."""
    return normal((shape.batch, shape.n_q_heads, shape.head_dim), seed_for(seed, 3, layer, step),
                  std=shape.q_std, dtype=shape.dtype, device=device)


def slot_inputs(shape: DraftShape, seed: int, layer: int, m: int, device="cpu"):
    """Slot hidden state H [B][hidden] and slot query q_g [B][Hq][D] for slot m of a layer."""
    h = normal((shape.batch, shape.hidden), seed_for(seed, 4, layer, m), std=shape.h_std,
               dtype=shape.dtype, device=device)
    qg = normal((shape.batch, shape.n_q_heads, shape.head_dim), seed_for(seed, 5, layer, m),
                std=shape.q_std, dtype=shape.dtype, device=device)
    return h, qg


def prefill_inputs(shape: DraftShape, seed: int, layer: int, P: int, ns: int, device="cpu"):
    """A whole prefix of one layer: raw K/V [B][P][Hkv][D] (row i-1 = position i), raw
    queries [B][P][Hq][D], slot hidden states [B][ns][hidden] and slot queries
    [B][ns][Hq][D] (row m-1 = slot m)."""
    k, v = token_kv(shape, seed, layer, 1, P, device)
    q = normal((shape.batch, P, shape.n_q_heads, shape.head_dim), seed_for(seed, 6, layer, P),
               std=shape.q_std, dtype=shape.dtype, device=device)
    h = normal((shape.batch, ns, shape.hidden), seed_for(seed, 7, layer, ns), std=shape.h_std,
               dtype=shape.dtype, device=device)
    qs = normal((shape.batch, ns, shape.n_q_heads, shape.head_dim), seed_for(seed, 8, layer, ns),
                std=shape.q_std, dtype=shape.dtype, device=device)
    return k, v, q, h, qs


def full_cache(batch: int, n_kv_heads: int, max_len: int, head_dim: int, seed: int,
               dtype: torch.dtype, std: float = 1.0, device="cpu"):
    """Contiguous full K/V cache [B][Hkv][max_len][D] (rows are positions 1..max_len)."""
    dims = (batch, n_kv_heads, max_len, head_dim)
    return (normal(dims, seed_for(seed, 11), std=std, dtype=dtype, device=device),
            normal(dims, seed_for(seed, 12), std=std, dtype=dtype, device=device))


def verify_query(shape: VerifyShape, seed: int, device="cpu"):
    """Verifier queries [B][n_q][Hq][D]."""
    return normal((shape.batch, shape.n_query, shape.n_q_heads, shape.head_dim),
                  seed_for(seed, 21), dtype=shape.dtype, device=device)
