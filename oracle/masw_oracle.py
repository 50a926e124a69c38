"""Plain, slow, fp64 CPU oracle for the MASW draft-attention hot path.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in ``oracle/``.
The HIP library never calls it, and it shares no code, header, table or helper with
the HIP library: it is written from the pages directly.

Pages cited (by title; section / equation / algorithm step on that page):

* [TR]  "Strong Drafts Need Compact Memories: A Technical Review of Memory-Augmented
         Sliding-Window (MASW) Drafting for Long-Context Speculative Decoding"
* [RN]  the Chinese reading notes on the same paper (title "强推理草稿也要瘦身：
         长上下文投机解码的记忆增强滑窗（MASW）阅读笔记"), which mirror [TR] section by section.

Notation follows [TR]: S sink tokens, W local-window width, r slot interval, t the
number of raw tokens in the cache *including* the current query token (Eq. 2 attends
over K_{<=t}), positions are 1-based, g_m is the m-th memory slot.

Readings taken where the pages leave a step open:

* R0  Eq. 2's sqrt(d) uses the per-head key dimension D; query head h reads KV head
      floor(h / G) with G = Hq / Hkv (grouped-query attention).
* R1  Slot g_m's structured mask ([TR] §3.2, Algorithm 1 step 2: sinks, the local
      window about to be evicted, earlier slots) is the memory the decode query saw
      r steps before g_m became visible: keylist(t_m - r).  Its local part is the exact
      W-window whose oldest r tokens are the block g_m compresses.
* R2  The number of visible slots is floor(max(0, t - S - W) / r); [TR] §3.1's
      "floor(t/r) memory slots" is read as an upper bound (I2 below).
* R3  Block B_m = positions S+(m-1)r+1 .. S+mr; g_m is materialized at
      t_m = S + W + m*r (after raw token t_m is appended, before the decode query at
      t_m) - exactly when B_m has left the local window.  A raw token and the slot
      holding it are never both visible.
* R4  g_m does not attend to itself unless ``include_self`` is set.
* R5  The slot's query vector q_g is an input (only K/V are mirrored, Algorithm 1 step 3).
* R6  Raw K/V and all queries arrive post-positional (the caller's rotary embedding is
      already applied); every workload draws them i.i.d.
* R11 Slot keys are rotated only when a rotary base theta is given ([TR] §3.2 Algorithm
      1 step 6 gives g_m the position id of the raw token right after it, a duplicate id).
      Ids are 0-based token indices, so raw position i has id i - 1 and g_m, whose block
      ends at position S + m r, gets id S + m r.  The rotation is RoFormer's: pairs of
      the head vector turn by pos * theta^(-2i/D), paired either as (i, i + D/2)
      ("rotate-half", the Llama-family layout) or as (2i, 2i + 1) ("interleaved").  It
      is applied to the fp64 projection before the cache rounds it; values are not
      touched.
* R7  1 <= r <= W for a memory with a slot chain.
* R8  r = 0 means no slot chain: the memory is sinks ++ the exact W-window, the
      sink-plus-window structure [TR] §3.1's sink bullet takes from StreamingLLM; with
      S = 0 it is the pure sliding window [TR] §3 opens with, which is also [TR] §4's SWA
      baseline (1,024-token window).  No slot is ever visible, the ring keeps C = W rows
      and every append is legal.
* R10 Draft prefill ([TR] §3.3 Algorithm 2 step 2: one pass over the prefix under the
      structured mask of Appendix C, which the pages do not print, slots materialized in
      the same pass) computes what decoding the prefix token by token would: the raw
      query at position i attends to keylist(i), slot g_m's query to keylist(t_m - r)
      (reading R1); slot K/V depend only on the slots' hidden states, so they are all
      projected first.
* R9  Rollback ([TR] §3.3 Algorithm 2 step 6): after the target accepts the first L_acc
      of the draft's candidates, the memory is what appending only the accepted tokens
      would have built: raw tokens past the accepted length t_acc are dropped and so is
      every slot materialized strictly after t_acc.  The retained raw-KV rollback window
      is read as `rollback` extra ring rows (C = W + r + rollback): a speculative append
      at position i <= t_acc + rollback evicts i - C <= t_acc - W - r, a token the memory
      at t_acc no longer needs, so undoing speculation moves no data.

Precision: every score, softmax and weighted sum is computed in fp64 on the stored
input values.  Stored slot K/V in a bf16 cache are rounded to bf16 with
round-to-nearest-even (``to_bf16``); in an fp32 cache they are kept unrounded.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

Key = Tuple[str, int]  # ("raw", position) or ("slot", m)


# ---------------------------------------------------------------------------
# Memory sets ([TR] §3.1, Eq. 4 and its three bullets)
# ---------------------------------------------------------------------------

def sink_positions(t: int, S: int) -> List[int]:
    """Sink set: exact raw KV of the first S tokens, never evicted ([TR] §3.1 Eq. 4, sink bullet)."""
    return list(range(1, min(S, t) + 1))


def local_positions(t: int, S: int, W: int) -> List[int]:
    """Local window {i : max(S+1, t-W+1) <= i <= t} ([TR] §3.1 Eq. 4, local bullet)."""
    lo = max(S + 1, t - W + 1)
    return list(range(lo, t + 1))


def visible_slot_count(t: int, S: int, W: int, r: int) -> int:
    """Slots visible at step t: one per r raw tokens that have left sink and window
    (reading R2); none without a slot chain (r = 0, reading R8)."""
    if r == 0:
        return 0
    return max(0, t - S - W) // r


def block_positions(m: int, S: int, r: int) -> List[int]:
    """Raw positions that slot g_m compresses (reading R3): S+(m-1)r+1 .. S+mr."""
    if r == 0:
        raise ValueError("no slot chain (r = 0)")
    return list(range(S + (m - 1) * r + 1, S + m * r + 1))


def boundary_step(m: int, S: int, W: int, r: int) -> int:
    """Step t_m at which g_m is materialized and becomes visible (reading R3)."""
    if r == 0:
        raise ValueError("no slot chain (r = 0)")
    return S + W + m * r


def is_boundary(t: int, S: int, W: int, r: int) -> int:
    """Return m if step t is the materialization step of slot m, else 0."""
    if r == 0:
        return 0
    d = t - S - W
    if d >= r and d % r == 0:
        return d // r
    return 0


def keylist(t: int, S: int, W: int, r: int) -> List[Key]:
    """Working memory M_t = sink ++ local ++ slots in that order ([TR] §3.1 Eq. 4)."""
    keys: List[Key] = [("raw", i) for i in sink_positions(t, S)]
    keys += [("raw", i) for i in local_positions(t, S, W)]
    keys += [("slot", m) for m in range(1, visible_slot_count(t, S, W, r) + 1)]
    return keys


def slot_query_keylist(m: int, S: int, W: int, r: int, include_self: bool = False) -> List[Key]:
    """Attention set A_m of slot g_m under the structured mask ([TR] §3.2 Algorithm 1 step 2).

    Reading R1: sinks, the W-window whose oldest r tokens are B_m, slots 1..m-1.
    """
    keys = keylist(boundary_step(m, S, W, r) - r, S, W, r)
    if include_self:
        keys.append(("slot", m))
    return keys


# ---------------------------------------------------------------------------
# Attention ([TR] §2.3, Eq. 2)
# ---------------------------------------------------------------------------

def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q K^T) V for one query vector, fp64 ([TR] §2.3 Eq. 2)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    s = (K @ q) * scale
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def softmax_weights(q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """The probability row of Eq. 2 (used by the one-hot-V support tests)."""
    s = (np.asarray(K, np.float64) @ np.asarray(q, np.float64)) * scale
    p = np.exp(s - s.max())
    return p / p.sum()


def default_scale(D: int) -> float:
    """1/sqrt(d) with d the per-head key dimension (reading R0)."""
    return 1.0 / math.sqrt(D)


def gqa_attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Grouped-query attention: q [Hq][D] over K, V [Hkv][n][D]; head h reads KV head h // G."""
    Hq = q.shape[0]
    Hkv = K.shape[0]
    G = Hq // Hkv
    out = np.empty(q.shape, dtype=np.float64)
    for h in range(Hq):
        out[h] = attend(q[h], K[h // G], V[h // G], scale)
    return out


# ---------------------------------------------------------------------------
# Rounding of stored slot K/V (bf16 cache) - round to nearest, ties to even
# ---------------------------------------------------------------------------

def to_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value of each fp64 element (ties to even), returned as fp64.

    bfloat16 has 8 significant bits and fp32's exponent range: normal numbers have
    quantum 2^(e-8) for x = f * 2^e, 0.5 <= |f| < 1; below 2^-126 the quantum is 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    finite = np.isfinite(x) & (x != 0)
    f, e = np.frexp(x[finite])
    e = np.maximum(e, -125)                     # subnormal range shares quantum 2^-133
    q = np.ldexp(np.rint(np.ldexp(x[finite], 8 - e)), e - 8)   # np.rint: half to even
    q[np.abs(q) >= 2.0 ** 128] = np.inf * np.sign(q[np.abs(q) >= 2.0 ** 128])
    out[finite] = q
    out[~finite] = x[~finite]
    return out


# ---------------------------------------------------------------------------
# Mirrored projection ([TR] §3.2 Algorithm 1 step 3)
# ---------------------------------------------------------------------------

def project_slot(h: np.ndarray, w_k: np.ndarray, w_v: np.ndarray, n_kv_heads: int,
                 head_dim: int, bf16_cache: bool, rope: Optional[Tuple[float, int]] = None,
                 pos=None) -> Tuple[np.ndarray, np.ndarray]:
    """K_g = H_g W_K,g and V_g = H_g W_V,g (row vector H, W [hidden][Hkv*D]).

    KV head k is the column block k*D .. k*D+D-1.  h may carry leading batch axes;
    returns [..., Hkv, D] each, rounded to bf16 when the cache stores bf16.  With
    rope = (theta, style) (theta > 0) K_g is rotated to position id pos (reading R11;
    pos broadcasts against h's leading axes) before the rounding.
    """
    h = np.asarray(h, np.float64)
    lead = h.shape[:-1]
    kg = (h @ np.asarray(w_k, np.float64)).reshape(lead + (n_kv_heads, head_dim))
    vg = (h @ np.asarray(w_v, np.float64)).reshape(lead + (n_kv_heads, head_dim))
    if rope is not None and rope[0] > 0:
        kg = rope_rotate(kg, np.asarray(pos, np.float64)[..., None], rope[0], rope[1])
    if bf16_cache:
        kg, vg = to_bf16(kg), to_bf16(vg)
    return kg, vg


# ---------------------------------------------------------------------------
# Rotary position of slot keys ([TR] §3.2 Algorithm 1 step 6; reading R11)
# ---------------------------------------------------------------------------

ROPE_ROTATE_HALF, ROPE_INTERLEAVED = 0, 1


def slot_position_id(m: int, S: int, r: int) -> int:
    """Position id of g_m: the id of the raw token right after its block B_m (a
    duplicate id).  With 0-based ids that token, position S + m r + 1, has id S + m r."""
    if r < 1 or m < 1:
        raise ValueError("slots exist only with a slot chain, from m = 1")
    return S + m * r


def rope_pairs(D: int, style: int) -> List[Tuple[int, int, int]]:
    """(a, b, i): the two components of a head vector rotated together, and the
    frequency index i of their angle."""
    half = D // 2
    if style == ROPE_ROTATE_HALF:
        return [(i, i + half, i) for i in range(half)]
    if style == ROPE_INTERLEAVED:
        return [(2 * i, 2 * i + 1, i) for i in range(half)]
    raise ValueError("unknown rotary pairing")


def rope_rotate(x: np.ndarray, pos, theta: float, style: int) -> np.ndarray:
    """Rotary embedding of head vectors x [..., D] at position id pos (a scalar, or an
    array broadcasting against x's leading axes): each pair (x_a, x_b) turns by the
    angle pos * theta^(-2i/D), x_a' = x_a cos - x_b sin, x_b' = x_a sin + x_b cos."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    pos = np.asarray(pos, np.float64)
    out = x.copy()
    for a, b, i in rope_pairs(D, style):
        ang = pos * float(theta) ** (-2.0 * i / D)
        c, s = np.cos(ang), np.sin(ang)
        out[..., a] = x[..., a] * c - x[..., b] * s
        out[..., b] = x[..., a] * s + x[..., b] * c
    return out


# ---------------------------------------------------------------------------
# The draft memory of one sequence in one layer, kept by logical identity
# ---------------------------------------------------------------------------

class DraftMemory:
    """Logical compact memory of one sequence in one layer ([TR] §3.1-§3.3).

    Every raw token ever appended is kept by position and every slot by index; the
    memory the method exposes at step t is selected by ``keylist``.  No ring buffer,
    no physical layout: the oracle only knows *which* entries are visible.
    """

    def __init__(self, S: int, W: int, r: int, n_kv_heads: int, head_dim: int,
                 bf16_cache: bool, rope_theta: float = 0.0, rope_style: int = ROPE_ROTATE_HALF):
        if not (0 <= r <= W) or S < 0 or W < 1:
            raise ValueError("need S >= 0, W >= 1 and 1 <= r <= W, or r = 0 (readings R7, R8)")
        self.S, self.W, self.r = S, W, r
        self.rope = (rope_theta, rope_style) if rope_theta > 0 else None
        self.Hkv, self.D = n_kv_heads, head_dim
        self.bf16 = bf16_cache
        self.t = 0
        self.raw: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}
        self.slots: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}

    # -- writes ------------------------------------------------------------
    def append(self, k_new: np.ndarray, v_new: np.ndarray) -> None:
        """Append raw tokens t+1..t+n (k_new, v_new [n][Hkv][D]); eviction is implicit.

        Values are kept as passed (an fp32 array holds bf16/fp32 inputs exactly) and
        widened to fp64 when gathered.
        """
        for j in range(k_new.shape[0]):
            self.t += 1
            self.raw[self.t] = (np.asarray(k_new[j]), np.asarray(v_new[j]))

    def pending_boundary(self) -> int:
        """m if the current step materializes g_m and it does not exist yet, else 0."""
        m = is_boundary(self.t, self.S, self.W, self.r)
        return m if (m and m not in self.slots) else 0

    def materialize(self, h: np.ndarray, w_k: np.ndarray, w_v: np.ndarray, q_slot: np.ndarray,
                    scale: float, include_self: bool = False) -> Optional[np.ndarray]:
        """Algorithm 1 steps 2-4 at boundary t_m: project, run the slot query, append.

        Returns o_g [Hq][D] (the slot query's attention output), or None when the
        current step is not a pending boundary.
        """
        m = self.pending_boundary()
        if not m:
            return None
        pos = slot_position_id(m, self.S, self.r) if self.rope else None
        kg, vg = project_slot(h, w_k, w_v, self.Hkv, self.D, self.bf16, self.rope, pos)
        self.add_slot(m, kg, vg)
        return self.slot_query(m, q_slot, scale, include_self)

    def add_slot(self, m: int, kg: np.ndarray, vg: np.ndarray) -> None:
        """Append g_m's K/V ([Hkv][D] each) to the slot chain (Algorithm 1 step 4)."""
        if m != len(self.slots) + 1:
            raise ValueError(f"slot {m} out of order (have {len(self.slots)})")
        self.slots[m] = (np.asarray(kg, np.float64), np.asarray(vg, np.float64))

    def slot_query(self, m: int, q_slot: np.ndarray, scale: float, include_self: bool = False) -> np.ndarray:
        """g_m's query under the structured mask (Algorithm 1 step 2, reading R1)."""
        keys = slot_query_keylist(m, self.S, self.W, self.r, include_self)
        K, V = self.gather(keys)
        return gqa_attend(np.asarray(q_slot, np.float64), K, V, scale)

    def rollback(self, t_acc: int) -> None:
        """Undo speculation past the accepted length t_acc (reading R9, [TR] §3.3
        Algorithm 2 step 6): drop raw tokens after t_acc and every slot materialized
        strictly after t_acc."""
        if not 0 <= t_acc <= self.t:
            raise ValueError("rollback target outside 0..t")
        for i in [i for i in self.raw if i > t_acc]:
            del self.raw[i]
        for m in [m for m in self.slots if boundary_step(m, self.S, self.W, self.r) > t_acc]:
            del self.slots[m]
        self.t = t_acc

    # -- reads -------------------------------------------------------------
    def gather(self, keys: Sequence[Key]) -> Tuple[np.ndarray, np.ndarray]:
        """Stack the K/V of the listed entries into [Hkv][n][D]."""
        ks, vs = [], []
        for kind, idx in keys:
            k, v = self.raw[idx] if kind == "raw" else self.slots[idx]
            ks.append(k)
            vs.append(v)
        return np.stack(ks, axis=1).astype(np.float64), np.stack(vs, axis=1).astype(np.float64)

    def decode(self, q: np.ndarray, scale: float) -> np.ndarray:
        """Draft decode attention at the current step over M_t ([TR] §3.3 Algorithm 2 step 4)."""
        keys = keylist(self.t, self.S, self.W, self.r)
        K, V = self.gather(keys)
        return gqa_attend(np.asarray(q, np.float64), K, V, scale)

    def decode_weights(self, q_head: np.ndarray, kv_head: int, scale: float) -> np.ndarray:
        keys = keylist(self.t, self.S, self.W, self.r)
        K, _ = self.gather(keys)
        return softmax_weights(q_head, K[kv_head], scale)


# ---------------------------------------------------------------------------
# Physical placement used by the bookkeeping checks (reading R3 / invariant I8)
# ---------------------------------------------------------------------------

def ring_capacity(W: int, r: int, rollback: int = 0) -> int:
    """A block leaves the window r-1 steps before its slot exists, so the ring keeps W + r
    rows; without a slot chain (r = 0) the window alone, W rows; plus the rollback rows
    that keep speculative appends undoable (reading R9)."""
    return W + r + rollback


def ring_cell(i: int, S: int, W: int, r: int, rollback: int = 0) -> int:
    """Ring row of non-sink raw position i: (i - S - 1) mod C."""
    return (i - S - 1) % ring_capacity(W, r, rollback)


def expected_ring(t: int, S: int, W: int, r: int, rollback: int = 0) -> List[Optional[int]]:
    """Closed form (I8): cell c holds the largest position i <= t, i > S, with ring_cell(i) = c."""
    C = ring_capacity(W, r, rollback)
    cells: List[Optional[int]] = [None] * C
    for c in range(C):
        i_first = S + 1 + c
        if i_first > t:
            continue
        cells[c] = i_first + ((t - i_first) // C) * C
    return cells


def append_is_legal(i: int, n_slots: int, S: int, W: int, r: int, rollback: int = 0) -> bool:
    """Writing raw position i may only overwrite a token whose block already has its slot."""
    if i <= S:
        return True
    if r == 0:
        return True            # nothing waits for a slot (reading R8)
    prev = i - ring_capacity(W, r, rollback)
    if prev <= S:
        return True
    m = -(-(prev - S) // r)   # block of the overwritten token, ceil((prev - S) / r)
    return n_slots >= m


def physical_keylist(t: int, S: int, W: int, r: int, rollback: int = 0) -> List[Tuple[int, int, int]]:
    """(segment, row, id) per logical key: segment 0 sink (row i-1), 1 ring (row
    (i-S-1) mod (W + r + rollback)), 2 slot (row m-1)."""
    out = []
    for kind, idx in keylist(t, S, W, r):
        if kind == "slot":
            out.append((2, idx - 1, idx))
        elif idx <= S:
            out.append((0, idx - 1, idx))
        else:
            out.append((1, ring_cell(idx, S, W, r, rollback), idx))
    return out


# ---------------------------------------------------------------------------
# Draft prefill (reading R10)
# ---------------------------------------------------------------------------

def prefill_attend(raw_k: np.ndarray, raw_v: np.ndarray, slot_k: np.ndarray, slot_v: np.ndarray,
                   q: np.ndarray, q_slot: np.ndarray, S: int, W: int, r: int,
                   scale: float, positions: Optional[Sequence[int]] = None,
                   slots: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of every prefix query under the decode-time memory of its step.

    raw_k/raw_v [P][Hkv][D] hold positions 1..P; slot_k/slot_v [n][Hkv][D] slots 1..n
    (n = n(P)); q [P][Hq][D] the raw queries, q_slot [n][Hq][D] the slot queries.
    Returns out [P][Hq][D] (query at position i over keylist(i)) and o_slot [n][Hq][D]
    (g_m over keylist(t_m - r)).  ``positions`` / ``slots`` (1-based) restrict the work
    to those queries; the other rows are left zero.
    """
    def gather(keys):
        ks = [raw_k[i - 1] if kind == "raw" else slot_k[i - 1] for kind, i in keys]
        vs = [raw_v[i - 1] if kind == "raw" else slot_v[i - 1] for kind, i in keys]
        return (np.stack(ks, axis=1).astype(np.float64), np.stack(vs, axis=1).astype(np.float64))

    P, n = q.shape[0], q_slot.shape[0]
    out = np.zeros(q.shape, np.float64)
    for i in (range(1, P + 1) if positions is None else positions):
        K, V = gather(keylist(i, S, W, r))
        out[i - 1] = gqa_attend(np.asarray(q[i - 1], np.float64), K, V, scale)
    o_slot = np.zeros(q_slot.shape, np.float64)
    for m in (range(1, n + 1) if slots is None else slots):
        K, V = gather(slot_query_keylist(m, S, W, r))
        o_slot[m - 1] = gqa_attend(np.asarray(q_slot[m - 1], np.float64), K, V, scale)
    return out, o_slot


# ---------------------------------------------------------------------------
# Full-KV baselines ([TR] §2.3 Eq. 2; §3.3 Algorithm 2 step 5)
# ---------------------------------------------------------------------------

def fullkv_decode(q: np.ndarray, K: np.ndarray, V: np.ndarray, t: int, scale: float) -> np.ndarray:
    """Decode at step t over the full cache rows 0..t-1: q [Hq][D], K/V [Hkv][N][D]."""
    return gqa_attend(q, np.asarray(K[:, :t], np.float64), np.asarray(V[:, :t], np.float64), scale)


def fullkv_verify(q: np.ndarray, K: np.ndarray, V: np.ndarray, t: int, scale: float) -> np.ndarray:
    """Verifier pass over n_q candidate positions ([TR] §3.3 Algorithm 2 step 5).

    q [n_q][Hq][D]; query j sits at position t - n_q + 1 + j and attends to keys
    1 .. t - n_q + 1 + j (causal over the appended candidates).
    """
    n_q = q.shape[0]
    out = np.empty(q.shape, dtype=np.float64)
    for j in range(n_q):
        out[j] = fullkv_decode(q[j], K, V, t - n_q + 1 + j, scale)
    return out


# ---------------------------------------------------------------------------
# Dense-mask brute force: an independent formulation of the same attention sets
# ---------------------------------------------------------------------------

def _masked_softmax_attend(q, entries_k, entries_v, allowed, scale):
    s = np.where(allowed, (entries_k @ q) * scale, -np.inf)
    p = np.exp(s - s[allowed].max())
    return (p @ entries_v) / p.sum()


def dense_mask_decode(q_head: np.ndarray, raw_k: np.ndarray, raw_v: np.ndarray,
                      slot_k: np.ndarray, slot_v: np.ndarray, t: int, S: int, W: int, r: int,
                      scale: float) -> np.ndarray:
    """Decode at step t by masking every entry ever created (one KV head).

    raw_k/raw_v [t][D] hold positions 1..t; slot_k/slot_v [n][D] hold every slot
    created so far.  A raw token is allowed iff it is a sink or inside the last W
    non-sink positions ([TR] Eq. 4); a slot is allowed iff its materialization step
    S + W + m*r has been reached.
    """
    entries_k = np.concatenate([raw_k[:t], slot_k], axis=0).astype(np.float64)
    entries_v = np.concatenate([raw_v[:t], slot_v], axis=0).astype(np.float64)
    allowed = np.zeros(entries_k.shape[0], dtype=bool)
    for i in range(1, t + 1):
        allowed[i - 1] = (i <= S) or (i > S and i > t - W)
    m = 1
    while r > 0 and m <= slot_k.shape[0]:
        if S + W + m * r <= t:
            allowed[t + m - 1] = True
        m += 1
    return _masked_softmax_attend(np.asarray(q_head, np.float64), entries_k, entries_v, allowed, scale)


def dense_mask_slot_query(q_head: np.ndarray, raw_k: np.ndarray, raw_v: np.ndarray,
                          slot_k: np.ndarray, slot_v: np.ndarray, m: int, S: int, W: int, r: int,
                          scale: float, include_self: bool = False) -> np.ndarray:
    """Slot g_m's query by masking every entry (one KV head); see reading R1.

    Allowed: sinks; the W raw positions starting at the first token of block B_m;
    slots created before g_m (and g_m itself with include_self).
    """
    n_raw = raw_k.shape[0]
    entries_k = np.concatenate([raw_k, slot_k], axis=0).astype(np.float64)
    entries_v = np.concatenate([raw_v, slot_v], axis=0).astype(np.float64)
    allowed = np.zeros(entries_k.shape[0], dtype=bool)
    first = S + (m - 1) * r + 1
    for i in range(1, n_raw + 1):
        allowed[i - 1] = (i <= S) or (first <= i < first + W)
    for mm in range(1, slot_k.shape[0] + 1):
        allowed[n_raw + mm - 1] = (mm < m) or (include_self and mm == m)
    return _masked_softmax_attend(np.asarray(q_head, np.float64), entries_k, entries_v, allowed, scale)
