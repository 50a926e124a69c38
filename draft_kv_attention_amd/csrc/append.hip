// append.hip - raw-token append with implicit eviction (Technical Review §3.2,
// Algorithm 1 step 5; §3.1 Eq. 4 local bullet).
//
// Position i <= S lands in sink row i-1; i > S in ring row (i-S-1) mod C, C = W + r
// plus the rollback rows.  The ring keeps at least W + r rows because a block leaves
// the W-window r-1 steps before its slot is materialized and the slot query still reads
// it (the rollback rows keep speculative appends undoable); overwriting a row therefore
// evicts the token i-C, which is legal only once that token's block has its slot.
// Each thread moves one 16-byte packet of K and of V; all packets of one token take
// the same decision (append_fate), so an illegal token is skipped whole, and so is a
// token a later position of the same call overwrites.  A prefill append takes a whole
// prefix per sequence and moves only the tokens the memory keeps after it.
#include "masw_internal.hpp"

namespace masw {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a) {
  constexpr int VEC = 16 / int(sizeof(T));
  const int b = blockIdx.y;
  const int per_tok = a.Hkv * a.D;
  const bool prefill = a.prefill_len > 0;
  // prefill: token slots [0, S) are the sinks, [S, S + C) the newest C positions
  const int n_tok = prefill ? a.g.S + a.g.C : a.n_new;
  const int packets = n_tok * per_tok / VEC;
  const int t = a.seq_len[b];
  if (prefill ? (t < 0 || t > a.prefill_len) : (t < a.n_new || (a.max_len > 0 && t > a.max_len))) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(a.err, MASW_DEV_SEQ_RANGE);
    return;
  }
  if (prefill && a.g.r > 0) {
    // the prefill's projection publishes n_slots = n(t); if it could not (it reported
    // why), the sequence is left alone
    const int dd = t - a.g.S - a.g.W;
    if (a.n_slots[b] != (dd > 0 ? dd / a.g.r : 0)) return;
  }
  const int first = prefill ? max(a.g.S, t - a.g.C) + 1 : 0;   // oldest ring position a prefill keeps
  int bits = 0;
  for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < packets; p += gridDim.x * blockDim.x) {
    const int e = p * VEC;
    const int j = e / per_tok;
    const int rem = e - j * per_tok;
    const int kvh = rem / a.D;
    const int d = rem - kvh * a.D;
    int i, src_row;
    if (prefill) {
      i = j < a.g.S ? j + 1 : first + (j - a.g.S);
      if (i > t) continue;
      src_row = i - 1;
    } else {
      i = t - a.n_new + 1 + j;
      src_row = j;
    }
    const size_t unit = size_t(b) * a.Hkv + kvh;
    T* dk;
    T* dv;
    size_t off;
    if (i <= a.g.S) {
      off = (unit * a.sink_cap + (i - 1)) * a.D + d;
      dk = static_cast<T*>(a.k_sink);
      dv = static_cast<T*>(a.v_sink);
    } else {
      const AppendFate f = append_fate(i, t, a.n_slots ? a.n_slots[b] : 0, a.g);
      if (f == kAppendIllegal) bits |= MASW_DEV_PENDING_SLOT;
      if (f != kAppendWrite) continue;
      off = (unit * a.g.C + (i - a.g.S - 1) % a.g.C) * a.D + d;
      dk = static_cast<T*>(a.k_ring);
      dv = static_cast<T*>(a.v_ring);
    }
    const int src_len = prefill ? a.prefill_len : a.n_new;
    const size_t src = ((size_t(b) * src_len + src_row) * a.Hkv + kvh) * a.D + d;
    *reinterpret_cast<uint4*>(dk + off) = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.k_new) + src);
    *reinterpret_cast<uint4*>(dv + off) = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.v_new) + src);
  }
  if (bits) atomicOr(a.err, bits);
}

// Rollback: one thread per sequence.  The accepted memory keeps the slots materialized
// at or before t_acc, n(t_acc) of them; the raw tokens need nothing (rollback rows).
__global__ void rollback_kernel(const MemGeom g, int rollback, const int32_t* seq_len, const int32_t* t_spec,
                                int32_t* n_slots, int32_t* err, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int t_acc = seq_len[b], ts = t_spec[b];
  if (t_acc < 0 || t_acc > ts || ts - t_acc > rollback) {
    atomicOr(err, MASW_DEV_ROLLBACK_RANGE);
    return;
  }
  const int d = t_acc - g.S - g.W;
  const int n = d > 0 && g.r > 0 ? d / g.r : 0;
  const int have = n_slots[b];
  if (have > n) n_slots[b] = n;
  else if (have < n) atomicOr(err, MASW_DEV_SLOT_MISSING);
}

}  // namespace

int launch_rollback(const MemGeom& g, int rollback, const int32_t* seq_len, const int32_t* t_spec,
                    int32_t* n_slots, int32_t* err, int B, hipStream_t s) {
  hipLaunchKernelGGL(rollback_kernel, dim3((B + 255) / 256), dim3(256), 0, s, g, rollback, seq_len, t_spec,
                     n_slots, err, B);
  return hipGetLastError() == hipSuccess ? MASW_OK : MASW_ERR_LAUNCH;
}

int launch_append(const AppendArgs& a, int dtype, hipStream_t s) {
  const int vec = dtype == MASW_BF16 ? 8 : 4;
  const long tokens = a.prefill_len > 0 ? long(a.g.S) + a.g.C : long(a.n_new);
  const long packets = tokens * a.Hkv * a.D / vec;
  const int blocks = int(std::min<long>((packets + 255) / 256, 1024));
  if (dtype == MASW_BF16)
    hipLaunchKernelGGL(append_kernel<uint16_t>, dim3(blocks, a.B), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(append_kernel<float>, dim3(blocks, a.B), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? MASW_OK : MASW_ERR_LAUNCH;
}

}  // namespace masw
