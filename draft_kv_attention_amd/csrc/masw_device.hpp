// masw_device.hpp - device helpers shared by the libmasw kernels (gfx950, wave64).
//
// The one key resolver below is used by every attention kernel and by the debug dump,
// so the segment bookkeeping the tests compare bit-exactly is the bookkeeping the
// attention actually reads through.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/masw.h"

namespace masw {

constexpr int kWave = 64;

// 16 bytes as a native vector (struct types such as uint4 can end up in scratch memory
// when indexed).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;          // LDS-DMA destination
// Cache policy of the LDS-DMA copies that stream K/V rows read once per launch (the
// decode kernel, the verifier): the non-temporal hint (`nt`), so the stream does not
// displace other lines in L2 and the Infinity Cache.  Measured: the 8B verifier layer
// 103 -> 92-94 us, the fused decode launch about 0.5 us faster.  The prefill re-reads
// its K/V tiles from L2 across query blocks and keeps the default policy.
constexpr int kStreamLoadNT = 2;
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;      // LDS transpose-read source

// Two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; a field at its maximum does not wait).  The compiler does not order a
// read of LDS after the asynchronous global->LDS copies that fill it: kernels wait
// with these explicitly.
constexpr int waitcnt_vm(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }
constexpr int kWaitLgkm0 = 0xf | (0x3 << 14) | (0x7 << 4);

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (bf16 = upper half of an IEEE binary32)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round to nearest, ties to even: add 0x7fff plus the lowest kept bit, then truncate.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static float to_f32(float x) { return x; }
  __device__ static float from_f32(float x) { return x; }
};
template <> struct Elem<uint16_t> {
  __device__ static float to_f32(uint16_t x) { return bf16_to_f32(x); }
  __device__ static uint16_t from_f32(float x) { return f32_to_bf16(x); }
};

// ---------------------------------------------------------------------------
// Cross-lane reductions
// ---------------------------------------------------------------------------
// v + (v of the lane a DPP control selects).  The identity as the "old" operand lets the
// compiler fold the move into the add (v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes of a DPP row (row_ror 8, 4, 2, 1): every lane gets the total.
__device__ __forceinline__ float row16_sum(float v) {
  return dpp_add<0x121>(dpp_add<0x122>(dpp_add<0x124>(dpp_add<0x128>(v))));
}

// Combine across the four 16-lane rows of a wave on the VALU.  v_permlane16_swap
// (v_permlane32_swap) with both operands a copy of v returns, in every lane, the values
// of the lane pair {l, l^16} ({l, l^32}) in a fixed order; no LDS round trip.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float rows4_max(float v) { return max_xor32(max_xor16(v)); }
__device__ __forceinline__ float rows4_sum(float v) { return sum_xor32(sum_xor16(v)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Split merge inside one launch (flash-decoding without a second kernel)
// ---------------------------------------------------------------------------
// Work-groups of one unit exchange partial results through memory.  On a multi-XCD
// part a device-scope __threadfence() writes back and invalidates the whole L2 of the
// issuing XCD, which costs far more than the partials themselves, so partials are
// written and read with agent-scope relaxed atomics (per-access write-through /
// L2-bypassing, coherent across XCDs).  Every work-group stores its partial, waits for
// the stores (s_waitcnt vmcnt(0)), then takes a ticket (split_arrive); the last arrival
// loads the others' partials and resets the ticket.  The decode kernel's split merge and
// the projection's hidden slices both work this way.

__device__ __forceinline__ void store_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_partial(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two adjacent 32-bit words (an 8-byte aligned pair) as one 64-bit access.
__device__ __forceinline__ void store_word2(void* p, uint32_t w0, uint32_t w1) {
  __hip_atomic_store(static_cast<uint64_t*>(p), (uint64_t(w1) << 32) | w0, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ u32x2_t load_word2(const void* p) {
  const uint64_t w = __hip_atomic_load(static_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x2_t{uint32_t(w), uint32_t(w >> 32)};
}

__device__ __forceinline__ void store_partial2(float* p, float v0, float v1) {
  store_word2(p, __float_as_uint(v0), __float_as_uint(v1));
}

__device__ __forceinline__ float2 load_partial2(const float* p) {
  const u32x2_t w = load_word2(p);
  return make_float2(__uint_as_float(w.x), __uint_as_float(w.y));
}

// Called by every thread of the work-group after its partial stores; true (for the
// whole work-group) when this is the last of n_valid arrivals.  The last arrival
// resets the counter with reset_ticket() once it has merged.
__device__ __forceinline__ bool split_arrive(int32_t* counter, int n_valid, int* sm_flag) {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's partial stores are done
  __syncthreads();
  if (threadIdx.x == 0)
    *sm_flag = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_valid - 1;
  __syncthreads();
  return *sm_flag != 0;
}

__device__ __forceinline__ void reset_ticket(int32_t* counter) {
  __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte slot swizzle of a 32-key K/V tile in LDS (rows of 256 bytes, as the matrix-core
// kernels stage them): slot = chunk ^ tile_swz(row), the row's two low
// bits moved above its next two.  With 64 LDS banks (256-byte rows, so slot s of every
// row is banks 4s..4s+3) both operand reads are conflict-free: the K read's 16 lanes per
// pass take rows 0..15 at one chunk (a bijection of the row), and the transposing V read's
// 32 lanes take 4 consecutive keys x 4 chunks of one aligned group (the keys' swizzles
// differ in the bits above the group).
__device__ __forceinline__ int tile_swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// ---------------------------------------------------------------------------
// Memory geometry and the key resolver (Technical Review §3.1, Eq. 4)
// ---------------------------------------------------------------------------
struct MemGeom {
  int S;          // sink count (a full cache is a memory whose every token is a sink)
  int W;          // local window
  int r;          // slot interval; 0 = no slot chain (sinks + window only)
  int C;          // ring rows, W + r (W without a slot chain)
  int max_slots;  // slot rows per (sequence, KV head)
};

// Counts of keylist(t): sinks, local window, slots; lo = first local position,
// ring0 = ring row of position lo.
struct KeySpan {
  int ns, nl, nslot, lo, ring0;
  __device__ int total() const { return ns + nl + nslot; }
};

__device__ __forceinline__ KeySpan key_span(int t, const MemGeom& g) {
  KeySpan k;
  k.ns = min(g.S, t);
  k.nl = min(max(t - g.S, 0), g.W);
  k.lo = t - k.nl + 1;
  int d = t - g.S - g.W;
  k.nslot = d > 0 && g.r > 0 ? d / g.r : 0;   // r = 0: no slot chain
  k.ring0 = k.nl > 0 ? (k.lo - g.S - 1) % g.C : 0;
  return k;
}

// Raw append ([TR] §3.2 Algorithm 1 step 5).  Writing non-sink position i into ring row
// (i-S-1) mod C evicts the token `victim` = i - C held there; that is legal once the
// victim's block has its slot (always without a slot chain, or for a sink/never-written
// row).
__device__ __forceinline__ bool evict_ok(int victim, int have, const MemGeom& g) {
  return victim <= g.S || g.r == 0 || have >= (victim - g.S + g.r - 1) / g.r;
}

enum AppendFate { kAppendWrite = 0, kAppendSuperseded = 1, kAppendIllegal = 2 };

// Fate of non-sink position i in an append call whose newest position is t, with `have`
// slots materialized.  A call may hold more than C positions; read sequentially, the
// positions landing in one row are written in order, and legality along that chain is
// monotone (each evicts a later token than the one before), so i's write is final iff
// it is legal and the next position of the chain (i + C, if in this call) does not
// legally overwrite it.  Illegal writes are suppressed and reported.
__device__ __forceinline__ AppendFate append_fate(int i, int t, int have, const MemGeom& g) {
  if (!evict_ok(i - g.C, have, g)) return kAppendIllegal;
  if (i + g.C <= t && evict_ok(i, have, g)) return kAppendSuperseded;
  return kAppendWrite;
}

// Slot index m whose boundary step is t ([TR] §3.2 Algorithm 1 step 1: g_m is
// materialized at t = S + W + m r) when the memory holds exactly m - 1 slots and has room
// for the m-th; 0 otherwise (no boundary, already done, out of order or out of room).
__device__ __forceinline__ int pending_slot(int t, int have, const MemGeom& g) {
  const int d = t - g.S - g.W;
  if (g.r < 1 || d < g.r || d % g.r) return 0;
  const int m = d / g.r;
  return have == m - 1 && m <= g.max_slots ? m : 0;
}

struct KeyRef {
  int seg;  // 0 sink, 1 ring, 2 slot
  int row;  // row inside that segment's [rows][D] block
  int id;   // raw position (sink / ring) or slot index m
};

// Logical key j (0-based, order sink ++ local ++ slots) -> physical row.
__device__ __forceinline__ KeyRef resolve_key(int j, const KeySpan& k, const MemGeom& g) {
  KeyRef r;
  if (j < k.ns) {
    r.seg = 0; r.row = j; r.id = j + 1;
  } else if (j < k.ns + k.nl) {
    int o = j - k.ns;
    int c = k.ring0 + o;
    if (c >= g.C) c -= g.C;
    r.seg = 1; r.row = c; r.id = k.lo + o;
  } else {
    int m = j - k.ns - k.nl;
    r.seg = 2; r.row = m; r.id = m + 1;
  }
  return r;
}

}  // namespace masw
