// masw_internal.hpp - argument blocks and launchers between the C ABI (capi.hip) and
// the kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "masw_device.hpp"
#include "decode_args.hpp"

namespace masw {

// Append raw tokens into a memory (sink + ring; a full cache is all sink).
struct AppendArgs {
  void* k_sink; void* v_sink;
  void* k_ring; void* v_ring;
  int sink_cap;             // rows per (sequence, KV head) of the sink block
  MemGeom g;
  const int32_t* seq_len;
  int32_t* err;
  const int32_t* n_slots;   // null for a full cache
  int max_len;              // full cache bound (0: none)
  const void* k_new; const void* v_new;   // [B][n_new][Hkv][D]
  int B, Hkv, D, n_new;
  // Prefill (> 0): k_new/v_new hold a whole prefix [B][prefill_len][Hkv][D], each
  // sequence appends its own seq_len[b] positions, and only the ones the memory keeps
  // (sinks and the newest C) are moved; n_new is unused.
  int prefill_len;
};

int launch_append(const AppendArgs& a, int dtype, hipStream_t s);

// Rollback rows a memory may keep (ring rows are W + r + rollback).
constexpr int kMaxRollback = 4096;
// Largest S, W and max_slots: positions and row indices stay far from int32 overflow
// (S + W + r + rollback and S + m r are formed in 32 bits).
constexpr int kMaxMemRows = 1 << 28;
// Largest batch and KV head count: they are grid dimensions (y/z at most 65535).
constexpr int kMaxGridDim = 65535;
int launch_rollback(const MemGeom& g, int rollback, const int32_t* seq_len, const int32_t* t_spec,
                    int32_t* n_slots, int32_t* err, int B, hipStream_t s);

// Mirrored projection of the slot hidden state into slot row m-1, plus the
// per-sequence boundary decision written to `active`.
struct ProjectArgs {
  const void* h;            // [B][hidden]
  const void* w_k; const void* w_v;   // [hidden][Hkv*D]
  void* k_slot; void* v_slot;         // [B][Hkv][max_slots][D]
  const int32_t* seq_len;
  int32_t* n_slots;         // read at a boundary; written by a prefill
  int32_t* err;
  int32_t* active;          // [B] workspace
  MemGeom g;
  int B, Hkv, D, hidden;
  // bf16: the hidden dimension is cut into ksplits slices of k_per_split rows (a
  // multiple of 128); with ksplits > 1 the slices' partial sums go through part
  // ([groups of 16 sequences][2][ksplits][16][Hkv*D] fp32) and the per-column-block
  // tickets counters ([groups][2][Hkv*D/64], zero between calls).
  int ksplits, k_per_split;
  float* part;
  int32_t* counters;
  // Rotary embedding of K_g (rope_theta > 0) at id S + m*r; rope_style 0: pairs
  // (j, j + D/2), 1: pairs (2j, 2j + 1).
  float rope_theta;
  int rope_style;
  // Prefill (> 0): h holds prefill_ns slot hidden states per sequence
  // ([B][prefill_ns][hidden]); rows are (sequence, slot) pairs and every slot
  // 1..n(seq_len[b]) is projected, after which n_slots[b] = n(seq_len[b]).  Needs
  // ksplits == 1; `active` is not used.
  int prefill_ns;
};

constexpr int kMaxProjectSplits = 8;
// Hidden rows per projection slice and the number of slices for a given hidden size.
inline int project_k_per_split(int hidden) {
  const int per = (hidden + kMaxProjectSplits - 1) / kMaxProjectSplits;
  return (per + 127) / 128 * 128;
}
inline int project_splits(int hidden) {
  const int per = project_k_per_split(hidden);
  return (hidden + per - 1) / per;
}

int launch_project(const ProjectArgs& a, int dtype, hipStream_t s);

// One launch for a bf16 slot boundary: the projection's work-groups (grid proj_x x 2 x
// proj_z, flattened) followed by the gated slot query's (splits x Hkv x B); `done` is a
// workspace ticket (zero between calls) and `publish` (the layer's n_slots) receives m.
struct BoundaryArgs {
  ProjectArgs p;
  DecodeArgs d;
  int proj_x, n_proj, n_wg;
  int32_t* done;
  int32_t* publish;
};

int launch_boundary(const BoundaryArgs& a, int D, hipStream_t s);

// Draft prefill attention (bf16, D = 128): every raw query of a prefix and every slot
// query, each under the memory of its own step.  One work-group per block of `qb`
// consecutive queries of one (sequence, KV head); blocks [0, raw_blocks) hold raw
// queries, [raw_blocks, raw_blocks + slot_blocks) slot queries.
struct PrefillArgs {
  const void* k; const void* v;             // raw prefix [B][p_max][Hkv][D]
  const void* k_slot; const void* v_slot;   // the layer's slots [B][Hkv][max_slots][D]
  const int32_t* n_slots;
  MemGeom g;
  const int32_t* seq_len;
  int32_t* err;
  const void* q;                            // [B][p_max][Hq][D]
  const void* q_slot;                       // [B][ns_max][Hq][D]
  void* out;                                // like q
  void* o_slot;                             // like q_slot
  int B, Hq, Hkv, p_max, ns_max;
  int qb, raw_blocks, slot_blocks;
  float scale_log2;
};

int prefill_rows_per_block();

// Matrix-core rate probe (measurement helper): work_groups x 256 threads.
int launch_mfma_rate(int work_groups, int iters, float* out, uint64_t* clocks, hipStream_t s);
int launch_prefill(const PrefillArgs& a, hipStream_t s);

// Multi-query verifier attention over a full cache on the matrix cores (bf16, D=128,
// Hq/Hkv * n_q <= 64 rows per KV head).  Same partial/merge protocol as DecodeArgs.
struct VerifyArgs {
  const void* k; const void* v;   // [B][Hkv][max_len][D]
  int max_len;
  const int32_t* seq_len;
  int32_t* err;
  const void* q;                  // [B][n_q][Hq][D]
  void* out;
  int32_t* counters;
  float* part_o;                  // [B][n_q*Hq][splits][D]
  float* part_ml;
  int B, Hq, Hkv, n_q, n_splits;
  float scale_log2;
};

int launch_verify_mfma(const VerifyArgs& a, hipStream_t s);
constexpr int kMaxVerifySplits = 64;   // splits the MFMA verifier merges (more are clamped)
// Verifier work-groups resident per CU: the streaming kernel holds ~132 KB of LDS.
inline int verify_resident_per_cu(int /*rows*/) { return 1; }

}  // namespace masw
