// masw_internal.hpp - argument blocks and launchers between the C ABI (capi.hip) and
// the kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "masw_device.hpp"

namespace masw {

// Decode streaming.  With MASW_DECODE_LDS_PIPE each wave keeps MASW_DECODE_PIPE_STAGES
// tiles in flight as asynchronous global->LDS copies (global_load_lds_dwordx4) and
// reduces the oldest one from registers, so the VALU work of one tile overlaps the
// memory time of the next ones.  Otherwise tiles are loaded straight into registers,
// optionally double-buffered.  MASW_DECODE_TILE_KEYS (0: per instantiation, see
// decode_tile_keys) and MASW_DECODE_NT (non-temporal hint) apply to the register path.
#ifndef MASW_DECODE_LDS_PIPE
#define MASW_DECODE_LDS_PIPE 1
#endif
#ifndef MASW_DECODE_PIPE_STAGES
#define MASW_DECODE_PIPE_STAGES 2
#endif
#ifndef MASW_DECODE_PIPE_STAGE_INSTR
#define MASW_DECODE_PIPE_STAGE_INSTR 8
#endif
#ifndef MASW_DECODE_TILE_KEYS
#define MASW_DECODE_TILE_KEYS 0
#endif
#ifndef MASW_DECODE_DOUBLE_BUFFER
#define MASW_DECODE_DOUBLE_BUFFER 0
#endif
#ifndef MASW_DECODE_NT
#define MASW_DECODE_NT 0
#endif
#ifndef MASW_DECODE_THREADS
#define MASW_DECODE_THREADS 256
#endif
constexpr bool kDecodeLdsPipe = MASW_DECODE_LDS_PIPE != 0;
constexpr int kPipeStages = MASW_DECODE_PIPE_STAGES;
constexpr int kPipeStageInstr = MASW_DECODE_PIPE_STAGE_INSTR;   // 1 KB load instructions per stage
constexpr bool kDecodeDoubleBuffer = MASW_DECODE_DOUBLE_BUFFER != 0;
constexpr bool kDecodeNonTemporal = MASW_DECODE_NT != 0;
constexpr int kDecodeThreads = MASW_DECODE_THREADS;
static_assert(!kDecodeLdsPipe || (kPipeStages >= 2 && kPipeStages <= 3), "two or three stages");
static_assert(!kDecodeLdsPipe || kPipeStageInstr * (kPipeStages - 1) <= 63, "s_waitcnt vmcnt holds 6 bits");
// LDS of the pipeline per work-group (it must leave room for the merge buffers).
constexpr int kPipeLdsBytes = (kDecodeThreads / 64) * kPipeStages * kPipeStageInstr * 1024;
static_assert(!kDecodeLdsPipe || kPipeLdsBytes <= 128 * 1024, "pipeline LDS fits beside the merge buffers");
// Decode work-groups per CU that the split heuristic aims for.  Measured on the 3B layer
// share (B = 8, 8 KV heads, 2.5K keys): one work-group per CU (4 splits) beats two
// (8 splits) for every loop variant, the extra partials and merge traffic costing more
// than the extra waves gain.
constexpr int kDecodeResidentPerCU = 1;

// Keys per wave tile.  Pipeline: one stage holds the K and V rows of a tile,
// kPipeStageInstr x 64 lanes x 16 bytes.  Register path: as many K/V bytes in flight
// per wave as fit beside the G query fragments and accumulators without dropping below
// two waves per SIMD (bf16, D = 128: 64 keys for G <= 3).
template <int ELEM_BYTES, int D, int G>
constexpr int decode_tile_keys() {
  if (kDecodeLdsPipe) return kPipeStageInstr * 1024 / (2 * D * ELEM_BYTES);
  if (MASW_DECODE_TILE_KEYS > 0) return MASW_DECODE_TILE_KEYS;
  if (ELEM_BYTES == 2) return G <= 3 || D == 64 ? 64 : 32;
  return 32;
}

// Split-K decode attention over one memory (three segments; a full cache is the sink
// segment alone).  One work-group per (split, KV head, sequence).  With several splits
// each work-group writes an (max, sum, o) partial and the last one to finish a
// (sequence, KV head) merges them, using a counter that it resets to zero.
struct DecodeArgs {
  const void* k[3];   // segment bases: sink, ring, slot
  const void* v[3];
  int cap[3];         // rows per (sequence, KV head) in each segment
  MemGeom g;
  const int32_t* seq_len;
  int32_t* err;
  const int32_t* n_slots;   // MASW decode: checked against n(t); null for a full cache
  const int32_t* active;    // slot-query mode: per-sequence slot index m (0 = skip)
  int32_t* n_slots_out;     // slot-query mode: set to m once the query is written
  int back;                 // keys of keylist(t - back)
  int self_slot;            // slot-query mode: also attend to the new slot itself
  int max_len;              // full cache: t must not exceed it (0: no bound)
  int min_t;                // t below this is out of range (besides t - back >= 1)
  // Fused append (n_new > 0): positions t-n_new+1..t are read from k_new/v_new
  // ([B][n_new][Hkv][D]) and written into the memory by split 0 of each KV head.
  const void* k_new;
  const void* v_new;
  int n_new;
  void* wk[2];              // write bases: sink (or the full cache), ring
  void* wv[2];
  int32_t* counters;        // [B*Hkv] split-merge tickets, zero between calls
  const void* q;            // q + b*qo_stride + h*D
  void* out;                // out + b*qo_stride + h*D
  long qo_stride;           // elements between sequences in q/out
  float* part_o;            // [B][Hq][splits][D]
  float* part_ml;           // [B][Hq][splits][2]  (running max in log2 units, sum)
  int B, Hq, Hkv, n_splits;
  float scale_log2;         // softmax scale times log2(e)
};

int launch_decode(const DecodeArgs& a, int dtype, int D, hipStream_t s);
int launch_debug_keylist(const MemGeom& g, const int32_t* seq_len, int B, int back,
                         int32_t* out, int max_keys, hipStream_t s);

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
// MASW_VERIFY_STREAM 1: waves stream their own key ranges through private LDS stages
// (verify_stream_kernel, one 128 KB work-group per CU); 0: work-group tiles staged
// through registers (verify_kernel).
#ifndef MASW_VERIFY_STREAM
#define MASW_VERIFY_STREAM 1
#endif
constexpr bool kVerifyStream = MASW_VERIFY_STREAM != 0;
// Verifier work-groups that stay resident per CU for `rows` = G * n_q query rows.  The
// streaming kernel holds 128 KB of LDS: one per CU.  The register-staged kernel, measured
// on 8B / 70B layer shares: 32-row blocks fill the chip best at one per CU, 64-row
// blocks at two.
inline int verify_resident_per_cu(int rows) { return kVerifyStream || rows <= 32 ? 1 : 2; }

}  // namespace masw
