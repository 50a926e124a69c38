// decode_args.hpp - the decode kernel's tuning switches, argument block and launchers
// (kept apart from the other kernels' argument blocks: the decode kernel is built from
// this header, masw_device.hpp and decode_attn.hip only).  Not installed; not part of the
// ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "masw_device.hpp"

namespace masw {

// Decode streaming: each wave keeps kPipeStages tiles in flight as asynchronous
// global->LDS copies (global_load_lds_dwordx4, kPipeStageInstr 1 KB copies per tile) and
// reduces the oldest one from registers, so the vector work of one tile overlaps the
// memory time of the next.  Measured on the 3B layer share (B = 8, t = 32768): three or
// four stages per wave, eight-wave work-groups and two work-groups per CU were all
// slower than two stages, four waves and one work-group per CU (see the design notes).
constexpr int kDecodeThreads = 256;
constexpr int kPipeStages = 2;
constexpr int kPipeStageInstr = 8;   // 1 KB load instructions per stage
// Decode work-groups per CU that the split heuristic aims for.
constexpr int kDecodeResidentPerCU = 1;

// Keys per wave tile: one stage holds the K and V rows of a tile.
template <int ELEM_BYTES, int D>
constexpr int decode_tile_keys() { return kPipeStageInstr * 1024 / (2 * D * ELEM_BYTES); }

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
  int gate_boundary;        // slot-query mode without `active`: decide m from seq_len, n_slots
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

}  // namespace masw
