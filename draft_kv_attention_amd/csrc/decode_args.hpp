// decode_args.hpp - the decode kernel's tuning switches, argument block and launchers
// (kept apart from the other kernels' argument blocks: the decode kernel is built from
// this header, masw_device.hpp and decode_attn.hip only).  Not installed; not part of the
// ABI.
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

}  // namespace masw
