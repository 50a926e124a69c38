/*
 * masw.h - C ABI of libmasw.so: the hot path of Memory-Augmented Sliding-Window (MASW)
 * drafting on AMD MI355X (gfx950).
 *
 * Pages cited (title; section / equation / algorithm step on that page):
 *   [TR] "Strong Drafts Need Compact Memories: A Technical Review of Memory-Augmented
 *        Sliding-Window (MASW) Drafting for Long-Context Speculative Decoding".
 *
 * Notation follows [TR]: S sink tokens, W local-window width, r slot interval,
 * t = number of raw tokens in a sequence's cache INCLUDING the token(s) being appended
 * or queried this step (Eq. 2 attends over K_{<=t}); positions are 1-based; g_m is the
 * m-th memory slot.  The draft memory at step t is ([TR] §3.1, Eq. 4)
 *     keylist(t) = sinks 1..min(S,t)  ++  local max(S+1, t-W+1)..t  ++  slots 1..n(t)
 * with n(t) = floor(max(0, t-S-W) / r).  Slot g_m compresses raw positions
 * S+(m-1)r+1 .. S+mr and is materialized at step t_m = S + W + m*r ([TR] §3.2,
 * Algorithm 1), after raw token t_m is appended and before the decode query at t_m.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Ownership: every pointer argument is DEVICE memory owned by the caller.  The
 *    library allocates nothing, keeps no global state and is thread-safe.
 *  - Streams: every call only enqueues kernels on `stream` (a hipStream_t; NULL is the
 *    legacy default stream).  No call synchronizes or reads device memory on the host,
 *    so a sequence of calls can be captured into a HIP graph.
 *  - Return value: MASW_OK or a negative MASW_ERR_* for errors found on the host before
 *    anything is enqueued (or MASW_ERR_LAUNCH if a launch fails).  Nothing is enqueued
 *    when a host error is returned.
 *  - Device errors: violations only the device can see (they depend on seq_len and
 *    n_slots) are OR-ed into the caller's sticky int32 error word `*err` as
 *    MASW_DEV_* bits, and the offending sequence's writes are suppressed (its output,
 *    cache rows or slot stay untouched).  The caller clears *err when it wants.
 *  - Layouts are row-major with the last index contiguous.  bf16 tensors hold IEEE
 *    bfloat16 bit patterns; results are rounded to nearest-even.  Accumulation is fp32.
 *  - Alignment: every tensor pointer (K/V caches and slots, q, out, k_new, v_new,
 *    hidden states, projection weights, slot queries and outputs) must be 16-byte
 *    aligned, since the kernels move rows in 16-byte pieces; a misaligned one is
 *    rejected with MASW_ERR_ARG.  int32 arrays (seq_len, n_slots, err) need only their
 *    natural alignment.
 *  - Workspace: ops that split the key range (flash-decoding split-K) need a scratch
 *    buffer of at least masw_workspace_bytes(...) bytes, 256-byte aligned, that no other
 *    call uses concurrently.  The caller zero-fills it once after allocating it; every
 *    call leaves the ticket counters it uses back at zero, so no later clearing is
 *    needed (the decode paths merge their splits in the same launch: the last
 *    work-group of each (sequence, KV head) combines the partials; fullkv_verify_attn
 *    merges them in a second kernel it enqueues on the same stream).  Where counters
 *    and partials sit depends on the plan, so a workspace serves one plan: calls may
 *    share it when they pass equal masw_dims (masw_draft_attn, masw_decode_step and
 *    masw_materialize_slot of one dims share a plan; the full-KV ops also need equal
 *    max_len, and n_q for the verifier).  Before a call with another plan uses it, the
 *    caller zero-fills it again, or uses another buffer: otherwise that plan's counters
 *    may lie where the previous plan left partial sums, and results are wrong.
 */
#ifndef MASW_H_
#define MASW_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MASW_API __attribute__((visibility("default")))
#define MASW_ABI_VERSION 6

/* ---- host status codes ------------------------------------------------------- */
enum {
  MASW_OK = 0,
  MASW_ERR_ARG = -1,           /* a null pointer, a negative size, r outside 1..W ... */
  MASW_ERR_DTYPE = -2,         /* dtype not MASW_F32 / MASW_BF16                     */
  MASW_ERR_SHAPE = -3,         /* Hq % Hkv != 0, head_dim not 64/128, group > 8 ...   */
  MASW_ERR_WORKSPACE = -4,     /* workspace missing, too small or misaligned          */
  MASW_ERR_LAUNCH = -5,        /* hipGetLastError() reported a launch failure         */
  MASW_ERR_UNIMPLEMENTED = -6  /* a valid request the library does not support        */
};

/* ---- device error bits (OR-ed into *err) -------------------------------------- */
enum {
  MASW_DEV_PENDING_SLOT = 1,  /* an append would overwrite a raw token whose block has
                                 no slot yet; that token's write was suppressed          */
  MASW_DEV_SLOT_CAPACITY = 2, /* a step needs more than max_slots slots                  */
  MASW_DEV_SEQ_RANGE = 4,     /* seq_len out of range (t < 1 for a query, t < n_new for
                                 an append, t > max_len for a full cache, t < n_q ...)   */
  MASW_DEV_SLOT_MISSING = 8,  /* a query needs slot n(t) (or a boundary needs slot m-1)
                                 but n_slots says it was never materialized              */
  MASW_DEV_ROLLBACK_RANGE = 16 /* a rollback reaches further back than the rollback rows
                                 keep (or forward); that sequence was left as it was      */
};

typedef enum { MASW_F32 = 0, MASW_BF16 = 1 } masw_dtype;

/* Pairing of a head vector's components in the rotary embedding of slot keys. */
typedef enum {
  MASW_ROPE_ROTATE_HALF = 0,  /* components i and i + D/2 turn together (Llama layout) */
  MASW_ROPE_INTERLEAVED = 1   /* components 2i and 2i + 1 turn together               */
} masw_rope_style;

/* Geometry and memory parameters.  S, W, r and max_slots are ignored by the
 * full-KV entry points. */
typedef struct {
  int32_t batch;       /* 1 <= B <= 65535 sequences (a grid dimension)              */
  int32_t n_q_heads;   /* Hq; query head h reads KV head h / (Hq/Hkv) (grouped)     */
  int32_t n_kv_heads;  /* Hkv <= 65535; Hq % Hkv == 0 and Hq/Hkv in {1,2,3,4,6,8}  */
  int32_t head_dim;    /* D in {64, 128}                                           */
  int32_t sink;        /* 0 <= S <= 2^28                                           */
  int32_t window;      /* 1 <= W <= 2^28                                           */
  int32_t interval;    /* r, 1 <= r <= W; the local ring holds C = W + r rows.
                          r = 0: no slot chain - sinks ++ the exact W-window only
                          (StreamingLLM-style with S > 0, a sliding window with
                          S = 0); the ring holds C = W rows and every append is
                          legal; masw_materialize_slot returns MASW_ERR_ARG        */
  int32_t max_slots;   /* slot rows allocated per (sequence, KV head), 0..2^28      */
  int32_t dtype;       /* masw_dtype of every K/V/q/out/h/w tensor                 */
  float scale;         /* softmax scale; <= 0 selects 1/sqrt(D) ([TR] §2.3 Eq. 2)  */
  int32_t num_splits;  /* split-K plan: 0 = library heuristic, else splits per
                          (sequence, KV head) in 1..256 (the MFMA verifier uses at
                          most 64).  Two calls over the same keys with the same
                          value give bitwise equal results.                        */
  int32_t rollback;    /* R >= 0 extra ring rows that keep speculative appends
                          undoable (masw_rollback): the ring holds C = W + r + R
                          rows.  0: no rollback.                                   */
  float rope_theta;    /* rotary base for slot keys ([TR] §3.2 Algorithm 1 step 6):
                          > 0: every projected K_g is rotated, before it is rounded
                          into the cache, to the position id of the raw token right
                          after its block, S + m*r (0-based ids: raw position i has
                          id i - 1); pair (a, b) of a head vector turns by
                          id * rope_theta^(-2j/D) for its frequency index j.
                          0: no rotation (raw K/V and queries are always the
                          caller's, already rotated).  V_g is never rotated.       */
  int32_t rope_style;  /* masw_rope_style of that rotation                          */
} masw_dims;

/* One layer's compact draft memory ([TR] §3.1 Eq. 4).  Layouts (C = W + r + rollback):
 *   k_sink, v_sink [B][Hkv][S][D]      sink cell i-1 holds position i (i <= S)
 *   k_ring, v_ring [B][Hkv][C][D]      ring cell (i-S-1) mod C holds position i > S
 *   k_slot, v_slot [B][Hkv][max_slots][D]  slot row m-1 holds g_m
 *   n_slots [B]                        slots materialized so far in THIS layer       */
typedef struct {
  void* k_sink;
  void* v_sink;
  void* k_ring;
  void* v_ring;
  void* k_slot;
  void* v_slot;
  int32_t* n_slots;
} masw_layer;

/* Per-sequence step state shared by all layers of a step. */
typedef struct {
  const int32_t* seq_len;  /* [B] t of each sequence (advanced by the caller once per
                              step, before that step's appends)                     */
  int32_t* err;            /* [1] sticky MASW_DEV_* bits                             */
} masw_seq;

/* Operation ids for masw_workspace_bytes. */
enum {
  MASW_OP_DRAFT_ATTN = 0,
  MASW_OP_MATERIALIZE = 1,
  MASW_OP_FULLKV_DECODE = 2,
  MASW_OP_FULLKV_VERIFY = 3
};

/* Raw append with implicit eviction ([TR] §3.2 Algorithm 1 step 5; Eq. 4 local bullet).
 * k_new, v_new [B][n_new][Hkv][D] hold positions t-n_new+1 .. t (t = seq_len[b]).
 * Position i <= S goes to sink cell i-1; i > S to ring cell (i-S-1) mod C
 * (C = W + r + rollback), which evicts the token i-C that occupied it.  That eviction is
 * legal only if the evicted token is a never-written cell or its block's slot already
 * exists (n_slots[b] >= ceil((i-C-S)/r)); otherwise the token is not written and
 * MASW_DEV_PENDING_SLOT is set.  Without a slot chain (r = 0) every eviction is legal.
 * t < n_new sets MASW_DEV_SEQ_RANGE and writes nothing.  n_new == 0 is a no-op. */
MASW_API int masw_evict_append(const masw_dims* dims, const masw_layer* layer,
                               const masw_seq* seq, const void* k_new, const void* v_new,
                               int32_t n_new, hipStream_t stream);

/* Slot materialization at a compression boundary ([TR] §3.2 Algorithm 1 steps 2-4).
 * For each sequence, the call acts only if t = seq_len[b] is the boundary of slot
 * m = (t-S-W)/r >= 1 and n_slots[b] == m-1; otherwise it leaves that sequence alone
 * (n_slots[b] == m: already done, silent; n_slots[b] < m-1: MASW_DEV_SLOT_MISSING;
 * m > max_slots: MASW_DEV_SLOT_CAPACITY).  For an acting sequence:
 *   1. mirrored projection (Algorithm 1 step 3): K_g = H W_K,g, V_g = H W_V,g with
 *      h [B][hidden], w_k_g, w_v_g [hidden][Hkv*D] (KV head k = columns k*D..k*D+D-1),
 *      K_g rotated to position id S + m*r when dims->rope_theta > 0 (Algorithm 1
 *      step 6), stored (rounded to the cache dtype) into slot row m-1;
 *   2. the slot query (Algorithm 1 step 2, structured mask): q_slot [B][Hq][D] attends
 *      over keylist(t - r) = sinks ++ the W-window whose oldest r tokens are the block
 *      g_m compresses ++ slots 1..m-1 (plus g_m itself if include_self != 0), and the
 *      result is written to o_slot [B][Hq][D];
 *   3. n_slots[b] = m (Algorithm 1 step 4).
 * q_slot is an input because only K/V projections are mirrored.  hidden >= 1. */
MASW_API int masw_materialize_slot(const masw_dims* dims, const masw_layer* layer,
                                   const masw_seq* seq, int32_t hidden, const void* h,
                                   const void* w_k_g, const void* w_v_g, const void* q_slot,
                                   void* o_slot, int32_t include_self, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* MASW draft decode attention ([TR] §2.3 Eq. 2 over §3.1 Eq. 4; §3.3 Algorithm 2 step 4).
 * q, out [B][Hq][D]: out[b][h] = softmax(scale * q K^T) V over keylist(seq_len[b]) of
 * KV head h / (Hq/Hkv).  Needs 1 <= t (else MASW_DEV_SEQ_RANGE), n(t) <= max_slots
 * (else MASW_DEV_SLOT_CAPACITY) and n_slots[b] >= n(t) (else MASW_DEV_SLOT_MISSING);
 * a sequence failing a check keeps its old output. */
MASW_API int masw_draft_attn(const masw_dims* dims, const masw_layer* layer,
                             const masw_seq* seq, const void* q, void* out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Fused decode step: masw_evict_append(k_new, v_new, n_new) followed by
 * masw_draft_attn, in one launch.  The n_new newest keys are read straight from
 * k_new/v_new while split 0 of each KV head writes them into the memory (same placement
 * and legality rule as masw_evict_append; an illegal eviction is reported and not
 * written, and the query still sees the new token).  n_new == 0 is masw_draft_attn.
 * t < n_new: MASW_DEV_SEQ_RANGE, nothing written. */
MASW_API int masw_decode_step(const masw_dims* dims, const masw_layer* layer, const masw_seq* seq,
                              const void* k_new, const void* v_new, int32_t n_new, const void* q,
                              void* out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* masw_decode_step without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The split partials and tickets live
 * in a fixed scratch array inside the library, one copy per GPU, held until the process
 * ends: MASW_STATIC_SCRATCH_BYTES in total, of which the tickets take the first
 * MASW_STATIC_MAX_UNITS int32 words (one per sequence and KV head: batch * n_kv_heads
 * must not exceed it) and the partials the rest (batch * n_q_heads * splits *
 * (head_dim + 2) * 4 bytes for the call's split plan, the same plan masw_decode_step
 * chooses).  A call whose plan does not fit returns MASW_ERR_WORKSPACE before anything
 * is enqueued.  The tickets start at zero and every call leaves them at zero.  All calls
 * on one GPU share that GPU's scratch: calls that overlap in time on one GPU (other
 * streams, other threads) race and give wrong results; serialize them.  The first call
 * on a device looks up the scratch address for that device (hipGetSymbolAddress) and
 * returns MASW_ERR_LAUNCH if that fails.  Otherwise exactly masw_decode_step. */
#define MASW_STATIC_SCRATCH_BYTES (8u << 20)
#define MASW_STATIC_MAX_UNITS 16384
MASW_API int masw_decode_step_static(const masw_dims* dims, const masw_layer* layer, const masw_seq* seq,
                                     const void* k_new, const void* v_new, int32_t n_new, const void* q,
                                     void* out, hipStream_t stream);

/* Rollback after verification ([TR] §3.3 Algorithm 2 step 6): the target accepted the
 * draft's candidates up to position t_acc = seq_len[b] (the caller has already set
 * seq_len back); t_spec[b] is the length the memory reached while drafting.  The call
 * drops every slot materialized strictly after t_acc (n_slots[b] = n(t_acc)); the raw
 * tokens past t_acc need no action, because with C = W + r + rollback ring rows a
 * speculative append evicts only tokens the memory at t_acc no longer needs - so the
 * layer is then exactly what appending only the accepted tokens would have built.
 * Requires 0 <= t_acc <= t_spec <= t_acc + rollback, else MASW_DEV_ROLLBACK_RANGE and
 * the sequence is left alone; n_slots[b] < n(t_acc) sets MASW_DEV_SLOT_MISSING.
 * t_spec [B] int32, device.  Call once per layer. */
MASW_API int masw_rollback(const masw_dims* dims, const masw_layer* layer, const masw_seq* seq,
                           const int32_t* t_spec, hipStream_t stream);

/* Draft prefill ([TR] §3.3 Algorithm 2 step 2): the draft processes a whole prefix of
 * P = seq_len[b] tokens per sequence in one call.  The structured prefill mask of the
 * review's Appendix C is not printed; this call computes what decoding the prefix one
 * token at a time would (materializing each slot at its boundary):
 *   1. (r > 0 and ns_max > 0) every slot g_1 .. g_n, n = n(P), is projected as in
 *      masw_materialize_slot step 1 from h_slot [B][ns_max][hidden] (row m-1 holds the
 *      hidden state of g_m) into slot rows 0 .. n-1, and n_slots[b] = n;
 *   2. the raw tokens the memory keeps after position P (sinks 1..min(S,P) and the
 *      newest C ring positions) are copied from k, v [B][p_max][Hkv][D] (row i-1 holds
 *      position i) into the layer, as masw_evict_append of positions 1..P would leave
 *      them;
 *   3. out[b][i-1] [B][p_max][Hq][D] = attention of q[b][i-1] over keylist(i) for every
 *      i = 1..P (Eq. 2 over Eq. 4), and o_slot[b][m-1] [B][ns_max][Hq][D] = attention of
 *      the slot query q_slot[b][m-1] over keylist(t_m - r) for m = 1..n (Algorithm 1
 *      step 2, include_self = 0).  Rows past P (past n) are untouched.
 * Keys are read from k, v and the projected slots, so the result does not depend on the
 * layer's earlier contents; the layer must start empty for r > 0 when no slots are
 * projected (n_slots[b] = 0).  bf16 with D = 128 only (else MASW_ERR_UNIMPLEMENTED);
 * hidden % 8 == 0.  Device errors: P < 0 or P > p_max: MASW_DEV_SEQ_RANGE;
 * n(P) > max_slots or > ns_max: MASW_DEV_SLOT_CAPACITY; that sequence's outputs and
 * memory are left alone.  P = 0 is a no-op for that sequence.  With r = 0 or
 * ns_max = 0, h_slot, w_k_g, w_v_g, q_slot and o_slot may be NULL.  No workspace. */
MASW_API int masw_prefill(const masw_dims* dims, const masw_layer* layer, const masw_seq* seq,
                          int32_t p_max, const void* k, const void* v, const void* q, void* out,
                          int32_t ns_max, int32_t hidden, const void* h_slot, const void* w_k_g,
                          const void* w_v_g, const void* q_slot, void* o_slot, hipStream_t stream);

/* Full-KV draft decode attention, the baseline ([TR] §2.3 Eq. 2 over K_{<=t}).
 * k, v [B][Hkv][max_len][D] (row i-1 holds position i); q, out [B][Hq][D]; keys 1..t.
 * Runs the same kernel as masw_draft_attn with a one-segment memory, so for
 * t <= S + W and equal num_splits both give bitwise equal outputs.
 * t < 1 or t > max_len: MASW_DEV_SEQ_RANGE, output untouched. */
MASW_API int fullkv_decode_attn(const masw_dims* dims, const void* k, const void* v,
                                int32_t max_len, const int32_t* seq_len, int32_t* err,
                                const void* q, void* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* Full-KV append: writes positions t-n_new+1..t to rows t-n_new..t-1 of
 * k, v [B][Hkv][max_len][D] from k_new, v_new [B][n_new][Hkv][D].  t < n_new or
 * t > max_len: MASW_DEV_SEQ_RANGE, nothing written. */
MASW_API int fullkv_append(const masw_dims* dims, void* k, void* v, int32_t max_len,
                           const int32_t* seq_len, int32_t* err, const void* k_new,
                           const void* v_new, int32_t n_new, hipStream_t stream);

/* Fused full-KV decode step: fullkv_append then fullkv_decode_attn in one launch
 * (the new rows are read from k_new/v_new and written by split 0). */
MASW_API int fullkv_decode_step(const masw_dims* dims, void* k, void* v, int32_t max_len,
                                const int32_t* seq_len, int32_t* err, const void* k_new,
                                const void* v_new, int32_t n_new, const void* q, void* out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Verifier attention over the full cache ([TR] §3.3 Algorithm 2 step 5): n_q candidate
 * positions checked in one parallel pass.  q, out [B][n_q][Hq][D]; query j sits at
 * position t-n_q+1+j (t = seq_len[b], the candidates already appended) and attends to
 * keys 1 .. t-n_q+1+j (causal among the candidates).  1 <= n_q <= 16.  bf16 with D = 128
 * and (Hq/Hkv)*n_q <= 64 runs on the matrix cores; other shapes run one vector-ALU
 * decode pass per candidate.
 * t < n_q or t > max_len: MASW_DEV_SEQ_RANGE, output untouched. */
MASW_API int fullkv_verify_attn(const masw_dims* dims, const void* k, const void* v,
                                int32_t max_len, const int32_t* seq_len, int32_t* err,
                                int32_t n_q, const void* q, void* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes an op needs.  max_keys: for the full-KV ops, max_len; ignored by the
 * MASW ops (their bound is S + W + max_slots + 1).  n_q: verifier candidates (others
 * ignore it).  Returns 0 for invalid dims. */
MASW_API size_t masw_workspace_bytes(const masw_dims* dims, int32_t op, int32_t max_keys,
                                     int32_t n_q);

/* Human-readable text of a MASW_OK / MASW_ERR_* code (static storage). */
MASW_API const char* masw_status_string(int status);

/* MASW_ABI_VERSION of the built library. */
MASW_API int masw_abi_version(void);

/* Test hook: the device key resolver used by every attention kernel, dumped.  For
 * each sequence b and logical key j of keylist(seq_len[b] - back) it writes
 * out[b][j] = {segment (0 sink, 1 ring, 2 slot), row, id (position or slot index)};
 * unused entries up to max_keys are {-1,-1,-1}.  out [B][max_keys][3] int32. */
MASW_API int masw_debug_keylist(const masw_dims* dims, const masw_seq* seq, int32_t back,
                                int32_t* out, int32_t max_keys, hipStream_t stream);

/* Measurement helper, not part of the method: a plain streaming read of
 * p[0..bytes) that adds every 32-bit word modulo 2^32 into the MASW_STREAM_SUMS
 * counters sums[] (device, caller-zeroed; calls accumulate): the wrapping total of
 * sums[] is the wrapping sum of the words.  Reports the HBM read rate a simple kernel
 * reaches on this device, the measured reference for the attention kernels' GB/s.
 * bytes must be a positive multiple of 16 and p 16-byte aligned (else MASW_ERR_ARG);
 * work_groups <= 0 picks 2048 contiguous chunks. */
#define MASW_STREAM_SUMS 256
MASW_API int masw_stream_read(const void* p, size_t bytes, int32_t work_groups, uint32_t* sums,
                              hipStream_t stream);

/* Measurement helper, not part of the method: work_groups work-groups of 256 threads,
 * each wave running iters rounds of four independent v_mfma_f32_32x32x16_bf16 on
 * register operands (2*32*32*16 FLOP each, so 4 waves x iters x 4 x 32768 FLOP per
 * work-group).  Every thread writes one float to out [work_groups * 256] (device; all
 * work-groups write the same values); clocks [2] (device) receives the shader-clock and
 * the 100 MHz real-time ticks the first wave of work-group 0 spent in its loop.  Reports
 * the matrix-core rate and shader clock this device sustains, the measured reference
 * for the matrix-core kernels' TFLOP/s.  work_groups >= 1 and iters >= 1, else
 * MASW_ERR_ARG. */
MASW_API int masw_mfma_rate(int32_t work_groups, int32_t iters, float* out, uint64_t* clocks,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MASW_H_ */
