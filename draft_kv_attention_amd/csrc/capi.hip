// capi.hip - the extern "C" entry points declared in include/masw.h: host-side
// validation, the split-K plan, workspace carving and kernel dispatch.  Nothing here
// touches device memory or synchronizes; every call only enqueues on `stream`.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "masw_internal.hpp"

using namespace masw;

// Scratch of masw_decode_step_static: [tickets: MASW_STATIC_MAX_UNITS int32][partials].
// Each GPU the library runs on holds its own copy (zero at load) until the process ends.
static __device__ __align__(256) unsigned char scratch[MASW_STATIC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxSplits = 256;   // split partials merged by one work-group
constexpr long kCUs = 256;
constexpr long kMinKeysPerSplit = 128;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool group_supported(int g) { return g == 1 || g == 2 || g == 3 || g == 4 || g == 6 || g == 8; }

int check_dims(const masw_dims* d, bool masw_memory) {
  if (!d) return MASW_ERR_ARG;
  if (d->dtype != MASW_F32 && d->dtype != MASW_BF16) return MASW_ERR_DTYPE;
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1) return MASW_ERR_SHAPE;
  if (d->batch > kMaxGridDim || d->n_kv_heads > kMaxGridDim) return MASW_ERR_SHAPE;
  if (d->n_q_heads % d->n_kv_heads) return MASW_ERR_SHAPE;
  if (!group_supported(d->n_q_heads / d->n_kv_heads)) return MASW_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return MASW_ERR_SHAPE;
  if (d->num_splits < 0 || d->num_splits > kMaxSplits) return MASW_ERR_ARG;
  if (masw_memory) {
    if (d->sink < 0 || d->window < 1 || d->interval < 0 || d->interval > d->window || d->max_slots < 0 ||
        d->rollback < 0 || d->rollback > kMaxRollback || d->sink > kMaxMemRows || d->window > kMaxMemRows ||
        d->max_slots > kMaxMemRows)
      return MASW_ERR_ARG;
    if (!(d->rope_theta >= 0.f) || std::isinf(d->rope_theta) ||
        (d->rope_style != MASW_ROPE_ROTATE_HALF && d->rope_style != MASW_ROPE_INTERLEAVED))
      return MASW_ERR_ARG;
  }
  return MASW_OK;
}

// Splits per (sequence, KV head): enough work-groups to fill every CU once with as many
// as stay resident together (`per_cu`), but at least ~128 keys each.  The kernels
// re-derive the chunk from the actual key count.
int choose_splits(const masw_dims* d, long max_keys, int per_cu = kDecodeResidentPerCU) {
  if (d->num_splits > 0) return d->num_splits;
  const long units = long(d->batch) * d->n_kv_heads;
  const long target = kCUs * per_cu;
  long s = (target + units - 1) / units;
  s = std::min(s, std::max(1L, (max_keys + kMinKeysPerSplit - 1) / kMinKeysPerSplit));
  return int(std::max(1L, std::min(s, long(kMaxSplits))));
}

long masw_max_keys(const masw_dims* d) { return long(d->sink) + d->window + d->max_slots + 1; }

struct WsPlan {
  size_t flags, counters, part_o, part_ml, proj_counters, proj_part, launch_done, total;
};

// [per-sequence flags][per-(sequence, KV head) split tickets][partial o][partial max/sum]
// and, for materialization, [projection tickets][projection partial sums][launch ticket].
WsPlan plan_workspace(const masw_dims* d, int splits, int rows_per_seq, bool projection = false) {
  WsPlan p;
  const size_t rows = size_t(d->batch) * rows_per_seq;
  p.flags = 0;
  p.counters = align_up(size_t(d->batch) * sizeof(int32_t));
  p.part_o = p.counters + align_up(size_t(d->batch) * d->n_kv_heads * sizeof(int32_t));
  const size_t po = splits > 1 ? rows * splits * d->head_dim * sizeof(float) : 0;
  p.part_ml = p.part_o + align_up(po);
  const size_t pml = splits > 1 ? rows * splits * 2 * sizeof(float) : 0;
  p.proj_counters = p.part_ml + align_up(pml);
  const size_t groups = (size_t(d->batch) + 15) / 16, N = size_t(d->n_kv_heads) * d->head_dim;
  const size_t pc = projection ? groups * 2 * (N / 64) * sizeof(int32_t) : 0;
  p.proj_part = p.proj_counters + align_up(pc);
  const size_t pp = projection ? groups * 2 * kMaxProjectSplits * 16 * N * sizeof(float) : 0;
  p.launch_done = p.proj_part + align_up(pp);
  p.total = p.launch_done + (projection ? kAlign : 0);
  return p;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need) return MASW_ERR_WORKSPACE;
  if (need && (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign))) return MASW_ERR_WORKSPACE;
  return MASW_OK;
}

float scale_log2(const masw_dims* d) {
  const float s = d->scale > 0.f ? d->scale : 1.0f / std::sqrt(float(d->head_dim));
  return s * 1.4426950408889634f;
}

MemGeom masw_geom(const masw_dims* d) {
  return MemGeom{d->sink, d->window, d->interval, d->window + d->interval + d->rollback, d->max_slots};
}

// A full cache is a memory in which every one of its max_len tokens is a sink.
MemGeom full_geom(int max_len) { return MemGeom{max_len, 1, 1, 2, 0}; }

void fill_common(DecodeArgs& a, const masw_dims* d, int splits, void* ws, const WsPlan& p) {
  a.B = d->batch;
  a.Hq = d->n_q_heads;
  a.Hkv = d->n_kv_heads;
  a.n_splits = splits;
  a.scale_log2 = scale_log2(d);
  a.qo_stride = long(d->n_q_heads) * d->head_dim;
  char* base = static_cast<char*>(ws);
  a.counters = splits > 1 ? reinterpret_cast<int32_t*>(base + p.counters) : nullptr;
  a.part_o = splits > 1 ? reinterpret_cast<float*>(base + p.part_o) : nullptr;
  a.part_ml = splits > 1 ? reinterpret_cast<float*>(base + p.part_ml) : nullptr;
}

const void* or_else(const void* p, const void* q) { return p ? p : q; }

// The three-segment memory of one layer as the decode kernel reads it.
void fill_masw_memory(DecodeArgs& a, const masw_dims* d, const masw_layer* L) {
  a.k[0] = or_else(L->k_sink, L->k_ring); a.k[1] = L->k_ring; a.k[2] = or_else(L->k_slot, L->k_ring);
  a.v[0] = or_else(L->v_sink, L->v_ring); a.v[1] = L->v_ring; a.v[2] = or_else(L->v_slot, L->v_ring);
  a.wk[0] = L->k_sink ? L->k_sink : L->k_ring; a.wk[1] = L->k_ring;
  a.wv[0] = L->v_sink ? L->v_sink : L->v_ring; a.wv[1] = L->v_ring;
  a.cap[0] = d->sink; a.cap[1] = d->window + d->interval + d->rollback; a.cap[2] = d->max_slots;
  a.g = masw_geom(d);
}

// A full cache [B][Hkv][max_len][D] as a one-segment memory.
void fill_full_memory(DecodeArgs& a, const void* k, const void* v, int32_t max_len) {
  for (int s = 0; s < 3; ++s) { a.k[s] = k; a.v[s] = v; }
  a.wk[0] = a.wk[1] = const_cast<void*>(k);
  a.wv[0] = a.wv[1] = const_cast<void*>(v);
  a.cap[0] = max_len; a.cap[1] = 0; a.cap[2] = 0;
  a.g = full_geom(max_len);
  a.max_len = max_len;
}

// Tensor pointers must be 16-byte aligned: the kernels move 16-byte pieces of rows.  A
// null pointer passes (its presence is checked where it is required).
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
template <typename... P>
bool all_aligned16(const P*... p) {
  return (aligned16(p) && ...);
}

int check_layer(const masw_dims* d, const masw_layer* L) {
  if (!L || !L->k_ring || !L->v_ring || !L->n_slots) return MASW_ERR_ARG;
  if (d->sink > 0 && (!L->k_sink || !L->v_sink)) return MASW_ERR_ARG;
  if (d->max_slots > 0 && (!L->k_slot || !L->v_slot)) return MASW_ERR_ARG;
  if (!all_aligned16(L->k_ring, L->v_ring, L->k_sink, L->v_sink, L->k_slot, L->v_slot)) return MASW_ERR_ARG;
  return MASW_OK;
}

}  // namespace

extern "C" {

MASW_API int masw_abi_version(void) { return MASW_ABI_VERSION; }

MASW_API const char* masw_status_string(int status) {
  switch (status) {
    case MASW_OK: return "ok";
    case MASW_ERR_ARG: return "invalid argument";
    case MASW_ERR_DTYPE: return "unsupported dtype";
    case MASW_ERR_SHAPE: return "unsupported shape";
    case MASW_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case MASW_ERR_LAUNCH: return "kernel launch failed";
    case MASW_ERR_UNIMPLEMENTED: return "not supported by this library";
    default: return "unknown status";
  }
}

MASW_API size_t masw_workspace_bytes(const masw_dims* d, int32_t op, int32_t max_keys, int32_t n_q) {
  const bool masw_op = op == MASW_OP_DRAFT_ATTN || op == MASW_OP_MATERIALIZE;
  if (check_dims(d, masw_op) != MASW_OK) return 0;
  if (masw_op) {
    const int splits = choose_splits(d, masw_max_keys(d));
    return plan_workspace(d, splits, d->n_q_heads, op == MASW_OP_MATERIALIZE).total;
  }
  if (max_keys < 1) return 0;
  if (op == MASW_OP_FULLKV_DECODE) return plan_workspace(d, choose_splits(d, max_keys), d->n_q_heads).total;
  if (op == MASW_OP_FULLKV_VERIFY) {
    if (n_q < 1) return 0;
    const int rows = d->n_q_heads / d->n_kv_heads * n_q;
    const bool mfma = d->dtype == MASW_BF16 && d->head_dim == 128 && rows <= 64;
    const int per_cu = mfma ? verify_resident_per_cu(rows) : kDecodeResidentPerCU;
    return plan_workspace(d, choose_splits(d, max_keys, per_cu), d->n_q_heads * n_q).total;
  }
  return 0;
}

MASW_API int masw_evict_append(const masw_dims* d, const masw_layer* L, const masw_seq* seq,
                               const void* k_new, const void* v_new, int32_t n_new,
                               hipStream_t stream) {
  int st = check_dims(d, true);
  if (st) return st;
  if ((st = check_layer(d, L))) return st;
  if (!seq || !seq->seq_len || !seq->err || n_new < 0) return MASW_ERR_ARG;
  if (n_new == 0) return MASW_OK;
  if (!k_new || !v_new || !all_aligned16(k_new, v_new)) return MASW_ERR_ARG;
  AppendArgs a{};
  a.k_sink = L->k_sink ? L->k_sink : L->k_ring;
  a.v_sink = L->v_sink ? L->v_sink : L->v_ring;
  a.k_ring = L->k_ring;
  a.v_ring = L->v_ring;
  a.sink_cap = d->sink;
  a.g = masw_geom(d);
  a.seq_len = seq->seq_len;
  a.err = seq->err;
  a.n_slots = L->n_slots;
  a.max_len = 0;
  a.k_new = k_new;
  a.v_new = v_new;
  a.B = d->batch;
  a.Hkv = d->n_kv_heads;
  a.D = d->head_dim;
  a.n_new = n_new;
  return launch_append(a, d->dtype, stream);
}

MASW_API int fullkv_append(const masw_dims* d, void* k, void* v, int32_t max_len, const int32_t* seq_len,
                           int32_t* err, const void* k_new, const void* v_new, int32_t n_new,
                           hipStream_t stream) {
  int st = check_dims(d, false);
  if (st) return st;
  if (!k || !v || !seq_len || !err || max_len < 1 || n_new < 0) return MASW_ERR_ARG;
  if (n_new == 0) return MASW_OK;
  if (!k_new || !v_new || !all_aligned16(k, v, k_new, v_new)) return MASW_ERR_ARG;
  AppendArgs a{};
  a.k_sink = k;
  a.v_sink = v;
  a.k_ring = k;
  a.v_ring = v;
  a.sink_cap = max_len;
  a.g = full_geom(max_len);
  a.seq_len = seq_len;
  a.err = err;
  a.n_slots = nullptr;
  a.max_len = max_len;
  a.k_new = k_new;
  a.v_new = v_new;
  a.B = d->batch;
  a.Hkv = d->n_kv_heads;
  a.D = d->head_dim;
  a.n_new = n_new;
  return launch_append(a, d->dtype, stream);
}

MASW_API int masw_draft_attn(const masw_dims* d, const masw_layer* L, const masw_seq* seq, const void* q,
                             void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return masw_decode_step(d, L, seq, nullptr, nullptr, 0, q, out, ws, ws_bytes, stream);
}

MASW_API int masw_decode_step(const masw_dims* d, const masw_layer* L, const masw_seq* seq,
                              const void* k_new, const void* v_new, int32_t n_new, const void* q,
                              void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(d, true);
  if (st) return st;
  if ((st = check_layer(d, L))) return st;
  if (!seq || !seq->seq_len || !seq->err || !q || !out || n_new < 0) return MASW_ERR_ARG;
  if (n_new > 0 && (!k_new || !v_new)) return MASW_ERR_ARG;
  if (!all_aligned16(q, out, k_new, v_new)) return MASW_ERR_ARG;
  const int splits = choose_splits(d, masw_max_keys(d));
  const WsPlan p = plan_workspace(d, splits, d->n_q_heads);
  if (splits > 1 && (st = check_ws(ws, ws_bytes, p.total))) return st;
  DecodeArgs a{};
  fill_masw_memory(a, d, L);
  a.seq_len = seq->seq_len;
  a.err = seq->err;
  a.n_slots = L->n_slots;
  a.k_new = k_new;
  a.v_new = v_new;
  a.n_new = n_new;
  a.q = q;
  a.out = out;
  fill_common(a, d, splits, ws, p);
  return launch_decode(a, d->dtype, d->head_dim, stream);
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` per device, once looked up

// Device address of this device's scratch copy (the array's name is a host-side stand-in
// and must never reach a kernel), looked up on the first call on each device.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

MASW_API int masw_decode_step_static(const masw_dims* d, const masw_layer* L, const masw_seq* seq,
                                     const void* k_new, const void* v_new, int32_t n_new, const void* q,
                                     void* out, hipStream_t stream) {
  int st = check_dims(d, true);
  if (st) return st;
  if ((st = check_layer(d, L))) return st;
  if (!seq || !seq->seq_len || !seq->err || !q || !out || n_new < 0) return MASW_ERR_ARG;
  if (n_new > 0 && (!k_new || !v_new)) return MASW_ERR_ARG;
  if (!all_aligned16(q, out, k_new, v_new)) return MASW_ERR_ARG;
  const int splits = choose_splits(d, masw_max_keys(d));
  const size_t units = size_t(d->batch) * d->n_kv_heads;
  const size_t rows = size_t(d->batch) * d->n_q_heads;
  const size_t ticket_bytes = align_up(size_t(MASW_STATIC_MAX_UNITS) * sizeof(int32_t));
  const size_t po = align_up(rows * splits * d->head_dim * sizeof(float));
  const size_t pml = align_up(rows * splits * 2 * sizeof(float));
  if (splits > 1 && (units > MASW_STATIC_MAX_UNITS || ticket_bytes + po + pml > MASW_STATIC_SCRATCH_BYTES))
    return MASW_ERR_WORKSPACE;
  char* base = static_cast<char*>(scratch_on_current_device());
  if (!base) return MASW_ERR_LAUNCH;
  DecodeArgs a{};
  fill_masw_memory(a, d, L);
  a.seq_len = seq->seq_len;
  a.err = seq->err;
  a.n_slots = L->n_slots;
  a.k_new = k_new;
  a.v_new = v_new;
  a.n_new = n_new;
  a.q = q;
  a.out = out;
  a.B = d->batch;
  a.Hq = d->n_q_heads;
  a.Hkv = d->n_kv_heads;
  a.n_splits = splits;
  a.scale_log2 = scale_log2(d);
  a.qo_stride = long(d->n_q_heads) * d->head_dim;
  a.counters = splits > 1 ? reinterpret_cast<int32_t*>(base) : nullptr;
  a.part_o = splits > 1 ? reinterpret_cast<float*>(base + ticket_bytes) : nullptr;
  a.part_ml = splits > 1 ? reinterpret_cast<float*>(base + ticket_bytes + po) : nullptr;
  return launch_decode(a, d->dtype, d->head_dim, stream);
}

MASW_API int fullkv_decode_attn(const masw_dims* d, const void* k, const void* v, int32_t max_len,
                                const int32_t* seq_len, int32_t* err, const void* q, void* out, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  return fullkv_decode_step(d, const_cast<void*>(k), const_cast<void*>(v), max_len, seq_len, err, nullptr,
                            nullptr, 0, q, out, ws, ws_bytes, stream);
}

MASW_API int fullkv_decode_step(const masw_dims* d, void* k, void* v, int32_t max_len, const int32_t* seq_len,
                                int32_t* err, const void* k_new, const void* v_new, int32_t n_new,
                                const void* q, void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(d, false);
  if (st) return st;
  if (!k || !v || !seq_len || !err || !q || !out || max_len < 1 || n_new < 0) return MASW_ERR_ARG;
  if (n_new > 0 && (!k_new || !v_new)) return MASW_ERR_ARG;
  if (!all_aligned16(k, v, q, out, k_new, v_new)) return MASW_ERR_ARG;
  const int splits = choose_splits(d, max_len);
  const WsPlan p = plan_workspace(d, splits, d->n_q_heads);
  if (splits > 1 && (st = check_ws(ws, ws_bytes, p.total))) return st;
  DecodeArgs a{};
  fill_full_memory(a, k, v, max_len);
  a.seq_len = seq_len;
  a.err = err;
  a.k_new = k_new;
  a.v_new = v_new;
  a.n_new = n_new;
  a.q = q;
  a.out = out;
  fill_common(a, d, splits, ws, p);
  return launch_decode(a, d->dtype, d->head_dim, stream);
}

MASW_API int masw_materialize_slot(const masw_dims* d, const masw_layer* L, const masw_seq* seq,
                                   int32_t hidden, const void* h, const void* w_k_g, const void* w_v_g,
                                   const void* q_slot, void* o_slot, int32_t include_self, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(d, true);
  if (st) return st;
  if ((st = check_layer(d, L))) return st;
  if (!seq || !seq->seq_len || !seq->err || !h || !w_k_g || !w_v_g || !q_slot || !o_slot || hidden < 1)
    return MASW_ERR_ARG;
  if (!all_aligned16(h, w_k_g, w_v_g, q_slot, o_slot)) return MASW_ERR_ARG;
  if (d->interval == 0) return MASW_ERR_ARG;   // no slot chain to materialize
  if (d->dtype == MASW_BF16 && hidden % 8) return MASW_ERR_SHAPE;
  const int splits = choose_splits(d, masw_max_keys(d));
  const WsPlan p = plan_workspace(d, splits, d->n_q_heads, true);
  if ((st = check_ws(ws, ws_bytes, p.total))) return st;
  char* base = static_cast<char*>(ws);
  int32_t* active = reinterpret_cast<int32_t*>(base + p.flags);

  ProjectArgs pa{};
  pa.h = h;
  pa.w_k = w_k_g;
  pa.w_v = w_v_g;
  pa.k_slot = L->k_slot;
  pa.v_slot = L->v_slot;
  pa.seq_len = seq->seq_len;
  pa.n_slots = L->n_slots;
  pa.err = seq->err;
  pa.active = active;
  pa.g = masw_geom(d);
  pa.B = d->batch;
  pa.Hkv = d->n_kv_heads;
  pa.D = d->head_dim;
  pa.hidden = hidden;
  pa.k_per_split = project_k_per_split(hidden);
  pa.ksplits = project_splits(hidden);
  pa.rope_theta = d->rope_theta;
  pa.rope_style = d->rope_style;
  pa.counters = reinterpret_cast<int32_t*>(base + p.proj_counters);
  pa.part = reinterpret_cast<float*>(base + p.proj_part);

  DecodeArgs a{};
  fill_masw_memory(a, d, L);
  a.seq_len = seq->seq_len;
  a.err = seq->err;
  a.n_slots_out = L->n_slots;
  a.back = d->interval;
  a.self_slot = include_self ? 1 : 0;
  a.q = q_slot;
  a.out = o_slot;
  fill_common(a, d, splits, ws, p);
  if (d->dtype == MASW_BF16 && !include_self) {
    // The slot query does not read the new slot: projection and query share one launch.
    BoundaryArgs ba{};
    ba.p = pa;
    a.n_slots = L->n_slots;
    a.gate_boundary = 1;
    a.n_slots_out = nullptr;   // published once every work-group has read n_slots
    ba.d = a;
    ba.publish = L->n_slots;
    ba.proj_x = d->n_kv_heads * d->head_dim / 64;
    ba.n_proj = ba.proj_x * 2 * pa.ksplits * ((d->batch + 15) / 16);
    const long n_wg = long(ba.n_proj) + long(splits) * d->n_kv_heads * d->batch;
    if (n_wg > 0x7fffffffL) return MASW_ERR_SHAPE;
    ba.n_wg = int(n_wg);
    ba.done = reinterpret_cast<int32_t*>(base + p.launch_done);
    return launch_boundary(ba, d->head_dim, stream);
  }
  // With include_self the query needs the projected slot: two launches, the query gated
  // by the projection's per-sequence decision.
  if ((st = launch_project(pa, d->dtype, stream))) return st;
  a.active = active;
  return launch_decode(a, d->dtype, d->head_dim, stream);
}

MASW_API int masw_rollback(const masw_dims* d, const masw_layer* L, const masw_seq* seq, const int32_t* t_spec,
                           hipStream_t stream) {
  int st = check_dims(d, true);
  if (st) return st;
  if ((st = check_layer(d, L))) return st;
  if (!seq || !seq->seq_len || !seq->err || !t_spec) return MASW_ERR_ARG;
  return launch_rollback(masw_geom(d), d->rollback, seq->seq_len, t_spec, L->n_slots, seq->err, d->batch, stream);
}

MASW_API int masw_prefill(const masw_dims* d, const masw_layer* L, const masw_seq* seq, int32_t p_max,
                          const void* k, const void* v, const void* q, void* out, int32_t ns_max, int32_t hidden,
                          const void* h_slot, const void* w_k_g, const void* w_v_g, const void* q_slot,
                          void* o_slot, hipStream_t stream) {
  int st = check_dims(d, true);
  if (st) return st;
  if ((st = check_layer(d, L))) return st;
  if (!seq || !seq->seq_len || !seq->err || !k || !v || !q || !out || p_max < 1 || ns_max < 0) return MASW_ERR_ARG;
  if (d->dtype != MASW_BF16 || d->head_dim != 128) return MASW_ERR_UNIMPLEMENTED;
  const bool slots = d->interval > 0 && ns_max > 0;
  if (slots && (!h_slot || !w_k_g || !w_v_g || !q_slot || !o_slot || hidden < 1)) return MASW_ERR_ARG;
  if (!all_aligned16(k, v, q, out) || (slots && !all_aligned16(h_slot, w_k_g, w_v_g, q_slot, o_slot)))
    return MASW_ERR_ARG;
  if (slots && hidden % 8) return MASW_ERR_SHAPE;
  const int G = d->n_q_heads / d->n_kv_heads;
  const int qb = prefill_rows_per_block() / G;
  const long raw_blocks = (long(p_max) + qb - 1) / qb, slot_blocks = slots ? (long(ns_max) + qb - 1) / qb : 0;
  const long groups = slots ? (long(d->batch) * ns_max + 15) / 16 : 0;
  if ((raw_blocks + slot_blocks) * d->n_kv_heads * d->batch > 0x7fffffffL || groups > 65535) return MASW_ERR_SHAPE;

  // 1. every slot of the prefix (Algorithm 1 step 3, all boundaries at once); n_slots = n(P)
  if (slots) {
    ProjectArgs pa{};
    pa.h = h_slot;
    pa.w_k = w_k_g;
    pa.w_v = w_v_g;
    pa.k_slot = L->k_slot;
    pa.v_slot = L->v_slot;
    pa.seq_len = seq->seq_len;
    pa.n_slots = L->n_slots;
    pa.err = seq->err;
    pa.g = masw_geom(d);
    pa.B = d->batch;
    pa.Hkv = d->n_kv_heads;
    pa.D = d->head_dim;
    pa.hidden = hidden;
    pa.ksplits = 1;
    pa.k_per_split = (hidden + 127) / 128 * 128;
    pa.prefill_ns = ns_max;
    pa.rope_theta = d->rope_theta;
    pa.rope_style = d->rope_style;
    if ((st = launch_project(pa, d->dtype, stream))) return st;
  }
  // 2. the raw tokens the memory keeps after the prefix (sinks and the newest C)
  AppendArgs aa{};
  aa.k_sink = L->k_sink ? L->k_sink : L->k_ring;
  aa.v_sink = L->v_sink ? L->v_sink : L->v_ring;
  aa.k_ring = L->k_ring;
  aa.v_ring = L->v_ring;
  aa.sink_cap = d->sink;
  aa.g = masw_geom(d);
  aa.seq_len = seq->seq_len;
  aa.err = seq->err;
  aa.n_slots = L->n_slots;
  aa.k_new = k;
  aa.v_new = v;
  aa.B = d->batch;
  aa.Hkv = d->n_kv_heads;
  aa.D = d->head_dim;
  aa.prefill_len = p_max;
  if ((st = launch_append(aa, d->dtype, stream))) return st;
  // 3. every raw query and slot query under the memory of its own step
  PrefillArgs a{};
  a.k = k;
  a.v = v;
  a.k_slot = or_else(L->k_slot, L->k_ring);
  a.v_slot = or_else(L->v_slot, L->v_ring);
  a.n_slots = L->n_slots;
  a.g = masw_geom(d);
  a.seq_len = seq->seq_len;
  a.err = seq->err;
  a.q = q;
  a.q_slot = q_slot;
  a.out = out;
  a.o_slot = o_slot;
  a.B = d->batch;
  a.Hq = d->n_q_heads;
  a.Hkv = d->n_kv_heads;
  a.p_max = p_max;
  a.ns_max = slots ? ns_max : 0;
  a.qb = qb;
  a.raw_blocks = int(raw_blocks);
  a.slot_blocks = int(slot_blocks);
  a.scale_log2 = scale_log2(d);
  return launch_prefill(a, stream);
}

MASW_API int fullkv_verify_attn(const masw_dims* d, const void* k, const void* v, int32_t max_len,
                                const int32_t* seq_len, int32_t* err, int32_t n_q, const void* q, void* out,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(d, false);
  if (st) return st;
  if (!k || !v || !seq_len || !err || !q || !out || max_len < 1 || n_q < 1 || n_q > 16) return MASW_ERR_ARG;
  if (!all_aligned16(k, v, q, out)) return MASW_ERR_ARG;
  const int rows = d->n_q_heads / d->n_kv_heads * n_q;
  const bool mfma = d->dtype == MASW_BF16 && d->head_dim == 128 && rows <= 64;
  int splits = choose_splits(d, max_len, mfma ? verify_resident_per_cu(rows) : kDecodeResidentPerCU);
  if (mfma) splits = std::min(splits, kMaxVerifySplits);   // its merge keeps [rows][splits] weights in LDS
  const WsPlan p = plan_workspace(d, splits, d->n_q_heads * n_q);
  if (splits > 1 && (st = check_ws(ws, ws_bytes, p.total))) return st;
  char* base = static_cast<char*>(ws);
  if (mfma) {
    VerifyArgs a{};
    a.k = k;
    a.v = v;
    a.max_len = max_len;
    a.seq_len = seq_len;
    a.err = err;
    a.q = q;
    a.out = out;
    a.counters = splits > 1 ? reinterpret_cast<int32_t*>(base + p.counters) : nullptr;
    a.part_o = splits > 1 ? reinterpret_cast<float*>(base + p.part_o) : nullptr;
    a.part_ml = splits > 1 ? reinterpret_cast<float*>(base + p.part_ml) : nullptr;
    a.B = d->batch;
    a.Hq = d->n_q_heads;
    a.Hkv = d->n_kv_heads;
    a.n_q = n_q;
    a.n_splits = splits;
    a.scale_log2 = scale_log2(d);
    return launch_verify_mfma(a, stream);
  }
  // Other shapes: one vector-ALU decode pass per candidate, query j over keys 1..t-n_q+1+j.
  const size_t esz = d->dtype == MASW_BF16 ? 2 : 4;
  const size_t step = size_t(d->n_q_heads) * d->head_dim * esz;
  for (int j = 0; j < n_q; ++j) {
    DecodeArgs a{};
    fill_full_memory(a, k, v, max_len);
    a.seq_len = seq_len;
    a.err = err;
    a.back = n_q - 1 - j;
    a.min_t = n_q;
    fill_common(a, d, splits, ws, p);
    a.q = static_cast<const char*>(q) + j * step;
    a.out = static_cast<char*>(out) + j * step;
    a.qo_stride = long(n_q) * d->n_q_heads * d->head_dim;
    if ((st = launch_decode(a, d->dtype, d->head_dim, stream))) return st;
  }
  return MASW_OK;
}

MASW_API int masw_mfma_rate(int32_t work_groups, int32_t iters, float* out, uint64_t* clocks, hipStream_t stream) {
  if (work_groups < 1 || iters < 1 || !out || !clocks) return MASW_ERR_ARG;
  return launch_mfma_rate(work_groups, iters, out, clocks, stream);
}

MASW_API int masw_debug_keylist(const masw_dims* d, const masw_seq* seq, int32_t back, int32_t* out,
                                int32_t max_keys, hipStream_t stream) {
  int st = check_dims(d, true);
  if (st) return st;
  if (!seq || !seq->seq_len || !out || max_keys < 1 || back < 0) return MASW_ERR_ARG;
  return launch_debug_keylist(masw_geom(d), seq->seq_len, d->batch, back, out, max_keys, stream);
}

}  // extern "C"
