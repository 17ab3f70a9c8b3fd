// C ABI entry points: argument marshalling, the plan upload through a pinned staging ring,
// kernel launches and kernel timing. The planner is in plan.cpp, the captured steps in
// graph.cpp, the kernels in the .hip files. Host code only.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "host.h"

namespace cb {

std::string& last_error() {
  thread_local std::string msg;
  return msg;
}

Tuning g_tuning;

namespace {

// ---- kernel timing ----------------------------------------------------------------------
struct ProfRec {
  int kernel;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
uint32_t g_prof_mask = ~0u;          // kernel ids (bits) that get an event pair
std::vector<ProfRec> g_prof;
std::vector<hipEvent_t> g_event_pool;     // events of earlier records, reused (no create per launch)

hipEvent_t pooled_event() {               // caller holds g_prof_mu
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  // timing only: no system-scope fence around the record, so the marker does not flush
  // caches between the kernels it brackets (elapsed times are read after a device wait)
  hipEvent_t e = nullptr;
  return hipEventCreateWithFlags(&e, hipEventDisableSystemFence) == hipSuccess ? e : nullptr;
}

struct ProfScope {
  int kernel;
  hipStream_t stream;
  hipEvent_t start = nullptr, stop = nullptr;
  ProfScope(int k, hipStream_t s) : kernel(k), stream(s) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on || !((g_prof_mask >> k) & 1u)) return;
    start = pooled_event();
    stop = pooled_event();
    if (!start || !stop) {
      if (start) g_event_pool.push_back(start);
      if (stop) g_event_pool.push_back(stop);
      start = stop = nullptr;
      return;
    }
    hipEventRecord(start, stream);
  }
  ~ProfScope() {
    if (!start) return;
    hipEventRecord(stop, stream);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof.push_back({kernel, start, stop});
  }
};

// ---- pinned staging ring for the plan upload -------------------------------------------
struct Staging {
  void* host = nullptr;
  void* host_dev = nullptr;     // the same pinned buffer as a device-side address
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool in_flight = false;
};
constexpr int kRing = 8;
std::mutex g_ring_mu;
Staging g_ring[kRing];
std::vector<void*> g_ring_retired;
int g_ring_next = 0;

// Copies `bytes` to device `dst` on `stream` through pinned memory: `fill(host)` writes the
// bytes straight into a staging slot, so a call makes no host allocation once the slots have
// grown to size (capacities are powers of two). A slot is reused only after its previous
// copy has completed (event wait). With the stage kernel the copy moves `bytes` rounded up to
// 16, so `dst` must have room for that.
//
// upload_with() leaves the device side to `launch(src_dev, src_host, bytes)`, which must
// enqueue on `stream` whatever reads the slot (the event after it guards the slot's reuse).
template <class Fill, class Launch>
int upload_with(size_t bytes, hipStream_t stream, Fill&& fill, Launch&& launch) {
  if (bytes == 0) return CB_OK;
  bytes = (bytes + 15) & ~static_cast<size_t>(15);
  std::lock_guard<std::mutex> lk(g_ring_mu);
  Staging& s = g_ring[g_ring_next];
  g_ring_next = (g_ring_next + 1) % kRing;
  if (s.in_flight) {
    if (hipEventSynchronize(s.ev) != hipSuccess) return fail(CB_ERR_HIP, "plan upload: event wait failed");
    s.in_flight = false;
  }
  // the event only tells the host that the copy has finished reading the slot
  if (!s.ev && hipEventCreateWithFlags(&s.ev, hipEventDisableTiming | hipEventDisableSystemFence) != hipSuccess)
    return fail(CB_ERR_HIP, "plan upload: hipEventCreate failed");
  if (s.cap < bytes) {
    // A kernel may have read the old buffer directly: it is kept (not freed) until the
    // process ends, which growth by powers of two bounds to the size of the last buffer.
    if (s.host) g_ring_retired.push_back(s.host);
    s.host = nullptr;
    s.cap = 0;
    size_t cap = size_t{1} << 16;
    while (cap < bytes) cap <<= 1;
    // coherent: the device reads what the host wrote before the launch, never a cached copy
    if (hipHostMalloc(&s.host, cap, hipHostMallocCoherent) != hipSuccess)
      return fail(CB_ERR_HIP, "plan upload: hipHostMalloc(%zu) failed", cap);
    if (hipHostGetDevicePointer(&s.host_dev, s.host, 0) != hipSuccess)
      return fail(CB_ERR_HIP, "plan upload: hipHostGetDevicePointer failed");
    s.cap = cap;
  }
  fill(static_cast<char*>(s.host));
  hipError_t e = launch(static_cast<const void*>(s.host_dev), static_cast<const void*>(s.host), bytes);
  if (e != hipSuccess) return fail(CB_ERR_HIP, "plan upload: %s", hipGetErrorString(e));
  if (hipEventRecord(s.ev, stream) != hipSuccess) return fail(CB_ERR_HIP, "plan upload: event record failed");
  s.in_flight = true;
  return CB_OK;
}

template <class Fill>
int upload(void* dst, size_t bytes, hipStream_t stream, Fill&& fill) {
  return upload_with(bytes, stream, fill, [&](const void* src_dev, const void* src_host, size_t n) {
    return g_tuning.stage_kernel ? launch_stage_copy(src_dev, dst, n, stream)
                                 : hipMemcpyAsync(dst, src_host, n, hipMemcpyHostToDevice, stream);
  });
}

// ---- side stream for running prefill tiles beside the decode rows ----------------------
// One non-blocking stream (default priority) and a fork/join event pair per device.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
std::vector<SideStream> g_side;

int side_stream(SideStream** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(CB_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_side_mu);
  if (static_cast<int>(g_side.size()) <= dev) g_side.resize(dev + 1);
  SideStream& ss = g_side[dev];
  if (!ss.stream) {
    if (hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess)
      return fail(CB_ERR_HIP, "could not create the side stream");
  }
  *out = &ss;
  return CB_OK;
}

}  // namespace

// Launches the attention kernels of plan `p`, whose work lists are already in the workspace
// at `ws` (plan offsets are relative to `ws`). `batch` holds device metadata pointers.
int launch_attention(const cb_shape* shape, const cb_batch* batch, const Plan& p, char* ws, const void* q,
                     const void* k_cache, const void* v_cache, float scale, void* o, hipStream_t s,
                     bool allow_side_stream) {
  const int eb = elem_bytes(shape);
  const float scale_log2 = static_cast<float>(static_cast<double>(scale) * kLog2e);
  hipError_t e = hipSuccess;
  int st = CB_OK;
  // Prefill tiles (MFMA-bound) and decode rows (HBM-bound) touch disjoint rows of O. With
  // "overlap_prefill" set, the prefill kernel runs on a side stream forked from `stream` and
  // joined back before the combine pass, so the two can share the device. It is off by
  // default: measured on config 2, co-resident prefill work-groups slowed the decode kernel
  // more than the overlap saved.
  hipStream_t ps = s;
  SideStream* side = nullptr;
  const bool fork =
      allow_side_stream && g_tuning.overlap_prefill && !p.mixed && !p.prefill.empty() && !p.splits.empty();
  if (fork) {
    if ((st = side_stream(&side))) return st;
    ps = side->stream;
    if (hipEventRecord(side->fork, s) != hipSuccess || hipStreamWaitEvent(ps, side->fork, 0) != hipSuccess)
      return fail(CB_ERR_HIP, "cb_ragged_attention: fork failed");
  }
  const PrefillArgs pa{q, k_cache, v_cache, o, reinterpret_cast<const PrefillItem*>(ws + p.off_prefill),
                       batch->cu_q_lens, batch->ctx_lens, batch->block_tables, static_cast<int32_t>(p.prefill.size()),
                       shape->num_q_heads, shape->num_kv_heads, batch->max_blocks_per_req, shape->num_blocks,
                       scale_log2, nullptr,
                       reinterpret_cast<float*>(ws + p.off_part_o), reinterpret_cast<float*>(ws + p.off_part_ml)};
  const RowArgs ra{q, k_cache, v_cache, o,
                   reinterpret_cast<float*>(ws + p.off_part_o), reinterpret_cast<float*>(ws + p.off_part_ml),
                   reinterpret_cast<const RowSplit*>(ws), batch->block_tables,
                   static_cast<int32_t>(p.splits.size()) * shape->num_kv_heads * p.n_sub,
                   shape->num_q_heads, shape->num_kv_heads, batch->max_blocks_per_req, shape->num_blocks, scale_log2,
                   p.group};
  if (p.mixed) {
    const MixedArgs ma{pa, ra, reinterpret_cast<const int32_t*>(ws + p.off_order),
                       static_cast<int32_t>(p.order.size())};
    ProfScope prof(CB_KERNEL_MIXED, s);
    e = launch_mixed(ma, shape->head_dim, s);
  } else {
    if (!p.prefill.empty()) {
      ProfScope prof(CB_KERNEL_PREFILL, ps);
      e = launch_prefill(pa, shape->head_dim, p.prefill_waves, ps);
    }
    if (e == hipSuccess && !p.splits.empty()) {
      ProfScope prof(CB_KERNEL_DECODE, s);
      e = p.mfma_decode ? launch_rows_mfma(ra, shape->head_dim, s) : launch_rows(ra, eb, shape->head_dim, p.group, s);
    }
  }
  // The side stream is joined back before the combine pass: split prefill tiles leave
  // partials that the combine merges, so it must follow the prefill kernel as well as the
  // decode kernel.
  if (fork) {
    if (hipEventRecord(side->join, ps) != hipSuccess || hipStreamWaitEvent(s, side->join, 0) != hipSuccess)
      return fail(CB_ERR_HIP, "cb_ragged_attention: join failed");
  }
  if (e == hipSuccess && !p.combine.empty()) {
    CombineArgs ca{o, reinterpret_cast<const float*>(ws + p.off_part_o),
                   reinterpret_cast<const float*>(ws + p.off_part_ml),
                   reinterpret_cast<const CombineRow*>(ws + p.off_combine), static_cast<int32_t>(p.combine.size()),
                   shape->num_q_heads};
    ProfScope prof(CB_KERNEL_COMBINE, s);
    e = launch_combine(ca, eb, shape->head_dim, s);
  }
  if (e != hipSuccess) return fail(CB_ERR_HIP, "cb_ragged_attention: launch failed: %s", hipGetErrorString(e));
  return CB_OK;
}

}  // namespace cb

using namespace cb;

extern "C" const char* cb_last_error(void) { return last_error().c_str(); }

extern "C" const char* cb_version(void) { return "cb 0.1 gfx950"; }

extern "C" int cb_debug_violations(uint32_t* count, int reset) {
  if (!count) return fail(CB_ERR_INVALID_ARG, "cb_debug_violations: count is NULL");
  *count = 0;
#ifdef CB_DEVICE_CHECKS
  if (hipDeviceSynchronize() != hipSuccess) return fail(CB_ERR_HIP, "cb_debug_violations: synchronize failed");
  for (auto* read : {violations_rows, violations_decode_gqa, violations_prefill, violations_mixed, violations_append,
                     violations_gemm}) {
    const hipError_t e = read(count, reset != 0);
    if (e != hipSuccess) return fail(CB_ERR_HIP, "cb_debug_violations: %s", hipGetErrorString(e));
  }
  return CB_OK;
#else
  (void)reset;
  return fail(CB_ERR_UNSUPPORTED, "cb_debug_violations: this copy of the library has no device checks "
                                  "(python -m ragged_continuous_batching_amd.build --device-checks)");
#endif
}

namespace {

// The tuning keys: name, field, and the values a key accepts (checked by cb_set_tuning;
// boolean keys store value != 0).
struct TuningKey {
  const char* name;
  int32_t Tuning::*field;
  enum Kind { kCount, kBool, kXcds, kWaves, kGroup, kHeads } kind;
};
constexpr TuningKey kTuningKeys[] = {
    {"split_blocks", &Tuning::split_blocks, TuningKey::kCount},
    {"target_waves", &Tuning::target_waves, TuningKey::kCount},
    {"overlap_prefill", &Tuning::overlap_prefill, TuningKey::kBool},
    {"xcds", &Tuning::xcds, TuningKey::kXcds},
    {"decode_group", &Tuning::decode_group, TuningKey::kGroup},
    {"decode_mfma", &Tuning::decode_mfma, TuningKey::kBool},
    {"stage_kernel", &Tuning::stage_kernel, TuningKey::kBool},
    {"prefill_snake", &Tuning::prefill_snake, TuningKey::kBool},
    {"prefill_waves", &Tuning::prefill_waves, TuningKey::kWaves},
    {"prefill_split", &Tuning::prefill_split, TuningKey::kBool},
    {"prefill_split_tiles", &Tuning::prefill_split_tiles, TuningKey::kCount},
    {"mixed_launch", &Tuning::mixed_launch, TuningKey::kBool},
    {"decode_order", &Tuning::decode_order, TuningKey::kBool},
    {"mixed_order", &Tuning::mixed_order, TuningKey::kBool},
    {"prefill_heads", &Tuning::prefill_heads, TuningKey::kHeads},
};

const TuningKey* find_tuning_key(const char* key) {
  if (!key) return nullptr;
  for (const TuningKey& k : kTuningKeys)
    if (std::strcmp(key, k.name) == 0) return &k;
  return nullptr;
}

}  // namespace

extern "C" int cb_set_tuning(const char* key, int32_t value) {
  const TuningKey* k = find_tuning_key(key);
  if (!k) return fail(CB_ERR_INVALID_ARG, "cb_set_tuning: unknown key '%s'", key ? key : "(null)");
  if (value < 0) return fail(CB_ERR_INVALID_ARG, "cb_set_tuning: negative value for '%s'", k->name);
  switch (k->kind) {
    case TuningKey::kBool: value = value != 0; break;
    case TuningKey::kXcds: value = std::max<int32_t>(1, value); break;
    case TuningKey::kWaves:
      if (value != 0 && value != 4 && value != 8)
        return fail(CB_ERR_INVALID_ARG, "cb_set_tuning: prefill_waves must be 0, 4 or 8");
      break;
    case TuningKey::kGroup:
      if (value != 1 && value != 2 && value != 4 && value != 8)
        return fail(CB_ERR_INVALID_ARG, "cb_set_tuning: decode_group must be 1, 2, 4 or 8");
      break;
    case TuningKey::kHeads:
      if (value != 0 && value != 1 && value != 2 && value != 4 && value != 8)
        return fail(CB_ERR_INVALID_ARG, "cb_set_tuning: prefill_heads must be 0, 1, 2, 4 or 8");
      break;
    case TuningKey::kCount: break;
  }
  g_tuning.*(k->field) = value;
  return CB_OK;
}

extern "C" int cb_get_tuning(const char* key, int32_t* value) {
  const TuningKey* k = find_tuning_key(key);
  if (!k) return fail(CB_ERR_INVALID_ARG, "cb_get_tuning: unknown key '%s'", key ? key : "(null)");
  if (!value) return fail(CB_ERR_INVALID_ARG, "cb_get_tuning: value is NULL");
  *value = g_tuning.*(k->field);
  return CB_OK;
}

extern "C" const char* cb_kernel_name(int k) {
  switch (k) {
    case CB_KERNEL_APPEND: return "kv_append_kernel";
    case CB_KERNEL_DECODE: return "row_attn_kernel";
    case CB_KERNEL_COMBINE: return "combine_kernel";
    case CB_KERNEL_PREFILL: return "prefill_kernel";
    case CB_KERNEL_GEMM: return "gemm_bt_kernel";
    case CB_KERNEL_MIXED: return "mixed_attn_kernel";
    default: return "";
  }
}

extern "C" int cb_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return CB_OK;
}

extern "C" int cb_profile_select(uint32_t mask) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_mask = mask ? mask : ~0u;
  return CB_OK;
}

extern "C" int cb_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof) {
    hipEventSynchronize(r.stop);
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_prof.clear();
  return CB_OK;
}

extern "C" int cb_profile_launches(int kernel_id, float* ms_out, int64_t capacity, int64_t* launches) {
  if (kernel_id < 0 || kernel_id >= CB_KERNEL_COUNT) return fail(CB_ERR_INVALID_ARG, "bad kernel id %d", kernel_id);
  if (capacity < 0 || (capacity > 0 && !ms_out)) return fail(CB_ERR_INVALID_ARG, "cb_profile_launches: bad buffer");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int64_t n = 0;
  for (auto& r : g_prof) {
    if (r.kernel != kernel_id) continue;
    if (n < capacity) {
      if (hipEventSynchronize(r.stop) != hipSuccess) return fail(CB_ERR_HIP, "cb_profile_launches: event wait failed");
      float ms = 0;
      if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
        return fail(CB_ERR_HIP, "cb_profile_launches: elapsed time failed");
      ms_out[n] = ms;
    }
    ++n;
  }
  if (launches) *launches = n;
  return CB_OK;
}

extern "C" int cb_profile_read(int kernel_id, double* total_ms, int64_t* launches) {
  if (kernel_id < 0 || kernel_id >= CB_KERNEL_COUNT) return fail(CB_ERR_INVALID_ARG, "bad kernel id %d", kernel_id);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double sum = 0;
  int64_t n = 0;
  for (auto& r : g_prof) {
    if (r.kernel != kernel_id) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return fail(CB_ERR_HIP, "cb_profile_read: event wait failed");
    float ms = 0;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      return fail(CB_ERR_HIP, "cb_profile_read: elapsed time failed");
    sum += ms;
    ++n;
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = n;
  return CB_OK;
}

extern "C" int cb_kv_append(const cb_shape* shape, const cb_batch* batch, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_batch(shape, batch))) return st;
  if (batch->num_tokens == 0) return CB_OK;
  if (!k_new || !v_new || !k_cache || !v_cache) return fail(CB_ERR_INVALID_ARG, "cb_kv_append: NULL tensor");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(CB_ERR_INVALID_ARG, "cb_kv_append: tensors must be 16-byte aligned");
  AppendArgs a{k_new, v_new, k_cache, v_cache, batch->cu_q_lens, batch->ctx_lens, batch->block_tables,
               batch->num_reqs, batch->num_tokens, batch->max_blocks_per_req, shape->num_kv_heads, shape->num_blocks};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  {
    ProfScope ps(CB_KERNEL_APPEND, s);
    e = launch_kv_append(a, elem_bytes(shape), shape->head_dim, s);
  }
  if (e != hipSuccess) return fail(CB_ERR_HIP, "cb_kv_append: launch failed: %s", hipGetErrorString(e));
  return CB_OK;
}

extern "C" size_t cb_ragged_attention_workspace_size(const cb_shape* shape, const cb_batch* batch) {
  if (check_shape(shape) || check_batch(shape, batch)) return 0;
  if (batch->num_tokens == 0) return 0;
  Plan p;
  make_plan(shape, batch, p);
  return p.total;
}

extern "C" int cb_plan_describe(const cb_shape* shape, const cb_batch* batch, cb_plan_info* out) {
  if (!out) return fail(CB_ERR_INVALID_ARG, "cb_plan_describe: out is null");
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_batch(shape, batch))) return st;
  *out = cb_plan_info{};
  if (batch->num_tokens == 0) return CB_OK;
  Plan p;
  make_plan(shape, batch, p);
  out->prefill_rows = p.prefill.empty() ? 0 : (32 * p.prefill_waves) >> p.prefill_heads_log2;
  out->prefill_heads = p.prefill.empty() ? 0 : 1 << p.prefill_heads_log2;
  out->prefill_items = static_cast<int32_t>(p.prefill.size());
  for (const PrefillItem& it : p.prefill)
    if (it.req >= 0 && it.part_base >= 0) ++out->prefill_split_items;
  out->decode_splits = static_cast<int32_t>(p.splits.size());
  out->decode_items = static_cast<int32_t>(p.splits.size()) * shape->num_kv_heads * p.n_sub;
  out->split_blocks = p.splits.empty() ? 0 : p.split_blocks;
  out->longest_first = 1;
  for (size_t i = 0; i < p.splits.size(); ++i) {
    const int32_t len = p.splits[i].blk_end - p.splits[i].blk_begin;
    out->split_min_blocks = i == 0 ? len : std::min(out->split_min_blocks, len);
    out->split_max_blocks = std::max(out->split_max_blocks, len);
    if (i > 0 && len > p.splits[i - 1].blk_end - p.splits[i - 1].blk_begin) out->longest_first = 0;
  }
  out->matrix_core_decode = !p.splits.empty() && p.mfma_decode;
  out->combine_rows = static_cast<int32_t>(p.combine.size());
  out->mixed = p.mixed;
  return CB_OK;
}

extern "C" int cb_ragged_attention(const cb_shape* shape, const cb_batch* batch, const void* q,
                                   const void* k_cache, const void* v_cache, float scale, void* o,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_batch(shape, batch))) return st;
  if (batch->num_tokens == 0) return CB_OK;
  if ((st = check_tensors(q, k_cache, v_cache, o, scale, "cb_ragged_attention"))) return st;
  Plan p;
  make_plan(shape, batch, p);
  if (workspace_bytes < p.total || (p.total > 0 && !workspace))
    return fail(CB_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed", workspace_bytes, p.total);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(CB_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if ((st = upload(ws, p.plan_bytes, s, [&](char* host) { write_plan(p, host); }))) return st;
  return launch_attention(shape, batch, p, ws, q, k_cache, v_cache, scale, o, s, true);
}

extern "C" size_t cb_step_workspace_size(const cb_shape* shape, int32_t num_reqs, int32_t num_tokens,
                                         int32_t max_blocks_per_req, const int32_t* h_cu_q_lens,
                                         const int32_t* h_ctx_lens) {
  if (check_shape(shape) || num_reqs < 0 || max_blocks_per_req < 0) return 0;
  cb_batch b = step_batch(num_reqs, num_tokens, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, nullptr,
                          step_layout(num_reqs, 0, num_tokens));
  if (check_batch(shape, &b) || num_tokens == 0) return 0;
  std::vector<int32_t> rows;
  const bool compact = slots_fit(shape);
  const int64_t nbt = compact ? compact_rows(num_reqs, h_cu_q_lens, h_ctx_lens, rows)
                              : static_cast<int64_t>(num_reqs) * max_blocks_per_req;
  const StepLayout l = step_layout(num_reqs, nbt, num_tokens);
  Plan p;
  make_plan(shape, &b, p, 0, true, compact ? rows.data() : nullptr);
  return l.plan_base + p.total;
}

extern "C" int cb_step_forward(const cb_shape* shape, int32_t num_reqs, int32_t num_tokens, int32_t max_blocks_per_req,
                               const int32_t* h_cu_q_lens, const int32_t* h_ctx_lens, const int32_t* h_block_tables,
                               const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               float scale, void* o, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if (num_reqs < 0 || max_blocks_per_req < 0) return fail(CB_ERR_INVALID_ARG, "cb_step_forward: negative count");
  char* ws = static_cast<char*>(workspace);
  cb_batch b = step_batch(num_reqs, num_tokens, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, nullptr,
                          step_layout(num_reqs, 0, num_tokens));
  if ((st = check_batch(shape, &b))) return st;
  if (num_tokens == 0) return CB_OK;
  // slots and the compact block table go together: with them, no kernel indexes the table
  // by max_blocks_per_req (the append takes slots, the rest take each item's bt_row)
  const bool slots = slots_fit(shape);
  // Marked rows need the staging kernel: their (row, slot) list stays in the pinned buffer,
  // after the bytes the append copies into the workspace, and the page work-groups read it there.
  const bool marks = slots && g_tuning.stage_kernel && sole_marks_apply(shape, num_reqs, h_cu_q_lens);
  std::vector<int32_t> bt_rows;
  const int64_t nbt = slots ? compact_rows(num_reqs, h_cu_q_lens, h_ctx_lens, bt_rows)
                            : static_cast<int64_t>(num_reqs) * max_blocks_per_req;
  const StepLayout l = step_layout(num_reqs, nbt, num_tokens);
  b = step_batch(num_reqs, num_tokens, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, ws, l);
  if ((st = check_block_ids(shape, num_reqs, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, h_block_tables,
                             "cb_step_forward")))
    return st;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))
    return fail(CB_ERR_INVALID_ARG, "cb_step_forward: new K/V must be non-NULL and 16-byte aligned");
  if ((st = check_tensors(q, k_cache, v_cache, o, scale, "cb_step_forward"))) return st;
  Plan p;
  make_plan(shape, &b, p, 0, true, slots ? bt_rows.data() : nullptr);
  if (!ws || workspace_bytes < l.plan_base + p.total)
    return fail(CB_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed", workspace_bytes,
                l.plan_base + p.total);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(CB_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

  // one upload: metadata, then the plan (then, not copied, the marked rows)
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t staged = l.plan_base + p.plan_bytes;
  const size_t off_marked = (staged + 15) & ~static_cast<size_t>(15);
  int32_t n_marked = 0;
  auto fill = [&](char* host) {
    std::memcpy(host + l.off_cu, h_cu_q_lens, static_cast<size_t>(num_reqs + 1) * 4);
    std::memcpy(host + l.off_ctx, h_ctx_lens, static_cast<size_t>(num_reqs) * 4);
    if (slots) {
      fill_compact(num_reqs, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, h_block_tables, bt_rows,
                   reinterpret_cast<int32_t*>(host + l.off_bt));
      n_marked = fill_slots(num_reqs, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, h_block_tables,
                            reinterpret_cast<int32_t*>(host + l.off_slots), marks,
                            marks ? reinterpret_cast<int32_t*>(host + off_marked) : nullptr);
    } else {
      std::memcpy(host + l.off_bt, h_block_tables, static_cast<size_t>(num_reqs) * max_blocks_per_req * 4);
    }
    write_plan(p, host + l.plan_base);
  };
  AppendArgs aa{k_new, v_new, k_cache, v_cache, b.cu_q_lens, b.ctx_lens, b.block_tables, num_reqs, num_tokens,
                max_blocks_per_req, shape->num_kv_heads, shape->num_blocks, nullptr,
                slots ? reinterpret_cast<const int32_t*>(ws + l.off_slots) : nullptr, nullptr, nullptr, 0,
                marks ? kSlotSoleWriter : 0};
  const int eb = elem_bytes(shape);
  hipError_t e = hipSuccess;
  if (g_tuning.stage_kernel && slots) {
    // The append launch also moves the staged bytes into the workspace, and takes its slots
    // straight from the pinned buffer: one kernel fewer per step.
    const size_t up = marks ? off_marked + static_cast<size_t>(num_tokens) * 8 : staged;
    st = upload_with(up, s, fill, [&](const void* src_dev, const void*, size_t) {
      aa.slots = reinterpret_cast<const int32_t*>(static_cast<const char*>(src_dev) + l.off_slots);
      aa.stage_src = src_dev;
      aa.stage_dst = ws;
      aa.stage_n16 = static_cast<int64_t>((staged + 15) / 16);
      aa.marked = n_marked ? reinterpret_cast<const int32_t*>(static_cast<const char*>(src_dev) + off_marked) : nullptr;
      aa.n_marked = n_marked;
      ProfScope prof(CB_KERNEL_APPEND, s);
      return e = launch_kv_append(aa, eb, shape->head_dim, s);
    });
    if (st) return st;
  } else {
    if ((st = upload(ws, l.plan_base + p.plan_bytes, s, fill))) return st;
    ProfScope prof(CB_KERNEL_APPEND, s);
    e = launch_kv_append(aa, eb, shape->head_dim, s);
  }
  if (e != hipSuccess) return fail(CB_ERR_HIP, "cb_step_forward: append launch failed: %s", hipGetErrorString(e));
  return launch_attention(shape, &b, p, ws + l.plan_base, q, k_cache, v_cache, scale, o, s, true);
}

static_assert(kSlotSoleWriter == CB_SLOT_SOLE_WRITER, "the staged sole-writer bit is the one cb.h documents");

extern "C" int32_t cb_paged_read_probe_sink_words(int32_t n_pages) { return n_pages > 0 ? paged_read_grid(n_pages) : 0; }

extern "C" int cb_paged_read_probe(const void* pages, int32_t n_pages, const int32_t* order, uint32_t* sink,
                                   void* stream) {
  if (n_pages < 1 || !pages || !order || !sink || !aligned16(pages))
    return fail(CB_ERR_INVALID_ARG, "cb_paged_read_probe: needs n_pages >= 1 and non-NULL pointers, pages 16-byte aligned");
  const hipError_t e = launch_paged_read(pages, n_pages, order, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(CB_ERR_HIP, "cb_paged_read_probe: launch failed: %s", hipGetErrorString(e));
  return CB_OK;
}

extern "C" int cb_step_slots(const cb_shape* shape, int32_t num_reqs, int32_t num_tokens, int32_t max_blocks_per_req,
                             const int32_t* h_cu_q_lens, const int32_t* h_ctx_lens, const int32_t* h_block_tables,
                             int32_t* out_slots) {
  int st = check_shape(shape);
  if (st) return st;
  if (num_reqs < 0 || max_blocks_per_req < 0) return fail(CB_ERR_INVALID_ARG, "cb_step_slots: negative count");
  cb_batch b = step_batch(num_reqs, num_tokens, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, nullptr,
                          step_layout(num_reqs, 0, num_tokens));
  if ((st = check_batch(shape, &b))) return st;
  if (num_tokens == 0) return CB_OK;
  if (!out_slots) return fail(CB_ERR_INVALID_ARG, "cb_step_slots: out_slots is null");
  if (!slots_fit(shape)) return fail(CB_ERR_UNSUPPORTED, "cb_step_slots: the pool is too large for host slots");
  if ((st = check_block_ids(shape, num_reqs, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, h_block_tables,
                            "cb_step_slots")))
    return st;
  fill_slots(num_reqs, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, h_block_tables, out_slots,
             sole_marks_apply(shape, num_reqs, h_cu_q_lens));
  return CB_OK;
}

extern "C" int cb_linear(int32_t M, int32_t N, int32_t K, const void* a, const void* w, void* c, void* stream) {
  if (M < 0 || N <= 0 || K <= 0 || N % 128 != 0 || K % 64 != 0 || K > kGemmMaxK)
    return fail(CB_ERR_UNSUPPORTED, "cb_linear: needs M >= 0, N a multiple of 128 and K a multiple of 64 "
                "up to %d (got %d, %d, %d)", kGemmMaxK, M, N, K);
  if (M == 0) return CB_OK;
  if (!a || !w || !c || !aligned16(a) || !aligned16(w) || !aligned16(c))
    return fail(CB_ERR_INVALID_ARG, "cb_linear: tensors must be non-NULL and 16-byte aligned");
  GemmArgs g{a, w, c, M, N, K, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, 0, 0, 0, 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  {
    ProfScope prof(CB_KERNEL_GEMM, s);
    e = launch_gemm(g, 0, s);
  }
  if (e != hipSuccess) return fail(CB_ERR_HIP, "cb_linear: launch failed: %s", hipGetErrorString(e));
  return CB_OK;
}

extern "C" int cb_qkv_project(const cb_shape* shape, const cb_batch* batch, int32_t d_model, const void* x,
                              const void* w_qkv, void* q, void* k_cache, void* v_cache, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_batch(shape, batch))) return st;
  if (shape->dtype != CB_BF16) return fail(CB_ERR_UNSUPPORTED, "cb_qkv_project: bf16 only");
  const int32_t qd = shape->num_q_heads * shape->head_dim, kd = shape->num_kv_heads * shape->head_dim;
  if (d_model <= 0 || d_model % 64 != 0 || d_model > kGemmMaxK || qd % 128 != 0 || kd % 128 != 0)
    return fail(CB_ERR_UNSUPPORTED, "cb_qkv_project: needs d_model a multiple of 64 up to %d and Hq*D, Hkv*D "
                "multiples of 128", kGemmMaxK);
  if (batch->num_tokens == 0) return CB_OK;
  if (!x || !w_qkv || !q || !k_cache || !v_cache || !aligned16(x) || !aligned16(w_qkv) || !aligned16(q) ||
      !aligned16(k_cache) || !aligned16(v_cache))
    return fail(CB_ERR_INVALID_ARG, "cb_qkv_project: tensors must be non-NULL and 16-byte aligned");
  GemmArgs g{x, w_qkv, q, batch->num_tokens, qd + 2 * kd, d_model, k_cache, v_cache, batch->cu_q_lens,
             batch->ctx_lens, batch->block_tables, batch->num_reqs, batch->max_blocks_per_req,
             shape->num_q_heads, shape->num_kv_heads, shape->head_dim, shape->num_blocks};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  {
    ProfScope prof(CB_KERNEL_GEMM, s);
    e = launch_gemm(g, 1, s);
  }
  if (e != hipSuccess) return fail(CB_ERR_HIP, "cb_qkv_project: launch failed: %s", hipGetErrorString(e));
  return CB_OK;
}
