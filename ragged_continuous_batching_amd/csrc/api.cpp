// C ABI entry points: argument validation, the launch planner, the plan upload, kernel
// launches and kernel timing. Host code only; the kernels live in the .hip files.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "cb.h"
#include "cb_common.h"
#include "cb_plan.h"

namespace cb {

std::string& last_error() {
  thread_local std::string msg;
  return msg;
}

hipError_t launch_kv_append(const AppendArgs& a, int elem_bytes, int head_dim, hipStream_t s);
hipError_t launch_rows(const RowArgs& a, int elem_bytes, int head_dim, int group, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int elem_bytes, int head_dim, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int waves, hipStream_t s);
hipError_t launch_rows_mfma(const RowArgs& a, int head_dim, hipStream_t s);
hipError_t launch_stage_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
hipError_t launch_stage_copy_desc(const void* src, void* dst, size_t max_bytes, hipStream_t s);
hipError_t launch_gemm(const GemmArgs& g, int epilogue, hipStream_t s);
hipError_t launch_mixed(const MixedArgs& a, int head_dim, hipStream_t s);

namespace {

constexpr double kLog2e = 1.4426950408889634;

// ---- tuning -----------------------------------------------------------------------------
struct Tuning {
  int32_t split_blocks = 0;       // 0 = automatic
  int32_t target_waves = 0;       // 0: 8192 wave items (vector-ALU decode), 4096 (matrix-core decode)
  int32_t overlap_prefill = 0;    // 1 = run prefill tiles on a side stream beside decode rows
  int32_t xcds = 8;               // XCDs that work-groups are dispatched over (MI355X: 8)
  int32_t prefill_touch = 0;      // 1: prefill pulls key tiles two steps ahead toward L2
  int32_t decode_group = 8;       // most query heads one decode wave handles (1, 2, 4 or 8)
  int32_t decode_mfma = 1;        // 1: grouped-query decode (4+ heads per kv head) on MFMA
  int32_t stage_kernel = 1;       // 1: uploads run as a copy kernel on the stream; 0: copy engine
  int32_t prefill_snake = 1;      // 1: alternate rounds of each XCD's prefill queue reversed
  int32_t prefill_waves = 0;      // waves per prefill work-group: 4, 8 (32 query rows each) or
                                  // 0 = 8 when that still gives two work-groups per CU, else 4
  int32_t prefill_split = 1;      // 1: split the key walk of long prefill tiles when the step
                                  // has fewer prefill work-groups than slots (partials merged
                                  // by the combine pass)
  int32_t prefill_split_tiles = 0;  // key tiles per split, forcing splits (tests); 0 = automatic
  int32_t mixed_launch = 0;       // 1: prefill tiles and matrix-core decode waves in one launch
  int32_t mixed_order = 0;        // 0: merge prefill and decode chunks in proportion to their
                                  // counts; 1: alternate them until one kind runs out
};
Tuning g_tuning;

// ---- kernel timing ----------------------------------------------------------------------
struct ProfRec {
  int kernel;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
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
    if (!g_prof_on) return;
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

// ---- validation -------------------------------------------------------------------------
inline int elem_bytes(const cb_shape* s) { return s->dtype == CB_BF16 ? 2 : 4; }
inline int32_t ceil_div(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(const cb_shape* s) {
  if (!s) return fail(CB_ERR_INVALID_ARG, "shape is NULL");
  if (s->num_q_heads < 1 || s->num_kv_heads < 1 || s->num_q_heads % s->num_kv_heads != 0)
    return fail(CB_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                s->num_q_heads, s->num_kv_heads);
  const int g = s->num_q_heads / s->num_kv_heads;
  if (!(g == 1 || g == 2 || g == 4 || g % 8 == 0))
    return fail(CB_ERR_UNSUPPORTED, "query group size %d not supported (1, 2, 4 or a multiple of 8)", g);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(CB_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", s->head_dim);
  if (s->block_size != kBlockSize) return fail(CB_ERR_UNSUPPORTED, "block_size must be %d", kBlockSize);
  if (s->num_blocks < 1) return fail(CB_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (s->dtype != CB_F32 && s->dtype != CB_BF16) return fail(CB_ERR_INVALID_ARG, "unknown dtype %d", s->dtype);
  return CB_OK;
}

int check_batch(const cb_shape* s, const cb_batch* b) {
  if (!b) return fail(CB_ERR_INVALID_ARG, "batch is NULL");
  if (b->num_reqs < 0 || b->num_tokens < 0 || b->max_blocks_per_req < 0)
    return fail(CB_ERR_INVALID_ARG, "negative count in batch");
  if (b->num_reqs == 0) {
    if (b->num_tokens != 0) return fail(CB_ERR_INVALID_ARG, "num_tokens > 0 with no requests");
    return CB_OK;
  }
  if (!b->h_cu_q_lens || !b->h_ctx_lens) return fail(CB_ERR_INVALID_ARG, "host mirrors are required");
  if (!b->cu_q_lens || !b->ctx_lens || !b->block_tables)
    return fail(CB_ERR_INVALID_ARG, "device metadata pointer is NULL");
  if (b->h_cu_q_lens[0] != 0) return fail(CB_ERR_INVALID_ARG, "cu_q_lens[0] must be 0");
  for (int32_t r = 0; r < b->num_reqs; ++r) {
    const int32_t q = b->h_cu_q_lens[r + 1] - b->h_cu_q_lens[r];
    const int32_t c = b->h_ctx_lens[r];
    if (q < 0) return fail(CB_ERR_INVALID_ARG, "cu_q_lens decreases at request %d", r);
    if (c < 0) return fail(CB_ERR_INVALID_ARG, "ctx_lens[%d] = %d is negative", r, c);
    if (q > 0 && ceil_div(static_cast<int64_t>(c) + q, s->block_size) > b->max_blocks_per_req)
      return fail(CB_ERR_INVALID_ARG, "request %d needs %d blocks but max_blocks_per_req is %d", r,
                  ceil_div(static_cast<int64_t>(c) + q, s->block_size), b->max_blocks_per_req);
    if (static_cast<int64_t>(c) + q > (int64_t{1} << 30)) return fail(CB_ERR_INVALID_ARG, "request %d too long", r);
  }
  if (static_cast<int64_t>(b->num_reqs) * b->max_blocks_per_req > INT32_MAX)
    return fail(CB_ERR_INVALID_ARG, "block table of %d x %d entries is too large", b->num_reqs, b->max_blocks_per_req);
  if (b->h_cu_q_lens[b->num_reqs] != b->num_tokens)
    return fail(CB_ERR_INVALID_ARG, "cu_q_lens[num_reqs] = %d but num_tokens = %d", b->h_cu_q_lens[b->num_reqs],
                b->num_tokens);
  return CB_OK;
}

// ---- the launch plan ----------------------------------------------------------------------
inline size_t align256(size_t x) { return (x + 255) & ~size_t{255}; }

struct Plan {
  std::vector<RowSplit> splits;
  std::vector<CombineRow> combine;
  std::vector<PrefillItem> prefill;
  int32_t n_parts = 0;
  int group = 1;         // query heads per decode wave
  bool mfma_decode = false;  // decode rows on the MFMA kernel
  int prefill_waves = 4;     // waves (x 32 query rows) per prefill work-group
  int n_sub = 1;         // decode waves per kv head
  bool mixed = false;    // prefill tiles and decode waves in one launch (order below)
  std::vector<int32_t> order;
  size_t off_combine = 0, off_prefill = 0, off_order = 0, plan_bytes = 0, off_part_o = 0, off_part_ml = 0,
         total = 0;
};

// Would a step with these rows take the mixed launch? bf16 steps with prefill chunks and
// matrix-core decode rows (the 4-wave prefill work-group then has the decode work-group's
// shape, and both fit two to a CU).
bool wants_mixed(const cb_shape* s, const cb_batch* b) {
  if (!g_tuning.mixed_launch || s->dtype != CB_BF16 || !g_tuning.decode_mfma) return false;
  if (s->num_q_heads / s->num_kv_heads < 4) return false;
  bool dec = false, pre = false;
  for (int32_t r = 0; r < b->num_reqs; ++r) {
    const int32_t q = b->h_cu_q_lens[r + 1] - b->h_cu_q_lens[r];
    dec |= q == 1;
    pre |= q > 1;
  }
  return dec && pre;
}

// force_waves (4 or 8) fixes the prefill work-group size; 0 takes the tuning / automatic choice.
// allow_mixed = false keeps prefill and decode in separate launches (captured steps).
// bt_rows (host, [num_reqs], nullable): where each request's block ids start in the device
// block table; null means the padded [num_reqs, max_blocks_per_req] layout of cb_batch.
void make_plan(const cb_shape* s, const cb_batch* b, Plan& p, int force_waves = 0, bool allow_mixed = true,
               const int32_t* bt_rows = nullptr) {
  auto bt_row = [&](int32_t r) {
    return bt_rows ? bt_rows[r] : static_cast<int32_t>(static_cast<int64_t>(r) * b->max_blocks_per_req);
  };
  const int q_per_kv = s->num_q_heads / s->num_kv_heads;
  // query heads per decode wave: all heads of the group up to decode_group; a larger group
  // is covered by n_sub waves on adjacent slots, which read the same pages back to back
  p.mfma_decode = s->dtype == CB_BF16 && q_per_kv >= 4 && g_tuning.decode_mfma;
  if (p.mfma_decode) {          // up to 16 heads fill the columns of one 16x16 tile
    p.group = q_per_kv % 16 == 0 ? 16 : (q_per_kv % 8 == 0 ? 8 : 4);
  } else {
    p.group = std::min(q_per_kv, static_cast<int>(g_tuning.decode_group));
    while (q_per_kv % p.group) p.group /= 2;
  }
  p.n_sub = q_per_kv / p.group;
  const bool mfma_prefill = s->dtype == CB_BF16;
  p.mixed = allow_mixed && wants_mixed(s, b);
  p.prefill_waves = p.mixed ? 4 : force_waves ? force_waves : g_tuning.prefill_waves;
  if (p.prefill_waves == 0) {
    // 256-row work-groups read each key/value tile once for twice the rows, but a CU holds
    // only one of them (registers); take them when there are enough to fill every CU twice
    int64_t items256 = 0;
    for (int32_t r = 0; r < b->num_reqs; ++r) {
      const int32_t q = b->h_cu_q_lens[r + 1] - b->h_cu_q_lens[r];
      if (q > 1 && mfma_prefill) items256 += ceil_div(q, 256) * static_cast<int64_t>(s->num_q_heads);
    }
    p.prefill_waves = items256 >= 2 * kNumCUs ? 8 : 4;
  }

  // rows that take the split-K path, longest first
  struct Row { int32_t token, req, kv_len; };
  struct PrefillGroup { std::vector<PrefillItem> items; int64_t cost = 0; };
  struct QTile { int32_t req, qb, n_kt, n_split; };      // one row tile of a prefill chunk
  std::vector<PrefillGroup> groups;
  std::vector<QTile> qtiles;
  std::vector<Row> rows;
  int64_t total_blocks = 0, total_tiles = 0;
  for (int32_t r = 0; r < b->num_reqs; ++r) {
    const int32_t t0 = b->h_cu_q_lens[r], q = b->h_cu_q_lens[r + 1] - t0, c = b->h_ctx_lens[r];
    if (q == 0) continue;
    if (q == 1 || !mfma_prefill) {
      for (int32_t i = 0; i < q; ++i) {
        rows.push_back({t0 + i, r, c + i + 1});
        total_blocks += ceil_div(c + i + 1, kBlockSize);
      }
    } else {
      const int32_t rows = 32 * p.prefill_waves;
      for (int32_t qt = ceil_div(q, rows) - 1; qt >= 0; --qt) {
        const int32_t qb = qt * rows;
        qtiles.push_back({r, qb, ceil_div(c + std::min(qb + rows, q), kPrefillKeys), 1});
        total_tiles += static_cast<int64_t>(qtiles.back().n_kt) * s->num_q_heads;
      }
    }
  }
  // Split-K for prefill tiles when a step has fewer prefill work-groups than the machine has
  // work-group slots: a late chunk of a long prompt has few rows but a long context, and its
  // few work-groups would each walk every key tile while most CUs idle. Tiles longer than
  // the step's work per slot (at least 16 key tiles) are then cut into near-equal key
  // ranges, which brings the count of work-groups up to about the slots. With as many
  // work-groups as slots or more, the CUs already share the work evenly (long and short
  // work-groups pair up on each CU), and splitting only adds partials: measured on the
  // Llama-2-7B-shaped mixed step, 512 work-groups, prefill 58 -> 62 us, combine 5 -> 15 us.
  // Every cut lies at or below the first row's last key ((c + qb) / 64 tiles are fully
  // visible to every row of the tile), so no row meets an empty range.
  const int64_t slots = static_cast<int64_t>(kNumCUs) * (p.prefill_waves == 8 ? 1 : 2);
  const int64_t pre_items = static_cast<int64_t>(qtiles.size()) * s->num_q_heads;
  if (!qtiles.empty() && g_tuning.prefill_split && (pre_items < slots || g_tuning.prefill_split_tiles > 0)) {
    const int64_t len = g_tuning.prefill_split_tiles > 0
                            ? g_tuning.prefill_split_tiles
                            : std::max<int64_t>(16, (total_tiles + slots - 1) / slots);
    for (QTile& t : qtiles) {
      const int32_t c = b->h_ctx_lens[t.req];
      const int32_t lim = (c + t.qb) / kPrefillKeys;
      int32_t n = static_cast<int32_t>(std::min<int64_t>((t.n_kt + len - 1) / len, 0xffff));
      while (n > 1 && static_cast<int64_t>(n - 1) * t.n_kt / n > lim) --n;
      t.n_split = std::max(n, 1);
    }
  }
  {
    // one group per (request, kv head): all its q-tiles and query heads read the same
    // key/value tiles, so they are kept on one XCD (shared L2) and run side by side
    const int32_t rows = 32 * p.prefill_waves;
    size_t i0 = 0;
    while (i0 < qtiles.size()) {
      size_t i1 = i0;
      while (i1 < qtiles.size() && qtiles[i1].req == qtiles[i0].req) ++i1;
      const int32_t r = qtiles[i0].req, t0 = b->h_cu_q_lens[r], q = b->h_cu_q_lens[r + 1] - t0;
      std::vector<int32_t> part_base(i1 - i0, -1);
      for (size_t i = i0; i < i1; ++i) {          // partial slots and combine rows of split tiles
        const QTile& t = qtiles[i];
        if (t.n_split == 1) continue;
        part_base[i - i0] = p.n_parts;
        const int32_t valid = std::min(rows, q - t.qb);
        for (int32_t k = 0; k < valid; ++k) p.combine.push_back({t0 + t.qb + k, p.n_parts + k * t.n_split, t.n_split, 0});
        p.n_parts += valid * t.n_split;
      }
      for (int32_t g = 0; g < s->num_kv_heads; ++g) {
        PrefillGroup grp;
        for (size_t i = i0; i < i1; ++i) {
          const QTile& t = qtiles[i];
          for (int32_t sp = 0; sp < t.n_split; ++sp) {
            const int32_t k0 = static_cast<int32_t>(static_cast<int64_t>(sp) * t.n_kt / t.n_split);
            const int32_t k1 = static_cast<int32_t>(static_cast<int64_t>(sp + 1) * t.n_kt / t.n_split);
            for (int32_t hh = 0; hh < q_per_kv; ++hh) {
              grp.items.push_back({r, t.qb, g * q_per_kv + hh, bt_row(r), k0, k1, part_base[i - i0],
                                   t.n_split > 1 ? (t.n_split << 16) | sp : 0});
              grp.cost += k1 - k0;
            }
          }
        }
        groups.push_back(std::move(grp));
      }
      i0 = i1;
    }
  }
  // Work-groups are dispatched round-robin over the XCDs (block b runs on XCD b % n). Groups
  // go, longest first, to the XCD with the least work so far; each XCD's queue is then
  // interleaved into the launch order. Unused slots hold an empty item (req = -1).
  if (!groups.empty()) {
    const int nx = std::max(1, g_tuning.xcds);
    std::stable_sort(groups.begin(), groups.end(),
                     [](const PrefillGroup& x, const PrefillGroup& y) { return x.cost > y.cost; });
    std::vector<std::vector<PrefillItem>> queue(nx);
    std::vector<int64_t> load(nx, 0);
    for (const PrefillGroup& grp : groups) {
      const int x = static_cast<int>(std::min_element(load.begin(), load.end()) - load.begin());
      load[x] += grp.cost;
      queue[x].insert(queue[x].end(), grp.items.begin(), grp.items.end());
    }
    // Within an XCD the first C = (CUs per XCD) work-groups go one to each CU, the next C
    // take each CU's second slot in the same order, and so on. A queue sorted longest first
    // would pair the longest first-round item with the longest second-round one; reversing
    // every other round of C pairs long with short, so the CUs finish closer together.
    if (g_tuning.prefill_snake) {
      const size_t C = static_cast<size_t>(std::max(1, kNumCUs / nx));
      for (auto& qx : queue)
        for (size_t k0 = C; k0 < qx.size(); k0 += 2 * C)
          std::reverse(qx.begin() + k0, qx.begin() + std::min(qx.size(), k0 + C));
    }
    size_t depth = 0;
    for (const auto& qx : queue) depth = std::max(depth, qx.size());
    p.prefill.assign(depth * nx, PrefillItem{-1, 0, 0, 0, 0, 0, -1, 0});
    for (int x = 0; x < nx; ++x)
      for (size_t k = 0; k < queue[x].size(); ++k) p.prefill[k * nx + x] = queue[x][k];
  }
  std::stable_sort(rows.begin(), rows.end(), [](const Row& x, const Row& y) { return x.kv_len > y.kv_len; });

  int32_t split = g_tuning.split_blocks;
  if (split <= 0) {
    const int64_t units = total_blocks * s->num_kv_heads * p.n_sub;
    // Longer splits mean fewer partials to write and merge; the target keeps enough items
    // to fill the machine a few times over (the matrix-core kernel runs 2 waves per SIMD,
    // the vector-ALU one more). Measured on configs 2, 3 and the trace replay.
    const int64_t target = g_tuning.target_waves > 0 ? g_tuning.target_waves : (p.mfma_decode ? 4096 : 8192);
    split = static_cast<int32_t>(std::clamp<int64_t>((units + target - 1) / target, 4, kMaxSplitBlocks));
  }
  split = std::min(split, kMaxSplitBlocks);
  for (const Row& row : rows) {
    const int32_t nb = ceil_div(row.kv_len, kBlockSize);
    const int32_t ns = ceil_div(nb, split);
    if (ns == 1) {
      p.splits.push_back({row.token, bt_row(row.req), 0, nb, row.kv_len, -1});
      continue;
    }
    p.combine.push_back({row.token, p.n_parts, ns, 0});
    for (int32_t k = 0; k < ns; ++k)
      p.splits.push_back({row.token, bt_row(row.req), k * split, std::min(nb, (k + 1) * split), row.kv_len,
                          p.n_parts + k});
    p.n_parts += ns;
  }

  if (p.mixed) {
    // Chunks of one work-group per XCD. mixed_order 0: prefill and decode chunks merged in
    // proportion to their counts, so prefill work-groups stay a minority of each CU's
    // slots throughout (the cache stream, the step's bound, keeps most of them; measured on
    // the trace replay: 594 us for the launch vs 621 us for the two kernels). mixed_order 1:
    // alternate until one kind runs out (half the slots go to prefill: 678 us). A prefill
    // chunk keeps the XCD positions its planner chose (the prefill list is laid out in
    // chunks of nx); the last decode chunk is padded with work-group indices past the
    // decode items.
    const int nx = std::max(1, g_tuning.xcds);
    const int64_t n_rows = static_cast<int64_t>(p.splits.size()) * s->num_kv_heads * p.n_sub;
    const int64_t n_dwg = (n_rows + 3) / 4;
    const int64_t pch = static_cast<int64_t>(p.prefill.size()) / nx, dch = (n_dwg + nx - 1) / nx;
    int64_t pc = 0, dc = 0;
    p.order.reserve(static_cast<size_t>((pch + dch) * nx));
    while (pc < pch || dc < dch) {
      const bool take_p = dc == dch || (pc < pch && (g_tuning.mixed_order ? pc <= dc : pc * dch <= dc * pch));
      for (int k = 0; k < nx; ++k)
        p.order.push_back(take_p ? static_cast<int32_t>(pc * nx + k) : static_cast<int32_t>(-1 - (dc * nx + k)));
      (take_p ? pc : dc) += 1;
    }
  }

  const size_t eb = 4;
  p.off_combine = align256(p.splits.size() * sizeof(RowSplit));
  p.off_prefill = p.off_combine + align256(p.combine.size() * sizeof(CombineRow));
  p.off_order = p.off_prefill + align256(p.prefill.size() * sizeof(PrefillItem));
  p.plan_bytes = p.off_order + p.order.size() * sizeof(int32_t);
  p.off_part_o = align256(p.plan_bytes);
  p.off_part_ml = p.off_part_o + align256(static_cast<size_t>(p.n_parts) * s->num_q_heads * s->head_dim * eb);
  p.total = p.off_part_ml + align256(static_cast<size_t>(p.n_parts) * s->num_q_heads * 2 * eb);
}

}  // namespace
}  // namespace cb

using namespace cb;

extern "C" const char* cb_last_error(void) { return last_error().c_str(); }

extern "C" const char* cb_version(void) { return "cb 0.1 gfx950"; }

extern "C" int cb_set_tuning(const char* key, int32_t value) {
  if (!key || value < 0) return fail(CB_ERR_INVALID_ARG, "cb_set_tuning: bad key or value");
  if (std::strcmp(key, "split_blocks") == 0) {
    g_tuning.split_blocks = value;
  } else if (std::strcmp(key, "target_waves") == 0) {
    g_tuning.target_waves = value;
  } else if (std::strcmp(key, "overlap_prefill") == 0) {
    g_tuning.overlap_prefill = value != 0;
  } else if (std::strcmp(key, "xcds") == 0) {
    g_tuning.xcds = std::max<int32_t>(1, value);
  } else if (std::strcmp(key, "prefill_touch") == 0) {
    g_tuning.prefill_touch = value != 0;
  } else if (std::strcmp(key, "decode_mfma") == 0) {
    g_tuning.decode_mfma = value != 0;
  } else if (std::strcmp(key, "prefill_waves") == 0) {
    if (value != 0 && value != 4 && value != 8)
      return fail(CB_ERR_INVALID_ARG, "cb_set_tuning: prefill_waves must be 0, 4 or 8");
    g_tuning.prefill_waves = value;
  } else if (std::strcmp(key, "prefill_snake") == 0) {
    g_tuning.prefill_snake = value != 0;
  } else if (std::strcmp(key, "prefill_split") == 0) {
    g_tuning.prefill_split = value != 0;
  } else if (std::strcmp(key, "prefill_split_tiles") == 0) {
    g_tuning.prefill_split_tiles = value;
  } else if (std::strcmp(key, "mixed_launch") == 0) {
    g_tuning.mixed_launch = value != 0;
  } else if (std::strcmp(key, "mixed_order") == 0) {
    g_tuning.mixed_order = value != 0;
  } else if (std::strcmp(key, "stage_kernel") == 0) {
    g_tuning.stage_kernel = value != 0;
  } else if (std::strcmp(key, "decode_group") == 0) {
    if (value != 1 && value != 2 && value != 4 && value != 8)
      return fail(CB_ERR_INVALID_ARG, "cb_set_tuning: decode_group must be 1, 2, 4 or 8");
    g_tuning.decode_group = value;
  } else {
    return fail(CB_ERR_INVALID_ARG, "cb_set_tuning: unknown key '%s'", key);
  }
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

namespace cb {
namespace {

// Launches the attention kernels of plan `p`, whose work lists are already in the workspace
// at `ws` (plan offsets are relative to `ws`). `batch` holds device metadata pointers.
int launch_attention(const cb_shape* shape, const cb_batch* batch, const Plan& p, char* ws, const void* q,
                     const void* k_cache, const void* v_cache, float scale, void* o, hipStream_t s) {
  const int eb = elem_bytes(shape);
  const float scale_log2 = static_cast<float>(static_cast<double>(scale) * kLog2e);
  hipError_t e = hipSuccess;
  int st = CB_OK;
  // Prefill tiles (MFMA-bound) and decode rows (HBM-bound) touch disjoint rows of O. With
  // "overlap_prefill" set, the prefill kernel runs on a side stream forked from `stream` and
  // joined back before the call returns, so the two can share the device. It is off by
  // default: measured on config 2, co-resident prefill work-groups slowed the decode kernel
  // more than the overlap saved.
  hipStream_t ps = s;
  SideStream* side = nullptr;
  const bool fork = g_tuning.overlap_prefill && !p.mixed && !p.prefill.empty() && !p.splits.empty();
  if (fork) {
    if ((st = side_stream(&side))) return st;
    ps = side->stream;
    if (hipEventRecord(side->fork, s) != hipSuccess || hipStreamWaitEvent(ps, side->fork, 0) != hipSuccess)
      return fail(CB_ERR_HIP, "cb_ragged_attention: fork failed");
  }
  const PrefillArgs pa{q, k_cache, v_cache, o, reinterpret_cast<const PrefillItem*>(ws + p.off_prefill),
                       batch->cu_q_lens, batch->ctx_lens, batch->block_tables, static_cast<int32_t>(p.prefill.size()),
                       shape->num_q_heads, shape->num_kv_heads, batch->max_blocks_per_req, shape->num_blocks,
                       scale_log2, g_tuning.prefill_touch, nullptr,
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
  if (e == hipSuccess && !p.combine.empty()) {
    CombineArgs ca{o, reinterpret_cast<const float*>(ws + p.off_part_o),
                   reinterpret_cast<const float*>(ws + p.off_part_ml),
                   reinterpret_cast<const CombineRow*>(ws + p.off_combine), static_cast<int32_t>(p.combine.size()),
                   shape->num_q_heads};
    ProfScope prof(CB_KERNEL_COMBINE, s);
    e = launch_combine(ca, eb, shape->head_dim, s);
  }
  if (fork) {
    if (hipEventRecord(side->join, ps) != hipSuccess || hipStreamWaitEvent(s, side->join, 0) != hipSuccess)
      return fail(CB_ERR_HIP, "cb_ragged_attention: join failed");
  }
  if (e != hipSuccess) return fail(CB_ERR_HIP, "cb_ragged_attention: launch failed: %s", hipGetErrorString(e));
  return CB_OK;
}

// Serialises the plan's work lists at their offsets into `out` (plan_bytes long).
void write_plan(const Plan& p, char* out) {
  if (!p.splits.empty()) std::memcpy(out, p.splits.data(), p.splits.size() * sizeof(RowSplit));
  if (!p.combine.empty()) std::memcpy(out + p.off_combine, p.combine.data(), p.combine.size() * sizeof(CombineRow));
  if (!p.prefill.empty())
    std::memcpy(out + p.off_prefill, p.prefill.data(), p.prefill.size() * sizeof(PrefillItem));
  if (!p.order.empty()) std::memcpy(out + p.off_order, p.order.data(), p.order.size() * sizeof(int32_t));
}

int check_tensors(const void* q, const void* k_cache, const void* v_cache, void* o, float scale, const char* fn) {
  if (!q || !k_cache || !v_cache || !o) return fail(CB_ERR_INVALID_ARG, "%s: NULL tensor", fn);
  if (!(scale > 0.f) || !(scale < 3.0e38f)) return fail(CB_ERR_INVALID_ARG, "%s: scale must be positive and finite", fn);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(CB_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  return CB_OK;
}

// Workspace layout of cb_step_forward: the step metadata (cu_q_lens, ctx_lens,
// block_tables, then each packed row's cache slot), then the attention plan and partials at
// `plan_base`.
struct StepLayout {
  size_t off_cu = 0, off_ctx = 0, off_bt = 0, off_slots = 0, meta_bytes = 0, plan_base = 0;
};

// bt_entries: block-table entries staged (the compact table's length, or R * max_blocks).
StepLayout step_layout(int32_t R, int64_t bt_entries, int32_t T) {
  StepLayout l;
  l.off_cu = 0;
  l.off_ctx = static_cast<size_t>(R + 1) * 4;
  l.off_bt = l.off_ctx + static_cast<size_t>(R) * 4;
  l.off_slots = l.off_bt + static_cast<size_t>(bt_entries) * 4;
  l.meta_bytes = l.off_slots + static_cast<size_t>(std::max(T, 0)) * 4;
  l.plan_base = align256(l.meta_bytes);
  return l;
}

// Cache slot (block * block_size + offset) of every packed row, from the host metadata
// (the slot rule of cb_kv_append: row i of request r sits at position ctx_lens[r] + i).
// Block ids were checked against the pool before this is called.
void fill_slots(int32_t R, int32_t maxb, const int32_t* cu, const int32_t* ctx, const int32_t* bt, int32_t* out) {
  for (int32_t r = 0; r < R; ++r) {
    const int32_t* row = bt + static_cast<size_t>(r) * maxb;
    for (int32_t t = cu[r], p = ctx[r]; t < cu[r + 1]; ++t, ++p) out[t] = row[p / kBlockSize] * kBlockSize + p % kBlockSize;
  }
}

// Slots fit an int32 for every pool this library accepts in practice; larger pools keep the
// device-side lookup.
inline bool slots_fit(const cb_shape* s) { return s->num_blocks <= INT32_MAX / kBlockSize; }

// The step entry points stage a compact block table: request r's ceil((c + q) / bs) ids (none
// for a request with no rows) start at rows[r]. The padded [R, max_blocks] table of a long
// request beside many short ones is mostly padding (the decode-only workload: 2.1 MB staged
// per step, 0.2 MB of it block ids). Returns the entry count.
int64_t compact_rows(int32_t R, const int32_t* cu, const int32_t* ctx, std::vector<int32_t>& rows) {
  rows.resize(static_cast<size_t>(R));
  int64_t n = 0;
  for (int32_t r = 0; r < R; ++r) {
    rows[r] = static_cast<int32_t>(n);
    const int32_t q = cu[r + 1] - cu[r];
    if (q > 0) n += ceil_div(static_cast<int64_t>(ctx[r]) + q, kBlockSize);
  }
  return n;
}

void fill_compact(int32_t R, int32_t maxb, const int32_t* cu, const int32_t* ctx, const int32_t* bt,
                  const std::vector<int32_t>& rows, int32_t* out) {
  for (int32_t r = 0; r < R; ++r) {
    const int32_t q = cu[r + 1] - cu[r];
    if (q > 0)
      std::memcpy(out + rows[r], bt + static_cast<size_t>(r) * maxb,
                  static_cast<size_t>(ceil_div(static_cast<int64_t>(ctx[r]) + q, kBlockSize)) * 4);
  }
}

}  // namespace
}  // namespace cb

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
  return launch_attention(shape, batch, p, ws, q, k_cache, v_cache, scale, o, s);
}

// Every block id a row of the step can touch lies in the pool (host mirrors, checked before
// any upload).
static int check_block_ids(const cb_shape* shape, int32_t num_reqs, int32_t max_blocks_per_req,
                           const int32_t* h_cu_q_lens, const int32_t* h_ctx_lens, const int32_t* h_block_tables,
                           const char* fn) {
  if (!h_block_tables) return fail(CB_ERR_INVALID_ARG, "%s: block tables are required", fn);
  for (int32_t r = 0; r < num_reqs; ++r) {
    if (h_cu_q_lens[r + 1] == h_cu_q_lens[r]) continue;
    const int32_t nb = ceil_div(static_cast<int64_t>(h_ctx_lens[r]) + h_cu_q_lens[r + 1] - h_cu_q_lens[r], kBlockSize);
    const int32_t* row = h_block_tables + static_cast<size_t>(r) * max_blocks_per_req;
    for (int32_t j = 0; j < nb; ++j)
      if (row[j] < 0 || row[j] >= shape->num_blocks)
        return fail(CB_ERR_INVALID_ARG, "%s: block id %d of request %d out of range", fn, row[j], r);
  }
  return CB_OK;
}

// A cb_batch over host metadata whose device pointers point into the step workspace.
static cb_batch step_batch(int32_t R, int32_t T, int32_t maxb, const int32_t* h_cu, const int32_t* h_ctx,
                           char* ws, const StepLayout& l) {
  // a non-null placeholder lets the host-side checks run before the workspace is known
  char* base = ws ? ws : reinterpret_cast<char*>(uintptr_t{256});
  return cb_batch{R, T, maxb, reinterpret_cast<const int32_t*>(base + l.off_cu),
                  reinterpret_cast<const int32_t*>(base + l.off_ctx), reinterpret_cast<const int32_t*>(base + l.off_bt),
                  h_cu, h_ctx};
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

  // one upload: metadata, then the plan
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto fill = [&](char* host) {
    std::memcpy(host + l.off_cu, h_cu_q_lens, static_cast<size_t>(num_reqs + 1) * 4);
    std::memcpy(host + l.off_ctx, h_ctx_lens, static_cast<size_t>(num_reqs) * 4);
    if (slots) {
      fill_compact(num_reqs, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, h_block_tables, bt_rows,
                   reinterpret_cast<int32_t*>(host + l.off_bt));
      fill_slots(num_reqs, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, h_block_tables,
                 reinterpret_cast<int32_t*>(host + l.off_slots));
    } else {
      std::memcpy(host + l.off_bt, h_block_tables, static_cast<size_t>(num_reqs) * max_blocks_per_req * 4);
    }
    write_plan(p, host + l.plan_base);
  };
  AppendArgs aa{k_new, v_new, k_cache, v_cache, b.cu_q_lens, b.ctx_lens, b.block_tables, num_reqs, num_tokens,
                max_blocks_per_req, shape->num_kv_heads, shape->num_blocks, nullptr,
                slots ? reinterpret_cast<const int32_t*>(ws + l.off_slots) : nullptr, nullptr, nullptr, 0};
  const int eb = elem_bytes(shape);
  hipError_t e = hipSuccess;
  if (g_tuning.stage_kernel && slots) {
    // The append launch also moves the staged bytes into the workspace, and takes its slots
    // straight from the pinned buffer: one kernel fewer per step.
    st = upload_with(l.plan_base + p.plan_bytes, s, fill, [&](const void* src_dev, const void*, size_t n) {
      aa.slots = reinterpret_cast<const int32_t*>(static_cast<const char*>(src_dev) + l.off_slots);
      aa.stage_src = src_dev;
      aa.stage_dst = ws;
      aa.stage_n16 = static_cast<int64_t>(n / 16);
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
  return launch_attention(shape, &b, p, ws + l.plan_base, q, k_cache, v_cache, scale, o, s);
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

// ---- captured steps ---------------------------------------------------------------------
// Hugging Face blog "Continuous batching from first principles", section "Continuous
// batching": graph capture (CUDA graphs, torch.compile) needs static tensor shapes, which a
// batch axis can only meet by padding every prompt to a fixed length. A captured step here
// keeps its buffers static instead: the caller's packed buffers hold up to max_tokens rows
// (the bucket), the workspace and staging buffers have fixed addresses, and the live sizes
// and work lists travel in the step header (StepDesc) that the replayed stage copy moves into
// the workspace. Before a replay, each kernel node's grid is set to the step's live count,
// so a replay launches no padded work.
namespace cb {
namespace {
enum GraphNode { kNodeStage = 0, kNodeAppend, kNodePrefill, kNodeDecode, kNodeCombine, kNodeCount };
}  // namespace
}  // namespace cb

struct cb_graph {
  cb_shape shape{};
  int32_t max_tokens = 0;
  const void* q = nullptr;
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  void* k_cache = nullptr;
  void* v_cache = nullptr;
  void* o = nullptr;
  float scale = 1.f;
  int device = 0;
  // what the current graphs were captured for
  bool captured = false;
  size_t cap_stage = 0, ws_bytes = 0;
  int prefill_waves = 0, group = 1, touch = 0;
  bool mfma_decode = false;
  void* ws = nullptr;                       // device workspace, owned
  struct Slot {                             // pinned staging buffer and the graph that reads it
    void* host = nullptr;
    void* host_dev = nullptr;
    size_t cap = 0;
    hipGraph_t graph = nullptr;             // kept: its kernel nodes are updated before replays
    hipGraphExec_t exec = nullptr;
    hipGraphNode_t node[cb::kNodeCount] = {};
    hipKernelNodeParams params[cb::kNodeCount] = {};
    hipEvent_t done = nullptr;
    bool in_flight = false;
  } slot[2];
  int next = 0;
  hipStream_t cap_stream = nullptr;
  int64_t replays = 0, captures = 0;
};

namespace cb {
namespace {

// Pinned staging buffers that a replay may have read: kept until the process ends, as the
// eager upload ring keeps its outgrown buffers.
std::mutex g_graph_retired_mu;
std::vector<void*> g_graph_retired;

void retire_pinned(void* p) {
  if (!p) return;
  std::lock_guard<std::mutex> lk(g_graph_retired_mu);
  g_graph_retired.push_back(p);
}

// Byte layout of a replayed step: header, metadata, then the plan at plan_base (plan offsets
// are relative to it). The stage copy moves [0, stage_bytes).
struct GraphLayout {
  size_t off_cu = 0, off_ctx = 0, off_bt = 0, off_slots = 0, plan_base = 0, stage_bytes = 0, total = 0;
};

GraphLayout graph_layout(int32_t R, int64_t bt_entries, int32_t T, const Plan& p) {
  GraphLayout l;
  l.off_cu = kDescBytes;
  l.off_ctx = l.off_cu + static_cast<size_t>(R + 1) * 4;
  l.off_bt = l.off_ctx + static_cast<size_t>(R) * 4;
  l.off_slots = l.off_bt + static_cast<size_t>(bt_entries) * 4;
  l.plan_base = align256(l.off_slots + static_cast<size_t>(T) * 4);
  l.stage_bytes = (l.plan_base + p.plan_bytes + 15) & ~size_t{15};
  l.total = std::max(l.plan_base + p.total, l.stage_bytes);
  return l;
}

// Buffer capacities at least double when a step outgrows them, so a trace whose steps keep
// growing (contexts lengthen, block tables widen) is captured again only a logarithmic
// number of times; each new capture waits for the replays in flight.
inline size_t grow_size(size_t need, size_t have) { return align256(std::max(2 * have, need + need / 2 + 4096)); }

void graph_wait_all(cb_graph* g) {
  for (auto& sl : g->slot)
    if (sl.in_flight) {
      hipEventSynchronize(sl.done);
      sl.in_flight = false;
    }
}

void graph_release(cb_graph::Slot& sl) {
  if (sl.exec) hipGraphExecDestroy(sl.exec);
  if (sl.graph) hipGraphDestroy(sl.graph);
  sl.exec = nullptr;
  sl.graph = nullptr;
  for (auto& n : sl.node) n = nullptr;
}

// Kernel nodes of a captured chain, in capture order.
int chain_nodes(hipGraph_t graph, std::vector<hipGraphNode_t>& out) {
  out.clear();
  size_t n = 1;
  hipGraphNode_t node = nullptr;
  if (hipGraphGetRootNodes(graph, &node, &n) != hipSuccess || n != 1)
    return fail(CB_ERR_HIP, "cb_graph_step: captured step is not a single chain");
  while (node) {
    hipGraphNodeType type;
    if (hipGraphNodeGetType(node, &type) != hipSuccess || type != hipGraphNodeTypeKernel)
      return fail(CB_ERR_HIP, "cb_graph_step: captured step holds a node that is not a kernel");
    out.push_back(node);
    hipGraphNode_t next = nullptr;
    size_t m = 0;
    if (hipGraphNodeGetDependentNodes(node, nullptr, &m) != hipSuccess || m > 1)
      return fail(CB_ERR_HIP, "cb_graph_step: captured step is not a single chain");
    if (m == 1 && hipGraphNodeGetDependentNodes(node, &next, &m) != hipSuccess)
      return fail(CB_ERR_HIP, "cb_graph_step: could not walk the captured step");
    node = m == 1 ? next : nullptr;
  }
  return CB_OK;
}

// Captures one graph per staging slot: stage copy, append, prefill tiles (bf16), decode
// rows and combine, every kernel reading the step header. Launch grids at capture are
// placeholders; cb_graph_step sets them per replay. Replays in flight
// finish first: the workspace and graphs are replaced.
int graph_capture(cb_graph* g, const Plan& p, const GraphLayout& l) {
  graph_wait_all(g);
  g->captured = false;                      // until every slot holds a complete graph again
  g->cap_stage = grow_size(l.stage_bytes, g->cap_stage);
  const size_t bytes = grow_size(std::max(l.total, g->cap_stage), g->ws_bytes);
  if (g->ws) hipFree(g->ws);
  g->ws = nullptr;
  g->ws_bytes = 0;
  if (hipMalloc(&g->ws, bytes) != hipSuccess) return fail(CB_ERR_HIP, "cb_graph_step: hipMalloc(%zu) failed", bytes);
  g->ws_bytes = bytes;
  g->prefill_waves = p.prefill_waves;
  g->mfma_decode = p.mfma_decode;
  g->group = p.group;
  g->touch = g_tuning.prefill_touch;

  const cb_shape* sh = &g->shape;
  const int eb = elem_bytes(sh);
  const bool prefill = sh->dtype == CB_BF16;          // fp32 prefill rows take the split-K path
  const bool fused = slots_fit(sh);                   // staging copy inside the append node
  const float scale_log2 = static_cast<float>(static_cast<double>(g->scale) * kLog2e);
  const StepDesc* desc = static_cast<const StepDesc*>(g->ws);
  for (auto& sl : g->slot) {
    graph_release(sl);
    if (sl.cap < g->cap_stage) {
      retire_pinned(sl.host);
      sl.host = sl.host_dev = nullptr;
      sl.cap = 0;
      // coherent: the replayed stage copy reads what the host wrote before the launch
      if (hipHostMalloc(&sl.host, g->cap_stage, hipHostMallocCoherent) != hipSuccess)
        return fail(CB_ERR_HIP, "cb_graph_step: hipHostMalloc(%zu) failed", g->cap_stage);
      if (hipHostGetDevicePointer(&sl.host_dev, sl.host, 0) != hipSuccess)
        return fail(CB_ERR_HIP, "cb_graph_step: hipHostGetDevicePointer failed");
      sl.cap = g->cap_stage;
    }
    hipStream_t cs = g->cap_stream;
    if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess)
      return fail(CB_ERR_HIP, "cb_graph_step: hipStreamBeginCapture failed");
    // With per-row slots (any pool up to 2^31 / 16 blocks) the append node also moves the
    // staged bytes: it reads the header and its slots from the pinned buffer and copies the
    // rest into the workspace, as cb_step_forward's append does. Otherwise a copy node
    // (bound: the capacity, an argument; grid set per replay) precedes it.
    hipError_t e = hipSuccess;
    AppendArgs aa{g->k_new, g->v_new, g->k_cache, g->v_cache, nullptr, nullptr, nullptr, 0, 1, 0,
                  sh->num_kv_heads, sh->num_blocks, desc};
    if (fused) {
      aa.desc = static_cast<const StepDesc*>(sl.host_dev);
      aa.stage_src = sl.host_dev;
      aa.stage_dst = g->ws;
      aa.stage_n16 = -static_cast<int64_t>(g->cap_stage / 16);
    } else {
      e = launch_stage_copy_desc(sl.host_dev, g->ws, g->cap_stage, cs);
    }
    if (e == hipSuccess) e = launch_kv_append(aa, eb, sh->head_dim, cs);
    if (e == hipSuccess && prefill) {
      PrefillArgs pa{g->q, g->k_cache, g->v_cache, g->o, nullptr, nullptr, nullptr, nullptr, 1,
                     sh->num_q_heads, sh->num_kv_heads, 0, sh->num_blocks, scale_log2, g->touch, desc};
      e = launch_prefill(pa, sh->head_dim, g->prefill_waves, cs);
    }
    if (e == hipSuccess) {
      RowArgs ra{g->q, g->k_cache, g->v_cache, g->o, nullptr, nullptr, nullptr, nullptr, 1,
                 sh->num_q_heads, sh->num_kv_heads, 0, sh->num_blocks, scale_log2, g->group, desc};
      e = g->mfma_decode ? launch_rows_mfma(ra, sh->head_dim, cs) : launch_rows(ra, eb, sh->head_dim, g->group, cs);
    }
    if (e == hipSuccess) {
      CombineArgs ca{g->o, nullptr, nullptr, nullptr, 1, sh->num_q_heads, desc};
      e = launch_combine(ca, eb, sh->head_dim, cs);
    }
    const hipError_t ec = hipStreamEndCapture(cs, &sl.graph);
    if (e != hipSuccess || ec != hipSuccess)
      return fail(CB_ERR_HIP, "cb_graph_step: capture failed: %s", hipGetErrorString(e != hipSuccess ? e : ec));
    std::vector<hipGraphNode_t> chain;
    int st = chain_nodes(sl.graph, chain);
    if (st) return st;
    const int kinds[] = {kNodeStage, kNodeAppend, kNodePrefill, kNodeDecode, kNodeCombine};
    std::vector<int> order;
    for (int k : kinds)
      if ((k != kNodePrefill || prefill) && (k != kNodeStage || !fused)) order.push_back(k);
    if (chain.size() != order.size())
      return fail(CB_ERR_HIP, "cb_graph_step: captured %zu kernels, expected %zu", chain.size(), order.size());
    for (size_t i = 0; i < chain.size(); ++i) {
      sl.node[order[i]] = chain[i];
      if (hipGraphKernelNodeGetParams(chain[i], &sl.params[order[i]]) != hipSuccess)
        return fail(CB_ERR_HIP, "cb_graph_step: could not read a kernel node");
    }
    e = hipGraphInstantiate(&sl.exec, sl.graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
      sl.exec = nullptr;
      return fail(CB_ERR_HIP, "cb_graph_step: hipGraphInstantiate failed: %s", hipGetErrorString(e));
    }
  }
  g->captured = true;
  ++g->captures;
  return CB_OK;
}

// Sets the grid of kernel node k of slot `sl` (unchanged grids are not set again).
int set_grid(cb_graph::Slot& sl, int k, dim3 grid) {
  if (!sl.node[k]) return CB_OK;
  hipKernelNodeParams& prm = sl.params[k];
  if (prm.gridDim.x == grid.x && prm.gridDim.y == grid.y && prm.gridDim.z == grid.z) return CB_OK;
  prm.gridDim = grid;
  if (hipGraphExecKernelNodeSetParams(sl.exec, sl.node[k], &prm) != hipSuccess)
    return fail(CB_ERR_HIP, "cb_graph_step: could not set a kernel node's grid");
  return CB_OK;
}

}  // namespace
}  // namespace cb

extern "C" int cb_graph_create(const cb_shape* shape, int32_t max_tokens, const void* q, const void* k_new,
                               const void* v_new, void* k_cache, void* v_cache, float scale, void* o, cb_graph** out) {
  if (!out) return fail(CB_ERR_INVALID_ARG, "cb_graph_create: out is NULL");
  *out = nullptr;
  int st = check_shape(shape);
  if (st) return st;
  if (max_tokens < 1) return fail(CB_ERR_INVALID_ARG, "cb_graph_create: max_tokens must be >= 1");
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))
    return fail(CB_ERR_INVALID_ARG, "cb_graph_create: new K/V must be non-NULL and 16-byte aligned");
  if ((st = check_tensors(q, k_cache, v_cache, o, scale, "cb_graph_create"))) return st;
  cb_graph* g = new cb_graph();
  g->shape = *shape;
  g->max_tokens = max_tokens;
  g->q = q;
  g->k_new = k_new;
  g->v_new = v_new;
  g->k_cache = k_cache;
  g->v_cache = v_cache;
  g->o = o;
  g->scale = scale;
  bool ok = hipGetDevice(&g->device) == hipSuccess &&
            hipStreamCreateWithFlags(&g->cap_stream, hipStreamNonBlocking) == hipSuccess;
  for (auto& sl : g->slot)
    ok = ok && hipEventCreateWithFlags(&sl.done, hipEventDisableTiming | hipEventDisableSystemFence) == hipSuccess;
  if (!ok) {
    cb_graph_destroy(g);
    return fail(CB_ERR_HIP, "cb_graph_create: could not create the capture stream or events");
  }
  *out = g;
  return CB_OK;
}

extern "C" int cb_graph_step(cb_graph* g, int32_t num_reqs, int32_t num_tokens, int32_t max_blocks_per_req,
                             const int32_t* h_cu_q_lens, const int32_t* h_ctx_lens, const int32_t* h_block_tables,
                             void* stream) {
  if (!g) return fail(CB_ERR_INVALID_ARG, "cb_graph_step: graph is NULL");
  if (num_reqs < 0 || max_blocks_per_req < 0) return fail(CB_ERR_INVALID_ARG, "cb_graph_step: negative count");
  if (num_tokens > g->max_tokens)
    return fail(CB_ERR_INVALID_ARG, "cb_graph_step: %d rows exceed the graph's %d", num_tokens, g->max_tokens);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != g->device)
    return fail(CB_ERR_INVALID_ARG, "cb_graph_step: the graph belongs to device %d, current is %d", g->device, dev);
  const cb_shape* sh = &g->shape;
  const StepLayout host_l = step_layout(num_reqs, 0, num_tokens);
  cb_batch b = step_batch(num_reqs, num_tokens, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, nullptr, host_l);
  int st = check_batch(sh, &b);
  if (st) return st;
  if (num_tokens == 0) return CB_OK;
  if ((st = check_block_ids(sh, num_reqs, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, h_block_tables,
                            "cb_graph_step")))
    return st;
  const bool slots = slots_fit(sh);           // with slots, the compact block table (as cb_step_forward)
  std::vector<int32_t> bt_rows;
  const int64_t nbt = slots ? compact_rows(num_reqs, h_cu_q_lens, h_ctx_lens, bt_rows)
                            : static_cast<int64_t>(num_reqs) * max_blocks_per_req;
  Plan p;
  make_plan(sh, &b, p, g->captured ? g->prefill_waves : 0, false, slots ? bt_rows.data() : nullptr);
  const GraphLayout l = graph_layout(num_reqs, nbt, num_tokens, p);
  const bool fits = g->captured && l.stage_bytes <= g->cap_stage && l.total <= g->ws_bytes &&
                    p.mfma_decode == g->mfma_decode && p.group == g->group && g_tuning.prefill_touch == g->touch;
  if (!fits && (st = graph_capture(g, p, l))) return st;

  cb_graph::Slot& sl = g->slot[g->next];
  if (sl.in_flight) {
    if (hipEventSynchronize(sl.done) != hipSuccess) return fail(CB_ERR_HIP, "cb_graph_step: event wait failed");
    sl.in_flight = false;
  }
  // live grids (a kind of work with no items keeps one work-group, which finds a zero count)
  const int32_t n_rows = static_cast<int32_t>(p.splits.size()) * sh->num_kv_heads * p.n_sub;
  const int32_t n_comb = static_cast<int32_t>(p.combine.size());
  const int32_t n_pre = static_cast<int32_t>(p.prefill.size());
  const int64_t n16 = static_cast<int64_t>(l.stage_bytes / 16);
  auto blocks = [](int64_t n, int64_t per) { return static_cast<unsigned>(std::max<int64_t>(1, (n + per - 1) / per)); };
  if ((st = set_grid(sl, kNodeStage, dim3(std::min(blocks(n16, 256), 1024u)))) ||
      (st = set_grid(sl, kNodeAppend, dim3(blocks(num_tokens, 16), blocks(sh->num_kv_heads, 4)))) ||
      (st = set_grid(sl, kNodePrefill, dim3(blocks(n_pre, 1)))) ||
      (st = set_grid(sl, kNodeDecode, dim3(blocks(n_rows, 4)))) ||
      (st = set_grid(sl, kNodeCombine, dim3(blocks(static_cast<int64_t>(n_comb) * sh->num_q_heads, 4)))))
    return st;

  char* host = static_cast<char*>(sl.host);
  StepDesc d{};
  d.stage_bytes = static_cast<int64_t>(l.stage_bytes);
  d.num_reqs = num_reqs;
  d.num_tokens = num_tokens;
  d.max_blocks = max_blocks_per_req;
  d.n_row_items = n_rows;
  d.n_combine_rows = n_comb;
  d.n_prefill = n_pre;
  d.off_cu = static_cast<int64_t>(l.off_cu);
  d.off_ctx = static_cast<int64_t>(l.off_ctx);
  d.off_bt = static_cast<int64_t>(l.off_bt);
  d.off_splits = static_cast<int64_t>(l.plan_base);
  d.off_combine = static_cast<int64_t>(l.plan_base + p.off_combine);
  d.off_prefill = static_cast<int64_t>(l.plan_base + p.off_prefill);
  d.off_part_o = static_cast<int64_t>(l.plan_base + p.off_part_o);
  d.off_part_ml = static_cast<int64_t>(l.plan_base + p.off_part_ml);
  d.off_slots = slots ? static_cast<int64_t>(l.off_slots) : 0;
  std::memcpy(host, &d, sizeof(d));
  std::memcpy(host + l.off_cu, h_cu_q_lens, static_cast<size_t>(num_reqs + 1) * 4);
  std::memcpy(host + l.off_ctx, h_ctx_lens, static_cast<size_t>(num_reqs) * 4);
  if (slots) {
    fill_compact(num_reqs, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, h_block_tables, bt_rows,
                 reinterpret_cast<int32_t*>(host + l.off_bt));
    fill_slots(num_reqs, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, h_block_tables,
               reinterpret_cast<int32_t*>(host + l.off_slots));
  } else {
    std::memcpy(host + l.off_bt, h_block_tables, static_cast<size_t>(num_reqs) * max_blocks_per_req * 4);
  }
  write_plan(p, host + l.plan_base);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipGraphLaunch(sl.exec, s);
  if (e != hipSuccess) return fail(CB_ERR_HIP, "cb_graph_step: hipGraphLaunch failed: %s", hipGetErrorString(e));
  if (hipEventRecord(sl.done, s) != hipSuccess) return fail(CB_ERR_HIP, "cb_graph_step: event record failed");
  sl.in_flight = true;
  g->next ^= 1;
  ++g->replays;
  return CB_OK;
}

extern "C" int cb_graph_stats(const cb_graph* g, int64_t* replays, int64_t* captures, size_t* workspace_bytes) {
  if (!g) return fail(CB_ERR_INVALID_ARG, "cb_graph_stats: graph is NULL");
  if (replays) *replays = g->replays;
  if (captures) *captures = g->captures;
  if (workspace_bytes) *workspace_bytes = g->ws_bytes;
  return CB_OK;
}

extern "C" void cb_graph_destroy(cb_graph* g) {
  if (!g) return;
  graph_wait_all(g);
  for (auto& sl : g->slot) {
    graph_release(sl);
    if (sl.done) hipEventDestroy(sl.done);
    retire_pinned(sl.host);
  }
  if (g->ws) hipFree(g->ws);
  if (g->cap_stream) hipStreamDestroy(g->cap_stream);
  delete g;
}
