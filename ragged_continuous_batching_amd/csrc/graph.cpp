// Captured steps (cb_graph_*): a whole step as a HIP graph with static buffers and live
// sizes in a device-side step header. Host code only.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "host.h"

using namespace cb;

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
  int prefill_waves = 0, group = 1;
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
// are relative to it). The stage copy moves [0, stage_bytes); the marked rows' (row, slot)
// pairs follow in the pinned buffer only (pinned_bytes), read there by the append node.
struct GraphLayout {
  size_t off_cu = 0, off_ctx = 0, off_bt = 0, off_slots = 0, plan_base = 0, stage_bytes = 0, total = 0;
  size_t pinned_bytes = 0;
};

GraphLayout graph_layout(int32_t R, int64_t bt_entries, int32_t T, const Plan& p) {
  GraphLayout l;
  l.off_cu = kDescBytes;
  l.off_ctx = l.off_cu + static_cast<size_t>(R + 1) * 4;
  l.off_bt = l.off_ctx + static_cast<size_t>(R) * 4;
  l.off_slots = l.off_bt + static_cast<size_t>(bt_entries) * 4;
  l.plan_base = align256(l.off_slots + static_cast<size_t>(T) * 4);
  l.stage_bytes = (l.plan_base + p.plan_bytes + 15) & ~size_t{15};
  l.pinned_bytes = l.stage_bytes + static_cast<size_t>(T) * 8;
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
  g->cap_stage = grow_size(l.pinned_bytes, g->cap_stage);
  const size_t bytes = grow_size(std::max(l.total, g->cap_stage), g->ws_bytes);
  if (g->ws) hipFree(g->ws);
  g->ws = nullptr;
  g->ws_bytes = 0;
  if (hipMalloc(&g->ws, bytes) != hipSuccess) return fail(CB_ERR_HIP, "cb_graph_step: hipMalloc(%zu) failed", bytes);
  g->ws_bytes = bytes;
  g->prefill_waves = p.prefill_waves;
  g->mfma_decode = p.mfma_decode;
  g->group = p.group;

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
                     sh->num_q_heads, sh->num_kv_heads, 0, sh->num_blocks, scale_log2, desc};
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
  const bool marks = slots && sole_marks_apply(sh, num_reqs, h_cu_q_lens);
  std::vector<int32_t> bt_rows;
  const int64_t nbt = slots ? compact_rows(num_reqs, h_cu_q_lens, h_ctx_lens, bt_rows)
                            : static_cast<int64_t>(num_reqs) * max_blocks_per_req;
  Plan p;
  make_plan(sh, &b, p, g->captured ? g->prefill_waves : 0, false, slots ? bt_rows.data() : nullptr);
  const GraphLayout l = graph_layout(num_reqs, nbt, num_tokens, p);
  const bool fits = g->captured && l.pinned_bytes <= g->cap_stage && l.total <= g->ws_bytes &&
                    p.mfma_decode == g->mfma_decode && p.group == g->group;
  if (!fits && (st = graph_capture(g, p, l))) return st;

  cb_graph::Slot& sl = g->slot[g->next];
  if (sl.in_flight) {
    if (hipEventSynchronize(sl.done) != hipSuccess) return fail(CB_ERR_HIP, "cb_graph_step: event wait failed");
    sl.in_flight = false;
  }
  char* host = static_cast<char*>(sl.host);
  int32_t n_marked = 0;
  if (slots)
    n_marked = fill_slots(num_reqs, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, h_block_tables,
                          reinterpret_cast<int32_t*>(host + l.off_slots), marks,
                          marks ? reinterpret_cast<int32_t*>(host + l.stage_bytes) : nullptr);
  // live grids (a kind of work with no items keeps one work-group, which finds a zero count)
  const int32_t n_rows = static_cast<int32_t>(p.splits.size()) * sh->num_kv_heads * p.n_sub;
  const int32_t n_comb = static_cast<int32_t>(p.combine.size());
  const int32_t n_pre = static_cast<int32_t>(p.prefill.size());
  const int64_t n16 = static_cast<int64_t>(l.stage_bytes / 16);
  auto blocks = [](int64_t n, int64_t per) { return static_cast<unsigned>(std::max<int64_t>(1, (n + per - 1) / per)); };
  if ((st = set_grid(sl, kNodeStage, dim3(std::min(blocks(n16, 256), 1024u)))) ||
      (st = set_grid(sl, kNodeAppend, append_grid(num_tokens, sh->num_kv_heads, elem_bytes(sh), sh->head_dim,
                                                  n_marked))) ||
      (st = set_grid(sl, kNodePrefill, dim3(blocks(n_pre, 1)))) ||
      (st = set_grid(sl, kNodeDecode, dim3(blocks(n_rows, 4)))) ||
      (st = set_grid(sl, kNodeCombine, dim3(blocks(static_cast<int64_t>(n_comb) * sh->num_q_heads, 4)))))
    return st;

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
  d.off_marked = static_cast<int64_t>(l.stage_bytes);
  d.n_marked = n_marked;
  d.sole_bit = marks ? kSlotSoleWriter : 0;
  std::memcpy(host, &d, sizeof(d));
  std::memcpy(host + l.off_cu, h_cu_q_lens, static_cast<size_t>(num_reqs + 1) * 4);
  std::memcpy(host + l.off_ctx, h_ctx_lens, static_cast<size_t>(num_reqs) * 4);
  if (slots) {
    fill_compact(num_reqs, max_blocks_per_req, h_cu_q_lens, h_ctx_lens, h_block_tables, bt_rows,
                 reinterpret_cast<int32_t*>(host + l.off_bt));
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
