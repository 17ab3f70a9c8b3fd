// Host-side declarations shared by the library's host translation units (no device code):
// the kernel launchers of the .hip files, tuning knobs, argument checks, the launch planner
// and the layouts a step stages into its workspace.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "cb.h"
#include "cb_common.h"
#include "cb_plan.h"

namespace cb {

hipError_t launch_kv_append(const AppendArgs& a, int elem_bytes, int head_dim, hipStream_t s);
// Grid of kv_append_kernel for num_tokens rows (256-thread work-groups); launch_kv_append and
// the captured step both take it from here.
dim3 append_grid(int64_t num_tokens, int32_t num_kv_heads, int elem_bytes, int head_dim, int32_t n_marked = 0);
// The paged-read probe (probe.hip): work-groups for n_pages, and its launch.
int32_t paged_read_grid(int32_t n_pages);
hipError_t launch_paged_read(const void* pages, int32_t n_pages, const int32_t* order, uint32_t* sink,
                             hipStream_t s);
hipError_t launch_rows(const RowArgs& a, int elem_bytes, int head_dim, int group, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int elem_bytes, int head_dim, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int waves, hipStream_t s);
hipError_t launch_rows_mfma(const RowArgs& a, int head_dim, hipStream_t s);
hipError_t launch_stage_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
hipError_t launch_stage_copy_desc(const void* src, void* dst, size_t max_bytes, hipStream_t s);
hipError_t launch_gemm(const GemmArgs& g, int epilogue, hipStream_t s);
hipError_t launch_mixed(const MixedArgs& a, int head_dim, hipStream_t s);

constexpr double kLog2e = 1.4426950408889634;

#ifdef CB_DEVICE_CHECKS
// The violation counters of the kernel sources (debug copy only): each adds its count to
// *sum, and zeroes it when `reset`.
hipError_t violations_rows(uint32_t* sum, bool reset);
hipError_t violations_decode_gqa(uint32_t* sum, bool reset);
hipError_t violations_prefill(uint32_t* sum, bool reset);
hipError_t violations_mixed(uint32_t* sum, bool reset);
hipError_t violations_append(uint32_t* sum, bool reset);
hipError_t violations_gemm(uint32_t* sum, bool reset);
#endif

// ---- tuning -----------------------------------------------------------------------------
struct Tuning {
  int32_t split_blocks = 0;       // 0 = automatic
  int32_t target_waves = 0;       // 0: 8192 wave items (vector-ALU decode), 4096 (matrix-core decode)
  int32_t overlap_prefill = 0;    // 1 = run prefill tiles on a side stream beside decode rows
  int32_t xcds = 8;               // XCDs that work-groups are dispatched over (MI355X: 8)
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
  int32_t decode_order = 1;       // 1: decode splits longest first; 0: rows longest first
  int32_t prefill_heads = 0;      // query heads per bf16 prefill work-group (one kv head's;
                                  // 0 = automatic)
  int32_t mixed_order = 0;        // 0: merge prefill and decode chunks in proportion to their
                                  // counts; 1: alternate them until one kind runs out
};
extern Tuning g_tuning;

// ---- argument checks (plan.cpp) -----------------------------------------------------------
inline int elem_bytes(const cb_shape* s) { return s->dtype == CB_BF16 ? 2 : 4; }
inline int32_t ceil_div(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int check_shape(const cb_shape* s);
int check_batch(const cb_shape* s, const cb_batch* b);
int check_tensors(const void* q, const void* k_cache, const void* v_cache, void* o, float scale, const char* fn);
// Every block id a row of the step can touch lies in the pool (host mirrors, checked before
// any upload).
int check_block_ids(const cb_shape* shape, int32_t num_reqs, int32_t max_blocks_per_req, const int32_t* h_cu_q_lens,
                    const int32_t* h_ctx_lens, const int32_t* h_block_tables, const char* fn);

// ---- the launch plan (plan.cpp) ------------------------------------------------------------
inline size_t align256(size_t x) { return (x + 255) & ~size_t{255}; }

struct Plan {
  std::vector<RowSplit> splits;
  std::vector<CombineRow> combine;
  std::vector<PrefillItem> prefill;
  int32_t n_parts = 0;
  int group = 1;         // query heads per decode wave
  bool mfma_decode = false;  // decode rows on the MFMA kernel
  int prefill_waves = 4;     // waves (x 32 query rows) per prefill work-group
  int prefill_heads_log2 = 0;  // query heads per prefill work-group (log2); rows = 32 waves / heads
  int n_sub = 1;         // decode waves per kv head
  int32_t split_blocks = 0;  // split length chosen for the split-K rows
  bool mixed = false;    // prefill tiles and decode waves in one launch (order below)
  std::vector<int32_t> order;
  size_t off_combine = 0, off_prefill = 0, off_order = 0, plan_bytes = 0, off_part_o = 0, off_part_ml = 0,
         total = 0;
};

// Builds the work lists of one step from its host mirrors. force_waves (4 or 8) fixes the
// prefill work-group size; 0 takes the tuning / automatic choice. allow_mixed = false keeps
// prefill and decode in separate launches (captured steps). bt_rows (host, [num_reqs],
// nullable): where each request's block ids start in the device block table; null means the
// padded [num_reqs, max_blocks_per_req] layout of cb_batch.
void make_plan(const cb_shape* s, const cb_batch* b, Plan& p, int force_waves = 0, bool allow_mixed = true,
               const int32_t* bt_rows = nullptr);
// Serialises the plan's work lists at their offsets into `out` (plan_bytes long).
void write_plan(const Plan& p, char* out);
// Launches the attention kernels of plan `p` on stream `s`; its work lists are already at
// `ws` (device), and its partials go to `ws` + the plan's partial offsets. With
// allow_side_stream and the "overlap_prefill" knob, the prefill kernel runs on the library's
// side stream (created on first use) and is joined back before the combine pass.
int launch_attention(const cb_shape* shape, const cb_batch* batch, const Plan& p, char* ws, const void* q,
                     const void* k_cache, const void* v_cache, float scale, void* o, hipStream_t s,
                     bool allow_side_stream);

// ---- step layouts (plan.cpp) ---------------------------------------------------------------
// Workspace layout of cb_step_forward: the step metadata (cu_q_lens, ctx_lens, the block
// ids, then each packed row's cache slot), then the attention plan and partials at
// `plan_base`.
struct StepLayout {
  size_t off_cu = 0, off_ctx = 0, off_bt = 0, off_slots = 0, meta_bytes = 0, plan_base = 0;
};

// bt_entries: block-table entries staged (the compact table's length, or R * max_blocks).
StepLayout step_layout(int32_t R, int64_t bt_entries, int32_t T);
// Cache slot of every packed row from the host metadata; with `mark`, rows that are the only
// row of the step writing into their block also carry kSlotSoleWriter, and `marked` (room for
// 2 * T values, or null) receives their (row, slot) pairs. Returns the number of marked rows.
int32_t fill_slots(int32_t R, int32_t maxb, const int32_t* cu, const int32_t* ctx, const int32_t* bt, int32_t* out,
                   bool mark, int32_t* marked = nullptr);
// Slots fit an int32 for every pool this library accepts in practice; larger pools keep the
// device-side lookup.
inline bool slots_fit(const cb_shape* s) { return s->num_blocks <= INT32_MAX / kBlockSize; }
// Whether a step's slots carry sole-writer marks: the bit must stay clear of every slot value
// (pools up to 2^26 blocks), and the step must hold decode rows only. With prefill rows a
// prefill kernel runs between the append and the decode rows, and the partly written lines
// of element-wise V^T writes are merged under it at no measured cost (the whole-page
// rewrites then only add work: the trace replay 0.6071 -> 0.6085 ms per step).
inline bool sole_marks_apply(const cb_shape* s, int32_t R, const int32_t* cu) {
  if (s->num_blocks > kSlotSoleWriter / kBlockSize) return false;
  for (int32_t r = 0; r < R; ++r)
    if (cu[r + 1] - cu[r] > 1) return false;
  return true;
}
// Offsets of each request's block ids in the compact table; returns the entry count.
int64_t compact_rows(int32_t R, const int32_t* cu, const int32_t* ctx, std::vector<int32_t>& rows);
void fill_compact(int32_t R, int32_t maxb, const int32_t* cu, const int32_t* ctx, const int32_t* bt,
                  const std::vector<int32_t>& rows, int32_t* out);
// A cb_batch over host metadata whose device pointers point into the step workspace.
cb_batch step_batch(int32_t R, int32_t T, int32_t maxb, const int32_t* h_cu, const int32_t* h_ctx, char* ws,
                    const StepLayout& l);

}  // namespace cb
