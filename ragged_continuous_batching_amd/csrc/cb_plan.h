// Work descriptors that the host planner writes into the workspace and the kernels read.
// Plain structs of int32 so that host and device agree on the layout byte for byte.
#pragma once

#include <cstdint>

namespace cb {

// One split of one single-row attention (a decode row, or any row of an fp32 prefill):
// keys [blk_begin*bs, min(blk_end*bs, kv_len)) of the row's request, for packed row `token`;
// the request's block ids start at block_tables[bt_row]. part < 0: the row has one split
// and the kernel writes O directly; otherwise the split's unnormalised output and
// (max, sum) go to partial slot `part` and a combine pass merges.
struct RowSplit {
  int32_t token;
  int32_t bt_row;
  int32_t blk_begin;
  int32_t blk_end;
  int32_t kv_len;
  int32_t part;
};

// A row with more than one split: partial slots part_begin .. part_begin+n_parts-1.
struct CombineRow {
  int32_t token;
  int32_t part_begin;
  int32_t n_parts;
  int32_t pad;
};

// One tile of a prefill chunk: rows q_begin .. q_begin+R-1 of request `req` and query heads
// head .. head + 2^heads_log2 - 1 (all of one kv head), key tiles kt_begin .. kt_end-1 (64
// keys each). The work-group's waves split into 2^heads_log2 heads x R/32 row blocks of 32,
// so R = 32 x waves / 2^heads_log2, clipped to the request's rows; every wave reads the same
// key/value tiles. req < 0 marks an empty slot. part_base < 0: the item
// walks all of its rows' keys and writes O. Otherwise it is split `split & 0xffff` of
// `split >> 16` over the key range: row i of the tile writes its unnormalised output and
// (max, sum) to partial slot part_base + i * (split >> 16) + (split & 0xffff), and the combine
// pass merges them. Every split boundary lies at or below the first row's last key, so each
// row sees at least one key of every split.
struct PrefillItem {
  int32_t req;
  int32_t q_begin;
  int32_t head;
  int32_t bt_row;       // the request's block ids start at block_tables[bt_row]
  int32_t kt_begin;
  int32_t kt_end;
  int32_t part_base;
  int32_t split;
  int32_t heads_log2;   // query heads per work-group, log2 (0: one head)
};

// Header at the start of a captured step's workspace (cb_graph_*). The host writes it into
// the staging slot ahead of the step's metadata and work lists. The replayed stage copy
// reads `stage_bytes` from it, and every replayed kernel reads its sizes and its arrays
// (offsets in bytes from this header) here rather than from launch arguments, whose grids
// are sized for the graph's capacity: work-groups past the live count exit at once.
struct StepDesc {
  int64_t stage_bytes;          // bytes the stage copy moves, this header included (x16)
  int32_t num_reqs, num_tokens, max_blocks;
  int32_t n_row_items;          // decode waves (RowArgs::n_items)
  int32_t n_combine_rows;       // rows merged by the combine pass
  int32_t n_prefill;            // prefill work-groups, empty launch-order slots included
  int64_t off_cu, off_ctx, off_bt, off_splits, off_combine, off_prefill, off_part_o, off_part_ml;
  int64_t off_slots;            // per-row cache slots (AppendArgs::slots); 0: none
  int64_t off_marked;           // (row, slot) pairs of the marked rows (AppendArgs::marked)
  int32_t n_marked, sole_bit;   // AppendArgs::n_marked and ::sole_bit
};
constexpr int kDescBytes = 256;        // the header's slot at the head of the workspace
static_assert(sizeof(StepDesc) <= kDescBytes, "the step header must fit its slot");

constexpr int kBlockSize = 16;         // KV positions per physical block
constexpr int kPrefillKeys = 64;       // keys per prefill K/V tile (4 blocks)
constexpr int kMaxSplitBlocks = 1024;  // blocks per decode split at most (16k positions)
constexpr int kNumCUs = 256;           // compute units of the target GPU (MI355X)

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* cu_q_lens;
  const int32_t* ctx_lens;
  const int32_t* block_tables;
  int32_t num_reqs, num_tokens, max_blocks, num_kv_heads, num_blocks;
  const StepDesc* desc;   // non-null in a replayed step: sizes and arrays come from here
  // Optional [num_tokens] cache slot of each packed row (block * block_size + offset), from
  // the host; null: each row's slot is looked up from cu_q_lens, ctx_lens and the tables.
  const int32_t* slots;
  // Optional staging copy done by the same launch: stage_n16 16-byte chunks from stage_src
  // (the pinned host buffer) to stage_dst (the workspace), for the kernels that follow.
  // stage_n16 < 0 (a replayed step): the count is the header's stage_bytes / 16, at most
  // -stage_n16.
  const void* stage_src;
  void* stage_dst;
  int64_t stage_n16;
  // kSlotSoleWriter when the host marks slots (see below), else 0: the bit is then part of
  // the slot value.
  int32_t sole_bit;
  // The marked rows as (packed row, slot) pairs, n_marked of them, read by the page
  // work-groups that follow the rows' (kPageRows marked rows each); null with n_marked = 0.
  const int32_t* marked;
  int32_t n_marked;
};

// Set in a host slot when its row is the only row of the step that writes into its block (a
// decode row, unless requests share a block): the append then rewrites that block's whole V^T
// page instead of one element per d-row. Used while num_blocks * block_size fits below the bit.
constexpr int32_t kSlotSoleWriter = 1 << 30;
constexpr int kPageRows = 2;             // marked rows per page work-group

struct RowArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  void* o;
  float* part_o;          // [n_parts, Hq, D] fp32
  float* part_ml;         // [n_parts, Hq, 2] fp32: running max (log2 units), sum
  const RowSplit* splits;
  const int32_t* block_tables;
  int32_t n_items;        // splits * num_kv_heads * (query heads per kv head / group)
  int32_t num_q_heads, num_kv_heads, max_blocks, num_blocks;
  float scale_log2;       // scale * log2(e)
  int32_t group;          // query heads per work item
  const StepDesc* desc;   // non-null in a replayed step: sizes and arrays come from here
};

struct CombineArgs {
  void* o;
  const float* part_o;
  const float* part_ml;
  const CombineRow* rows;
  int32_t n_rows;
  int32_t num_q_heads;
  const StepDesc* desc;   // non-null in a replayed step: sizes and arrays come from here
};

struct PrefillArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  void* o;
  const PrefillItem* items;
  const int32_t* cu_q_lens;
  const int32_t* ctx_lens;
  const int32_t* block_tables;
  int32_t n_items;
  int32_t num_q_heads, num_kv_heads, max_blocks, num_blocks;
  float scale_log2;
  const StepDesc* desc;   // non-null in a replayed step: sizes and arrays come from here
  float* part_o;          // partial outputs of split items, as RowArgs::part_o / part_ml
  float* part_ml;
};

// One launch holding a step's prefill tiles and its matrix-core decode waves (4-wave
// work-groups of both kinds). order[b] >= 0: work-group b is prefill slot order[b];
// order[b] < 0: it is decode work-group -1 - order[b] (its waves take items 4w..4w+3;
// indices past the decode items exit at once).
struct MixedArgs {
  PrefillArgs prefill;
  RowArgs decode;
  const int32_t* order;
  int32_t n_blocks;
};

// Largest reduction length of the token-wise GEMM: the work-group's loads go through buffer
// resources whose byte range (256 weight rows x K x 2 bytes) is a 32-bit count.
constexpr int kGemmMaxK = 1 << 20;

// C[M, N] = A[M, K] B[N, K]^T (bf16 in, fp32 accumulation, bf16 out). With the QKV
// epilogue, columns [0, Hq*D) are Q rows written to `c` ([M, Hq*D]); the next Hkv*D columns
// are K rows and the last Hkv*D are V rows, written into the paged cache at each row's slot
// (request found from cu_q_lens, position ctx + row offset, block from the block table).
struct GemmArgs {
  const void* a;
  const void* b;
  void* c;
  int32_t M, N, K;
  void* k_cache;
  void* v_cache;
  const int32_t* cu_q_lens;
  const int32_t* ctx_lens;
  const int32_t* block_tables;
  int32_t num_reqs, max_blocks, num_q_heads, num_kv_heads, head_dim, num_blocks;
};

}  // namespace cb
