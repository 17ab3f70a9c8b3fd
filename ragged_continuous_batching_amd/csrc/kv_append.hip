// KV append: scatter this step's new keys and values into the paged cache.
//
// zhangchitc "continuous-batching", section "Inside the kernel": once the QKV projection
// has produced a step's keys and values, each row is stored in the cache slot of the
// request it belongs to, and only then does attention read the cache. The cache is paged
// (fixed-size physical blocks, hassanahmed "How continuous batching speeds up LLM serving",
// paged-memory section).
//
// Layout (include/cb.h): K pages are [block_size][D], V pages are [D][block_size] (V is
// stored transposed). A work-group takes 16 consecutive packed rows and one kv head (two at
// D = 64 in bf16, see append_heads):
//   1. every thread loads its 16-byte chunks of the new K and V rows, while the first 16
//      threads find each row's block and slot (from the host's slot list when the step
//      entry point provides one, else from the request's context length and block table);
//      called from the step entry point, the launch also copies the step's staged
//      metadata and plan into the workspace (no separate copy kernel);
//   2. K chunks go straight to their slots (key rows stay contiguous); V rows are staged in
//      LDS;
//   3. V^T leaves LDS per d-row: a group of 16/ES rows that occupies consecutive, aligned
//      slots of one block (rows of a prefill chunk) is written as one 16-byte store;
//   4. other rows (decode rows, the edges of a chunk) are written element by element, except
//      rows the host marks as the only row of the step writing into their block (decode
//      rows of a decode-only step): extra work-groups at the start of the grid, two marked
//      rows each, rewrite those blocks' whole V^T pages. A page is read, the row's element
//      put into each d-row, and every chunk stored back, the other slots with their own
//      bits. One element per 32-byte d-row leaves partly written cache lines, which memory
//      merges later at the cost of a read and a write each: skipping those writes
//      altogether (a timing copy) took 12-13 us off a step of 64 decode rows x 32 kv heads
//      or 256 x 8, most of it in the kernels after the append. A prefill kernel between the
//      append and the decode rows hides that merge, so the host marks rows only in
//      decode-only steps.
#include <algorithm>
#include <type_traits>

#include "cb_device.h"

namespace cb {

// Packed rows per work-group. More rows per work-group (fewer, longer work-groups) measured
// slower: config 2's append 21.7 -> 24.7 us at 32 or 64 rows, the chunked-prefill-heavy step's
// 50.5 -> 59.5-61.5 us (the trace's steps 24.1 -> 23.4-23.8 us).
constexpr int kAppendRows = 16;

// kv heads per work-group: as few as give every thread a whole number of 16-byte chunks
// (one head at D = 128 in bf16). More, smaller work-groups finish the scattered V^T stores
// sooner: one head instead of four measured 17.3 -> 12.4 us on 256 decode rows (Hkv = 8)
// and 22.3 -> 18.2 us on a 2048-row mixed step (Hkv = 32).
template <int ES, int D>
constexpr int append_heads() {
  return 256 / (kAppendRows * (D * ES / 16)) > 1 ? 256 / (kAppendRows * (D * ES / 16)) : 1;
}

// Whole V^T pages of marked rows m0 .. m0 + kPageRows - 1, kv heads g0 .. g0 + nheads - 1.
// Chunk c of a page holds d-row c / CPR, slots (c % CPR) * VEC ..; the chunk that holds the
// row's slot takes its new element (straight from v_new), every other one keeps its bits.
// All chunks are loaded before any is stored.
template <int ES, int D, int HEADS>
__device__ __forceinline__ void append_pages(const AppendArgs& a, int m0, int g0, int nheads, int tid) {
  constexpr int VEC = 16 / ES;
  constexpr int PCH = D * kBlockSize * ES / 16;        // 16-byte chunks per V^T page
  constexpr int CPR = kBlockSize / VEC;                // chunks per d-row
  constexpr int NCH = kPageRows * HEADS * PCH / 256;   // chunks per thread
  static_assert(NCH * 256 == kPageRows * HEADS * PCH, "page chunks must split evenly over 256 threads");
  using E = typename std::conditional<ES == 2, uint16_t, uint32_t>::type;
  u32x4 buf[NCH];
  int64_t at[NCH];                                     // chunk index in the V cache, -1: none
  uint32_t val[NCH], keep[NCH];                        // new element in place; bits kept
  int dw[NCH];                                         // dword that takes it, -1: none
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int w = tid + u * 256;
    const int c = w % PCH, hh = (w / PCH) % HEADS, m = m0 + w / (PCH * HEADS);
    at[u] = -1;
    dw[u] = -1;
    val[u] = 0u;
    keep[u] = 0xffffffffu;
    if (m >= a.n_marked || hh >= nheads) continue;
    const int t = a.marked[2 * m], sl = a.marked[2 * m + 1];
    const int blk = sl / kBlockSize, off = sl % kBlockSize;
    if (sl < 0 || static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks) ||
        static_cast<unsigned>(t) >= static_cast<unsigned>(a.num_tokens)) {
      note_violation(sl >= 0 && static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks));
      continue;
    }
    at[u] = (static_cast<int64_t>(blk) * a.num_kv_heads + g0 + hh) * PCH + c;
    buf[u] = reinterpret_cast<const u32x4*>(a.v_cache)[at[u]];
    if (c % CPR == off / VEC) {
      const int e = off % VEC, sh = (e * ES % 4) * 8;
      dw[u] = e * ES / 4;
      keep[u] = ES == 4 ? 0u : ~(0xffffu << sh);
      val[u] = static_cast<uint32_t>(
                   static_cast<const E*>(a.v_new)[(static_cast<int64_t>(t) * a.num_kv_heads + g0 + hh) * D + c / CPR])
               << sh;
    }
  }
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    if (at[u] < 0) continue;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k == dw[u]) buf[u][k] = (buf[u][k] & keep[u]) | val[u];
    reinterpret_cast<u32x4*>(a.v_cache)[at[u]] = buf[u];
  }
}

template <int ES, int D>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  constexpr int VEC = 16 / ES;              // elements per 16-byte chunk
  constexpr int CH = D / VEC;               // chunks per row
  constexpr int ROWS = kAppendRows, HEADS = append_heads<ES, D>();
  static_assert(ROWS <= 64, "the marked rows of a work-group are one 64-bit mask");
  constexpr int LS = D + 16 / ES;           // LDS row stride (elements): spreads banks
  using E = typename std::conditional<ES == 2, uint16_t, uint32_t>::type;
  __shared__ __align__(16) E vt[HEADS * ROWS * LS];
  __shared__ int32_t info_blk[ROWS], info_off[ROWS];
  __shared__ int32_t info_run[ROWS / VEC];
  __shared__ uint64_t info_sole;               // bit r: row r rewrites its whole V^T page

  if (a.desc) resolve_desc(a);
  // The page work-groups come first, so that their longer chains (pinned list, page, stores)
  // start early; they load no rows.
  const int n_pagex = (max(a.n_marked, 0) + kPageRows - 1) / kPageRows;
  const bool pages = static_cast<int>(blockIdx.x) < n_pagex;     // a whole-page work-group
  const int t0 = (static_cast<int>(blockIdx.x) - n_pagex) * ROWS;
  const int g0 = blockIdx.y * HEADS;
  const int tid = threadIdx.x;
  const int nrows = pages ? 0 : min(ROWS, a.num_tokens - t0);   // page work-groups load no rows
  const int nheads = min(HEADS, a.num_kv_heads - g0);
  // The new K and V chunks of the work-group are requested first; the slot lookup (a binary
  // search over cu_q_lens, then ctx_lens and the block table: a chain of dependent loads)
  // runs while they are in flight.
  constexpr int NPT = HEADS * ROWS * CH / 256;   // chunks per thread
  static_assert(NPT * 256 == HEADS * ROWS * CH, "chunks must split evenly over 256 threads");
  u32x4 kv[NPT], vv[NPT];
#pragma unroll
  for (int u = 0; u < NPT; ++u) {
    const int e = tid + u * 256;
    const int c = e % CH, row = (e / CH) % ROWS, hh = e / (CH * ROWS);
    kv[u] = vv[u] = u32x4{0u, 0u, 0u, 0u};
    if (row < nrows && hh < nheads) {
      const int64_t src = ((static_cast<int64_t>(t0 + row) * a.num_kv_heads + g0 + hh) * D + c * VEC) * ES;
      vv[u] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.v_new) + src);
      kv[u] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.k_new) + src);
    }
  }
  if (a.stage_src) {
    // The step's metadata and plan, from the pinned staging buffer into the workspace (the
    // kernels after this one read them there): spread over all work-groups, issued while the
    // new K/V rows above are in flight.
    const int64_t stride = static_cast<int64_t>(gridDim.x) * gridDim.y * 256;
    const int64_t n16 = a.stage_n16 >= 0 ? a.stage_n16 : min(a.desc->stage_bytes / 16, -a.stage_n16);
    const u32x4* src = static_cast<const u32x4*>(a.stage_src);
    u32x4* dst = static_cast<u32x4*>(a.stage_dst);
    for (int64_t i = (static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x) * 256 + tid; i < n16; i += stride)
      dst[i] = src[i];
  }
  if (pages) {
    append_pages<ES, D, HEADS>(a, blockIdx.x * kPageRows, g0, nheads, tid);
    return;
  }
  if (t0 >= a.num_tokens) return;              // past the live rows
  if (tid < ROWS) {
    int blk = -1, off = 0;
    bool sole = false;
    if (tid < nrows) {
      const int t = t0 + tid;
      if (a.slots) {                            // the host's slot: one load instead of a chain
        int sl = a.slots[t];
        if (sl >= 0 && (sl & a.sole_bit) != 0) {
          sole = true;
          sl &= ~a.sole_bit;
        }
        blk = sl >= 0 ? sl / kBlockSize : -1;
        off = sl >= 0 ? sl % kBlockSize : 0;
      } else {
        const int r = find_request(a.cu_q_lens, a.num_reqs, t);
        const int p = a.ctx_lens[r] + (t - a.cu_q_lens[r]);
        blk = a.block_tables[static_cast<int64_t>(r) * a.max_blocks + p / kBlockSize];
        off = p % kBlockSize;
      }
      if (static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks)) {
        note_violation(blk >= 0 || !a.slots);   // a host slot of -1 marks no row, not a bad id
        blk = -1;
      }
    }
    info_blk[tid] = blk;
    info_off[tid] = off;
    const uint64_t sole_rows = __ballot(sole && blk >= 0);   // the first ROWS lanes of wave 0
    if (tid == 0) info_sole = sole_rows;
  }
  // V rows into LDS
#pragma unroll
  for (int u = 0; u < NPT; ++u) {
    const int e = tid + u * 256;
    const int c = e % CH, row = (e / CH) % ROWS, hh = e / (CH * ROWS);
    if (row < nrows && hh < nheads) *reinterpret_cast<u32x4*>(&vt[(hh * ROWS + row) * LS + c * VEC]) = vv[u];
  }
  __syncthreads();
  if (tid < ROWS / VEC) {                       // does row group tid fill one aligned run?
    const int r0 = tid * VEC;
    bool run = r0 + VEC <= nrows && info_blk[r0] >= 0 && info_off[r0] % VEC == 0;
    for (int i = 1; i < VEC && run; ++i)
      run = info_blk[r0 + i] == info_blk[r0] && info_off[r0 + i] == info_off[r0] + i;
    info_run[tid] = run;
  }
  // K rows straight to their slots
#pragma unroll
  for (int u = 0; u < NPT; ++u) {
    const int e = tid + u * 256;
    const int c = e % CH, row = (e / CH) % ROWS, hh = e / (CH * ROWS);
    if (row >= nrows || hh >= nheads) continue;
    const int blk = info_blk[row];
    if (blk < 0) continue;
    const int64_t page = static_cast<int64_t>(blk) * a.num_kv_heads + g0 + hh;
    *reinterpret_cast<u32x4*>(static_cast<char*>(a.k_cache) +
                              ((page * kBlockSize + info_off[row]) * D + c * VEC) * ES) = kv[u];
  }
  __syncthreads();

  // V^T: a group of VEC rows that fill VEC consecutive, aligned slots of one block (the rows
  // of a prefill chunk, as a rule) leaves as one 16-byte store per d-row; in other groups the
  // unmarked rows store element by element and the marked ones are left to the page
  // work-groups.
  constexpr int GROUPS = ROWS / VEC;
  for (int e = tid; e < HEADS * D * GROUPS; e += 256) {
    const int grp = e % GROUPS, d = (e / GROUPS) % D, hh = e / (GROUPS * D);
    if (hh >= nheads) continue;
    const int r0 = grp * VEC;
    if (r0 >= nrows) continue;
    const E* src = &vt[(hh * ROWS + r0) * LS + d];
    if (info_run[grp]) {
      const int64_t page = static_cast<int64_t>(info_blk[r0]) * a.num_kv_heads + g0 + hh;
      E vals[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) vals[i] = src[i * LS];
      u32x4 w;
      __builtin_memcpy(&w, vals, 16);
      *reinterpret_cast<u32x4*>(static_cast<E*>(a.v_cache) + (page * D + d) * kBlockSize + info_off[r0]) = w;
    } else {
      for (int i = 0; i < VEC && r0 + i < nrows; ++i) {
        const int blk = info_blk[r0 + i];
        if (blk < 0 || ((info_sole >> (r0 + i)) & 1u) != 0) continue;
        const int64_t page = static_cast<int64_t>(blk) * a.num_kv_heads + g0 + hh;
        static_cast<E*>(a.v_cache)[(page * D + d) * kBlockSize + info_off[r0 + i]] = src[i * LS];
      }
    }
  }
}

dim3 append_grid(int64_t num_tokens, int32_t num_kv_heads, int elem_bytes, int head_dim, int32_t n_marked) {
  const int h = elem_bytes == 2 ? (head_dim == 128 ? append_heads<2, 128>() : append_heads<2, 64>())
                                : (head_dim == 128 ? append_heads<4, 128>() : append_heads<4, 64>());
  // at least one work-group in each dimension (a captured step may replay with no rows; the
  // kernel exits for rows and heads past the end); the page work-groups follow the rows'
  const int64_t x = (num_tokens + kAppendRows - 1) / kAppendRows + (std::max(n_marked, 0) + kPageRows - 1) / kPageRows,
                y = (num_kv_heads + h - 1) / h;
  return dim3(static_cast<unsigned>(x > 0 ? x : 1), static_cast<unsigned>(y > 0 ? y : 1));
}

template <int ES, int D>
static hipError_t launch_append_t(const AppendArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL((kv_append_kernel<ES, D>), append_grid(a.num_tokens, a.num_kv_heads, ES, D, a.n_marked),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_kv_append(const AppendArgs& a, int elem_bytes, int head_dim, hipStream_t s) {
  if (elem_bytes == 2) return head_dim == 128 ? launch_append_t<2, 128>(a, s) : launch_append_t<2, 64>(a, s);
  return head_dim == 128 ? launch_append_t<4, 128>(a, s) : launch_append_t<4, 64>(a, s);
}

CB_VIOLATION_READER(violations_append)

}  // namespace cb
