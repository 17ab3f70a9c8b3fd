// KV append: scatter this step's new keys and values into the paged cache.
//
// zhangchitc "continuous-batching", section "Inside the kernel": once the QKV projection
// has produced a step's keys and values, each row is stored in the cache slot of the
// request it belongs to, and only then does attention read the cache. The cache is paged (fixed-size physical blocks,
// hassanahmed "How continuous batching speeds up LLM serving", paged-memory section).
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
//      slots of one block (rows of a prefill chunk) is written as one 16-byte store; other
//      rows (decode rows, the edges of a chunk) element by element, as the layout implies.
#include <type_traits>

#include "cb_device.h"

namespace cb {

// kv heads per work-group: as few as give every thread a whole number of 16-byte chunks
// (one head at D = 128 in bf16). More, smaller work-groups finish the scattered V^T stores
// sooner: one head instead of four measured 17.3 -> 12.4 us on 256 decode rows (Hkv = 8)
// and 22.3 -> 18.2 us on a 2048-row mixed step (Hkv = 32).
template <int ES, int D>
constexpr int append_heads() {
  return 256 / (16 * (D * ES / 16)) > 1 ? 256 / (16 * (D * ES / 16)) : 1;
}

template <int ES, int D>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  constexpr int VEC = 16 / ES;              // elements per 16-byte chunk
  constexpr int CH = D / VEC;               // chunks per row
  constexpr int ROWS = 16, HEADS = append_heads<ES, D>();
  constexpr int LS = D + 16 / ES;           // LDS row stride (elements): spreads banks
  using E = typename std::conditional<ES == 2, uint16_t, uint32_t>::type;
  __shared__ __align__(16) E vt[HEADS * ROWS * LS];
  __shared__ int32_t info_blk[ROWS], info_off[ROWS];
  __shared__ int32_t info_run[ROWS / VEC];

  if (a.desc) resolve_desc(a);
  const int t0 = blockIdx.x * ROWS;
  if (t0 >= a.num_tokens) return;              // past the live rows of a replayed step
  const int g0 = blockIdx.y * HEADS;
  const int tid = threadIdx.x;
  const int nrows = min(ROWS, a.num_tokens - t0);
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
  if (tid < ROWS) {
    int blk = -1, off = 0;
    if (tid < nrows) {
      const int t = t0 + tid;
      if (a.slots) {                            // the host's slot: one load instead of a chain
        const int sl = a.slots[t];
        blk = sl >= 0 ? sl / kBlockSize : -1;
        off = sl >= 0 ? sl % kBlockSize : 0;
      } else {
        const int r = find_request(a.cu_q_lens, a.num_reqs, t);
        const int p = a.ctx_lens[r] + (t - a.cu_q_lens[r]);
        blk = a.block_tables[static_cast<int64_t>(r) * a.max_blocks + p / kBlockSize];
        off = p % kBlockSize;
      }
      if (static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks)) blk = -1;
    }
    info_blk[tid] = blk;
    info_off[tid] = off;
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
  // of a prefill chunk, as a rule) leaves as one 16-byte store per d-row; other groups (decode
  // rows, chunk edges) store element by element.
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
        if (blk < 0) continue;
        const int64_t page = static_cast<int64_t>(blk) * a.num_kv_heads + g0 + hh;
        static_cast<E*>(a.v_cache)[(page * D + d) * kBlockSize + info_off[r0 + i]] = src[i * LS];
      }
    }
  }
}

dim3 append_grid(int64_t num_tokens, int32_t num_kv_heads, int elem_bytes, int head_dim) {
  const int h = elem_bytes == 2 ? (head_dim == 128 ? append_heads<2, 128>() : append_heads<2, 64>())
                                : (head_dim == 128 ? append_heads<4, 128>() : append_heads<4, 64>());
  // at least one work-group in each dimension (a captured step may replay with no rows; the
  // kernel exits for rows and heads past the end)
  const int64_t x = (num_tokens + 15) / 16, y = (num_kv_heads + h - 1) / h;
  return dim3(static_cast<unsigned>(x > 0 ? x : 1), static_cast<unsigned>(y > 0 ? y : 1));
}

template <int ES, int D>
static hipError_t launch_append_t(const AppendArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL((kv_append_kernel<ES, D>), append_grid(a.num_tokens, a.num_kv_heads, ES, D), dim3(256), 0, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_kv_append(const AppendArgs& a, int elem_bytes, int head_dim, hipStream_t s) {
  if (elem_bytes == 2) return head_dim == 128 ? launch_append_t<2, 128>(a, s) : launch_append_t<2, 64>(a, s);
  return head_dim == 128 ? launch_append_t<4, 128>(a, s) : launch_append_t<4, 64>(a, s);
}

}  // namespace cb
