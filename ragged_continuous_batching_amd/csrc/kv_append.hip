// KV append: scatter this step's new keys and values into the paged cache.
//
// zhangchitc "continuous-batching", section "Inside the kernel": after the QKV projection
// the new keys and values are written into the KV cache, each into its own request's entry,
// before attention reads the cache back. The cache is paged (fixed-size physical blocks,
// hassanahmed "How continuous batching speeds up LLM serving", paged-memory section).
//
// Layout (include/cb.h): K pages are [block_size][D], V pages are [D][block_size] (V is
// stored transposed). A work-group takes 16 consecutive packed rows and up to 4 kv heads:
//   1. the first 16 threads find each row's request, block and slot;
//   2. K rows are copied chunk by chunk (16 bytes per thread, key rows stay contiguous);
//      V rows are staged in LDS;
//   3. V elements leave LDS with 16 consecutive lanes on 16 consecutive rows of one d-row,
//      so the rows of a prefill chunk that share a block land as one contiguous run of the
//      transposed page (a decode row writes one element per d-row, as the layout implies).
#include <type_traits>

#include "cb_device.h"

namespace cb {

template <int ES, int D>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  constexpr int VEC = 16 / ES;              // elements per 16-byte chunk
  constexpr int CH = D / VEC;               // chunks per row
  constexpr int ROWS = 16, HEADS = 4;
  constexpr int LS = D + 16 / ES;           // LDS row stride (elements): spreads banks
  using E = typename std::conditional<ES == 2, uint16_t, uint32_t>::type;
  __shared__ __align__(16) E vt[HEADS * ROWS * LS];
  __shared__ int32_t info_blk[ROWS], info_off[ROWS];

  const int t0 = blockIdx.x * ROWS;
  const int g0 = blockIdx.y * HEADS;
  const int tid = threadIdx.x;
  const int nrows = min(ROWS, a.num_tokens - t0);
  const int nheads = min(HEADS, a.num_kv_heads - g0);
  if (tid < ROWS) {
    int blk = -1, off = 0;
    if (tid < nrows) {
      const int t = t0 + tid;
      const int r = find_request(a.cu_q_lens, a.num_reqs, t);
      const int p = a.ctx_lens[r] + (t - a.cu_q_lens[r]);
      blk = a.block_tables[static_cast<int64_t>(r) * a.max_blocks + p / kBlockSize];
      off = p % kBlockSize;
      if (static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks)) blk = -1;
    }
    info_blk[tid] = blk;
    info_off[tid] = off;
  }
  __syncthreads();

  // K rows straight to their slots; V rows into LDS
  for (int e = tid; e < HEADS * ROWS * CH; e += 256) {
    const int c = e % CH, row = (e / CH) % ROWS, hh = e / (CH * ROWS);
    if (row >= nrows || hh >= nheads) continue;
    const int64_t src = ((static_cast<int64_t>(t0 + row) * a.num_kv_heads + g0 + hh) * D + c * VEC) * ES;
    const u32x4 vv = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.v_new) + src);
    *reinterpret_cast<u32x4*>(&vt[(hh * ROWS + row) * LS + c * VEC]) = vv;
    const int blk = info_blk[row];
    if (blk < 0) continue;
    const u32x4 kv = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.k_new) + src);
    const int64_t page = static_cast<int64_t>(blk) * a.num_kv_heads + g0 + hh;
    *reinterpret_cast<u32x4*>(static_cast<char*>(a.k_cache) +
                              ((page * kBlockSize + info_off[row]) * D + c * VEC) * ES) = kv;
  }
  __syncthreads();

  // V^T: lane-consecutive rows within one d-row
  for (int e = tid; e < HEADS * D * ROWS; e += 256) {
    const int row = e % ROWS, d = (e / ROWS) % D, hh = e / (ROWS * D);
    if (row >= nrows || hh >= nheads) continue;
    const int blk = info_blk[row];
    if (blk < 0) continue;
    const int64_t page = static_cast<int64_t>(blk) * a.num_kv_heads + g0 + hh;
    static_cast<E*>(a.v_cache)[(page * D + d) * kBlockSize + info_off[row]] = vt[(hh * ROWS + row) * LS + d];
  }
}

template <int ES, int D>
static hipError_t launch_append_t(const AppendArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL((kv_append_kernel<ES, D>), dim3((a.num_tokens + 15) / 16, (a.num_kv_heads + 3) / 4), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

hipError_t launch_kv_append(const AppendArgs& a, int elem_bytes, int head_dim, hipStream_t s) {
  if (elem_bytes == 2) return head_dim == 128 ? launch_append_t<2, 128>(a, s) : launch_append_t<2, 64>(a, s);
  return head_dim == 128 ? launch_append_t<4, 128>(a, s) : launch_append_t<4, 64>(a, s);
}

}  // namespace cb
