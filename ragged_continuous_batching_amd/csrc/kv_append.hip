// KV append: scatter this step's new keys and values into the paged cache.
//
// zhangchitc "continuous-batching", section "Inside the kernel": after the QKV projection
// the new keys and values are written into the KV cache, each into its own request's entry,
// before attention reads the cache back. The cache is paged (fixed-size physical blocks,
// hassanahmed "How continuous batching speeds up LLM serving", paged-memory section).
//
// Layout (include/cb.h): K pages are [block_size][D] (one 16-byte chunk of a key row per
// thread, stored as is); V pages are [D][block_size] (the thread's VEC elements go to VEC
// different d-rows at slot `off`). One thread moves one 16-byte chunk of K and of V.
#include "cb_device.h"

namespace cb {

template <int ES, int D>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  constexpr int VEC = 16 / ES;       // elements per 16-byte chunk
  constexpr int CH = D / VEC;        // chunks per row
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t rows = static_cast<int64_t>(a.num_tokens) * a.num_kv_heads;
  if (gid >= rows * CH) return;
  const int c = static_cast<int>(gid % CH);
  const int64_t row = gid / CH;                       // t * Hkv + g
  const int g = static_cast<int>(row % a.num_kv_heads);
  const int t = static_cast<int>(row / a.num_kv_heads);
  const int r = find_request(a.cu_q_lens, a.num_reqs, t);
  const int p = a.ctx_lens[r] + (t - a.cu_q_lens[r]);
  const int blk = a.block_tables[static_cast<int64_t>(r) * a.max_blocks + p / kBlockSize];
  if (static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks)) return;
  const int off = p % kBlockSize;
  const int64_t page = static_cast<int64_t>(blk) * a.num_kv_heads + g;

  const u32x4 kv = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.k_new) + (row * D + c * VEC) * ES);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.v_new) + (row * D + c * VEC) * ES);
  *reinterpret_cast<u32x4*>(static_cast<char*>(a.k_cache) + ((page * kBlockSize + off) * D + c * VEC) * ES) = kv;

  char* vpage = static_cast<char*>(a.v_cache) + page * D * kBlockSize * ES;
  if constexpr (ES == 2) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(vpage) + (c * VEC) * kBlockSize + off;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dst[(2 * w) * kBlockSize] = static_cast<uint16_t>(vv[w] & 0xffffu);
      dst[(2 * w + 1) * kBlockSize] = static_cast<uint16_t>(vv[w] >> 16);
    }
  } else {
    uint32_t* dst = reinterpret_cast<uint32_t*>(vpage) + (c * VEC) * kBlockSize + off;
#pragma unroll
    for (int w = 0; w < 4; ++w) dst[w * kBlockSize] = vv[w];
  }
}

template <int ES, int D>
static hipError_t launch_append_t(const AppendArgs& a, hipStream_t s) {
  constexpr int CH = D / (16 / ES);
  const int64_t threads = static_cast<int64_t>(a.num_tokens) * a.num_kv_heads * CH;
  if (threads == 0) return hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((kv_append_kernel<ES, D>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_kv_append(const AppendArgs& a, int elem_bytes, int head_dim, hipStream_t s) {
  if (elem_bytes == 2) return head_dim == 128 ? launch_append_t<2, 128>(a, s) : launch_append_t<2, 64>(a, s);
  return head_dim == 128 ? launch_append_t<4, 128>(a, s) : launch_append_t<4, 64>(a, s);
}

}  // namespace cb
