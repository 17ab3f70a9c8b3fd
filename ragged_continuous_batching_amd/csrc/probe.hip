// Measurement aid, not part of a step: the read rate the GPU attains on the cache's access
// pattern, so that the bench can state the decode kernels' bandwidth against what this box
// delivers for that pattern as well as against the vendor figure. The decode kernels read
// whole 4 KiB pages (one kv head of one block) in an order the block tables scatter over the
// pool, with non-temporal 16-byte loads; this kernel does the same and nothing else. Each wave
// reads kProbePages pages, all requested before the first is used (as many bytes in flight as
// the memory takes: the rate is a ceiling for the pattern); the values are folded into one
// word that is stored only if it matches a constant, so the loads stay live and almost nothing
// is written.
#include "cb_device.h"

namespace cb {

namespace {
constexpr int kProbePages = 16;                  // pages per wave
constexpr int kPageBytes = 4096;
constexpr int kLoads = kPageBytes / (64 * 16);   // 16-byte loads per lane per page
}  // namespace

__global__ __launch_bounds__(256) void paged_read_kernel(const char* __restrict__ base, const int32_t* __restrict__ order,
                                                         int32_t n_pages, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t p0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kProbePages;
  // the wave's page ids, one per lane, read once: a per-page index load would make each
  // page's loads wait for the previous page's (the load counter drains in order)
  int32_t ids = -1;
  if (lane < kProbePages && p0 + lane < n_pages) ids = order[p0 + lane];
  uint32_t acc = 0;
#pragma unroll
  for (int k = 0; k < kProbePages; k += 2) {
    u32x4 v[2][kLoads];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int32_t pg = __builtin_amdgcn_readlane(ids, k + h);      // the same in every lane
      const bool ok = static_cast<uint32_t>(pg) < static_cast<uint32_t>(n_pages);
#pragma unroll
      for (int j = 0; j < kLoads; ++j)
        v[h][j] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                           base + static_cast<int64_t>(pg) * kPageBytes + (j * 64 + lane) * 16))
                     : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < kLoads; ++j) acc ^= v[h][j][0] ^ v[h][j][1] ^ v[h][j][2] ^ v[h][j][3];
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

int32_t paged_read_grid(int32_t n_pages) { return (n_pages + 4 * kProbePages - 1) / (4 * kProbePages); }

hipError_t launch_paged_read(const void* pages, int32_t n_pages, const int32_t* order, uint32_t* sink,
                             hipStream_t s) {
  hipLaunchKernelGGL(paged_read_kernel, dim3(paged_read_grid(n_pages)), dim3(256), 0, s,
                     static_cast<const char*>(pages), order, n_pages, sink);
  return hipGetLastError();
}

}  // namespace cb
