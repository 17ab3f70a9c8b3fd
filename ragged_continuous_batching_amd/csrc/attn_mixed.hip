// Prefill tiles and decode waves of one step in a single launch.
//
// Hugging Face blog "Continuous batching from first principles", section "Continuous
// batching": a ragged step mixes prefill chunks with decode tokens. The two halves stress
// different units: prefill tiles are bound by the matrix cores (O(n^2 d) work per chunk),
// decode rows by the cache read (section "KV-cache"). Launched one after the other they take
// turns on every CU. Here one grid holds both kinds of 4-wave work-group, interleaved by
// the host planner in proportion to their counts, so that the dispatcher places prefill and
// decode work-groups side by side on each CU and the matrix-core work runs under the cache
// stream. Both halves run the same code as their own kernels (prefill_tile,
// row_attn_mfma_waves). The order is interleaved in runs of one work-group per XCD, so a
// prefill slot keeps the XCD its planner chose for it.
#include "attn_decode_gqa.h"
#include "attn_prefill.h"

namespace cb {

template <int D>
__global__ __launch_bounds__(256, 2) void mixed_attn_kernel(MixedArgs a) {
  const int e = a.order[blockIdx.x];
  if (e >= 0)
    prefill_tile<D, 4>(a.prefill, e);
  else
    row_attn_mfma_waves<D>(a.decode, -1 - e);
}

hipError_t launch_mixed(const MixedArgs& a, int head_dim, hipStream_t s) {
  if (a.n_blocks == 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(mixed_attn_kernel<128>, dim3(a.n_blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(mixed_attn_kernel<64>, dim3(a.n_blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

CB_VIOLATION_READER(violations_mixed)

}  // namespace cb
