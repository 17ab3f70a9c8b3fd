// Prefill-chunk attention kernel (bf16 MFMA tiles); the tile itself is prefill_tile in
// attn_prefill.h, shared with the mixed prefill/decode launch.
#include "attn_prefill.h"

namespace cb {

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void prefill_kernel(PrefillArgs a) {
  prefill_tile<D, NW>(a, static_cast<int>(blockIdx.x));
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int waves, hipStream_t s) {
  if (a.n_items == 0) return hipSuccess;
  if (waves == 8) {
    if (head_dim == 128)
      hipLaunchKernelGGL((prefill_kernel<128, 8>), dim3(a.n_items), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((prefill_kernel<64, 8>), dim3(a.n_items), dim3(512), 0, s, a);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((prefill_kernel<128, 4>), dim3(a.n_items), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((prefill_kernel<64, 4>), dim3(a.n_items), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

CB_VIOLATION_READER(violations_prefill)

}  // namespace cb
