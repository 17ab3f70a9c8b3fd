// Grouped-query decode kernel on the matrix cores; the per-wave work is row_attn_mfma_waves
// in attn_decode_gqa.h, shared with the mixed prefill/decode launch.
#include "attn_decode_gqa.h"

namespace cb {

template <int D>
__global__ __launch_bounds__(256, 2) void row_attn_mfma_kernel(RowArgs a) {
  row_attn_mfma_waves<D>(a, static_cast<int>(blockIdx.x));
}

hipError_t launch_rows_mfma(const RowArgs& a, int head_dim, hipStream_t s) {
  if (a.n_items == 0) return hipSuccess;
  const int blocks = (a.n_items + 3) / 4;
  if (head_dim == 128)
    hipLaunchKernelGGL(row_attn_mfma_kernel<128>, dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(row_attn_mfma_kernel<64>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

CB_VIOLATION_READER(violations_decode_gqa)

}  // namespace cb
