// Moves a step's host-staged metadata and work lists into the workspace on the compute
// queue: the kernel reads the pinned host buffer directly over the host link and writes
// device memory. Kept on the same queue as the kernels that consume the data, the copy
// needs no hand-over between a copy engine and the compute queue before the next launch.
#include <algorithm>

#include "cb_device.h"

namespace cb {

__global__ __launch_bounds__(256) void stage_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// `bytes` is rounded up to 16; both buffers must hold the rounded size and be 16-aligned.
hipError_t launch_stage_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const int64_t n16 = static_cast<int64_t>((bytes + 15) / 16);
  if (n16 == 0) return hipSuccess;
  const int blocks = static_cast<int>(std::min<int64_t>((n16 + 255) / 256, 1024));
  hipLaunchKernelGGL(stage_copy_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

// The replayed form: the copy's length is the header's stage_bytes, read from the pinned
// slot itself (the host writes the header before it launches the graph); at most max16
// chunks, the capacity the graph was captured for.
__global__ __launch_bounds__(256) void stage_copy_desc_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                              int64_t max16) {
  const int64_t n16 = min(reinterpret_cast<const StepDesc*>(src)->stage_bytes / 16, max16);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

hipError_t launch_stage_copy_desc(const void* src, void* dst, size_t max_bytes, hipStream_t s) {
  const int64_t max16 = static_cast<int64_t>(max_bytes / 16);
  const int blocks = static_cast<int>(std::clamp<int64_t>((max16 + 255) / 256, 1, 1024));
  hipLaunchKernelGGL(stage_copy_desc_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), max16);
  return hipGetLastError();
}

}  // namespace cb
