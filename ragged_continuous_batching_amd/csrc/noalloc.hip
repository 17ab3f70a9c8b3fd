// cb_ragged_attention_noalloc: ragged attention for callers that cannot allocate memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// It runs exactly the kernels of cb_ragged_attention. Where that call takes a caller
// workspace (the launch plan's work lists, then the fp32 split-K partials), this one uses a
// fixed array in device memory, `scratch`, of kNoAllocScratchBytes. The plan goes there with
// one host-to-device copy from ordinary host memory on the caller's stream; no device or
// pinned memory is allocated, freed or registered by the call.
//
// The array is a file-scope __device__ variable, so each GPU holds its own copy at its own
// address until the process ends. In host code `scratch` names a host-side stand-in, not a
// device address: its device address is read once per device with hipGetSymbolAddress and
// kept, and only that pointer is ever given to copies and kernels.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "host.h"

namespace cb {
namespace {

constexpr size_t kNoAllocScratchBytes = size_t{CB_NOALLOC_SCRATCH_BYTES};
static_assert(kNoAllocScratchBytes % 256 == 0, "the plan layout assumes a 256-byte aligned array");

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;     // per device: device address of `scratch` (null: not yet read)

// Device address of this device's copy of `scratch` (the current device). The first call on
// a device reads it with hipGetSymbolAddress, with that device current.
int scratch_address(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CB_ERR_HIP, "cb_ragged_attention_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (static_cast<int>(g_scratch_ptr.size()) <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(CB_ERR_HIP, "cb_ragged_attention_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return CB_OK;
}

}  // namespace
}  // namespace cb

using namespace cb;

extern "C" int cb_ragged_attention_noalloc(const cb_shape* shape, const cb_batch* batch, const void* q,
                                           const void* k_cache, const void* v_cache, float scale, void* o,
                                           void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_batch(shape, batch))) return st;
  if (batch->num_tokens == 0) return CB_OK;
  if ((st = check_tensors(q, k_cache, v_cache, o, scale, "cb_ragged_attention_noalloc"))) return st;
  Plan p;
  make_plan(shape, batch, p);
  if (p.total > kNoAllocScratchBytes)
    return fail(CB_ERR_WORKSPACE_TOO_SMALL,
                "cb_ragged_attention_noalloc: this batch needs %zu bytes of workspace, more than the fixed %zu "
                "(use cb_ragged_attention with a caller workspace)", p.total, kNoAllocScratchBytes);
  char* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.plan_bytes > 0) {
    // The plan's host image: ordinary (pageable) host memory, reused by later calls on this
    // thread. The copy is ordered on `s` after earlier work that reads the array.
    thread_local std::vector<char> host_plan;
    if (host_plan.size() < p.plan_bytes) host_plan.resize(p.plan_bytes);
    write_plan(p, host_plan.data());
    hipError_t e = hipMemcpyAsync(ws, host_plan.data(), p.plan_bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess)
      return fail(CB_ERR_HIP, "cb_ragged_attention_noalloc: plan copy failed: %s", hipGetErrorString(e));
  }
  return launch_attention(shape, batch, p, ws, q, k_cache, v_cache, scale, o, s, false);
}
