// Device helpers for the gfx950 kernels: bf16 bit handling, DPP/lane reductions, vector types.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "cb_plan.h"

namespace cb {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource word 3 for CDNA: 32-bit data format, no swizzle, raw (stride 0) access.
constexpr int kBufferFlags = 0x00020000;

// Device checks (the debug copy of the library, built with CB_DEVICE_CHECKS). The host checks
// a step's block ids against the pool before it launches anything, from its host mirrors; a
// kernel reads the device block table. Where a kernel meets an id outside the pool it reads
// block 0 instead, or skips the write, so it never faults; in the debug copy it also adds one
// to the violation counter of its code object (every kernel source has its own counter and
// its own reader, CB_VIOLATION_READER), which cb_debug_violations() sums. In the normal build
// the count compiles to nothing.
#ifdef CB_DEVICE_CHECKS
static __device__ unsigned int g_violations;
__device__ __forceinline__ void note_violation(bool bad) {
  if (bad) __hip_atomic_fetch_add(&g_violations, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Host reader of this source's counter: adds it to *sum, then zeroes it when `reset`.
#define CB_VIOLATION_READER(name)                                                              \
  hipError_t name(uint32_t* sum, bool reset) {                                                 \
    unsigned int v = 0;                                                                        \
    hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_violations), sizeof(v), 0, hipMemcpyDeviceToHost); \
    if (e != hipSuccess) return e;                                                             \
    *sum += v;                                                                                 \
    if (!reset) return hipSuccess;                                                             \
    const unsigned int zero = 0;                                                               \
    return hipMemcpyToSymbol(HIP_SYMBOL(g_violations), &zero, sizeof(zero), 0, hipMemcpyHostToDevice); \
  }
#else
__device__ __forceinline__ void note_violation(bool) {}
#define CB_VIOLATION_READER(name)
#endif

// bf16 stored as 16-bit patterns; a 32-bit word holds two (low half = lower address).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> two bf16 (round to nearest even), packed low = a. gfx950 has a native
// conversion instruction for this.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float a) {
  return static_cast<uint16_t>(pack_bf16x2(a, 0.f) & 0xffffu);
}

// Data-parallel-primitive lane moves (gfx9 DPP control codes).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

// Sum / max over aligned groups of W consecutive lanes; every lane gets the group result.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (W >= 2) v += dpp_mov<kDppXor1>(v);
  if constexpr (W >= 4) v += dpp_mov<kDppXor2>(v);
  if constexpr (W >= 8) v += dpp_mov<kDppHalfMirror>(v);
  if constexpr (W >= 16) v += dpp_mov<kDppMirror>(v);
  if constexpr (W >= 32) v += __shfl_xor(v, 16);
  if constexpr (W >= 64) v += __shfl_xor(v, 32);
  return v;
}

// Sum / max across lanes whose ids differ only in bits >= log2(STRIDE) (i.e. lane groups
// STRIDE apart), for STRIDE in {1..32}; every lane gets the result.
template <int STRIDE>
__device__ __forceinline__ float strided_sum(float v) {
  if constexpr (STRIDE <= 1) v += dpp_mov<kDppXor1>(v);
  if constexpr (STRIDE <= 2) v += dpp_mov<kDppXor2>(v);
  if constexpr (STRIDE <= 4) v += __shfl_xor(v, 4);
  if constexpr (STRIDE <= 8) v += __shfl_xor(v, 8);
  if constexpr (STRIDE <= 16) v += __shfl_xor(v, 16);
  if constexpr (STRIDE <= 32) v += __shfl_xor(v, 32);
  return v;
}

template <int STRIDE>
__device__ __forceinline__ float strided_max(float v) {
  if constexpr (STRIDE <= 1) v = fmaxf(v, dpp_mov<kDppXor1>(v));
  if constexpr (STRIDE <= 2) v = fmaxf(v, dpp_mov<kDppXor2>(v));
  if constexpr (STRIDE <= 4) v = fmaxf(v, __shfl_xor(v, 4));
  if constexpr (STRIDE <= 8) v = fmaxf(v, __shfl_xor(v, 8));
  if constexpr (STRIDE <= 16) v = fmaxf(v, __shfl_xor(v, 16));
  if constexpr (STRIDE <= 32) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Request owning packed row t: largest r with cu[r] <= t (cu nondecreasing, cu[0] = 0).
__device__ __forceinline__ int find_request(const int32_t* __restrict__ cu, int num_reqs, int t) {
  int lo = 0, hi = num_reqs;          // invariant: cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// A replayed step (StepDesc non-null) takes its sizes and work arrays from the header the
// stage copy wrote at the head of the workspace; its kernels are launched for the graph's
// capacity, so these run before the first bounds check.
template <class T>
__device__ __forceinline__ T* desc_array(const StepDesc* d, int64_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(const_cast<StepDesc*>(d)) + off);
}

__device__ __forceinline__ void resolve_desc(AppendArgs& a) {
  const StepDesc* d = a.desc;
  a.num_reqs = d->num_reqs;
  a.num_tokens = d->num_tokens;
  a.max_blocks = d->max_blocks;
  a.cu_q_lens = desc_array<const int32_t>(d, d->off_cu);
  a.ctx_lens = desc_array<const int32_t>(d, d->off_ctx);
  a.block_tables = desc_array<const int32_t>(d, d->off_bt);
  a.slots = d->off_slots ? desc_array<const int32_t>(d, d->off_slots) : nullptr;
  a.n_marked = d->n_marked;
  a.sole_bit = d->sole_bit;
  a.marked = d->n_marked ? desc_array<const int32_t>(d, d->off_marked) : nullptr;
}

__device__ __forceinline__ void resolve_desc(RowArgs& a) {
  const StepDesc* d = a.desc;
  a.n_items = d->n_row_items;
  a.max_blocks = d->max_blocks;
  a.splits = desc_array<const RowSplit>(d, d->off_splits);
  a.block_tables = desc_array<const int32_t>(d, d->off_bt);
  a.part_o = desc_array<float>(d, d->off_part_o);
  a.part_ml = desc_array<float>(d, d->off_part_ml);
}

__device__ __forceinline__ void resolve_desc(CombineArgs& a) {
  const StepDesc* d = a.desc;
  a.n_rows = d->n_combine_rows;
  a.rows = desc_array<const CombineRow>(d, d->off_combine);
  a.part_o = desc_array<const float>(d, d->off_part_o);
  a.part_ml = desc_array<const float>(d, d->off_part_ml);
}

__device__ __forceinline__ void resolve_desc(PrefillArgs& a) {
  const StepDesc* d = a.desc;
  a.n_items = d->n_prefill;
  a.max_blocks = d->max_blocks;
  a.items = desc_array<const PrefillItem>(d, d->off_prefill);
  a.cu_q_lens = desc_array<const int32_t>(d, d->off_cu);
  a.ctx_lens = desc_array<const int32_t>(d, d->off_ctx);
  a.block_tables = desc_array<const int32_t>(d, d->off_bt);
  a.part_o = desc_array<float>(d, d->off_part_o);
  a.part_ml = desc_array<float>(d, d->off_part_ml);
}

}  // namespace cb
