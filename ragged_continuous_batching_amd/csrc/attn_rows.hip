// Single-row attention over the paged cache, split-K, bandwidth-bound (decode rows).
//
// zhangchitc "continuous-batching", section "Inside the kernel": per request, the cache is
// read one physical block at a time; the block's scores weight its values and the result is
// accumulated into a running state (online softmax). Hugging Face blog, section
// "KV-cache": a decode token reads every cached key and value once, so the cost is the
// O(n) cache read.
//
// Work item = (split of a row's blocks, kv head): one 64-lane wave. The wave handles all G
// query heads that share the kv head, so each K/V page is read from HBM once per group.
// Per block (16 positions, one kv head):
//   K page [16][D], 4 KiB in bf16 at D=128: every lane loads 16-byte chunks, and a lane
//     group of RL lanes covers one key row. Dot products are per-lane partial sums
//     reduced over the group with DPP moves.
//   V page [D][16] (stored transposed): every lane loads 16 bytes = VEC positions of one
//     d-row, so P.V is a per-lane FMA chain over those positions.
//   The probabilities move from the K layout to the V layout through a 16-float LDS slot
//   per head.
// The running max lives in log2 units (scores pre-multiplied by scale*log2(e)) so that
// exp2 is the only transcendental. A row with one split writes O directly. Otherwise each
// split writes (unnormalised o, max, sum) and combine_kernel merges the splits:
//   M = max_s m_s,  O = sum_s 2^(m_s-M) o_s / sum_s 2^(m_s-M) l_s.
#include "cb_device.h"

namespace cb {

template <int ES, int D>
struct RowGeom {
  static constexpr int ROWB = D * ES;           // bytes of one key row
  static constexpr int RL = ROWB / 16;          // lanes per key row
  static constexpr int TPL = 64 / RL;           // key rows per load instruction
  static constexpr int NLK = kBlockSize / TPL;  // K loads per lane per page
  static constexpr int VEC = 16 / ES;           // elements per 16-byte chunk
  static constexpr int VL = kBlockSize * ES / 16;  // lanes per V d-row
  static constexpr int DPL = 64 / VL;           // d-rows per V load instruction
  static constexpr int NLV = D / DPL;           // V loads per lane per page
  static_assert(RL * TPL == 64 && NLK * TPL == kBlockSize, "K page must split over 64 lanes");
  static_assert(VL * VEC == kBlockSize && NLV * DPL == D, "V page must split over 64 lanes");
};

template <int ES>
__device__ __forceinline__ float dot_chunk(const u32x4& a, const u32x4& b, float acc) {
  if constexpr (ES == 2) {
    // Words are copied out through memcpy: this compiler miscompiles a bit_cast of a vector
    // element straight into the dot2 operand (it reuses element 0 for every word).
    uint32_t aw[4] = {a[0], a[1], a[2], a[3]}, bw[4] = {b[0], b[1], b[2], b[3]};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      bf16x2 x, y;
      __builtin_memcpy(&x, &aw[w], 4);
      __builtin_memcpy(&y, &bw[w], 4);
      acc = __builtin_amdgcn_fdot2_f32_bf16(x, y, acc, false);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = fmaf(__uint_as_float(a[w]), __uint_as_float(b[w]), acc);
  }
  return acc;
}

// Elements of a 16-byte chunk as fp32.
template <int ES>
__device__ __forceinline__ void chunk_to_f32(const u32x4& c, float (&out)[16 / ES]) {
  if constexpr (ES == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      out[2 * w] = bf16_lo(c[w]);
      out[2 * w + 1] = bf16_hi(c[w]);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) out[w] = __uint_as_float(c[w]);
  }
}

__device__ __forceinline__ void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int ES, int D, int G>
__global__ __launch_bounds__(256) void row_attn_kernel(RowArgs a) {
  using Geo = RowGeom<ES, D>;
  constexpr int RL = Geo::RL, NLK = Geo::NLK, VEC = Geo::VEC, VL = Geo::VL, DPL = Geo::DPL, NLV = Geo::NLV;
  static_assert(G <= RL, "one writer lane per head");
  __shared__ __align__(16) float p_lds[4][G][kBlockSize];

  if (a.desc) resolve_desc(a);
  const int lane = lane_id();
  const int wave = wave_id();
  const int item = blockIdx.x * 4 + wave;
  if (item >= a.n_items) return;
  const int hkv = a.num_kv_heads;
  const int q_per_kv = a.num_q_heads / hkv;
  const int n_sub = q_per_kv / G;
  const int split = item / (hkv * n_sub);
  const int rem = item - split * hkv * n_sub;
  const int g = rem / n_sub;
  const int h0 = g * q_per_kv + (rem - g * n_sub) * G;   // first q head of this item

  const RowSplit sp = a.splits[split];
  const int kg = lane / RL, kc = lane % RL;               // K layout: row group, 16-byte chunk
  const int vd = lane / VL, vt = (lane % VL) * VEC;       // V layout: d-row offset, first slot

  // query chunks of the G heads (dims kc*VEC .. +VEC)
  u32x4 qv[G];
  {
    const char* qbase = static_cast<const char*>(a.q) + (static_cast<int64_t>(sp.token) * a.num_q_heads + h0) * D * ES;
#pragma unroll
    for (int j = 0; j < G; ++j) qv[j] = *reinterpret_cast<const u32x4*>(qbase + (j * D + kc * VEC) * ES);
  }

  float m_run[G], l_run[G], acc[G][NLV];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
#pragma unroll
    for (int i = 0; i < NLV; ++i) acc[j][i] = 0.f;
  }

  const int32_t* bt = a.block_tables + sp.bt_row;
  const int64_t page_elems = static_cast<int64_t>(kBlockSize) * D;
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);

  auto load_block = [&](int b, u32x4 (&kr)[NLK], u32x4 (&vr)[NLV]) {
    int blk = bt[b];
    if (static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks)) {
      note_violation(lane == 0);
      blk = 0;
    }
    const int64_t page = (static_cast<int64_t>(blk) * hkv + g) * page_elems * ES;
    // each page is read once per step: non-temporal loads keep it from displacing lines
    // that other waves still need (measured: +8% streaming read bandwidth on MI355X)
    const char* kp = kbase + page + (kg * NLK * D + kc * VEC) * ES;
#pragma unroll
    for (int i = 0; i < NLK; ++i) kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + i * D * ES));
    const char* vp = vbase + page + lane * 16;
#pragma unroll
    for (int i = 0; i < NLV; ++i) vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + i * 1024));
  };

  float* pw = &p_lds[wave][0][0];

  auto process = [&](int b, const u32x4 (&kr)[NLK], const u32x4 (&vr)[NLV]) {
    const int pos0 = b * kBlockSize;
    // scores s[j][i] for key rows kg*NLK + i
    float s[G][NLK];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int i = 0; i < NLK; ++i) s[j][i] = group_sum<RL>(dot_chunk<ES>(qv[j], kr[i], 0.f)) * a.scale_log2;
    if (pos0 + kBlockSize > sp.kv_len) {
#pragma unroll
      for (int i = 0; i < NLK; ++i)
        if (pos0 + kg * NLK + i >= sp.kv_len)
#pragma unroll
          for (int j = 0; j < G; ++j) s[j][i] = -INFINITY;
    }
    float alpha[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float bm = s[j][0];
#pragma unroll
      for (int i = 1; i < NLK; ++i) bm = fmaxf(bm, s[j][i]);
      bm = strided_max<RL>(bm);
      const float m_new = fmaxf(m_run[j], bm);
      alpha[j] = __builtin_amdgcn_exp2f(m_run[j] - m_new);
      m_run[j] = m_new;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < NLK; ++i) {
        s[j][i] = __builtin_amdgcn_exp2f(s[j][i] - m_new);
        ps += s[j][i];
      }
      l_run[j] = l_run[j] * alpha[j] + ps;
    }
    // probabilities to LDS in position order: head j is written by the lanes with kc == j
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (kc == j) {
#pragma unroll
        for (int i = 0; i < NLK; ++i) pw[j * kBlockSize + kg * NLK + i] = s[j][i];
      }
    }
    wave_fence();
    float vf[NLV][VEC];
#pragma unroll
    for (int i = 0; i < NLV; ++i) chunk_to_f32<ES>(vr[i], vf[i]);
    if (pos0 + kBlockSize > sp.kv_len) {   // stale slots past the end may hold anything
#pragma unroll
      for (int u = 0; u < VEC; ++u)
        if (pos0 + vt + u >= sp.kv_len)
#pragma unroll
          for (int i = 0; i < NLV; ++i) vf[i][u] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float pr[VEC];
#pragma unroll
      for (int u = 0; u < VEC; ++u) pr[u] = pw[j * kBlockSize + vt + u];
#pragma unroll
      for (int i = 0; i < NLV; ++i) {
        float t = acc[j][i] * alpha[j];
#pragma unroll
        for (int u = 0; u < VEC; ++u) t = fmaf(pr[u], vf[i][u], t);
        acc[j][i] = t;
      }
    }
    wave_fence();
  };

  // Two blocks in flight. In the steady-state loop every load is issued on every path, so the
  // compiler's wait before each block's first use counts exactly the loads issued after it:
  // loads issued only on some paths (the split's last blocks) would make it wait, on every
  // path, as if they were never issued, draining the next block's loads before this one's
  // dot products start. A split of one block reads it twice (its second load is never used).
  u32x4 kA[NLK], vA[NLV], kB[NLK], vB[NLV];
  const int b0 = sp.blk_begin, b1 = sp.blk_end;
  load_block(b0, kA, vA);
  load_block(min(b0 + 1, b1 - 1), kB, vB);
  int b = b0;
  for (; b + 3 < b1; b += 2) {
    process(b, kA, vA);
    __builtin_amdgcn_sched_barrier(0);     // the next loads reuse this block's registers
    load_block(b + 2, kA, vA);
    process(b + 1, kB, vB);
    __builtin_amdgcn_sched_barrier(0);
    load_block(b + 3, kB, vB);
  }
  // the last one to three blocks
  process(b, kA, vA);
  if (b + 2 < b1) load_block(b + 2, kA, vA);
  if (b + 1 < b1) process(b + 1, kB, vB);
  if (b + 2 < b1) process(b + 2, kA, vA);

  // reduce over the VL lanes that share a d-row, and the sums over key-row groups
  const bool writer = (lane % VL) == 0;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float l_tot = strided_sum<RL>(l_run[j]);
    const int h = h0 + j;
#pragma unroll
    for (int i = 0; i < NLV; ++i) {
      const float v = group_sum<VL>(acc[j][i]);
      const int d = i * DPL + vd;
      if (writer) {
        if (sp.part < 0) {
          const float o = v / l_tot;
          const int64_t idx = (static_cast<int64_t>(sp.token) * a.num_q_heads + h) * D + d;
          if constexpr (ES == 2)
            static_cast<uint16_t*>(a.o)[idx] = to_bf16_bits(o);
          else
            static_cast<float*>(a.o)[idx] = o;
        } else {
          a.part_o[(static_cast<int64_t>(sp.part) * a.num_q_heads + h) * D + d] = v;
        }
      }
    }
    if (sp.part >= 0 && lane == 0) {
      float* ml = a.part_ml + (static_cast<int64_t>(sp.part) * a.num_q_heads + h) * 2;
      ml[0] = m_run[j];
      ml[1] = l_tot;
    }
  }
}

// Merge the splits of one row and query head: one wave per (row, head). Lane s holds split
// s's (max, sum); the weights 2^(m_s - M) are broadcast from their lanes while every lane
// accumulates D/64 output dims.
template <int ES, int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  if (a.desc) resolve_desc(a);
  const int item = blockIdx.x * 4 + wave_id();
  if (item >= a.n_rows * a.num_q_heads) return;
  const int lane = lane_id();
  const CombineRow row = a.rows[item / a.num_q_heads];
  const int h = item % a.num_q_heads;
  const int64_t stride = static_cast<int64_t>(a.num_q_heads);
  const float* ml = a.part_ml + (static_cast<int64_t>(row.part_begin) * stride + h) * 2;
  const float* po = a.part_o + (static_cast<int64_t>(row.part_begin) * stride + h) * D + lane;

  float mx = -INFINITY;
  for (int s = lane; s < row.n_parts; s += 64) mx = fmaxf(mx, ml[s * stride * 2]);
  mx = strided_max<1>(mx);
  float den = 0.f;
  float num[D / 64];
#pragma unroll
  for (int k = 0; k < D / 64; ++k) num[k] = 0.f;
  for (int s0 = 0; s0 < row.n_parts; s0 += 64) {
    const int s = s0 + lane;
    float w = 0.f;
    if (s < row.n_parts) {
      w = __builtin_amdgcn_exp2f(ml[s * stride * 2] - mx);
      den = fmaf(w, ml[s * stride * 2 + 1], den);
    }
    const int n = min(64, row.n_parts - s0);
    int t = 0;
    for (; t + 4 <= n; t += 4) {
      float wt[4], v[4][D / 64];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wt[u] = __shfl(w, t + u);
#pragma unroll
        for (int k = 0; k < D / 64; ++k) v[u][k] = po[(s0 + t + u) * stride * D + k * 64];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < D / 64; ++k) num[k] = fmaf(wt[u], v[u][k], num[k]);
    }
    for (; t < n; ++t) {
      const float wt = __shfl(w, t);
#pragma unroll
      for (int k = 0; k < D / 64; ++k) num[k] = fmaf(wt, po[(s0 + t) * stride * D + k * 64], num[k]);
    }
  }
  den = strided_sum<1>(den);
  const float inv = 1.f / den;
  const int64_t base = (static_cast<int64_t>(row.token) * a.num_q_heads + h) * D + lane;
#pragma unroll
  for (int k = 0; k < D / 64; ++k) {
    if constexpr (ES == 2)
      static_cast<uint16_t*>(a.o)[base + k * 64] = to_bf16_bits(num[k] * inv);
    else
      static_cast<float*>(a.o)[base + k * 64] = num[k] * inv;
  }
}

template <int ES, int D, int G>
static hipError_t launch_rows_t(const RowArgs& a, hipStream_t s) {
  const int blocks = (a.n_items + 3) / 4;
  hipLaunchKernelGGL((row_attn_kernel<ES, D, G>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int ES, int D>
static hipError_t launch_rows_d(const RowArgs& a, int g, hipStream_t s) {
  switch (g) {
    case 1: return launch_rows_t<ES, D, 1>(a, s);
    case 2: return launch_rows_t<ES, D, 2>(a, s);
    case 4: return launch_rows_t<ES, D, 4>(a, s);
    default: return launch_rows_t<ES, D, 8>(a, s);
  }
}

// group: query heads handled per wave (1, 2, 4 or 8; a larger group is covered by several
// sub-groups of 8, counted in n_items).
hipError_t launch_rows(const RowArgs& a, int elem_bytes, int head_dim, int group, hipStream_t s) {
  if (a.n_items == 0) return hipSuccess;
  if (elem_bytes == 2) return head_dim == 128 ? launch_rows_d<2, 128>(a, group, s) : launch_rows_d<2, 64>(a, group, s);
  return head_dim == 128 ? launch_rows_d<4, 128>(a, group, s) : launch_rows_d<4, 64>(a, group, s);
}

hipError_t launch_combine(const CombineArgs& a, int elem_bytes, int head_dim, hipStream_t s) {
  if (a.n_rows == 0) return hipSuccess;
  auto k = elem_bytes == 2 ? (head_dim == 128 ? combine_kernel<2, 128> : combine_kernel<2, 64>)
                           : (head_dim == 128 ? combine_kernel<4, 128> : combine_kernel<4, 64>);
  const int64_t waves = static_cast<int64_t>(a.n_rows) * a.num_q_heads;
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

CB_VIOLATION_READER(violations_rows)

}  // namespace cb
