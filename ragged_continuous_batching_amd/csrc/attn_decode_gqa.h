// Single-row (decode) attention for grouped-query heads, split-K, with the per-block
// contractions on the matrix cores.
//
// Same work and the same online softmax as row_attn_kernel (zhangchitc "continuous-batching",
// section "Inside the kernel": the cache is read one physical block at a time and each
// block's scores weight its values into a running state). When G = Hq/Hkv query heads share
// a kv head, one block of one kv head meets G queries. Scoring it is a [16 keys x D] by
// [D x G] product, and weighting its values is a [D x 16] by [16 x G] product. With G >= 4
// these run on v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x16_bf16, with the G heads as
// the 16 columns (G < 16 leaves columns empty). The vector-ALU form of the same step would
// be compute-bound at G = 8, while this form stays bound by the cache read.
//
// Work item = (split, kv head, group of up to 16 query heads): one wave.
//   S^T[key][head] = K Q^T   A = K page rows (lane: key l%16, 8 dims), B = Q (registers)
//   O^T[d][head]  += V^T P^T A = V^T page rows (lane: d-row l%16, 4 keys = 8 contiguous
//                            bytes), B = P^T, which is the S^T accumulator layout as is
// Each lane owns head l%16 and keys 4*(l/16)..+3 of the block, so the row statistics need
// two cross-lane steps (lanes l^16, l^32). Splits, partial outputs and the combine pass are
// shared with row_attn_kernel.
#pragma once

#include "cb_device.h"

namespace cb {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// The four waves of decode work-group `wg`: wave w takes work item 4*wg + w.
template <int D>
__device__ __forceinline__ void row_attn_mfma_waves(RowArgs a, int wg) {
  constexpr int KC = D / 32;            // 16x16x32 steps over the head dim (scores)
  constexpr int DT = D / 16;            // 16-row output tiles over the head dim
  if (a.desc) resolve_desc(a);
  const int lane = lane_id();
  const int wave = wave_id();
  const int item = wg * 4 + wave;
  if (item >= a.n_items) return;
  const int hkv = a.num_kv_heads;
  const int q_per_kv = a.num_q_heads / hkv;
  const int gw = a.group;                                  // heads per wave (4, 8 or 16)
  const int n_sub = q_per_kv / gw;
  const int split = item / (hkv * n_sub);
  const int rem = item - split * hkv * n_sub;
  const int g = rem / n_sub;
  const int h0 = g * q_per_kv + (rem - g * n_sub) * gw;
  const RowSplit sp = a.splits[split];
  const int col = lane & 15, grp = lane >> 4;            // head column, key / k group
  const bool head_ok = col < gw;

  // Q^T as the B operand: lane holds Q[head col][32*kc + 8*grp .. +8]
  bf16x8 qb[KC];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<int64_t>(sp.token) * a.num_q_heads + h0 + (head_ok ? col : 0)) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qp + kc * 32 + grp * 8);
      if (!head_ok) v = u32x4{0u, 0u, 0u, 0u};
      qb[kc] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int32_t* bt = a.block_tables + sp.bt_row;
  const int64_t page_elems = static_cast<int64_t>(kBlockSize) * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache);

  auto load_block = [&](int b, u32x4 (&kr)[KC], u32x2 (&vr)[DT]) {
    int blk = bt[b];
    if (static_cast<unsigned>(blk) >= static_cast<unsigned>(a.num_blocks)) {
      note_violation(threadIdx.x % 64 == 0);
      blk = 0;
    }
    const int64_t page = (static_cast<int64_t>(blk) * hkv + g) * page_elems;
    // K row `col`, dims 32*kc + 8*grp: each load reads 64 contiguous bytes of every row
    const uint16_t* kp = kbase + page + col * D + grp * 8;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) kr[kc] = *reinterpret_cast<const u32x4*>(kp + kc * 32);
    // V^T rows 16t+col, keys 4*grp..+3: each load reads 512 contiguous bytes
    const uint16_t* vp = vbase + page + col * kBlockSize + grp * 4;
#pragma unroll
    for (int t = 0; t < DT; ++t)
      vr[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vp + t * 16 * kBlockSize));
  };

  auto process = [&](int b, const u32x4 (&kr)[KC], u32x2 (&vr)[DT]) {
    const int pos0 = b * kBlockSize + grp * 4;           // position of this lane's first key
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kc]), qb[kc], st, 0, 0, 0);
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = pos0 + i < sp.kv_len ? st[i] * a.scale_log2 : -INFINITY;
    float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
      bm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float m_new = fmaxf(m_run, bm);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(s[i] - m_new);
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    const uint32_t w0 = pack_bf16x2(p[0], p[1]), w1 = pack_bf16x2(p[2], p[3]);
    const s16x4 pbv = __builtin_bit_cast(s16x4, u32x2{w0, w1});
    if (b * kBlockSize + kBlockSize > sp.kv_len) {       // stale slots past the end: zero V
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const int q0 = pos0 + 2 * w;
          vr[t][w] &= (q0 < sp.kv_len ? 0x0000ffffu : 0u) | (q0 + 1 < sp.kv_len ? 0xffff0000u : 0u);
        }
    }
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      oacc[t] *= alpha;
      oacc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vr[t]), pbv, oacc[t], 0, 0, 0);
    }
  };

  // three blocks in flight per wave (two waves per SIMD: measured slightly ahead of two
  // blocks at three waves per SIMD)
  u32x4 kA[KC], kB[KC], kC[KC];
  u32x2 vA[DT], vB[DT], vC[DT];
  const int b0 = sp.blk_begin, b1 = sp.blk_end;
  load_block(b0, kA, vA);
  if (b0 + 1 < b1) load_block(b0 + 1, kB, vB);
  for (int b = b0; b < b1; b += 3) {
    if (b + 2 < b1) load_block(b + 2, kC, vC);
    process(b, kA, vA);
    if (b + 3 < b1) load_block(b + 3, kA, vA);
    if (b + 1 < b1) process(b + 1, kB, vB);
    if (b + 4 < b1) load_block(b + 4, kB, vB);
    if (b + 2 < b1) process(b + 2, kC, vC);
  }

  // each lane summed its own keys; add the other three key groups
  float l_tot = l_run + __shfl_xor(l_run, 16);
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_tot), __float_as_uint(l_tot), false, false);
    l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (!head_ok) return;
  const int h = h0 + col;
  // lane holds O^T rows d = 16t + 4*grp + i (i = 0..3) of head h
  if (sp.part < 0) {
    const float inv = 1.f / l_tot;
    uint16_t* op = static_cast<uint16_t*>(a.o) + (static_cast<int64_t>(sp.token) * a.num_q_heads + h) * D + grp * 4;
#pragma unroll
    for (int t = 0; t < DT; ++t)
      *reinterpret_cast<u32x2*>(op + t * 16) =
          u32x2{pack_bf16x2(oacc[t][0] * inv, oacc[t][1] * inv), pack_bf16x2(oacc[t][2] * inv, oacc[t][3] * inv)};
  } else {
    float* po = a.part_o + (static_cast<int64_t>(sp.part) * a.num_q_heads + h) * D + grp * 4;
#pragma unroll
    for (int t = 0; t < DT; ++t) *reinterpret_cast<f32x4*>(po + t * 16) = oacc[t];
    if (grp == 0) {
      float* ml = a.part_ml + (static_cast<int64_t>(sp.part) * a.num_q_heads + h) * 2;
      ml[0] = m_run;
      ml[1] = l_tot;
    }
  }
}

}  // namespace cb
