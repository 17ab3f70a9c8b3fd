// Prefill-chunk attention with bf16 MFMA tiles and an fp32 online softmax.
//
// Hugging Face blog "Continuous batching from first principles": scores cost O(n^2 d)
// (section "Attention"); a chunk attends to the cached keys of its own request plus its own
// keys, with the causal mask cut "in the middle" (section "Chunked prefill"); requests
// never see each other (section "Continuous batching"). zhangchitc "continuous-batching":
// masked pairs are not computed at all, and the cache is read one block at a time into a
// running online-softmax state.
//
// One work-group (4 or 8 waves) = 32 query rows per wave of one request: 128 or 256 rows of
// one query head, or fewer rows of several query heads that share one kv head (grouped-query
// attention: the waves then split into heads x row blocks and read the same key/value
// tiles). Each wave owns 32 rows of one head. Keys stream through LDS in tiles of 64 (4 cache blocks),
// double-buffered, and the global loads of later tiles overlap the current tile's math.
// The products are computed transposed so that the query index stays the lane index:
//   S^T[key][q] = K Q^T      A = K tile rows from LDS, B = the wave's Q rows (registers)
//   O^T[d][q]  += V^T P^T    A = V^T rows from LDS (the cache stores V transposed),
//                            B = P^T, which is exactly the S^T accumulator layout
// with v_mfma_f32_32x32x16_bf16. Each lane owns one query column, so the row max, the
// rescale factor and the row sum are per-lane values. Only the two lane halves (keys split
// across lanes l and l^32) exchange the max. Within a 16-key MFMA step the key order is
// permuted identically for A and B, so that P needs no shuffles. Tiles that lie past every
// row of a wave are skipped, and the causal mask is only evaluated on tiles that cross the
// diagonal.
#pragma once

#include "cb_device.h"

namespace cb {

template <int D>
struct PrefillGeom {
  static constexpr int KS = D + 8;                    // K tile row stride (elements)
  static constexpr int VS = kPrefillKeys + 8;         // V^T tile row stride (elements, 16-B rows)
  static constexpr int K_TILE = kPrefillKeys * KS;
  static constexpr int V_TILE = D * VS;
  static constexpr int LDS_ELEMS = 2 * (K_TILE + V_TILE);
  static constexpr int DCH = D / 16;                  // MFMA k-steps over the head dim
  static constexpr int DT = D / 32;                   // 32-wide output tiles over the head dim
};

// instruction classes for __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x0002;
constexpr int kSchedMfma = 0x0008;
constexpr int kSchedDsRead = 0x0100;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One prefill work-group's tile (work-group `slot` of the launch order). Every thread of the
// work-group calls it; it holds the LDS staging buffers of the kernel that inlines it.
template <int D, int NW>
__device__ __forceinline__ void prefill_tile(PrefillArgs a, int slot) {
  using Geo = PrefillGeom<D>;
  constexpr int NT = 64 * NW;                           // threads
  constexpr int ROWS = 32 * NW;                         // row x head pairs of the work-group
  constexpr int KS = Geo::KS, VS = Geo::VS, DCH = Geo::DCH, DT = Geo::DT;
  __shared__ __align__(16) uint16_t lds[Geo::LDS_ELEMS];

  if (a.desc) resolve_desc(a);
  if (slot >= a.n_items) return;                              // past a replayed step's items
  const PrefillItem it = a.items[slot];
  if (it.req < 0) return;                                     // padding slot of the launch order
  const int hl = it.heads_log2;                               // query heads of the work-group
  const int rows_wg = ROWS >> hl;                             // query rows of the work-group
  const int r = it.req;
  const int hkv = a.num_kv_heads;
  const int g = it.head / (a.num_q_heads / hkv);
  const int t0 = a.cu_q_lens[r];
  const int nq = a.cu_q_lens[r + 1] - t0;
  const int c = a.ctx_lens[r];
  const int kv_len = c + nq;
  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = wave_id();
  const int col = lane & 31, grp = lane >> 5;
  const int h = it.head + (wave & ((1 << hl) - 1));          // this wave's query head
  const int wave_row0 = it.q_begin + (wave >> hl) * 32;      // first row of this wave
  const int qrow = wave_row0 + col;                           // this lane's row in the request
  const bool wave_active = wave_row0 < nq;
  const int wave_keys = c + min(wave_row0 + 31, nq - 1) + 1;  // keys any row of the wave sees
  const int wg_keys = c + min(it.q_begin + rows_wg - 1, nq - 1) + 1;
  const int kt0 = it.kt_begin;                                // absolute first key tile
  const int n_tiles = it.kt_end - kt0;                        // tiles of this item (local 0..)
  const int32_t* bt = a.block_tables + it.bt_row;
  const int64_t page_elems = static_cast<int64_t>(kBlockSize) * D;
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);

  // the wave's query rows as the B operand of K Q^T: Q[qrow][16*dc + 8*grp .. +8]
  bf16x8 qf[DCH];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (static_cast<int64_t>(t0 + qrow) * a.num_q_heads + h) * D;
#pragma unroll
    for (int dc = 0; dc < DCH; ++dc) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qrow < nq) v = *reinterpret_cast<const u32x4*>(qp + dc * 16 + grp * 8);
      qf[dc] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // global -> registers for key tile j. Every load instruction of a wave reads one page of
  // the tile (positions 64j+16p .. +15), so its block id is a scalar and each thread's offset
  // inside the page is fixed: K row tl/(D/8), chunk tl%(D/8); V^T bytes tl*16 (d-row tl/2,
  // key octet tl%2). At D = 128 a page is one 16-byte chunk per thread (4 loads cover the 4
  // pages); at D = 64 the two halves of the work-group take two pages per load. Only the
  // tile that reaches wg_keys (the last key any row of this work-group sees) clamps pages
  // and zeroes positions past it.
  constexpr int TPP = 2 * D;                                       // threads per page (16 B each)
  constexpr int PPL = NT / TPP;                                    // pages per load
  constexpr int NL = 4 / PPL;                                      // loads per tile
  static_assert(NL * PPL == 4, "a tile is 4 pages");
  // Register staging: with 8 waves (one work-group per CU) there are registers for two
  // sets, so tiles are requested two steps before they are stored to LDS; with 4 waves one.
  constexpr int NSET = NW == 8 ? 2 : 1;
  u32x4 kreg[NSET][NL], vreg[NSET][NL];
  const int tl = tid % TPP;                                        // thread within its page
  // Block id of key page pidx (clamped to the last page the work-group sees). The index is
  // wave-uniform, so the id comes through the scalar cache straight into a scalar register;
  // ids outside the pool read block 0.
  const int last_page = __builtin_amdgcn_readfirstlane((wg_keys - 1) / kBlockSize);
  auto page_block = [&](int pidx) -> int {
    const int i = __builtin_amdgcn_readfirstlane(min(pidx, last_page));
    const int blk = __builtin_amdgcn_readfirstlane(__builtin_nontemporal_load(bt + i));
    return static_cast<unsigned>(blk) < static_cast<unsigned>(a.num_blocks) ? blk : 0;
  };
  auto load_tile = [&](int j, int set) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int page = u * PPL + tid / TPP;                // wave-uniform
      const int64_t base = (static_cast<int64_t>(page_block(j * 4 + page)) * hkv + g) * page_elems;
      kreg[set][u] = *reinterpret_cast<const u32x4*>(kc + base + (tl / (D / 8)) * D + (tl % (D / 8)) * 8);
      vreg[set][u] = *reinterpret_cast<const u32x4*>(vc + base + tl * 8);
    }
    if ((j + 1) * kPrefillKeys > wg_keys) {        // the last tile: zero keys >= wg_keys
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int page = u * PPL + tid / TPP;
        const int kpos = j * kPrefillKeys + page * kBlockSize + tl / (D / 8);
        if (kpos >= wg_keys) kreg[set][u] = u32x4{0u, 0u, 0u, 0u};
        const int vpos = j * kPrefillKeys + page * kBlockSize + (tl % 2) * 8;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int p0 = vpos + 2 * w;
          vreg[set][u][w] &= (p0 < wg_keys ? 0x0000ffffu : 0u) | (p0 + 1 < wg_keys ? 0xffff0000u : 0u);
        }
      }
    }
  };
  auto store_tile = [&](int buf, int set) {
    uint16_t* kl = lds + buf * Geo::K_TILE;
    uint16_t* vl = lds + 2 * Geo::K_TILE + buf * Geo::V_TILE;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int page = u * PPL + tid / TPP;
      *reinterpret_cast<u32x4*>(kl + (page * kBlockSize + tl / (D / 8)) * KS + (tl % (D / 8)) * 8) = kreg[set][u];
      // Inside each 16-key page, key k sits at position (k&3) + 4*(k>>3) + 8*((k>>2)&1):
      // positions 0..7 then hold keys 0-3 and 8-11, positions 8..15 keys 4-7 and 12-15, the
      // two key sets that lanes 0-31 and 32-63 take in one 32x32x16 step (the S^T accumulator
      // layout). The thread's octet tl%2 = h (keys 8h..8h+7) goes to positions 4h.. and 8+4h..
      uint16_t* vrow = vl + (tl / 2) * VS + page * kBlockSize + (tl % 2) * 4;
      *reinterpret_cast<u32x2*>(vrow) = u32x2{vreg[set][u][0], vreg[set][u][1]};
      *reinterpret_cast<u32x2*>(vrow + 8) = u32x2{vreg[set][u][2], vreg[set][u][3]};
    }
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int qpos = c + qrow;

  // S^T for the 64 keys of the tile in LDS buffer `buf`: two 32-key accumulators
  auto compute_s = [&](int buf, f32x16 (&st)[2]) {
    const uint16_t* kl = lds + buf * Geo::K_TILE;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st[kt][i] = 0.f;
#pragma unroll
    for (int dc = 0; dc < DCH; ++dc)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {   // two independent accumulation chains, interleaved
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kl + (kt * 32 + col) * KS + dc * 16 + grp * 8);
        st[kt] = mfma32(ka, qf[dc], st[kt]);
      }
  };

  // Row max of a 64-key score tile (four independent chains, then lanes l and l^32)
  auto tile_max = [&](const f32x16 (&st)[2]) -> float {
    float mq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) mq[q] = fmaxf(st[q >> 1][(q & 1) * 8], st[q >> 1][(q & 1) * 8 + 1]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 2; i < 8; ++i) mq[q] = fmaxf(mq[q], st[q >> 1][(q & 1) * 8 + i]);
    const float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };

  // One key tile j whose scores are in s_cur and whose unmasked row max is mx: mask,
  // softmax, O += V P. The scores of tile j+1 (other LDS buffer) are computed into s_next in
  // the same straight-line block as the exp2 work of tile j, and their row max at its end,
  // beside the P.V MFMAs, so the matrix core and the vector ALU overlap within the wave.
  // Only tiles that cross the causal diagonal need a mask (every key of another tile is
  // visible to every row of the wave), and only those recompute the max after it.
  auto tile_step = [&](int u, f32x16 (&s_cur)[2], f32x16 (&s_next)[2], float& mx) {
    const int buf = u & 1;                       // local index: buffers and register sets
    const int j = kt0 + u;                       // absolute tile: positions and masks
    if (!wave_active || j * kPrefillKeys >= wave_keys) return;
    const bool diag = __builtin_amdgcn_readfirstlane(j * kPrefillKeys + kPrefillKeys - 1 > c + wave_row0);
    if (diag) {                                  // causal mask, only on tiles crossing it
      const int rel = qpos - j * kPrefillKeys - grp * 4;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kt * 32 + (i >> 2) * 8 + (i & 3) > rel) s_cur[kt][i] = -INFINITY;
      mx = tile_max(s_cur);
    }
    // Lazy rescaling: the reference max only moves when some lane's max grew by more than
    // 8 (log2 units). Until then probabilities may reach 2^8, which fp32 sums and bf16 P
    // hold as well as values below 1; O and l share the reference, so O / l is unchanged.
    // The scale is positive, so max(scale*s) = scale*max(s) and it folds into the fma.
    const float m_cand = fmaxf(m_run, mx * a.scale_log2);
    if (__builtin_amdgcn_readfirstlane(__ballot(m_cand > m_run + 8.f) != 0)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_cand);
      m_run = m_cand;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
    }
    compute_s(buf ^ 1, s_next);
    const float m_ref = m_run;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};          // four independent sum chains
    bf16x8 pb[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s_cur[kt][half * 8 + 2 * e], a.scale_log2, -m_ref));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s_cur[kt][half * 8 + 2 * e + 1], a.scale_log2, -m_ref));
          ps[kt * 2 + half] += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pb[kt * 2 + half] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
      }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    // O^T += V^T P^T over four 16-key steps; one 16-byte read per A operand (the key order
    // inside each 16-key page of the V^T tile matches the P layout, see store_tile)
    const uint16_t* vl = lds + 2 * Geo::K_TILE + buf * Geo::V_TILE;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)               // DT independent accumulators back to back
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vl + (dt * 32 + col) * VS + grp * 8 + ks * 16);
        oacc[dt] = mfma32(va, pb[ks], oacc[dt]);
      }
    mx = tile_max(s_next);
    // Instruction order for the block above (scheduler groups): each of its 32 MFMAs (the
    // next tile's scores, and the P.V products as soon as their quarter of P is packed)
    // is followed by an LDS operand read, issued four MFMAs ahead of its use, and three
    // vector instructions (the exp2/pack work of this tile, then the next tile's max).
    // Spreading the vector work over all 32 MFMAs measured 5% faster than over the 16
    // score MFMAs with the P.V MFMAs left bare.
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int k = 0; k < 2 * DCH + 4 * DT; ++k) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 3, 0);
    }
  };

  // prologue: tiles 0 and 1 in LDS, the scores of tile 0 computed, the next NSET tiles in
  // flight (tile t is staged in register set t % NSET)
  load_tile(kt0, 0);
  store_tile(0, 0);
  if (n_tiles > 1) load_tile(kt0 + 1, 1 % NSET);
  __syncthreads();
  f32x16 sa[2], sb[2];
  float mx = 0.f;                                // unmasked row max of the next tile's scores
  if (wave_active) {
    compute_s(0, sa);
    mx = tile_max(sa);
  }
  if (n_tiles > 1) {
    store_tile(1, 1 % NSET);
    if (n_tiles > 2) load_tile(kt0 + 2, 0);
    if (NSET == 2 && n_tiles > 3) load_tile(kt0 + 3, 1 % NSET);
  }
  __syncthreads();
  // Per tile j: step (reads buffer j&1, scores of j+1 from the other buffer), a barrier
  // (buffer j&1 is free), tile j+2 from its register set into it, the loads of tile
  // j+2+NSET into the same set, a barrier.
  // (A variant with separate key and value buffer rings and one barrier per tile measured
  // slower: the first barrier keeps the waves of the work-group in step.)
  auto advance = [&](int j) {
    __syncthreads();
    if (j + 2 < n_tiles) {
      store_tile(j & 1, j % NSET);
      if (j + 2 + NSET < n_tiles) load_tile(kt0 + j + 2 + NSET, j % NSET);
    }
    __syncthreads();
  };
  for (int j = 0; j < n_tiles; j += 2) {
    tile_step(j, sa, sb, mx);
    advance(j);
    if (j + 1 < n_tiles) {
      tile_step(j + 1, sb, sa, mx);
      advance(j + 1);
    }
  }

  if (!wave_active) return;
  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
  const float l_tot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
  if (qrow >= nq) return;
  if (it.part_base >= 0) {                     // one split of the key range: partials
    const int n_split = it.split >> 16;
    const int64_t part = it.part_base + static_cast<int64_t>(qrow - it.q_begin) * n_split + (it.split & 0xffff);
    float* po = a.part_o + (part * a.num_q_heads + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(po + dt * 32 + q4 * 8 + grp * 4) =
            f32x4{oacc[dt][q4 * 4 + 0], oacc[dt][q4 * 4 + 1], oacc[dt][q4 * 4 + 2], oacc[dt][q4 * 4 + 3]};
    if (grp == 0) {
      float* ml = a.part_ml + (part * a.num_q_heads + h) * 2;
      ml[0] = m_run;
      ml[1] = l_tot;
    }
    return;
  }
  const float inv = 1.f / l_tot;
  uint16_t* op = static_cast<uint16_t*>(a.o) + (static_cast<int64_t>(t0 + qrow) * a.num_q_heads + h) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = dt * 32 + q4 * 8 + grp * 4;
      const uint32_t w0 = pack_bf16x2(oacc[dt][q4 * 4 + 0] * inv, oacc[dt][q4 * 4 + 1] * inv);
      const uint32_t w1 = pack_bf16x2(oacc[dt][q4 * 4 + 2] * inv, oacc[dt][q4 * 4 + 3] * inv);
      *reinterpret_cast<u32x2*>(op + d) = u32x2{w0, w1};
    }
}

}  // namespace cb
