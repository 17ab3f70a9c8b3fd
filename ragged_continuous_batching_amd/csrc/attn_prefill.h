// Prefill-chunk attention with bf16 MFMA tiles and an fp32 online softmax.
//
// Hugging Face blog "Continuous batching from first principles": scores cost O(n^2 d)
// (section "Attention"); a chunk attends to the cached keys of its own request plus its own
// keys, its rows sitting after the cached positions so the causal mask is aligned to the
// bottom right (section "Chunked prefill"); requests never see each other (section
// "Continuous batching"). zhangchitc "continuous-batching":
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
// across lanes l and l^32) exchange the max. The K rows are fed to the score MFMA in a
// permuted order (see compute_s) that makes the S^T accumulator hold each lane's keys in
// natural order, so P^T needs no shuffles and V^T is read as it is stored. Tiles that lie
// past every row of a wave are skipped, and the causal mask is only evaluated on tiles that
// cross the diagonal.
//
// Key and value tiles go from the cache straight into LDS (buffer_load_dwordx4 ... lds: no
// staging registers and no LDS store instructions) through two K buffers and two V
// buffers; in an eight-wave work-group only waves 0-3 issue them (see the direct loads).
// Tile t's keys are first read one step before its values (the scores of tile t
// are computed while tile t-1's probabilities are applied), so K(t+3) and V(t+2) are
// requested right after the barrier that ends step t, and waited for at the end of step
// t+1: one barrier per tile.
#pragma once

#include "cb_device.h"

namespace cb {

template <int D>
struct PrefillGeom {
  static constexpr int PAGE_BYTES = kBlockSize * D * 2;   // one cache page: 16 positions x D bf16
  static constexpr int TILE_BYTES = 4 * PAGE_BYTES;       // 64 keys
  static constexpr int IPP = PAGE_BYTES / 1024;           // 1-KB direct loads per page (D / 32)
  static constexpr int DCH = D / 16;                      // MFMA k-steps over the head dim
  static constexpr int DT = D / 32;                       // 32-wide output tiles over the head dim
};

// instruction classes for __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x0002;
constexpr int kSchedMfma = 0x0008;
constexpr int kSchedDsRead = 0x0100;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16 bytes at byte offset `off` (per lane) of the buffer `rs` into LDS at lds_base + lane * 16
// (lds_base uniform). The buffer form (not the flat global one): the compiler counts a flat
// access to LDS as able to finish out of order with LDS reads, and would then make every
// wait for an LDS operand a full wait.
__device__ __forceinline__ void load_to_lds(__amdgpu_buffer_rsrc_t rs, uint32_t off, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds_base), 16, off, 0, 0, 0);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt not waited for): every global load of this wave,
// the direct-to-LDS ones included, has landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// One prefill work-group's tile (work-group `slot` of the launch order). Every thread of the
// work-group calls it; it holds the LDS buffers of the kernel that inlines it.
template <int D, int NW>
__device__ __forceinline__ void prefill_tile(PrefillArgs a, int slot) {
  using Geo = PrefillGeom<D>;
  constexpr int ROWS = 32 * NW;                         // row x head pairs of the work-group
  constexpr int DCH = Geo::DCH, DT = Geo::DT, PAGE = Geo::PAGE_BYTES, IPP = Geo::IPP;
  // LDS layout of one tile (4 pages of 16 positions):
  //   K buffer: page p at p*PAGE, stored chunk-major: the 16-byte chunk c (elements
  //     8c..8c+7) of position r at c*256 + r*16. A score MFMA operand (16 lanes on 16
  //     positions, one chunk) then spans all 64 banks, and the chunks of an operand
  //     differ by a constant offset.
  //   V buffer: page p at p*PAGE, d-row d (the page's 16 positions of dimension d, 32 bytes)
  //     at d*32, its two 8-position halves swapped in rows with bit 3 of d set (half h at
  //     16*(h ^ bit3(d))), so a P.V operand (16 lanes on 16 d-rows, one half) spans all 64
  //     banks.
  // Each buffer is its own array, so that the compiler sees that a direct load into one
  // buffer never aliases a read of another and adds no waits for it.
  __shared__ __align__(1024) uint8_t kb0[Geo::TILE_BYTES], kb1[Geo::TILE_BYTES];
  __shared__ __align__(1024) uint8_t vb0[Geo::TILE_BYTES], vb1[Geo::TILE_BYTES];

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
  const uint8_t* kc = static_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vc = static_cast<const uint8_t*>(a.v_cache);

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

  // Direct loads: a tile is four cache pages of keys and four of values, each page IPP 1-KB
  // pieces. Only waves 0-3 load: loading wave w takes page w of every tile, its IPP pieces of
  // keys and of values. Each lane's source offset inside its cache page is fixed; only the
  // page's block id changes from tile to tile (one id per wave and tile, the same in every
  // lane). A CU's load path moves about 64 bytes per clock, so a tile's 32 KB keep it busy
  // for about 512 clocks, and a wave that issues a load waits until the path takes it. In an
  // eight-wave work-group waves w and w+4 share a SIMD, so while the loading wave of a SIMD
  // waits, its partner keeps the matrix core busy (config 4 measured 3409 -> 3136 clocks per
  // key tile and wave; when all eight waves loaded, both waves of a SIMD waited together).
  // Four-wave work-groups have one wave per SIMD, and every wave loads.
  constexpr int NL = 4;                                            // waves that load tiles
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  const bool loader = wave < NL;
  const int pw = wave;                                             // page of a loading wave
  // LDS offset of this wave's page in a buffer. Made opaque where it is used, so the
  // compiler computes each piece's LDS address at its load instead of keeping all of them in
  // scalar registers through the loop (which spilled them into vector-register lanes).
  auto page_lds = [&]() {
    int o = pw * PAGE;
    asm volatile("" : "+s"(o));
    return static_cast<uint32_t>(o);
  };
  uint32_t ksrc[IPP], vsrc[IPP];
#pragma unroll
  for (int part = 0; part < IPP; ++part) {
    // keys: chunks 4*part .. 4*part+3 of positions 0..15 (lane: chunk 4*part + lane/16,
    // position lane%16)
    ksrc[part] = (lane % 16) * (2 * D) + (4 * part + lane / 16) * 16;
    // values: d-rows 32*part .. +31 (lane: row 32*part + lane/2, stored half lane%2)
    const int d = 32 * part + lane / 2;
    vsrc[part] = d * 32 + ((lane & 1) ^ ((d >> 3) & 1)) * 16;
  }
  // Block id of key page pidx (clamped to the last page the work-group sees; ids outside the
  // pool read block 0). The index is wave-uniform.
  const int last_page = __builtin_amdgcn_readfirstlane((wg_keys - 1) / kBlockSize);
  auto page_of = [&](int t) { return min((kt0 + t) * 4 + pw, last_page); };   // this wave's page of tile t
  auto valid_block = [&](int blk) {
    const bool ok = static_cast<unsigned>(blk) < static_cast<unsigned>(a.num_blocks);
    note_violation(!ok && lane == 0);
    return ok ? blk : 0;
  };
  // a buffer resource over one cache page (its byte range bounds the lanes' offsets)
  auto page_rsrc = [&](const uint8_t* cache, int blk) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(cache + (static_cast<int64_t>(blk) * hkv + g) * PAGE),
                                             0, PAGE, kBufferFlags);
  };
  auto load_k = [&](uint8_t* dst, int blk) {
    const __amdgpu_buffer_rsrc_t rs = page_rsrc(kc, blk);
    const uint32_t base = page_lds();
#pragma unroll
    for (int part = 0; part < IPP; ++part) load_to_lds(rs, ksrc[part], dst + base + part * 1024);
  };
  auto load_v = [&](uint8_t* dst, int blk) {
    const __amdgpu_buffer_rsrc_t rs = page_rsrc(vc, blk);
    const uint32_t base = page_lds();
#pragma unroll
    for (int part = 0; part < IPP; ++part) load_to_lds(rs, vsrc[part], dst + base + part * 1024);
  };
  // The tile that reaches wg_keys (the last key any row of this work-group sees): value
  // positions at or past it may hold anything (stale slots of the last page, or pages past
  // it, clamped to it), and a zero probability times a non-finite value is not zero, so each
  // lane of a loading wave zeroes them in the 16-byte pieces it loaded itself (after its own
  // loads landed).
  auto zero_tail = [&](uint8_t* vbuf, int t) {
    const int lim = wg_keys - (kt0 + t) * kPrefillKeys;            // valid positions of the tile
    if (lim >= kPrefillKeys) return;
#pragma unroll
    for (int part = 0; part < IPP; ++part) {
      const int d = 32 * part + lane / 2;
      const int hf = (lane & 1) ^ ((d >> 3) & 1);                  // half of the page held here
      const int k0 = pw * kBlockSize + hf * 8;                     // its first position in the tile
      if (k0 + 8 > lim) {
        u32x4* q = reinterpret_cast<u32x4*>(vbuf + pw * PAGE + part * 1024 + lane * 16);
        u32x4 v = *q;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          v[w] &= (k0 + 2 * w < lim ? 0x0000ffffu : 0u) | (k0 + 2 * w + 1 < lim ? 0xffff0000u : 0u);
        *q = v;
      }
    }
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int qpos = c + qrow;

  // Operand addresses (bytes inside a buffer). Score MFMA: lane (col, grp) supplies row
  // `col` of the 32-key block, fed from key position perm(col), where perm swaps bits 2 and
  // 3 of the position inside each group of 16: the accumulator element (i, j) of lane grp
  // (row 8i + 4grp + j) then holds key 16*(i/2) + 8*grp + 4*(i%2) + j, i.e. the 16-key step
  // i/2 of the P.V product finds its 8 keys in natural order at 8*grp.. (its B operand), and
  // the V^T operand is 8 consecutive positions of one d-row.
  const int kperm = (col & 3) | ((col & 4) << 1) | ((col & 8) >> 1);
  const int ka_off = (col >> 4) * PAGE + grp * 256 + kperm * 16;     // + kt*2*PAGE + dc*512
  const int va_off = col * 32 + ((grp ^ (col >> 3)) & 1) * 16;       // + dt*1024 + ks*PAGE

  // S^T for the 64 keys of the tile in K buffer kbuf: two 32-key accumulators
  auto compute_s = [&](const uint8_t* kbuf, f32x16 (&st)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st[kt][i] = 0.f;
#pragma unroll
    for (int dc = 0; dc < DCH; ++dc)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {   // two independent accumulation chains, interleaved
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kbuf + ka_off + kt * 2 * PAGE + dc * 512);
        st[kt] = mfma32(ka, qf[dc], st[kt]);
      }
  };

  // Row max of a 64-key score tile (four independent chains, then lanes l and l^32). The
  // NaN-propagating maximum (v_maximum3_f32) needs no quieting of its MFMA-result inputs,
  // which fmaxf does (one extra instruction per chain); the scores it sees are finite or
  // -inf, except past the end of a request, which only diagonal tiles hold and which are
  // masked and their max taken again before use.
  auto tile_max = [&](const f32x16 (&st)[2]) -> float {
    float mq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) mq[q] = __builtin_elementwise_maximum(st[q >> 1][(q & 1) * 8], st[q >> 1][(q & 1) * 8 + 1]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 2; i < 8; ++i) mq[q] = __builtin_elementwise_maximum(mq[q], st[q >> 1][(q & 1) * 8 + i]);
    const float mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mq[0], mq[1]),
                                                   __builtin_elementwise_maximum(mq[2], mq[3]));
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };

  // One key tile u whose scores are in s_cur and whose unmasked row max is mx: mask,
  // softmax, O += V P, with the tile's values in vbuf. The scores of tile u+1 (K buffer knext)
  // are computed into s_next in the same straight-line block as the exp2 work of tile u, and
  // their row max at its end, beside the P.V MFMAs, so the matrix core and the vector ALU
  // overlap within the wave. Only tiles that cross the causal diagonal need a mask (every key
  // of another tile is visible to every row of the wave), and only those recompute the max
  // after it.
  // Lazy rescaling: the reference max only moves when some lane's max grew by more than
  // 8 (log2 units). Until then probabilities may reach 2^8, which fp32 sums and bf16 P
  // hold as well as values below 1; O and l share the reference, so O / l is unchanged.
  // The scale is positive, so max(scale*s) = scale*max(s) and it folds into the fma.
  // The test for a tile is made as soon as its row max is known (at the end of the step
  // before, beside the last MFMAs), so the step itself starts with a scalar branch.
  auto rescale_due = [&](float m) -> bool {
    return __builtin_amdgcn_ballot_w64(fmaxf(m_run, m * a.scale_log2) > m_run + 8.f) != 0;
  };
  auto tile_step = [&](int u, const uint8_t* vbuf, const uint8_t* knext, f32x16 (&s_cur)[2],
                       f32x16 (&s_next)[2], float& mx, bool& resc) {
    const int j = kt0 + u;                       // absolute tile: positions and masks
    if (!wave_active || j * kPrefillKeys >= wave_keys) return;
    const bool diag = j * kPrefillKeys + kPrefillKeys - 1 > c + wave_row0;   // uniform (scalar) values
    if (diag) {                                  // causal mask, only on tiles crossing it
      const int rel = qpos - j * kPrefillKeys - grp * 8;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kt * 32 + (i >> 3) * 16 + ((i >> 2) & 1) * 4 + (i & 3) > rel) s_cur[kt][i] = -INFINITY;
      mx = tile_max(s_cur);
      resc = rescale_due(mx);
    }
    if (resc) {                                  // wave-uniform: a scalar branch
      const float m_cand = fmaxf(m_run, mx * a.scale_log2);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_cand);
      m_run = m_cand;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
    }
    compute_s(knext, s_next);
    const float m_ref = m_run;
    float ps[4];                                 // four independent sum chains
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
          ps[kt * 2 + half] = e == 0 ? p0 + p1 : ps[kt * 2 + half] + (p0 + p1);   // no add of 0 first
          w[e] = pack_bf16x2(p0, p1);
        }
        pb[kt * 2 + half] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
      }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    // O^T += V^T P^T over four 16-key steps (one per page of the tile); one 16-byte read per
    // A operand: 8 consecutive positions of one d-row
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)               // DT independent accumulators back to back
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vbuf + va_off + dt * 1024 + ks * PAGE);
        oacc[dt] = mfma32(va, pb[ks], oacc[dt]);
      }
    mx = tile_max(s_next);
    resc = rescale_due(mx);
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

  // Block ids of the tiles requested at the next barrier (values of tile u+2, keys of tile
  // u+3 after step u), loaded one step ahead into vector registers (all lanes read the same
  // id): a scalar load in flight during a step would force full waits on the LDS operand
  // reads, which share its counter.
  int32_t id_v = 0, id_k = 0;
  auto fetch_ids = [&](int tv, int tk) {
    id_v = __builtin_nontemporal_load(bt + page_of(tv));
    id_k = __builtin_nontemporal_load(bt + page_of(tk));
  };

  // prologue: keys of tiles 0 and 1 and values of tile 0 in LDS, the scores of tile 0, then
  // the values of tile 1 and keys of tile 2 requested. The block ids of the item's first 64
  // pages come in one load, one per lane, so the first three tiles wait for one id load
  // rather than one each.
  const int ids0 = __builtin_nontemporal_load(bt + min(kt0 * 4 + lane, last_page));
  auto first_block = [&](int t) { return valid_block(__builtin_amdgcn_readlane(ids0, t * 4 + pw)); };
  if (loader) {
    const int b0 = first_block(0);
    load_k(kb0, b0);
    load_v(vb0, b0);
    if (n_tiles > 1) load_k(kb1, first_block(1));
  }
  wait_vmem();
  if (loader && n_tiles == 1) zero_tail(vb0, 0);
  __syncthreads();
  f32x16 sa[2], sb[2];
  float mx = 0.f;                                // unmasked row max of the next tile's scores
  bool resc = false;                             // its rescale test (lanes of the whole wave)
  if (wave_active) {
    compute_s(kb0, sa);
    mx = tile_max(sa);
    resc = rescale_due(mx);
  }
  __syncthreads();                               // K buffer 0 is read: it takes tile 2
  if (loader) {
    if (n_tiles > 1) load_v(vb1, first_block(1));
    if (n_tiles > 2) load_k(kb0, first_block(2));
    fetch_ids(2, 3);
  }
  // After step u (values of tile u in V buffer u&1, keys of tile u+1 in K buffer (u+1)&1):
  // wait for the requests of the previous barrier (values u+1, keys u+2, block ids), zero
  // the last tile's value tail, barrier (both buffers of step u are free), then request
  // values u+2 into V buffer u&1 and keys u+3 into K buffer (u+1)&1, and the block ids of
  // the tiles after them.
  auto advance = [&](int u, uint8_t* vfree, uint8_t* kfree, uint8_t* vnext) {
    wait_vmem();
    if (loader && u + 1 == n_tiles - 1) zero_tail(vnext, u + 1);
    __syncthreads();
    if (loader) {
      const int blk_v = valid_block(__builtin_amdgcn_readfirstlane(id_v));
      const int blk_k = valid_block(__builtin_amdgcn_readfirstlane(id_k));
      if (u + 2 < n_tiles) load_v(vfree, blk_v);
      if (u + 3 < n_tiles) load_k(kfree, blk_k);
      fetch_ids(u + 3, u + 4);
    }
  };
  int u = 0;
  for (; u + 1 < n_tiles; u += 2) {
    tile_step(u, vb0, kb1, sa, sb, mx, resc);
    advance(u, vb0, kb1, vb1);
    tile_step(u + 1, vb1, kb0, sb, sa, mx, resc);
    if (u + 2 < n_tiles) advance(u + 1, vb1, kb0, vb0);
  }
  if (u < n_tiles) tile_step(u, vb0, kb1, sa, sb, mx, resc);

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
