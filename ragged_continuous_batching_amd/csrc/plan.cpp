// The launch planner and step layouts: from a step's host metadata to the work lists the
// kernels read (decode splits, combine rows, prefill tiles, the mixed launch order) and the
// byte layout a step stages into its workspace. Also the host-side argument checks. Host
// code only.
#include <algorithm>
#include <cstring>
#include <vector>

#include "host.h"

namespace cb {

int check_shape(const cb_shape* s) {
  if (!s) return fail(CB_ERR_INVALID_ARG, "shape is NULL");
  if (s->num_q_heads < 1 || s->num_kv_heads < 1 || s->num_q_heads % s->num_kv_heads != 0)
    return fail(CB_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                s->num_q_heads, s->num_kv_heads);
  const int g = s->num_q_heads / s->num_kv_heads;
  if (!(g == 1 || g == 2 || g == 4 || g % 8 == 0))
    return fail(CB_ERR_UNSUPPORTED, "query group size %d not supported (1, 2, 4 or a multiple of 8)", g);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(CB_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", s->head_dim);
  if (s->block_size != kBlockSize) return fail(CB_ERR_UNSUPPORTED, "block_size must be %d", kBlockSize);
  if (s->num_blocks < 1) return fail(CB_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (s->dtype != CB_F32 && s->dtype != CB_BF16) return fail(CB_ERR_INVALID_ARG, "unknown dtype %d", s->dtype);
  return CB_OK;
}

int check_batch(const cb_shape* s, const cb_batch* b) {
  if (!b) return fail(CB_ERR_INVALID_ARG, "batch is NULL");
  if (b->num_reqs < 0 || b->num_tokens < 0 || b->max_blocks_per_req < 0)
    return fail(CB_ERR_INVALID_ARG, "negative count in batch");
  if (b->num_reqs == 0) {
    if (b->num_tokens != 0) return fail(CB_ERR_INVALID_ARG, "num_tokens > 0 with no requests");
    return CB_OK;
  }
  if (!b->h_cu_q_lens || !b->h_ctx_lens) return fail(CB_ERR_INVALID_ARG, "host mirrors are required");
  if (!b->cu_q_lens || !b->ctx_lens || !b->block_tables)
    return fail(CB_ERR_INVALID_ARG, "device metadata pointer is NULL");
  if (b->h_cu_q_lens[0] != 0) return fail(CB_ERR_INVALID_ARG, "cu_q_lens[0] must be 0");
  for (int32_t r = 0; r < b->num_reqs; ++r) {
    const int32_t q = b->h_cu_q_lens[r + 1] - b->h_cu_q_lens[r];
    const int32_t c = b->h_ctx_lens[r];
    if (q < 0) return fail(CB_ERR_INVALID_ARG, "cu_q_lens decreases at request %d", r);
    if (c < 0) return fail(CB_ERR_INVALID_ARG, "ctx_lens[%d] = %d is negative", r, c);
    if (q > 0 && ceil_div(static_cast<int64_t>(c) + q, s->block_size) > b->max_blocks_per_req)
      return fail(CB_ERR_INVALID_ARG, "request %d needs %d blocks but max_blocks_per_req is %d", r,
                  ceil_div(static_cast<int64_t>(c) + q, s->block_size), b->max_blocks_per_req);
    if (static_cast<int64_t>(c) + q > (int64_t{1} << 30)) return fail(CB_ERR_INVALID_ARG, "request %d too long", r);
  }
  if (static_cast<int64_t>(b->num_reqs) * b->max_blocks_per_req > INT32_MAX)
    return fail(CB_ERR_INVALID_ARG, "block table of %d x %d entries is too large", b->num_reqs, b->max_blocks_per_req);
  if (b->h_cu_q_lens[b->num_reqs] != b->num_tokens)
    return fail(CB_ERR_INVALID_ARG, "cu_q_lens[num_reqs] = %d but num_tokens = %d", b->h_cu_q_lens[b->num_reqs],
                b->num_tokens);
  return CB_OK;
}

// Would a step with these rows take the mixed launch? bf16 steps with prefill chunks and
// matrix-core decode rows (the 4-wave prefill work-group then has the decode work-group's
// shape, and both fit two to a CU).
static bool wants_mixed(const cb_shape* s, const cb_batch* b) {
  if (!g_tuning.mixed_launch || s->dtype != CB_BF16 || !g_tuning.decode_mfma) return false;
  if (s->num_q_heads / s->num_kv_heads < 4) return false;
  bool dec = false, pre = false;
  for (int32_t r = 0; r < b->num_reqs; ++r) {
    const int32_t q = b->h_cu_q_lens[r + 1] - b->h_cu_q_lens[r];
    dec |= q == 1;
    pre |= q > 1;
  }
  return dec && pre;
}

// force_waves (4 or 8) fixes the prefill work-group size; 0 takes the tuning / automatic choice.
// allow_mixed = false keeps prefill and decode in separate launches (captured steps).
// bt_rows (host, [num_reqs], nullable): where each request's block ids start in the device
// block table; null means the padded [num_reqs, max_blocks_per_req] layout of cb_batch.
void make_plan(const cb_shape* s, const cb_batch* b, Plan& p, int force_waves, bool allow_mixed,
               const int32_t* bt_rows) {
  auto bt_row = [&](int32_t r) {
    return bt_rows ? bt_rows[r] : static_cast<int32_t>(static_cast<int64_t>(r) * b->max_blocks_per_req);
  };
  const int q_per_kv = s->num_q_heads / s->num_kv_heads;
  // query heads per decode wave: all heads of the group up to decode_group; a larger group
  // is covered by n_sub waves on adjacent slots, which read the same pages back to back
  p.mfma_decode = s->dtype == CB_BF16 && q_per_kv >= 4 && g_tuning.decode_mfma;
  if (p.mfma_decode) {          // up to 16 heads fill the columns of one 16x16 tile
    p.group = q_per_kv % 16 == 0 ? 16 : (q_per_kv % 8 == 0 ? 8 : 4);
  } else {
    p.group = std::min(q_per_kv, static_cast<int>(g_tuning.decode_group));
    while (q_per_kv % p.group) p.group /= 2;
  }
  p.n_sub = q_per_kv / p.group;
  const bool mfma_prefill = s->dtype == CB_BF16;
  p.mixed = allow_mixed && wants_mixed(s, b);
  p.prefill_waves = p.mixed ? 4 : force_waves ? force_waves : g_tuning.prefill_waves;
  if (p.prefill_waves == 0) {
    // 256-row work-groups read each key/value tile once for twice the rows, but a CU holds
    // only one of them (registers), so nothing hides a work-group's start (its query rows
    // and first tiles) and end. Take them when there are enough to fill every CU twice and
    // they are long (16+ key tiles on average: the 2048-token chunks with long contexts);
    // short fresh chunks (the trace replay) run 2% faster as 128-row work-groups, two per
    // CU. Also take them when there are fewer than CUs but long ones (32+ key tiles on
    // average): the split over key ranges then makes the work-groups, and the halved
    // key/value traffic counts (a late 256-row chunk after 16k cached tokens: prefill
    // 104.7 -> 95.5 us).
    int64_t items256 = 0, tiles256 = 0;
    for (int32_t r = 0; r < b->num_reqs; ++r) {
      const int32_t q = b->h_cu_q_lens[r + 1] - b->h_cu_q_lens[r], c = b->h_ctx_lens[r];
      if (q <= 1 || !mfma_prefill) continue;
      for (int32_t qb = 0; qb < q; qb += 256) {
        items256 += s->num_q_heads;
        tiles256 += static_cast<int64_t>(ceil_div(c + std::min(qb + 256, q), kPrefillKeys)) * s->num_q_heads;
      }
    }
    const bool few_long = items256 < kNumCUs && tiles256 >= 32 * items256 && g_tuning.prefill_split;
    const bool many_long = items256 >= 2 * kNumCUs && tiles256 >= 16 * items256;
    p.prefill_waves = many_long || few_long ? 8 : 4;
  }

  // Query heads per prefill work-group (one kv head's heads side by side, each wave 32 rows of
  // one head): the tuning key, else up to 4. The waves of a work-group then share its rows'
  // causal extent (no wave idles on the diagonal tiles while the others finish) and one
  // stream of key/value tiles serves several heads. Measured on the trace replay (G = 8):
  // prefill 152.7 us per step with one head, 146.1 / 145.3 / 145.5 us with 2 / 4 / 8.
  p.prefill_heads_log2 = 0;
  const int want_heads = g_tuning.prefill_heads > 0 ? g_tuning.prefill_heads : 4;
  if (mfma_prefill && want_heads > 1) {
    int gh = std::min<int>({want_heads, q_per_kv, p.prefill_waves});
    while (q_per_kv % gh) gh /= 2;
    while ((1 << (p.prefill_heads_log2 + 1)) <= gh) ++p.prefill_heads_log2;
  }
  const int32_t pre_rows = (32 * p.prefill_waves) >> p.prefill_heads_log2;   // rows per prefill item
  const int32_t pre_heads = 1 << p.prefill_heads_log2;

  // rows that take the split-K path, longest first
  struct Row { int32_t token, req, kv_len; };
  struct PrefillGroup { std::vector<PrefillItem> items; int64_t cost = 0; };
  struct QTile { int32_t req, qb, n_kt, n_split; };      // one row tile of a prefill chunk
  std::vector<PrefillGroup> groups;
  std::vector<QTile> qtiles;
  std::vector<Row> rows;
  int64_t total_blocks = 0, total_tiles = 0;
  for (int32_t r = 0; r < b->num_reqs; ++r) {
    const int32_t t0 = b->h_cu_q_lens[r], q = b->h_cu_q_lens[r + 1] - t0, c = b->h_ctx_lens[r];
    if (q == 0) continue;
    if (q == 1 || !mfma_prefill) {
      for (int32_t i = 0; i < q; ++i) {
        rows.push_back({t0 + i, r, c + i + 1});
        total_blocks += ceil_div(c + i + 1, kBlockSize);
      }
    } else {
      for (int32_t qt = ceil_div(q, pre_rows) - 1; qt >= 0; --qt) {
        const int32_t qb = qt * pre_rows;
        qtiles.push_back({r, qb, ceil_div(c + std::min(qb + pre_rows, q), kPrefillKeys), 1});
        total_tiles += static_cast<int64_t>(qtiles.back().n_kt) * (s->num_q_heads / pre_heads);
      }
    }
  }
  // Split-K for prefill tiles when a step has fewer prefill work-groups than the machine has
  // work-group slots: a late chunk of a long prompt has few rows but a long context, and its
  // few work-groups would each walk every key tile while most CUs idle. Tiles longer than
  // the step's work per slot (at least 16 key tiles) are then cut into near-equal key
  // ranges, which brings the count of work-groups up to about the slots. With as many
  // work-groups as slots or more, the CUs already share the work evenly (long and short
  // work-groups pair up on each CU), and splitting only adds partials: measured on the
  // Llama-2-7B-shaped mixed step, 512 work-groups, prefill 58 -> 62 us, combine 5 -> 15 us;
  // as 256 work-groups of 256 rows, unsplit 61-63 us and cut into 14- or 20-tile ranges
  // 63-70 us with the combine at 12-17 us (128-row work-groups unsplit: 52 us, 4.6 us).
  // Every cut lies at or below the first row's last key ((c + qb) / 64 tiles are fully
  // visible to every row of the tile), so no row meets an empty range.
  const int64_t slots = static_cast<int64_t>(kNumCUs) * (p.prefill_waves == 8 ? 1 : 2);
  const int64_t pre_items = static_cast<int64_t>(qtiles.size()) * (s->num_q_heads / pre_heads);
  if (!qtiles.empty() && g_tuning.prefill_split && (pre_items < slots || g_tuning.prefill_split_tiles > 0)) {
    const int64_t len = g_tuning.prefill_split_tiles > 0
                            ? g_tuning.prefill_split_tiles
                            : std::max<int64_t>(16, (total_tiles + slots - 1) / slots);
    for (QTile& t : qtiles) {
      const int32_t c = b->h_ctx_lens[t.req];
      const int32_t lim = (c + t.qb) / kPrefillKeys;
      int32_t n = static_cast<int32_t>(std::min<int64_t>((t.n_kt + len - 1) / len, 0xffff));
      while (n > 1 && static_cast<int64_t>(n - 1) * t.n_kt / n > lim) --n;
      t.n_split = std::max(n, 1);
    }
  }
  {
    // one group per (request, kv head): all its q-tiles and query heads read the same
    // key/value tiles, so they are kept on one XCD (shared L2) and run side by side
    const int32_t rows = pre_rows;
    size_t i0 = 0;
    while (i0 < qtiles.size()) {
      size_t i1 = i0;
      while (i1 < qtiles.size() && qtiles[i1].req == qtiles[i0].req) ++i1;
      const int32_t r = qtiles[i0].req, t0 = b->h_cu_q_lens[r], q = b->h_cu_q_lens[r + 1] - t0;
      std::vector<int32_t> part_base(i1 - i0, -1);
      for (size_t i = i0; i < i1; ++i) {          // partial slots and combine rows of split tiles
        const QTile& t = qtiles[i];
        if (t.n_split == 1) continue;
        part_base[i - i0] = p.n_parts;
        const int32_t valid = std::min(rows, q - t.qb);
        for (int32_t k = 0; k < valid; ++k) p.combine.push_back({t0 + t.qb + k, p.n_parts + k * t.n_split, t.n_split, 0});
        p.n_parts += valid * t.n_split;
      }
      for (int32_t g = 0; g < s->num_kv_heads; ++g) {
        PrefillGroup grp;
        for (size_t i = i0; i < i1; ++i) {
          const QTile& t = qtiles[i];
          for (int32_t sp = 0; sp < t.n_split; ++sp) {
            const int32_t k0 = static_cast<int32_t>(static_cast<int64_t>(sp) * t.n_kt / t.n_split);
            const int32_t k1 = static_cast<int32_t>(static_cast<int64_t>(sp + 1) * t.n_kt / t.n_split);
            for (int32_t hh = 0; hh < q_per_kv; hh += pre_heads) {
              grp.items.push_back({r, t.qb, g * q_per_kv + hh, bt_row(r), k0, k1, part_base[i - i0],
                                   t.n_split > 1 ? (t.n_split << 16) | sp : 0, p.prefill_heads_log2});
              grp.cost += k1 - k0;
            }
          }
        }
        groups.push_back(std::move(grp));
      }
      i0 = i1;
    }
  }
  // Work-groups are dispatched round-robin over the XCDs (block b runs on XCD b % n). Groups
  // go, longest first, to the XCD with the least work so far; each XCD's queue is then
  // interleaved into the launch order. Unused slots hold an empty item (req = -1).
  if (!groups.empty()) {
    const int nx = std::max(1, g_tuning.xcds);
    // A group costlier than one XCD's share of the step (the long chunk of a request with
    // few kv heads: one or two groups hold nearly all the work) is cut, in item order, into
    // pieces of about that share, so it does not leave the other XCDs idle.
    int64_t total_cost = 0;
    for (const PrefillGroup& grp : groups) total_cost += grp.cost;
    const int64_t share = (total_cost + nx - 1) / nx;
    std::vector<PrefillGroup> pieces;
    for (PrefillGroup& grp : groups) {
      if (grp.cost <= share || grp.items.size() < 2) {
        pieces.push_back(std::move(grp));
        continue;
      }
      PrefillGroup cur;
      for (const PrefillItem& it : grp.items) {
        const int64_t c = it.kt_end - it.kt_begin;
        if (cur.cost > 0 && cur.cost + c > share) {
          pieces.push_back(std::move(cur));
          cur = PrefillGroup();
        }
        cur.items.push_back(it);
        cur.cost += c;
      }
      if (!cur.items.empty()) pieces.push_back(std::move(cur));
    }
    groups.swap(pieces);
    std::stable_sort(groups.begin(), groups.end(),
                     [](const PrefillGroup& x, const PrefillGroup& y) { return x.cost > y.cost; });
    std::vector<std::vector<PrefillItem>> queue(nx);
    std::vector<int64_t> load(nx, 0);
    for (const PrefillGroup& grp : groups) {
      const int x = static_cast<int>(std::min_element(load.begin(), load.end()) - load.begin());
      load[x] += grp.cost;
      queue[x].insert(queue[x].end(), grp.items.begin(), grp.items.end());
    }
    // Within an XCD the first C = (CUs per XCD) work-groups go one to each CU, the next C
    // take each CU's second slot in the same order, and so on. A queue sorted longest first
    // would pair the longest first-round item with the longest second-round one; reversing
    // every other round of C pairs long with short, so the CUs finish closer together.
    if (g_tuning.prefill_snake) {
      const size_t C = static_cast<size_t>(std::max(1, kNumCUs / nx));
      for (auto& qx : queue)
        for (size_t k0 = C; k0 < qx.size(); k0 += 2 * C)
          std::reverse(qx.begin() + k0, qx.begin() + std::min(qx.size(), k0 + C));
    }
    size_t depth = 0;
    for (const auto& qx : queue) depth = std::max(depth, qx.size());
    p.prefill.assign(depth * nx, PrefillItem{-1, 0, 0, 0, 0, 0, -1, 0, 0});
    for (int x = 0; x < nx; ++x)
      for (size_t k = 0; k < queue[x].size(); ++k) p.prefill[k * nx + x] = queue[x][k];
  }
  std::stable_sort(rows.begin(), rows.end(), [](const Row& x, const Row& y) { return x.kv_len > y.kv_len; });

  int32_t split = g_tuning.split_blocks;
  if (split <= 0) {
    const int64_t units = total_blocks * s->num_kv_heads * p.n_sub;
    // Longer splits mean fewer partials to write and merge and fewer waves, each of which
    // pays a start (its query rows, its first pages) and an end (its stores, which queue
    // behind the cache stream); the target keeps enough items to fill the machine about
    // twice (the matrix-core kernel runs 2 waves per SIMD, the vector-ALU one 3). Measured
    // on configs 2, 3 and the trace replay: 2048 and 4096 (was 4096 and 8192 with splits
    // capped at 64 blocks): decode 490 -> 481 us on config 3, 433 -> 419 us on the trace,
    // 367 -> 360 us on config 2.
    const int64_t target = g_tuning.target_waves > 0 ? g_tuning.target_waves : (p.mfma_decode ? 2048 : 4096);
    split = static_cast<int32_t>(std::clamp<int64_t>((units + target - 1) / target, 4, kMaxSplitBlocks));
  }
  split = std::min(split, kMaxSplitBlocks);
  p.split_blocks = split;
  for (const Row& row : rows) {
    const int32_t nb = ceil_div(row.kv_len, kBlockSize);
    const int32_t ns = ceil_div(nb, split);
    if (ns == 1) {
      p.splits.push_back({row.token, bt_row(row.req), 0, nb, row.kv_len, -1});
      continue;
    }
    // near-equal splits (a 209-block row at split 64: 53/52/52/52, not 64/64/64/17), so no
    // wave pays a full start-up for a sliver of a row
    p.combine.push_back({row.token, p.n_parts, ns, 0});
    for (int32_t k = 0; k < ns; ++k)
      p.splits.push_back({row.token, bt_row(row.req), static_cast<int32_t>(static_cast<int64_t>(k) * nb / ns),
                          static_cast<int32_t>(static_cast<int64_t>(k + 1) * nb / ns), row.kv_len, p.n_parts + k});
    p.n_parts += ns;
  }
  // waves longest first (a long row's splits are shorter than a shorter row's single split)
  if (g_tuning.decode_order == 1)
    std::stable_sort(p.splits.begin(), p.splits.end(),
                     [](const RowSplit& x, const RowSplit& y) { return x.blk_end - x.blk_begin > y.blk_end - y.blk_begin; });

  if (p.mixed) {
    // Chunks of one work-group per XCD. mixed_order 0: prefill and decode chunks merged in
    // proportion to their counts, so prefill work-groups stay a minority of each CU's
    // slots throughout (the cache stream, the step's bound, keeps most of them; measured on
    // the trace replay: 594 us for the launch vs 621 us for the two kernels). mixed_order 1:
    // alternate until one kind runs out (half the slots go to prefill: 678 us). A prefill
    // chunk keeps the XCD positions its planner chose (the prefill list is laid out in
    // chunks of nx); the last decode chunk is padded with work-group indices past the
    // decode items.
    const int nx = std::max(1, g_tuning.xcds);
    const int64_t n_rows = static_cast<int64_t>(p.splits.size()) * s->num_kv_heads * p.n_sub;
    const int64_t n_dwg = (n_rows + 3) / 4;
    const int64_t pch = static_cast<int64_t>(p.prefill.size()) / nx, dch = (n_dwg + nx - 1) / nx;
    int64_t pc = 0, dc = 0;
    p.order.reserve(static_cast<size_t>((pch + dch) * nx));
    while (pc < pch || dc < dch) {
      const bool take_p = dc == dch || (pc < pch && (g_tuning.mixed_order ? pc <= dc : pc * dch <= dc * pch));
      for (int k = 0; k < nx; ++k)
        p.order.push_back(take_p ? static_cast<int32_t>(pc * nx + k) : static_cast<int32_t>(-1 - (dc * nx + k)));
      (take_p ? pc : dc) += 1;
    }
  }

  const size_t eb = 4;
  p.off_combine = align256(p.splits.size() * sizeof(RowSplit));
  p.off_prefill = p.off_combine + align256(p.combine.size() * sizeof(CombineRow));
  p.off_order = p.off_prefill + align256(p.prefill.size() * sizeof(PrefillItem));
  p.plan_bytes = p.off_order + p.order.size() * sizeof(int32_t);
  p.off_part_o = align256(p.plan_bytes);
  p.off_part_ml = p.off_part_o + align256(static_cast<size_t>(p.n_parts) * s->num_q_heads * s->head_dim * eb);
  p.total = p.off_part_ml + align256(static_cast<size_t>(p.n_parts) * s->num_q_heads * 2 * eb);
}

// Serialises the plan's work lists at their offsets into `out` (plan_bytes long).
void write_plan(const Plan& p, char* out) {
  if (!p.splits.empty()) std::memcpy(out, p.splits.data(), p.splits.size() * sizeof(RowSplit));
  if (!p.combine.empty()) std::memcpy(out + p.off_combine, p.combine.data(), p.combine.size() * sizeof(CombineRow));
  if (!p.prefill.empty())
    std::memcpy(out + p.off_prefill, p.prefill.data(), p.prefill.size() * sizeof(PrefillItem));
  if (!p.order.empty()) std::memcpy(out + p.off_order, p.order.data(), p.order.size() * sizeof(int32_t));
}

int check_tensors(const void* q, const void* k_cache, const void* v_cache, void* o, float scale, const char* fn) {
  if (!q || !k_cache || !v_cache || !o) return fail(CB_ERR_INVALID_ARG, "%s: NULL tensor", fn);
  if (!(scale > 0.f) || !(scale < 3.0e38f)) return fail(CB_ERR_INVALID_ARG, "%s: scale must be positive and finite", fn);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(CB_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  return CB_OK;
}



// bt_entries: block-table entries staged (the compact table's length, or R * max_blocks).
StepLayout step_layout(int32_t R, int64_t bt_entries, int32_t T) {
  StepLayout l;
  l.off_cu = 0;
  l.off_ctx = static_cast<size_t>(R + 1) * 4;
  l.off_bt = l.off_ctx + static_cast<size_t>(R) * 4;
  l.off_slots = l.off_bt + static_cast<size_t>(bt_entries) * 4;
  l.meta_bytes = l.off_slots + static_cast<size_t>(std::max(T, 0)) * 4;
  l.plan_base = align256(l.meta_bytes);
  return l;
}

// Cache slot (block * block_size + offset) of every packed row, from the host metadata
// (the slot rule of cb_kv_append: row i of request r sits at position ctx_lens[r] + i).
// Block ids were checked against the pool before this is called.
//
// With `mark`, a row that is the only row of the step writing into its block also carries
// kSlotSoleWriter. Rows are counted per block (not per request) in an open-addressing table
// of the blocks the step writes, so a block that holds two rows of a chunk, or that two
// requests share, is never marked.
int32_t fill_slots(int32_t R, int32_t maxb, const int32_t* cu, const int32_t* ctx, const int32_t* bt, int32_t* out,
                   bool mark, int32_t* marked) {
  if (!mark) {
    for (int32_t r = 0; r < R; ++r) {
      const int32_t* row = bt + static_cast<size_t>(r) * maxb;
      for (int32_t t = cu[r], p = ctx[r]; t < cu[r + 1]; ++t, ++p)
        out[t] = row[p / kBlockSize] * kBlockSize + p % kBlockSize;
    }
    return 0;
  }
  int32_t n_marked = 0;
  thread_local std::vector<int32_t> keys;      // block id, -1: empty
  thread_local std::vector<uint8_t> counts;    // rows written into it, saturating at 2
  int bits = 6;
  while ((size_t{1} << bits) < 2 * static_cast<size_t>(std::max(cu[R], 1))) ++bits;
  const size_t mask = (size_t{1} << bits) - 1;
  keys.assign(mask + 1, -1);
  counts.assign(mask + 1, 0);
  auto entry = [&](int32_t b) {                // Fibonacci hashing, linear probing
    size_t h = (static_cast<uint32_t>(b) * 0x9E3779B1u) >> (32 - bits);
    while (keys[h] != b && keys[h] != -1) h = (h + 1) & mask;
    keys[h] = b;
    return h;
  };
  for (int pass = 0; pass < 2; ++pass) {
    for (int32_t r = 0; r < R; ++r) {
      const int32_t q = cu[r + 1] - cu[r];
      if (q <= 0) continue;
      const int32_t* row = bt + static_cast<size_t>(r) * maxb;
      const int32_t p0 = ctx[r], p1 = ctx[r] + q - 1;
      for (int32_t j = p0 / kBlockSize; j <= p1 / kBlockSize; ++j) {
        const int32_t lo = std::max(p0, j * kBlockSize), hi = std::min(p1, j * kBlockSize + kBlockSize - 1);
        const size_t h = entry(row[j]);
        if (pass == 0) {
          counts[h] = static_cast<uint8_t>(std::min(2, counts[h] + hi - lo + 1));
        } else {
          const int32_t flag = counts[h] == 1 ? kSlotSoleWriter : 0;
          for (int32_t p = lo; p <= hi; ++p) {
            const int32_t t = cu[r] + p - p0, slot = row[j] * kBlockSize + p % kBlockSize;
            out[t] = slot | flag;
            if (flag && marked) {
              marked[2 * n_marked] = t;
              marked[2 * n_marked + 1] = slot;
            }
            n_marked += flag != 0;
          }
        }
      }
    }
  }
  return n_marked;
}


// The step entry points stage a compact block table: request r's ceil((c + q) / bs) ids (none
// for a request with no rows) start at rows[r]. The padded [R, max_blocks] table of a long
// request beside many short ones is mostly padding (the decode-only workload: 2.1 MB staged
// per step, 0.2 MB of it block ids). Returns the entry count.
int64_t compact_rows(int32_t R, const int32_t* cu, const int32_t* ctx, std::vector<int32_t>& rows) {
  rows.resize(static_cast<size_t>(R));
  int64_t n = 0;
  for (int32_t r = 0; r < R; ++r) {
    rows[r] = static_cast<int32_t>(n);
    const int32_t q = cu[r + 1] - cu[r];
    if (q > 0) n += ceil_div(static_cast<int64_t>(ctx[r]) + q, kBlockSize);
  }
  return n;
}

void fill_compact(int32_t R, int32_t maxb, const int32_t* cu, const int32_t* ctx, const int32_t* bt,
                  const std::vector<int32_t>& rows, int32_t* out) {
  for (int32_t r = 0; r < R; ++r) {
    const int32_t q = cu[r + 1] - cu[r];
    if (q > 0)
      std::memcpy(out + rows[r], bt + static_cast<size_t>(r) * maxb,
                  static_cast<size_t>(ceil_div(static_cast<int64_t>(ctx[r]) + q, kBlockSize)) * 4);
  }
}

// Every block id a row of the step can touch lies in the pool (host mirrors, checked before
// any upload).
int check_block_ids(const cb_shape* shape, int32_t num_reqs, int32_t max_blocks_per_req,
                           const int32_t* h_cu_q_lens, const int32_t* h_ctx_lens, const int32_t* h_block_tables,
                           const char* fn) {
  if (!h_block_tables) return fail(CB_ERR_INVALID_ARG, "%s: block tables are required", fn);
  for (int32_t r = 0; r < num_reqs; ++r) {
    if (h_cu_q_lens[r + 1] == h_cu_q_lens[r]) continue;
    const int32_t nb = ceil_div(static_cast<int64_t>(h_ctx_lens[r]) + h_cu_q_lens[r + 1] - h_cu_q_lens[r], kBlockSize);
    const int32_t* row = h_block_tables + static_cast<size_t>(r) * max_blocks_per_req;
    for (int32_t j = 0; j < nb; ++j)
      if (row[j] < 0 || row[j] >= shape->num_blocks)
        return fail(CB_ERR_INVALID_ARG, "%s: block id %d of request %d out of range", fn, row[j], r);
  }
  return CB_OK;
}

// A cb_batch over host metadata whose device pointers point into the step workspace.
cb_batch step_batch(int32_t R, int32_t T, int32_t maxb, const int32_t* h_cu, const int32_t* h_ctx,
                           char* ws, const StepLayout& l) {
  // a non-null placeholder lets the host-side checks run before the workspace is known
  char* base = ws ? ws : reinterpret_cast<char*>(uintptr_t{256});
  return cb_batch{R, T, maxb, reinterpret_cast<const int32_t*>(base + l.off_cu),
                  reinterpret_cast<const int32_t*>(base + l.off_ctx), reinterpret_cast<const int32_t*>(base + l.off_bt),
                  h_cu, h_ctx};
}

}  // namespace cb
