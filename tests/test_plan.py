"""The launch planner's choices, from host metadata only (cb_plan_describe; no GPU).

Each test builds a batch from (query rows, cached tokens) pairs, with placeholder device
pointers (the planner reads only the host mirrors), and checks one rule of the planner:
the prefill work-group size, the split over key ranges, the decode split sizing and its
near-equal lengths, the longest-first order and the kernel choice.
"""
import ctypes
import math

import numpy as np
import pytest

from ragged_continuous_batching_amd import cb

_KEEP = []


def batch(reqs, block_size=16):
    """cb_batch over host mirrors for [(q_len, ctx_len), ...]."""
    q = np.array([r[0] for r in reqs], dtype=np.int32)
    c = np.array([r[1] for r in reqs], dtype=np.int32)
    cu = np.zeros(len(reqs) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q)
    maxb = max(1, max(-(-(int(a) + int(b)) // block_size) for a, b in zip(q, c)))
    _KEEP.append((cu, c))
    fake = ctypes.c_void_p(256)        # never dereferenced: the planner reads host mirrors
    return cb.cb_batch(len(reqs), int(cu[-1]), maxb, fake, fake, fake, cu.ctypes.data, c.ctypes.data)


def describe(reqs, hq, hkv, d=128, dtype="bf16", **tune):
    shape = cb.make_shape(hq, hkv, d, 1 << 24, dtype)
    try:
        for k, v in tune.items():
            cb.cb_set_tuning(k, v)
        return cb.cb_plan_describe(shape, batch(reqs))
    finally:
        defaults = {"split_blocks": 0, "target_waves": 0, "prefill_waves": 0, "decode_order": 1,
                    "mixed_launch": 0, "prefill_split_tiles": 0, "decode_mfma": 1, "prefill_heads": 0}
        for k in tune:
            cb.cb_set_tuning(k, defaults[k])


def test_long_chunks_take_256_row_work_groups():
    """Four 2048-row chunks with long contexts (the chunked-prefill-heavy step): 1024
    row tiles of 256 rows averaging about 106 key tiles, so 256-row work-groups."""
    info = describe([(2048, 2048), (2048, 6144), (2048, 14336), (2048, 0)], 32, 32)
    assert info["prefill_rows"] == 256
    assert info["decode_splits"] == 0 and info["prefill_split_items"] == 0


def test_short_fresh_chunks_take_128_row_work_groups():
    """Many short fresh prompts (the trace's steps): enough 256-row tiles, but only about 4
    key tiles each, so 4-wave work-groups, two per CU; with 8 query heads per kv head each
    takes 4 heads x 32 rows."""
    info = describe([(256, 0)] * 16 + [(1, 700)] * 8, 64, 8)
    assert info["prefill_rows"] * info["prefill_heads"] == 128
    assert info["prefill_heads"] == 4


def test_late_chunk_takes_256_rows_split_over_key_ranges():
    """One 256-row chunk after 16384 cached tokens: few but long row tiles, so 256-row
    work-groups split over key ranges (about one per CU)."""
    info = describe([(256, 16384)], 32, 32)
    assert info["prefill_rows"] == 256
    assert info["prefill_split_items"] > 0
    assert info["combine_rows"] == 256        # every row of the chunk merges its ranges


def test_mixed_step_keeps_128_rows_and_decode_on_vector_alu():
    """The Llama-2-7B-shaped step (64 decodes, two 992-row chunks, Hq = Hkv): 128-row
    prefill work-groups, unsplit key ranges, decode rows on the vector-ALU kernel."""
    rng = np.random.default_rng(1)
    reqs = [(1, int(c)) for c in rng.integers(512, 4097, size=64)] + [(992, 1024), (992, 0)]
    info = describe(reqs, 32, 32)
    assert info["prefill_rows"] == 128 and info["prefill_split_items"] == 0
    assert info["decode_splits"] >= 64 and info["matrix_core_decode"] == 0
    assert info["decode_items"] == info["decode_splits"] * 32


def test_grouped_query_decode_on_matrix_cores():
    """Four or more query heads per kv head: decode rows on the matrix-core kernel, one wave
    per (split, kv head) with up to 8 heads."""
    info = describe([(1, 2000 + 37 * i) for i in range(64)], 32, 8)
    assert info["matrix_core_decode"] == 1
    assert info["decode_items"] == info["decode_splits"] * 8


def test_split_sizing_targets_the_wave_count():
    """Automatic split length = ceil(row-blocks x kv heads / target), target 2048 wave items
    for the matrix-core kernel, at least 4 and at most 1024 blocks."""
    ctx = [16 * 200 - 1] * 256                   # 200 blocks per row with the new token
    info = describe([(1, c) for c in ctx], 32, 8)
    units = 256 * 200 * 8
    assert info["split_blocks"] == min(1024, max(4, math.ceil(units / 2048)))
    # a smaller target gives longer splits
    longer = describe([(1, c) for c in ctx], 32, 8, target_waves=512)
    assert longer["split_blocks"] > info["split_blocks"]


def test_splits_are_near_equal():
    """A 209-block row at split length 64 takes 4 splits of 53/52/52/52 blocks, not
    64/64/64/17 (no tail sliver)."""
    info = describe([(1, 16 * 209 - 1)], 32, 8, split_blocks=64)
    assert info["decode_splits"] == 4
    assert (info["split_min_blocks"], info["split_max_blocks"]) == (52, 53)
    assert info["combine_rows"] == 1


def test_splits_launch_longest_first():
    """decode_order = 1 lists the splits in non-increasing length; a long row's splits can be
    shorter than a short row's single split, so ordering rows (decode_order = 0) does not
    order the splits."""
    reqs = [(1, 16 * 130 - 1), (1, 16 * 70 - 1), (1, 16 * 20 - 1)]
    assert describe(reqs, 32, 8, split_blocks=64)["longest_first"] == 1
    by_rows = describe(reqs, 32, 8, split_blocks=64, decode_order=0)
    assert by_rows["longest_first"] == 0         # 43/43/44 (130 blocks) then 35/35 (70): not sorted by split


def test_mixed_launch_needs_both_kinds_of_rows():
    """With mixed_launch set, a bf16 step with prefill chunks and matrix-core decode rows
    takes one launch; a decode-only step does not."""
    both = describe([(300, 0), (1, 900), (1, 2000)], 16, 2, mixed_launch=1)
    assert both["mixed"] == 1 and both["prefill_rows"] * both["prefill_heads"] == 128   # 4-wave groups
    decode_only = describe([(1, 900), (1, 2000)], 16, 2, mixed_launch=1)
    assert decode_only["mixed"] == 0


def test_fp32_prefill_rows_take_the_split_k_path():
    """fp32 steps have no MFMA prefill tiles: every row of a chunk is a split-K row."""
    info = describe([(40, 100), (1, 50)], 4, 2, d=64, dtype="f32")
    assert info["prefill_rows"] == 0 and info["prefill_items"] == 0
    assert info["decode_splits"] >= 41


def test_empty_batch():
    shape = cb.make_shape(8, 2, 128, 1024, "bf16")
    info = cb.cb_plan_describe(shape, cb.cb_batch(0, 0, 0, None, None, None, None, None))
    assert all(v == 0 for v in info.values())


def test_rejects_a_batch_that_overflows_its_block_table():
    shape = cb.make_shape(8, 2, 128, 1024, "bf16")
    b = batch([(10, 100)])
    b.max_blocks_per_req = 2                     # 110 positions need 7 blocks
    with pytest.raises(cb.CbError):
        cb.cb_plan_describe(shape, b)


@pytest.mark.parametrize("heads,hq,hkv,waves,rows,got_heads", [
    (8, 64, 8, 8, 32, 8), (4, 64, 8, 8, 64, 4), (8, 8, 2, 8, 64, 4), (8, 64, 8, 4, 32, 4), (2, 32, 32, 8, 256, 1)])
def test_prefill_heads_cut_rows(heads, hq, hkv, waves, rows, got_heads):
    """prefill_heads: a work-group takes up to that many query heads of one kv head (capped by
    the group size and the waves), and its rows shrink to 32 x waves / heads."""
    d = describe([(300, 100)], hq, hkv, prefill_heads=heads, prefill_waves=waves)
    assert (d["prefill_heads"], d["prefill_rows"]) == (got_heads, rows), d
    tiles = -(-300 // rows)
    assert d["prefill_items"] >= tiles * hq // got_heads


def test_a_dominant_group_is_cut_across_xcds():
    """A 100-row chunk after 65,536 cached tokens with one kv head: its split items all belong
    to one (request, kv head) group, which would put them on one XCD (1952 launch slots, 7 of
    8 XCDs idle). The group is cut into pieces of about one XCD's share, so the launch order
    holds the 248 items in 8 near-even queues."""
    info = describe([(1, 131071), (100, 65536), (70, 0)], 8, 1)
    assert info["prefill_split_items"] == 244
    assert info["prefill_items"] <= 8 * (-(-248 // 8) + 4), info
    # a step whose groups are all below the share keeps one group per XCD queue as before
    assert describe([(2048, 2048), (2048, 6144), (2048, 14336), (2048, 0)], 32, 32)["prefill_items"] == 1024


# ---- staged slots and sole-writer marks (cb_step_slots) -------------------------------------

SOLE = cb.CB_SLOT_SOLE_WRITER


def staged_slots(reqs, tables, num_blocks=4096):
    """cb_step_slots for [(q_len, ctx_len), ...] with explicit per-request block lists."""
    q = np.array([r[0] for r in reqs], np.int32)
    c = np.array([r[1] for r in reqs], np.int32)
    cu = np.concatenate([[0], np.cumsum(q)]).astype(np.int32)
    maxb = max(1, max(len(t) for t in tables))
    bt = np.full((len(reqs), maxb), -1, np.int32)
    for i, t in enumerate(tables):
        bt[i, :len(t)] = t
    shape = cb.make_shape(8, 8, 128, num_blocks, "bf16")
    return cb.cb_step_slots(shape, len(reqs), int(cu[-1]), maxb, cu, c, bt), cu, c, bt


def rule_slots(cu, ctx, bt, bs=16):
    """The slot rule written out (cb_kv_append's): row i of request r at p = ctx[r] + i."""
    out = []
    for r in range(len(ctx)):
        for i in range(cu[r + 1] - cu[r]):
            p = ctx[r] + i
            out.append(bt[r, p // bs] * bs + p % bs)
    return np.array(out, np.int64)


def brute_marks(slots, bs=16):
    """A row is marked iff no other row of the step writes into its block."""
    blocks = slots // bs
    return np.array([(blocks == b).sum() == 1 for b in blocks], bool)


def test_decode_only_steps_mark_rows_alone_in_their_block():
    """A step of decode rows marks each row that no other row of the step writes beside;
    the same rows beside one prefill chunk are not marked (a prefill kernel then runs between
    the append and the decode rows)."""
    reqs = [(1, 40), (1, 15), (1, 16), (1, 31)]
    tables = [[5, 9, 11], [7], [20, 21], [30, 31]]
    out, cu, ctx, bt = staged_slots(reqs, tables)
    assert np.array_equal(out & ~SOLE, rule_slots(cu, ctx, bt))
    assert ((out & SOLE) != 0).all()
    out, cu, ctx, bt = staged_slots(reqs + [(20, 0)], tables + [[40, 41]])
    assert np.array_equal(out & ~SOLE, rule_slots(cu, ctx, bt))
    assert not ((out & SOLE) != 0).any()


def test_rows_of_requests_sharing_a_block_are_not_marked():
    """Two decode rows whose requests (wrongly) share their last block: neither may rewrite the
    page, or one would overwrite the other's new position; a request with no rows shares
    blocks without counting."""
    reqs = [(1, 3), (1, 4), (0, 7), (1, 0)]
    tables = [[8], [8], [40], [40]]
    out, cu, ctx, bt = staged_slots(reqs, tables)
    assert np.array_equal(out & ~SOLE, rule_slots(cu, ctx, bt))
    assert ((out & SOLE) != 0).tolist() == [False, False, True]


def test_marks_match_brute_force_on_a_random_permuted_pool():
    """Many decode rows on a randomly permuted pool (so the marks' hash table sees
    collisions), a few of them sharing a block with another request."""
    rng = np.random.default_rng(5)
    reqs, tables = [], []
    pool = rng.permutation(1 << 16).astype(np.int32)
    nxt = 0
    for _ in range(3000):
        c = int(rng.integers(0, 200))
        nb = c // 16 + 1
        t = pool[nxt:nxt + nb].tolist()
        nxt += nb
        if rng.random() < 0.03 and tables and len(tables[-1]) >= nb:
            t = tables[-1][:nb]                 # share the previous request's blocks
        reqs.append((1, c))
        tables.append(t)
    out, cu, ctx, bt = staged_slots(reqs, tables, num_blocks=1 << 16)
    ref = rule_slots(cu, ctx, bt)
    assert np.array_equal(out & ~SOLE, ref)
    assert np.array_equal((out & SOLE) != 0, brute_marks(ref))
    assert 2500 < ((out & SOLE) != 0).sum() < 3000


def test_marks_stop_where_the_bit_would_be_a_slot_bit():
    reqs, tables = [(1, 3)], [[5]]
    out, *_ = staged_slots(reqs, tables, num_blocks=1 << 26)
    assert out[0] == (5 * 16 + 3) | SOLE
    out, *_ = staged_slots(reqs, tables, num_blocks=(1 << 26) + 1)
    assert out[0] == 5 * 16 + 3
    with pytest.raises(cb.CbError):            # beyond int32 slots: the device looks them up
        staged_slots(reqs, tables, num_blocks=(1 << 27) + 1)


def test_step_slots_checks_block_ids():
    with pytest.raises(cb.CbError):
        staged_slots([(1, 20)], [[3]])         # position 20 needs a second block id
    with pytest.raises(cb.CbError):
        staged_slots([(1, 3)], [[5000]], num_blocks=4096)


def test_step_slots_agree_with_the_reference_scheduler():
    """Along a reference-scheduler trace (arrivals, chunked prefill, decode, EOS), the staged
    slots without their marks are the scheduler's slot mapping, and only decode-only steps
    carry marks."""
    from oracle.scheduler import RefScheduler
    rng = np.random.default_rng(3)
    s = RefScheduler(token_budget=256, block_size=16, num_blocks=2048)
    rid, seen_decode_only = 0, 0
    for step_i in range(80):
        for _ in range(int(rng.poisson(2 if step_i < 30 else 0))):
            s.add(rid, int(rng.integers(1, 300)), int(rng.integers(1, 40)))
            rid += 1
        st = s.build()
        if st.num_tokens == 0:
            s.commit()
            continue
        shape = cb.make_shape(8, 8, 128, 2048, "bf16")
        out = cb.cb_step_slots(shape, st.num_reqs, st.num_tokens, st.block_tables.shape[1], st.cu_q_lens,
                               st.ctx_lens, st.block_tables)
        assert np.array_equal(out & ~SOLE, st.slot_mapping), f"step {step_i}"
        decode_only = (np.diff(st.cu_q_lens) <= 1).all()
        want = brute_marks(st.slot_mapping.astype(np.int64)) if decode_only else np.zeros(st.num_tokens, bool)
        assert np.array_equal((out & SOLE) != 0, want), f"step {step_i}"
        seen_decode_only += int(decode_only)
        s.commit()
    assert seen_decode_only >= 5
