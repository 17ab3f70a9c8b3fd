"""Every tuning key away from its default, against the fp64 oracle (needs an MI355X).

Knobs that only reorder work (launch order, XCD placement, the stream the prefill kernel
runs on) must leave every output bit-identical to the default; knobs that change how the
work is cut (split sizes, wave groups) are checked against the oracle at the usual bars
(bf16 max-abs <= 2e-2, mean-abs <= 2e-3; fp32 max-abs <= 1e-4).
"""
import numpy as np
import pytest
import torch

from ragged_continuous_batching_amd import cb
from ragged_continuous_batching_amd.cb import tuned
from ragged_continuous_batching_amd.runner import DeviceRun

from test_gpu_parity import check, oracle_full, run_one_step, small_workload, step_forward

pytestmark = pytest.mark.gpu


def both_entry_points(wl):
    """Output of the two-call form (cb_kv_append + cb_ragged_attention) and of
    cb_step_forward on a second, fresh run of the same step."""
    run, step, batch, o = run_one_step(wl)
    run2 = DeviceRun(wl)
    st2 = run2.sched.build()
    run2.write_history(st2)
    q, k, v = run2.step_inputs(st2)
    o2 = step_forward(run2, st2, q, k, v)
    torch.cuda.synchronize()
    return step, o, o2


@pytest.mark.parametrize("name,hq,hkv,d,split_tiles", [
    ("late_chunk", 4, 4, 128, 0), ("late_chunk", 8, 1, 128, 0), ("late_chunk", 4, 2, 64, 0),
    ("mixed", 8, 2, 128, 2), ("mixed", 4, 4, 64, 2), ("long_decode", 16, 2, 128, 3)])
def test_overlap_prefill_side_stream(name, hq, hkv, d, split_tiles):
    """Prefill tiles on the side stream beside the decode rows. The late chunk beside decode
    rows and the forced splits give prefill partials that the combine pass must read only
    after the side stream is joined back; the result is bit-identical to one stream."""
    wl = small_workload(name, hq, hkv, d, "bf16")
    with tuned(prefill_split_tiles=split_tiles):
        step, base, base2 = both_entry_points(wl)
        desc = cb.cb_plan_describe(cb.make_shape(hq, hkv, d, wl.num_blocks, "bf16"), cb.Batch.from_step(step).struct)
        assert desc["prefill_split_items"] > 0 and desc["decode_splits"] > 0, desc
        with tuned(overlap_prefill=1):
            for rep in range(3):            # the side stream's timing varies between repeats
                _, o, o2 = both_entry_points(wl)
                assert torch.equal(o, base), f"repeat {rep}: two-call form differs from one stream"
                assert torch.equal(o2, base2), f"repeat {rep}: cb_step_forward differs from one stream"
    check(o, oracle_full(wl, step), "bf16", f"overlap_prefill {name} Hq={hq} Hkv={hkv} D={d}")


@pytest.mark.parametrize("setting", [dict(xcds=1), dict(xcds=3), dict(xcds=16), dict(prefill_snake=0),
                                     dict(xcds=3, prefill_snake=0)])
@pytest.mark.parametrize("name,hq,hkv,d,waves", [("mixed", 8, 2, 128, 4), ("tile_edges", 4, 4, 128, 8),
                                                 ("late_chunk", 8, 8, 64, 0)])
def test_prefill_placement_knobs_keep_bits(setting, name, hq, hkv, d, waves):
    """XCD count and the snake order only move prefill work-groups around the launch."""
    wl = small_workload(name, hq, hkv, d, "bf16")
    with tuned(prefill_waves=waves):
        _, _, _, base = run_one_step(wl)
        with tuned(**setting):
            run, step, batch, o = run_one_step(wl)
    assert torch.equal(o, base), setting
    check(o, oracle_full(wl, step), "bf16", f"{setting} {name} Hq={hq} Hkv={hkv} D={d}")


@pytest.mark.parametrize("group", [1, 2, 4])
@pytest.mark.parametrize("hq,hkv,dtype", [(8, 1, "bf16"), (16, 2, "bf16"), (4, 1, "f32"), (8, 2, "f32")])
def test_decode_group_vector_alu(group, hq, hkv, dtype):
    """Fewer query heads per vector-ALU decode wave (several waves per kv head)."""
    wl = small_workload("long_decode", hq, hkv, 128, dtype)
    with tuned(decode_mfma=0, decode_group=group):
        run, step, batch, o = run_one_step(wl)
    check(o, oracle_full(wl, step), dtype, f"decode_group={group} Hq={hq} Hkv={hkv} {dtype}")


@pytest.mark.parametrize("target", [1, 64, 100000])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 2)])
def test_target_waves_split_sizing(target, hq, hkv):
    """The automatic split length aimed at other wave counts (1: one split per row unless
    the row exceeds the split cap; 100000: the shortest splits allowed)."""
    wl = small_workload("long_decode", hq, hkv, 128, "bf16")
    with tuned(target_waves=target):
        run, step, batch, o = run_one_step(wl)
    check(o, oracle_full(wl, step), "bf16", f"target_waves={target} Hq={hq} Hkv={hkv}")


@pytest.mark.parametrize("heads", [2, 4, 8])
@pytest.mark.parametrize("name,hq,hkv,d,waves,split_tiles", [
    ("mixed", 8, 2, 128, 8, 0), ("mixed", 8, 1, 128, 4, 0), ("tile_edges", 16, 2, 128, 8, 0),
    ("tile_edges", 32, 2, 64, 4, 0), ("late_chunk", 8, 1, 128, 0, 0), ("mixed", 16, 4, 64, 8, 2),
    ("long_decode", 64, 8, 128, 8, 3), ("mixed", 4, 2, 128, 4, 1)])
def test_prefill_heads_per_work_group(heads, name, hq, hkv, d, waves, split_tiles):
    """Several query heads of one kv head per prefill work-group (waves split into heads x
    32-row blocks over shared key/value tiles), with forced key-range splits in some cases;
    the heads per work-group are capped by the group size and the waves."""
    wl = small_workload(name, hq, hkv, d, "bf16")
    with tuned(prefill_heads=heads, prefill_waves=waves, prefill_split_tiles=split_tiles):
        run, step, batch, o = run_one_step(wl)
        desc = cb.cb_plan_describe(cb.make_shape(hq, hkv, d, wl.num_blocks, "bf16"), cb.Batch.from_step(step).struct)
    assert desc["prefill_heads"] == min(heads, hq // hkv, waves or 8) or waves == 0, desc
    check(o, oracle_full(wl, step), "bf16", f"prefill_heads={heads} {name} Hq={hq} Hkv={hkv} D={d} w={waves}")


@pytest.mark.parametrize("heads", [2, 8])
def test_prefill_heads_mixed_launch_and_graph(heads):
    """Shared-kv-head prefill items in the mixed launch (4-wave work-groups) and in a captured
    step: bit-identical to the two-launch eager step with the same items."""
    wl = small_workload("mixed", 16, 2, 128, "bf16")
    with tuned(prefill_heads=heads, prefill_waves=4):
        _, step, _, base = run_one_step(wl)
        with tuned(mixed_launch=1):
            _, _, _, o_mixed = run_one_step(wl)
        run = DeviceRun(wl)
        st = run.sched.build()
        run.write_history(st)
        q, k, v = run.step_inputs(st)
        o_g = torch.full_like(q, float("nan"))
        g = cb.cb_graph_create(run.shape, st.num_tokens, q, k, v, run.k_cache, run.v_cache, wl.scale, o_g)
        try:
            cb.cb_graph_step(g, st.num_reqs, st.num_tokens, st.max_blocks_per_req, st.cu_q_lens, st.ctx_lens,
                             st.block_tables, run.stream)
            torch.cuda.synchronize()
        finally:
            cb.cb_graph_destroy(g)
    assert torch.equal(o_mixed, base)
    assert torch.equal(o_g, base)
    check(base, oracle_full(wl, step), "bf16", f"prefill_heads={heads} mixed/graph")
