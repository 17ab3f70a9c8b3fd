"""cb_ragged_attention_noalloc against cb_ragged_attention, through the C ABI (needs an MI355X).

The entry point for callers that cannot allocate runs the same kernels as the workspace
form, with its plan and split-K partials in the library's fixed device array, so its
output must be bit-identical. Two calls in a row, the second on a smaller batch that reuses
what the first left in the array; each output is also checked against the fp64 oracle
(bf16 max-abs <= 2e-2, mean-abs <= 2e-3; fp32 max-abs <= 1e-4).
"""
import numpy as np
import pytest
import torch

import workloads as W
from ragged_continuous_batching_amd import cb
from ragged_continuous_batching_amd.runner import DeviceRun

from test_gpu_parity import check, oracle_full, oracle_rows, sample_rows, small_workload

pytestmark = pytest.mark.gpu


def both_forms(run, step):
    """(workspace form, no-alloc form) outputs of one built step; the cache is appended once."""
    run.write_history(step)
    batch = cb.Batch.from_step(step, device=run.device)
    q, k, v = run.step_inputs(step)
    run.append(batch, k, v)
    o_ws = run.attention(batch, q)
    o_na = torch.full_like(q, float("nan"))
    cb.cb_ragged_attention_noalloc(run.shape, batch.struct, q, run.k_cache, run.v_cache, run.wl.scale, o_na,
                                   run.stream)
    torch.cuda.synchronize()
    return batch, o_ws, o_na


def test_noalloc_matches_workspace_form_on_two_calls():
    # first call: the Llama-2-7B-shaped mixed step (split decode rows and split prefill tiles,
    # 2.3 MiB of plan and partials); second call: a smaller grouped-query mix
    wl1 = W.config(2, value_reading="unit")
    run1 = DeviceRun(wl1)
    step1 = run1.sched.build()
    batch1, o1_ws, o1_na = both_forms(run1, step1)
    need1 = cb.cb_ragged_attention_workspace_size(run1.shape, batch1.struct)
    wl2 = small_workload("long_decode", 16, 2, 128, "bf16")
    run2 = DeviceRun(wl2)
    step2 = run2.sched.build()
    batch2, o2_ws, o2_na = both_forms(run2, step2)
    need2 = cb.cb_ragged_attention_workspace_size(run2.shape, batch2.struct)
    assert 0 < need2 < need1 <= cb.NOALLOC_SCRATCH_BYTES, (need1, need2)
    assert torch.equal(o1_na, o1_ws), "first call differs from the workspace form"
    assert torch.equal(o2_na, o2_ws), "second (smaller) call differs from the workspace form"
    rows, ref = oracle_rows(wl1, step1, list(range(step1.num_decode)) +
                            [t for t in sample_rows(step1, 16, np.random.default_rng(31)) if t >= step1.num_decode])
    check(o1_na[torch.from_numpy(rows).cuda()], ref, "bf16", "no-alloc call 1 (config 2)")
    check(o2_na, oracle_full(wl2, step2), "bf16", "no-alloc call 2 (small mix)")


@pytest.mark.parametrize("name,hq,hkv,d,dtype", [("late_chunk", 8, 8, 128, "bf16"), ("mixed", 4, 2, 64, "bf16"),
                                                 ("mixed", 2, 2, 64, "f32")])
def test_noalloc_other_shapes(name, hq, hkv, d, dtype):
    """Prefill split partials (late chunk), D = 64, and the fp32 path, each after the calls
    above left other contents in the array."""
    wl = small_workload(name, hq, hkv, d, dtype)
    run = DeviceRun(wl)
    step = run.sched.build()
    _, o_ws, o_na = both_forms(run, step)
    assert torch.equal(o_na, o_ws)
    check(o_na, oracle_full(wl, step), dtype, f"no-alloc {name} Hq={hq} Hkv={hkv} D={d} {dtype}")
