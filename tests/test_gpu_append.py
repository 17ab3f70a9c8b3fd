"""The KV append is bit-exact, on every entry path that writes the cache (needs an MI355X).

zhangchitc "continuous-batching", section "Inside the kernel": a step's new keys and values
are stored in the cache slots of their own request before attention reads them. Every test
starts from caches filled with NaN, writes through one path, then reads back every position
of every request through its block table and compares the stored bits with the pool values
(int16 views for bf16, int32 for fp32). Slots no request owns must still hold NaN, so a
write to a wrong slot is caught even where it holds a plausible value.
"""
import numpy as np
import pytest
import torch

import workloads as W
from ragged_continuous_batching_amd import cb
from ragged_continuous_batching_amd.cb import tuned
from ragged_continuous_batching_amd.runner import DeviceRun

from test_gpu_parity import check, oracle_full, small_workload

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def check_cache(run, step, chunk=1 << 16):
    """Every position 0..c+q-1 of every request of `step` holds its pool value bit for bit,
    and every other slot of both caches is still NaN."""
    bs = run.wl.block_size
    L = (step.ctx_lens + np.diff(step.cu_q_lens)).astype(np.int64)
    req = np.repeat(np.arange(step.num_reqs), L)
    pos = np.concatenate([np.arange(n) for n in L]) if len(L) else np.zeros(0, np.int64)
    rids = step.req_ids[req]
    blk = step.block_tables[req, pos // bs].astype(np.int64)
    off = pos % bs
    assert (blk >= 0).all()
    slots = blk * bs + off
    assert len(np.unique(slots)) == len(slots), "two positions share a cache slot"
    for s in range(0, len(pos), chunk):
        e = min(len(pos), s + chunk)
        b = torch.from_numpy(blk[s:e]).to(run.device)
        o = torch.from_numpy(off[s:e]).to(run.device)
        k = run.k_cache[b, :, o, :]                        # [n, Hkv, D]
        v = run.v_cache[b, :, :, o]                        # [n, Hkv, D]
        ek = run.gather(W.KIND_K, rids[s:e], pos[s:e])
        ev = run.gather(W.KIND_V, rids[s:e], pos[s:e])
        assert torch.equal(bits(k), bits(ek)), f"K differs in positions {s}..{e}"
        assert torch.equal(bits(v), bits(ev)), f"V differs in positions {s}..{e}"
    # pool values are finite, so the NaN count proves that nothing else was written
    per_slot = run.wl.num_kv_heads * run.wl.head_dim
    free = (run.wl.num_blocks * bs - len(slots)) * per_slot
    for name, c in (("K", run.k_cache), ("V", run.v_cache)):
        nan = int(torch.isnan(c).sum().item())
        assert nan == free, f"{name} cache: {nan} NaN values, expected {free} (a stray or missing write)"


def fresh_step(wl):
    run = DeviceRun(wl)
    step = run.sched.build()
    run.write_history(step)                       # cached prefixes through cb_kv_append
    q, k, v = run.step_inputs(step)
    return run, step, q, k, v


SHAPES = [  # (Hq, Hkv, D, dtype)
    (8, 1, 128, "bf16"), (8, 8, 128, "bf16"), (32, 32, 128, "bf16"), (8, 1, 64, "bf16"), (16, 8, 64, "bf16"),
    (32, 32, 64, "bf16"), (4, 1, 128, "f32"), (8, 8, 128, "f32"), (32, 32, 64, "f32"), (16, 8, 64, "f32"),
]


@pytest.mark.parametrize("path", ["append", "step_forward", "step_forward_copy_engine", "graph"])
@pytest.mark.parametrize("hq,hkv,d,dtype", SHAPES)
def test_append_bit_exact_from_nan_cache(path, hq, hkv, d, dtype):
    wl = small_workload("mixed", hq, hkv, d, dtype)
    run, step, q, k, v = fresh_step(wl)
    T = step.num_tokens
    o = torch.full_like(q, float("nan"))
    if path == "append":
        run.append(cb.Batch.from_step(step, device=run.device), k, v)
        o = run.attention(cb.Batch.from_step(step, device=run.device), q)
    elif path in ("step_forward", "step_forward_copy_engine"):
        need = cb.cb_step_workspace_size(run.shape, step.num_reqs, T, step.max_blocks_per_req, step.cu_q_lens,
                                         step.ctx_lens)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        with tuned(stage_kernel=int(path == "step_forward")):
            cb.cb_step_forward(run.shape, step.num_reqs, T, step.max_blocks_per_req, step.cu_q_lens, step.ctx_lens,
                               step.block_tables, q, k, v, run.k_cache, run.v_cache, wl.scale, o, ws, need, run.stream)
    else:
        g = cb.cb_graph_create(run.shape, T, q, k, v, run.k_cache, run.v_cache, wl.scale, o)
        try:
            cb.cb_graph_step(g, step.num_reqs, T, step.max_blocks_per_req, step.cu_q_lens, step.ctx_lens,
                             step.block_tables, run.stream)
            torch.cuda.synchronize()
        finally:
            cb.cb_graph_destroy(g)
    torch.cuda.synchronize()
    check_cache(run, step)
    check(o, oracle_full(wl, step), dtype, f"append {path} Hq={hq} Hkv={hkv} D={d} {dtype}")


@pytest.mark.parametrize("config,path", [(3, "append"), (4, "append"), (4, "step_forward"), (2, "step_forward")])
def test_append_bit_exact_full_size(config, path):
    """The named workloads at full size: config 3's 256 lognormal contexts on a permuted pool
    (about 0.9 M cached positions), config 4's four 2048-row chunks (8192 rows appended in one
    call), config 2's mixed step."""
    wl = W.config(config)
    run, step, q, k, v = fresh_step(wl)
    if path == "append":
        run.append(cb.Batch.from_step(step, device=run.device), k, v)
    else:
        T = step.num_tokens
        need = cb.cb_step_workspace_size(run.shape, step.num_reqs, T, step.max_blocks_per_req, step.cu_q_lens,
                                         step.ctx_lens)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        o = torch.empty_like(q)
        cb.cb_step_forward(run.shape, step.num_reqs, T, step.max_blocks_per_req, step.cu_q_lens, step.ctx_lens,
                           step.block_tables, q, k, v, run.k_cache, run.v_cache, wl.scale, o, ws, need, run.stream)
    torch.cuda.synchronize()
    check_cache(run, step)


def test_append_bit_exact_over_trace_steps():
    """Sixty steps of the scheduler trace through cb_step_forward: after each step every
    running request's cache (the positions appended in earlier steps, in blocks allocated
    as it grew, and this step's rows) holds its pool values; evicted requests' blocks are
    reused by later admissions without leaking old rows into them."""
    wl = W.config(5)
    run = DeviceRun(wl)
    ws = torch.empty(0, dtype=torch.uint8, device="cuda")
    for kstep in range(60):
        for r in wl.arrivals[kstep]:
            run.sched.add(r.req_id, r.prompt_len, r.out_len)
        step = run.sched.build()
        q, k, v = run.step_inputs(step)
        T = step.num_tokens
        need = cb.cb_step_workspace_size(run.shape, step.num_reqs, T, step.max_blocks_per_req, step.cu_q_lens,
                                         step.ctx_lens)
        if ws.numel() < need:
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        o = torch.empty_like(q)
        cb.cb_step_forward(run.shape, step.num_reqs, T, step.max_blocks_per_req, step.cu_q_lens, step.ctx_lens,
                           step.block_tables, q, k, v, run.k_cache, run.v_cache, wl.scale, o, ws, ws.numel(),
                           run.stream)
        torch.cuda.synchronize()
        if kstep % 10 == 9:
            check_cache_live(run, step)
        run.sched.commit()


def check_cache_live(run, step):
    """Like check_cache for the requests of `step`, without the NaN count (blocks of evicted
    requests keep their old rows until they are reused)."""
    bs = run.wl.block_size
    L = (step.ctx_lens + np.diff(step.cu_q_lens)).astype(np.int64)
    req = np.repeat(np.arange(step.num_reqs), L)
    pos = np.concatenate([np.arange(n) for n in L])
    blk = torch.from_numpy(step.block_tables[req, pos // bs].astype(np.int64)).to(run.device)
    off = torch.from_numpy(pos % bs).to(run.device)
    rids = step.req_ids[req]
    assert torch.equal(bits(run.k_cache[blk, :, off, :]), bits(run.gather(W.KIND_K, rids, pos)))
    assert torch.equal(bits(run.v_cache[blk, :, :, off]), bits(run.gather(W.KIND_V, rids, pos)))
