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


@pytest.mark.parametrize("path", ["step_forward", "graph"])
@pytest.mark.parametrize("with_chunk", [False, True])
@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 1), (6, 3)])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_whole_page_rewrites_keep_every_other_slot(dtype, d, hq, hkv, with_chunk, path):
    """In a decode-only step, rows alone in their block rewrite its whole transposed V page
    (cb_step_slots marks them); the other positions of that page must come back with the
    bits they held (finite values, and NaN where nothing was written). A hand-built step:
    decode rows alone in their blocks at the first, middle and last slot, and two decode rows
    whose requests share one block (not marked: each writes its element). With a prefill
    chunk added, no row is marked and every row writes element by element. The whole cache is
    compared bit for bit with the expected one, after cb_step_forward or a captured step.
    Odd kv head counts leave the last page work-group of two heads (D = 64 in bf16) with one."""
    nb, bs = 48, 16
    shape = cb.make_shape(hq, hkv, d, nb, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(11)
    # (q_len, ctx, table)
    reqs = [(1, 20, [3, 4]), (1, 5, [7]), (1, 2, [9]), (1, 6, [9]), (1, 16, [10, 11]), (1, 31, [12, 13]),
            (1, 47, [20, 21, 22])]
    if with_chunk:
        reqs.append((17, 16, [30, 31, 32]))
    cu = np.concatenate([[0], np.cumsum([r[0] for r in reqs])]).astype(np.int32)
    ctx = np.array([r[1] for r in reqs], np.int32)
    maxb = max(len(r[2]) for r in reqs)
    bt = np.full((len(reqs), maxb), -1, np.int32)
    for i, r in enumerate(reqs):
        bt[i, :len(r[2])] = r[2]
    T = int(cu[-1])
    slots = cb.cb_step_slots(shape, len(reqs), T, maxb, cu, ctx, bt)
    marked = (slots & cb.CB_SLOT_SOLE_WRITER) != 0
    want = [False] * T if with_chunk else [True, True, False, False, True, True, True]
    assert marked.tolist() == want
    slots = slots & ~cb.CB_SLOT_SOLE_WRITER
    # caches: referenced blocks hold finite values in their first half, NaN in the rest;
    # unreferenced blocks are NaN
    k_cache = torch.full((nb, hkv, bs, d), float("nan"), dtype=tdt)
    v_cache = torch.full((nb, hkv, d, bs), float("nan"), dtype=tdt)
    for b in sorted({b for r in reqs for b in r[2]}):
        k_cache[b, :, :8, :] = torch.randn(hkv, 8, d, generator=g).to(tdt)
        v_cache[b, :, :, :8] = torch.randn(hkv, d, 8, generator=g).to(tdt)
    k_new = torch.randn(T, hkv, d, generator=g).to(tdt)
    v_new = torch.randn(T, hkv, d, generator=g).to(tdt)
    q = torch.randn(T, hq, d, generator=g).to(tdt)
    k_exp, v_exp = k_cache.clone(), v_cache.clone()
    for t in range(T):
        b, o = int(slots[t]) // bs, int(slots[t]) % bs
        k_exp[b, :, o, :] = k_new[t]
        v_exp[b, :, :, o] = v_new[t]
    kc, vc = k_cache.cuda(), v_cache.cuda()
    qd, kd, vd = q.cuda(), k_new.cuda(), v_new.cuda()
    out = torch.empty_like(qd)
    stream = torch.cuda.current_stream().cuda_stream
    if path == "step_forward":
        need = cb.cb_step_workspace_size(shape, len(reqs), T, maxb, cu, ctx)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        cb.cb_step_forward(shape, len(reqs), T, maxb, cu, ctx, bt, qd, kd, vd, kc, vc, d ** -0.5, out, ws, need,
                           stream)
    else:
        gr = cb.cb_graph_create(shape, T, qd, kd, vd, kc, vc, d ** -0.5, out)
        try:
            cb.cb_graph_step(gr, len(reqs), T, maxb, cu, ctx, bt, stream)
            torch.cuda.synchronize()
        finally:
            cb.cb_graph_destroy(gr)
    torch.cuda.synchronize()
    assert torch.equal(bits(kc.cpu()), bits(k_exp))
    assert torch.equal(bits(vc.cpu()), bits(v_exp))
