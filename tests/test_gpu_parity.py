"""HIP path against the fp64 oracle, through the C ABI (needs an MI355X).

Inputs come from the seeded pools in ``workloads``. The oracle reads them on the CPU
straight from the pools and never sees anything the GPU produced. Every cache slot starts
as NaN, so any read outside a request's visible keys would surface as a NaN.
Bars: bf16 max-abs <= 2e-2 and mean-abs <= 2e-3; fp32 max-abs <= 1e-4; the KV append and
all indexing are bit-exact.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from ragged_continuous_batching_amd import cb
from ragged_continuous_batching_amd.runner import DeviceRun

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-4, 1e-4)}


def check(o_gpu, o_ref, dtype, what=""):
    o = o_gpu.detach().float().cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - o_ref)
    mx, mean = TOL[dtype]
    print(f"{what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} (n={err.size})", flush=True)
    assert err.max() <= mx, f"{what}: max abs err {err.max():.3e} > {mx}"
    assert err.mean() <= mean, f"{what}: mean abs err {err.mean():.3e} > {mean}"
    return err


def oracle_full(wl, step):
    """fp64 oracle of every row of a step (inputs regenerated from the pools)."""
    owner = step.token_to_req
    rids = step.req_ids[owner]
    pos = step.ctx_lens[owner] + (np.arange(step.num_tokens) - step.cu_q_lens[owner])
    q = wl.token_values(W.KIND_Q, rids, pos)
    k = wl.token_values(W.KIND_K, rids, pos)
    v = wl.token_values(W.KIND_V, rids, pos)
    hk = [wl.values(W.KIND_K, int(r), np.arange(c)) for r, c in zip(step.req_ids, step.ctx_lens)]
    hv = [wl.values(W.KIND_V, int(r), np.arange(c)) for r, c in zip(step.req_ids, step.ctx_lens)]
    return A.ragged_attention(q, k, v, hk, hv, step.cu_q_lens, step.ctx_lens, wl.scale)


def oracle_positions(wl, req_ids, positions, workers=None):
    """fp64 oracle of query rows given as (request id, absolute position) pairs, in the
    order given. A token's values depend only on its request and position, so all rows of
    one request (from one step or from several) are one oracle call over that request's
    keys 0..max position. Requests run on a thread pool (BLAS single-threaded inside) when
    there are many of them, else one at a time with threaded BLAS."""
    import concurrent.futures as cf
    import os
    from threadpoolctl import threadpool_limits
    req_ids = np.asarray(req_ids, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    out = np.zeros((len(req_ids), wl.num_q_heads, wl.head_dim))
    order = np.argsort(req_ids, kind="stable")
    bounds = np.flatnonzero(np.diff(req_ids[order])) + 1
    groups = np.split(order, bounds) if len(order) else []
    wl.raw_pool(W.KIND_Q)                         # build the pools once, before the threads

    def one(idx):
        rid, pos = int(req_ids[idx[0]]), positions[idx]
        L = int(pos.max()) + 1
        keys = wl.values(W.KIND_K, rid, np.arange(L))
        vals = wl.values(W.KIND_V, rid, np.arange(L))
        out[idx] = A.attend(wl.values(W.KIND_Q, rid, pos), keys, vals, pos, wl.scale)

    n = workers or min(16, len(os.sched_getaffinity(0)))
    if len(groups) >= 4 * n:
        with threadpool_limits(1), cf.ThreadPoolExecutor(n) as ex:
            list(ex.map(one, groups))
    else:
        for g in groups:
            one(g)
    return out


def step_positions(step, rows):
    rows = np.asarray(rows, dtype=np.int64)
    owner = step.token_to_req[rows]
    return step.req_ids[owner].astype(np.int64), step.ctx_lens[owner] + (rows - step.cu_q_lens[owner])


def oracle_rows(wl, step, rows):
    """fp64 oracle of selected packed rows of one step (sorted, duplicates dropped)."""
    rows = np.asarray(sorted(set(int(t) for t in rows)), dtype=np.int64)
    rids, pos = step_positions(step, rows)
    return rows, oracle_positions(wl, rids, pos)


def run_one_step(wl, **kw):
    run = DeviceRun(wl, **kw)
    step, batch, q, k, v, o = run.run_step()
    torch.cuda.synchronize()
    return run, step, batch, o


# --------------------------------------------------------------------------------------
def test_config1_tiny_step():
    wl = W.config(1)
    run, step, batch, o = run_one_step(wl)
    check(o, oracle_full(wl, step), "f32", "config 1")


def test_config1_listed_order_is_a_permutation():
    """The step listed as prefill-first runs bit-identically to the decode-first order."""
    wl = W.config(1)
    run, step, batch, o = run_one_step(wl)
    perm = [2, 0, 1]
    rows = np.concatenate([np.arange(step.cu_q_lens[r], step.cu_q_lens[r + 1]) for r in perm])
    lens = np.diff(step.cu_q_lens)[perm]
    b2 = cb.Batch(np.concatenate([[0], np.cumsum(lens)]), step.ctx_lens[perm], step.block_tables[perm])
    q, _, _ = run.step_inputs(step)
    o2 = run.attention(b2, q[torch.from_numpy(rows).cuda()].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o2, o[torch.from_numpy(rows).cuda()])


SMALL = {
    # (requests as (cached, prompt, generated) ; None cached = fresh prompt)
    "mixed": [(37, 37, 1), (0, 1, 0), (None, 130, 0), (5, 20, 0), (16, 16, 1), (None, 1, 0), (200, 300, 0)],
    "tile_edges": [(None, 129, 0), (63, 64 + 63 + 65, 0), (127, 127, 1), (None, 2, 0), (15, 15 + 17, 0)],
    "long_decode": [(2100, 2100, 1), (777, 777, 1), (None, 300, 0)],
    # a 256-row chunk after 4000 cached tokens: few, long prefill tiles, so the automatic
    # choice takes 256-row work-groups split over key ranges
    "late_chunk": [(4000, 4256, 0), (1500, 1500, 1), (None, 40, 0)],
}


def small_workload(name, hq, hkv, d, dtype, seed=3):
    reqs = []
    for i, (cached, prompt, gen) in enumerate(SMALL[name]):
        if cached is None:
            reqs.append(W.Request(i, prompt, 1 << 20))
        else:
            reqs.append(W.Request(i, prompt, 1 << 20, cached=cached, generated=gen))
    return W.custom(reqs, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype, seed=seed)


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("hq,hkv,d,dtype", [
    (4, 4, 128, "bf16"), (8, 2, 128, "bf16"), (16, 2, 128, "bf16"), (32, 2, 128, "bf16"), (4, 2, 64, "bf16"),
    (2, 2, 64, "f32"), (4, 1, 128, "f32"), (8, 8, 64, "bf16"),
])
def test_small_steps_full_oracle(name, hq, hkv, d, dtype):
    wl = small_workload(name, hq, hkv, d, dtype)
    run, step, batch, o = run_one_step(wl)
    check(o, oracle_full(wl, step), dtype, f"{name} Hq={hq} Hkv={hkv} D={d} {dtype}")


@pytest.mark.parametrize("hq,hkv,d,dtype", [(8, 1, 128, "bf16"), (2, 1, 64, "f32")])
def test_very_long_contexts(hq, hkv, d, dtype):
    """The largest contexts of any test: a decode row after 131,071 cached tokens (8192 cache
    blocks: thousands of short decode splits merged by one combine row), a 100-row chunk
    after 65,536 cached tokens (1026 key tiles per item, split over key ranges), and a fresh
    prompt. Every row against the oracle."""
    reqs = [W.Request(0, 131071, 1 << 20, cached=131071, generated=1),
            W.Request(1, 65636, 1 << 20, cached=65536, generated=0),
            W.Request(2, 70, 1 << 20)]
    wl = W.custom(reqs, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype, seed=11)
    run, step, batch, o = run_one_step(wl)
    assert list(np.diff(step.cu_q_lens)) == [1, 100, 70] and list(step.ctx_lens) == [131071, 65536, 0]
    rows, ref = oracle_rows(wl, step, range(step.num_tokens))
    check(o[torch.from_numpy(rows).cuda()], ref, dtype, f"very long contexts Hq={hq} Hkv={hkv} D={d} {dtype}")


def test_small_steps_normal_values_unit_scale():
    """Sharper softmax (scale 1, N(0,1) values) on the same ragged mix."""
    wl = small_workload("mixed", 8, 2, 128, "bf16")
    wl.scale = 0.25
    run, step, batch, o = run_one_step(wl)
    check(o, oracle_full(wl, step), "bf16", "mixed scale=0.25")


def test_append_is_bit_exact_and_stays_in_its_slots():
    wl = small_workload("mixed", 4, 2, 128, "bf16")
    run, step, batch, o = run_one_step(wl)
    for i, rid in enumerate(step.req_ids.tolist()):
        L = int(step.ctx_lens[i] + step.cu_q_lens[i + 1] - step.cu_q_lens[i])
        k, v = run.gather_cache(step.block_tables[i], L)
        ek = run.gather(W.KIND_K, np.full(L, rid), np.arange(L))
        ev = run.gather(W.KIND_V, np.full(L, rid), np.arange(L))
        assert torch.equal(k.view(torch.int16), ek.view(torch.int16))
        assert torch.equal(v.view(torch.int16), ev.view(torch.int16))
    # slots never written are still NaN (nothing outside a request's slots was touched)
    kc = run.k_cache.float()
    written = torch.zeros(kc.shape[0], kc.shape[2], dtype=torch.bool, device=kc.device)
    for i in range(step.num_reqs):
        L = int(step.ctx_lens[i] + step.cu_q_lens[i + 1] - step.cu_q_lens[i])
        for p in range(L):
            written[int(step.block_tables[i][p // 16]), p % 16] = True
    assert torch.isnan(kc.permute(0, 2, 1, 3)[~written]).all()


def step_forward(run, step, q, k, v):
    """The fused entry point: one upload of host metadata + plan, append, attention."""
    need = cb.cb_step_workspace_size(run.shape, step.num_reqs, step.num_tokens, step.max_blocks_per_req,
                                     step.cu_q_lens, step.ctx_lens)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    cb.cb_step_forward(run.shape, step.num_reqs, step.num_tokens, step.max_blocks_per_req, step.cu_q_lens,
                       step.ctx_lens, step.block_tables, q, k, v, run.k_cache, run.v_cache, run.wl.scale, o, ws,
                       need, run.stream)
    return o


@pytest.mark.parametrize("name,hq,hkv,d,dtype", [("mixed", 8, 2, 128, "bf16"), ("tile_edges", 4, 4, 128, "bf16"),
                                                 ("long_decode", 16, 2, 128, "bf16"), ("mixed", 2, 2, 64, "f32")])
def test_step_forward_matches_two_calls_and_oracle(name, hq, hkv, d, dtype):
    wl = small_workload(name, hq, hkv, d, dtype)
    run, step, batch, o = run_one_step(wl)           # append + attention through the two calls
    q, k, v = run.step_inputs(step)
    o2 = step_forward(run, step, q, k, v)            # appends the same rows again, then attends
    torch.cuda.synchronize()
    assert torch.equal(o2, o)
    check(o2, oracle_full(wl, step), dtype, f"step_forward {name} Hq={hq} Hkv={hkv} D={d} {dtype}")


def test_copy_engine_and_stage_kernel_uploads_agree():
    """The metadata upload as a copy kernel (default) or through the copy engine: same bits."""
    wl = small_workload("mixed", 8, 2, 128, "bf16")
    outs = []
    try:
        for mode in (0, 1, 0):
            cb.cb_set_tuning("stage_kernel", mode)
            run = DeviceRun(wl)
            step = run.sched.build()
            run.write_history(step)
            q, k, v = run.step_inputs(step)
            outs.append(step_forward(run, step, q, k, v))
            outs.append(run.attention(cb.Batch.from_step(step, device=run.device), q))
    finally:
        cb.cb_set_tuning("stage_kernel", 1)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    check(outs[0], oracle_full(wl, step), "bf16", "uploads")


def test_step_forward_fresh_cache_config2():
    """Config 2 through the fused entry point alone (history appended beforehand)."""
    wl = W.config(2, value_reading="unit")
    run = DeviceRun(wl)
    step = run.sched.build()
    run.write_history(step)
    q, k, v = run.step_inputs(step)
    o = step_forward(run, step, q, k, v)
    torch.cuda.synchronize()
    rows = list(range(step.num_decode)) + [t for t in sample_rows(step, 16, np.random.default_rng(9))
                                           if t >= step.num_decode]
    rows, ref = oracle_rows(wl, step, rows)
    check(o[torch.from_numpy(rows).cuda()], ref, "bf16", "step_forward config 2")


@pytest.mark.parametrize("name,hq,hkv,d", [("mixed", 8, 2, 128), ("tile_edges", 4, 4, 128), ("mixed", 4, 2, 64)])
def test_prefill_eight_wave_work_groups(name, hq, hkv, d):
    """256 query rows per prefill work-group (8 waves) against the oracle."""
    wl = small_workload(name, hq, hkv, d, "bf16")
    try:
        cb.cb_set_tuning("prefill_waves", 8)
        run, step, batch, o = run_one_step(wl)
    finally:
        cb.cb_set_tuning("prefill_waves", 0)
    check(o, oracle_full(wl, step), "bf16", f"prefill 8 waves {name} Hq={hq} Hkv={hkv} D={d}")


@pytest.mark.parametrize("waves", [4, 8])
def test_config4_prefill_waves(waves):
    """Config 4 with each prefill work-group size forced (the default picks one by size)."""
    wl = W.config(4)
    try:
        cb.cb_set_tuning("prefill_waves", waves)
        run, step, batch, o = run_one_step(wl)
    finally:
        cb.cb_set_tuning("prefill_waves", 0)
    rows, ref = oracle_rows(wl, step, sample_rows(step, 20, np.random.default_rng(4)) + [255, 256, 257, 511, 512])
    check(o[torch.from_numpy(rows).cuda()], ref, "bf16", f"config 4, {waves}-wave prefill")


@pytest.mark.parametrize("hq,hkv", [(8, 2), (16, 2), (32, 2)])
def test_gqa_decode_vector_alu_kernel(hq, hkv):
    """The vector-ALU decode kernel also serves grouped-query rows when the matrix-core
    kernel is switched off ("decode_mfma" = 0)."""
    wl = small_workload("long_decode", hq, hkv, 128, "bf16")
    cb.cb_set_tuning("decode_mfma", 0)
    try:
        run, step, batch, o = run_one_step(wl)
    finally:
        cb.cb_set_tuning("decode_mfma", 1)
    check(o, oracle_full(wl, step), "bf16", f"vector-ALU decode Hq={hq} Hkv={hkv}")


@pytest.mark.parametrize("split", [4, 7, 64])
def test_split_count_invariance(split):
    wl = small_workload("long_decode", 8, 2, 128, "bf16")
    cb.cb_set_tuning("split_blocks", split)
    try:
        run, step, batch, o = run_one_step(wl)
    finally:
        cb.cb_set_tuning("split_blocks", 0)
    check(o, oracle_full(wl, step), "bf16", f"split_blocks={split}")


def test_block_permutation_invariance():
    """Physical block ids do not change the result (bit-identical)."""
    base = small_workload("mixed", 8, 2, 128, "bf16")
    outs = []
    for fl in (None, np.random.default_rng(5).permutation(base.num_blocks).astype(np.int32)):
        wl = small_workload("mixed", 8, 2, 128, "bf16")
        wl.free_list = fl
        run, step, batch, o = run_one_step(wl)
        outs.append(o.clone())
    assert torch.equal(outs[0], outs[1])


# --------------------------------------------------------------------------------------
# the named workloads at full size
# --------------------------------------------------------------------------------------
def sample_rows(step, per_req, rng):
    rows = []
    for i in range(step.num_reqs):
        s, e = int(step.cu_q_lens[i]), int(step.cu_q_lens[i + 1])
        n = e - s
        pick = {s, e - 1} | {s + int(x) for x in rng.integers(0, n, size=min(per_req, n))}
        if n > 128:
            pick |= {s + 127, s + 128}
        rows += sorted(pick)
    return rows


@pytest.mark.parametrize("reading", ["literal", "unit"])
def test_config2_mixed_step(reading):
    wl = W.config(2, value_reading=reading)
    run, step, batch, o = run_one_step(wl)
    rng = np.random.default_rng(0)
    dec = list(range(step.num_decode))
    pre = [t for t in sample_rows(step, 24, rng) if t >= step.num_decode]
    rows, ref = oracle_rows(wl, step, dec + pre)
    got = o[torch.from_numpy(rows).cuda()]
    check(got, ref, "bf16", f"config 2 ({reading})")
    if reading == "unit":
        g = got.float().cpu().numpy().astype(np.float64)
        assert np.linalg.norm(g - ref) / np.linalg.norm(ref) <= 1e-2


def test_config3_decode_gqa():
    """Every row of the decode-only step (256 requests, lognormal contexts up to 32k)."""
    wl = W.config(3)
    run, step, batch, o = run_one_step(wl)
    rows, ref = oracle_rows(wl, step, range(step.num_tokens))
    assert len(rows) == 256
    check(o[torch.from_numpy(rows).cuda()], ref, "bf16", "config 3 (all rows)")


def chunk_edge_rows(step, tile=256, boundary=128):
    """Every row of each prefill chunk's first and last `tile` rows, and the two rows on each
    side of every multiple of `boundary` inside the chunk (work-group and key-tile edges)."""
    rows = set()
    for i in range(step.num_reqs):
        s, e = int(step.cu_q_lens[i]), int(step.cu_q_lens[i + 1])
        rows |= set(range(s, min(e, s + tile))) | set(range(max(s, e - tile), e))
        for b in range(boundary, e - s, boundary):
            rows |= {s + b - 1, s + b}
    return sorted(rows)


def test_config4_chunked_prefill():
    wl = W.config(4)
    run, step, batch, o = run_one_step(wl)
    rows, ref = oracle_rows(wl, step, chunk_edge_rows(step))
    assert len(rows) == 4 * 512 + 4 * 2 * 12
    check(o[torch.from_numpy(rows).cuda()], ref, "bf16", "config 4 (chunk edges)")


def test_largest_step():
    """A step four times config 4's width: 32,768 packed rows (a decode row and fifteen
    2048-row chunks after contexts 0..28,672, one 2047-row chunk), Hq = 8, Hkv = 1. Sampled
    rows (first and last rows of each chunk, work-group edges) against the oracle; the decode
    row too."""
    reqs = [W.Request(0, 3000, 1 << 20, cached=3000, generated=1)]
    for i in range(15):
        c = 2048 * i
        reqs.append(W.Request(1 + i, c + 2048, 1 << 20, cached=c, generated=0))
    reqs.append(W.Request(16, 2047, 1 << 20))
    wl = W.custom(reqs, num_q_heads=8, num_kv_heads=1, head_dim=128, dtype="bf16", seed=13)
    run, step, batch, o = run_one_step(wl)
    assert step.num_tokens == 1 + 15 * 2048 + 2047 == 32768
    rows, ref = oracle_rows(wl, step, chunk_edge_rows(step, tile=40, boundary=512))
    check(o[torch.from_numpy(rows).cuda()], ref, "bf16", f"largest step ({len(rows)} sampled rows)")


def test_config5_trace_replay():
    """500 steps of the scheduler trace with append + attention every step. The first and the
    last row of every request in the contiguous window of steps 150..199 (about 30k rows;
    a token's values depend only on its request and position, so each request's rows from
    all 50 steps are one oracle call), plus sampled rows of every 50th step."""
    wl = W.config(5)
    run = DeviceRun(wl, stale=None)
    rng = np.random.default_rng(5)
    checked = 0
    win_rid, win_pos, win_got, win_step = [], [], [], []
    for k in range(wl.steps):
        for r in wl.arrivals[k]:
            run.sched.add(r.req_id, r.prompt_len, r.out_len)
        step, batch, q, kn, vn, o = run.run_step()
        if 150 <= k < 200:
            rows = np.array(sorted(set(step.cu_q_lens[:-1].tolist()) | set((step.cu_q_lens[1:] - 1).tolist())))
            rid, pos = step_positions(step, rows)
            win_rid.append(rid)
            win_pos.append(pos)
            win_got.append(o[torch.from_numpy(rows).cuda()].float().cpu())
            win_step.append(np.full(len(rows), k))
        if k % 50 == 49 or k == 0:
            torch.cuda.synchronize()
            cand = sample_rows(step, 2, rng)
            rows, ref = oracle_rows(wl, step, rng.choice(cand, size=min(64, len(cand)), replace=False))
            check(o[torch.from_numpy(rows).cuda()], ref, "bf16", f"config 5 step {k} (T={step.num_tokens})")
            checked += 1
        run.sched.commit()
    assert checked == 11
    ref = oracle_positions(wl, np.concatenate(win_rid), np.concatenate(win_pos))
    got = torch.cat(win_got)
    assert len(got) > 20000
    check(got, ref, "bf16", "config 5 steps 150-199, first and last row of every request")


@pytest.mark.parametrize("batch_size", [1, 3])
def test_static_batching_steps(batch_size):
    """Naive padded batching runs through the same kernels: every row of every step,
    pad rows and the rows of finished members included, matches the oracle (cache values
    depend only on (request, position), so a pad slot that a decode row later overwrites
    holds the same value either way)."""
    reqs = [W.Request(0, 37, 3), W.Request(1, 5, 6), W.Request(2, 130, 2), W.Request(3, 1, 4), W.Request(4, 64, 1)]
    wl = W.custom(reqs, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16", seed=9)
    run = DeviceRun(wl)
    run.sched.set_static(batch_size)
    n = 0
    while True:
        step = run.sched.build()
        if step.num_reqs == 0:
            break
        _, batch, q, k, v, o = run.run_step(step)
        torch.cuda.synchronize()
        check(o, oracle_full(wl, step), "bf16", f"static B={batch_size} step {n} (T={step.num_tokens})")
        run.sched.commit()
        n += 1
    expect = 0
    for i in range(0, len(reqs), batch_size):
        expect += max(r.out_len for r in reqs[i:i + batch_size])
    assert n == expect


def test_preemption_recompute_steps():
    """A pool too small for every running request: preempted requests come back and prefill
    their prompt and generated tokens again. Every row of every step matches the oracle."""
    reqs = [W.Request(i, p, o) for i, (p, o) in enumerate([(40, 45), (25, 60), (60, 30), (18, 50), (33, 40)])]
    wl = W.custom(reqs, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16", seed=4, token_budget=96,
                  num_blocks=14)
    run = DeviceRun(wl)
    run.sched.set_preemption(True)
    n, preempted, rows = 0, 0, 0
    while True:
        step = run.sched.build()
        preempted += len(step.preempted)
        if step.num_reqs == 0 and run.sched.stats()[:2] == (0, 0):
            break
        if step.num_reqs:
            _, batch, q, k, v, o = run.run_step(step)
            torch.cuda.synchronize()
            check(o, oracle_full(wl, step), "bf16", f"preemption step {n} (T={step.num_tokens})")
            rows += step.num_tokens
        run.sched.commit()
        n += 1
        assert n < 2000
    assert preempted > 0
    assert rows > sum(r.prompt_len + r.out_len - 1 for r in reqs)


# --------------------------------------------------------------------------------------
# token-wise layers (QKV projection with the fused paged append, output projection)
# --------------------------------------------------------------------------------------
from oracle import layer as LY  # noqa: E402


def bf16_tensor(values):
    bits = W.bf16_bits_from_f32(np.asarray(values, dtype=np.float32))
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def check_rounded(got, ref, what):
    """bf16 outputs of an fp32-accumulated product: within half an ulp of bf16 (2^-8 of the
    magnitude) plus a small absolute slack for the fp32 accumulation."""
    g = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4
    print(f"{what}: max_abs={err.max():.3e} worst_ratio={(err / bound).max():.3f}", flush=True)
    assert np.isfinite(g).all()
    assert (err <= bound).all(), f"{what}: {(err > bound).sum()} elements beyond the rounding bound"


@pytest.mark.parametrize("M,N,K", [(1, 128, 64), (77, 256, 192), (300, 384, 512), (1024, 128, 4096), (2048, 12288, 4096), (600, 4096, 4096)])
def test_linear_parity(M, N, K):
    rng = np.random.default_rng(M + N + K)
    a = W.f32_from_bf16_bits(W.bf16_bits_from_f32(rng.standard_normal((M, K)).astype(np.float32)))
    w = W.f32_from_bf16_bits(W.bf16_bits_from_f32((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)))
    c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    cb.cb_linear(M, N, K, bf16_tensor(a), bf16_tensor(w), c)
    torch.cuda.synchronize()
    check_rounded(c, LY.linear(a, w), f"linear M={M} N={N} K={K}")


def qkv_inputs(wl, step, d_model, history=False):
    """Layer inputs of the step's rows (or of every request's cached history)."""
    if history:
        rids = np.concatenate([np.full(c, r) for r, c in zip(step.req_ids, step.ctx_lens)]).astype(np.int64)
        pos = np.concatenate([np.arange(c) for c in step.ctx_lens]).astype(np.int64)
    else:
        owner = step.token_to_req
        rids = step.req_ids[owner]
        pos = step.ctx_lens[owner] + (np.arange(step.num_tokens) - step.cu_q_lens[owner])
    return rids, pos, wl.x_values(rids, pos, d_model)


def project_history(run, step, w_qkv_t, d_model):
    """Writes every request's cached positions through the fused projection (one packed call)."""
    wl = run.wl
    lens = step.ctx_lens.astype(np.int32)
    if lens.sum() == 0:
        return
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    batch = cb.Batch(cu, np.zeros(len(lens), np.int32), step.block_tables, device=run.device)
    _, _, x = qkv_inputs(wl, step, d_model, history=True)
    q = torch.empty(int(cu[-1]), wl.num_q_heads, wl.head_dim, dtype=torch.bfloat16, device="cuda")
    cb.cb_qkv_project(run.shape, batch.struct, d_model, bf16_tensor(x), w_qkv_t, q, run.k_cache, run.v_cache)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 1)])
def test_qkv_project_writes_q_and_cache(hq, hkv):
    d_model = 256
    wl = small_workload("mixed", hq, hkv, 128, "bf16")
    run = DeviceRun(wl)
    step = run.sched.build()
    n_out = (hq + 2 * hkv) * 128
    w = W.f32_from_bf16_bits(W.layer_weights(wl.seed, 0, n_out, d_model))
    batch = cb.Batch.from_step(step, device=run.device)
    rids, pos, x = qkv_inputs(wl, step, d_model)
    q = torch.empty(step.num_tokens, hq, 128, dtype=torch.bfloat16, device="cuda")
    cb.cb_qkv_project(run.shape, batch.struct, d_model, bf16_tensor(x), bf16_tensor(w), q, run.k_cache, run.v_cache)
    torch.cuda.synchronize()
    qr, kr, vr = LY.qkv_split(LY.linear(x, w), hq, hkv, 128)
    check_rounded(q.reshape(step.num_tokens, -1), qr.reshape(step.num_tokens, -1), f"qkv Q Hq={hq} Hkv={hkv}")
    # keys and values at each row's slot (K pages [blk][g][off][d], V pages [blk][g][d][off])
    blk = torch.from_numpy((step.slot_mapping // 16).astype(np.int64)).cuda()
    off = torch.from_numpy((step.slot_mapping % 16).astype(np.int64)).cuda()
    kc = run.k_cache[blk, :, off, :]
    vc = run.v_cache[blk, :, :, off]
    check_rounded(kc.reshape(step.num_tokens, -1), kr.reshape(step.num_tokens, -1), "qkv K pages")
    check_rounded(vc.reshape(step.num_tokens, -1), vr.reshape(step.num_tokens, -1), "qkv V pages")
    # slots of the step's blocks that no row wrote keep their stale fill
    used = set(step.slot_mapping.tolist())
    free = [b * 16 + o for b in set((step.slot_mapping // 16).tolist()) for o in range(16) if b * 16 + o not in used]
    if free:
        fb = torch.tensor([f // 16 for f in free], device="cuda")
        fo = torch.tensor([f % 16 for f in free], device="cuda")
        assert torch.isnan(run.k_cache[fb, :, fo, :].float()).all()


def test_layer_step_end_to_end():
    """x -> fused QKV projection (+ paged append) -> ragged attention -> output projection,
    against the fp64 chain (no intermediate rounding) on a mixed step with cached history."""
    hq, hkv, d, d_model = 8, 2, 128, 256
    wl = small_workload("mixed", hq, hkv, d, "bf16")
    run = DeviceRun(wl)
    step = run.sched.build()
    run._pending_history.clear()                     # history comes from the projection here
    w_qkv = W.f32_from_bf16_bits(W.layer_weights(wl.seed, 0, (hq + 2 * hkv) * d, d_model))
    w_o = W.f32_from_bf16_bits(W.layer_weights(wl.seed, 1, d_model, hq * d))
    wq_t, wo_t = bf16_tensor(w_qkv), bf16_tensor(w_o)
    project_history(run, step, wq_t, d_model)
    batch = cb.Batch.from_step(step, device=run.device)
    _, _, x = qkv_inputs(wl, step, d_model)
    q = torch.empty(step.num_tokens, hq, d, dtype=torch.bfloat16, device="cuda")
    cb.cb_qkv_project(run.shape, batch.struct, d_model, bf16_tensor(x), wq_t, q, run.k_cache, run.v_cache)
    attn = run.attention(batch, q)
    y = torch.empty(step.num_tokens, d_model, dtype=torch.bfloat16, device="cuda")
    cb.cb_linear(step.num_tokens, d_model, hq * d, attn.reshape(step.num_tokens, -1), wo_t, y)
    torch.cuda.synchronize()
    # fp64 chain
    qr, kr, vr = LY.qkv_split(LY.linear(x, w_qkv), hq, hkv, d)
    _, _, xh = qkv_inputs(wl, step, d_model, history=True)
    _, khr, vhr = LY.qkv_split(LY.linear(xh, w_qkv), hq, hkv, d) if len(xh) else (None, np.zeros((0, hkv, d)),
                                                                                    np.zeros((0, hkv, d)))
    hk, hv, o0 = [], [], 0
    for c in step.ctx_lens.tolist():
        hk.append(khr[o0:o0 + c])
        hv.append(vhr[o0:o0 + c])
        o0 += c
    attn_ref = A.ragged_attention(qr, kr, vr, hk, hv, step.cu_q_lens, step.ctx_lens, wl.scale)
    y_ref = LY.linear(attn_ref.reshape(step.num_tokens, -1), w_o)
    check(y, y_ref, "bf16", "layer step y")


# --------------------------------------------------------------------------------------
# prefill tiles and grouped-query decode waves in one launch ("mixed_launch")
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("name,hq,hkv,d,order", [("mixed", 8, 2, 128, 0), ("mixed", 16, 2, 128, 0),
                                                 ("tile_edges", 16, 4, 128, 0), ("long_decode", 32, 2, 128, 0),
                                                 ("mixed", 8, 1, 64, 0), ("mixed", 64, 8, 128, 0),
                                                 ("mixed", 16, 2, 128, 1), ("tile_edges", 16, 4, 128, 1)])
def test_mixed_launch_matches_two_launches_and_oracle(name, hq, hkv, d, order):
    """The mixed launch runs the same tile and wave code as the two kernels (with 128-row
    prefill work-groups), so its output is bit-identical, in either work-group order; and
    it matches the oracle."""
    wl = small_workload(name, hq, hkv, d, "bf16")
    outs = []
    try:
        cb.cb_set_tuning("prefill_waves", 4)
        cb.cb_set_tuning("mixed_order", order)
        for mixed in (0, 1):
            cb.cb_set_tuning("mixed_launch", mixed)
            cb.cb_profile_reset()
            cb.cb_profile_enable(True)
            run, step, batch, o = run_one_step(wl)
            cb.cb_profile_enable(False)
            launched = {k: cb.cb_profile_read(v)[1] for k, v in cb.KERNELS.items()}
            assert launched["mixed"] == mixed and launched["prefill"] == 1 - mixed, launched
            outs.append(o)
    finally:
        cb.cb_profile_enable(False)
        cb.cb_profile_reset()
        cb.cb_set_tuning("mixed_launch", 0)
        cb.cb_set_tuning("mixed_order", 0)
        cb.cb_set_tuning("prefill_waves", 0)
    assert torch.equal(outs[0], outs[1])
    check(outs[1], oracle_full(wl, step), "bf16", f"mixed launch {name} Hq={hq} Hkv={hkv} D={d}")


def test_profile_select_times_only_the_selected_kernels():
    """cb_profile_select restricts the event pairs to the selected kernel ids; None restores
    every kernel. The outputs do not depend on it."""
    wl = small_workload("mixed", 8, 8, 128, "bf16")
    outs, launched = [], []
    try:
        for sel in ([cb.KERNELS["decode"]], None):
            cb.cb_profile_reset()
            cb.cb_profile_select(sel)
            cb.cb_profile_enable(True)
            run, step, batch, o = run_one_step(wl)
            cb.cb_profile_enable(False)
            launched.append({k: cb.cb_profile_read(v)[1] for k, v in cb.KERNELS.items()})
            outs.append(o)
    finally:
        cb.cb_profile_enable(False)
        cb.cb_profile_select(None)
        cb.cb_profile_reset()
    assert launched[0] == {k: int(k == "decode") for k in cb.KERNELS}, launched[0]
    assert launched[1]["append"] >= 1 and launched[1]["decode"] == 1 and launched[1]["prefill"] == 1, launched[1]
    assert torch.equal(outs[0], outs[1])


def test_mixed_launch_trace_replay():
    """The first 150 steps of the scheduler trace with the mixed launch; sampled rows of
    every 30th step against the oracle."""
    wl = W.config(5)
    run = DeviceRun(wl, stale=None)
    rng = np.random.default_rng(15)
    cb.cb_set_tuning("mixed_launch", 1)
    checked = 0
    try:
        for k in range(150):
            for r in wl.arrivals[k]:
                run.sched.add(r.req_id, r.prompt_len, r.out_len)
            step, batch, q, kn, vn, o = run.run_step()
            if k % 30 == 29:
                torch.cuda.synchronize()
                cand = sample_rows(step, 2, rng)
                rows, ref = oracle_rows(wl, step, rng.choice(cand, size=min(64, len(cand)), replace=False))
                check(o[torch.from_numpy(rows).cuda()], ref, "bf16", f"mixed trace step {k} (T={step.num_tokens})")
                checked += 1
            run.sched.commit()
    finally:
        cb.cb_set_tuning("mixed_launch", 0)
    assert checked == 5


# --------------------------------------------------------------------------------------
# split-K of long prefill tiles ("prefill_split"); partials merged by the combine pass
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("name,hq,hkv,d,waves,split_tiles,mixed", [
    ("mixed", 8, 2, 128, 4, 2, 0), ("tile_edges", 4, 4, 128, 4, 1, 0), ("mixed", 4, 2, 64, 4, 3, 0),
    ("tile_edges", 8, 2, 128, 8, 2, 0), ("mixed", 16, 2, 128, 4, 2, 1), ("long_decode", 16, 4, 128, 4, 5, 0)])
def test_prefill_split_against_oracle(name, hq, hkv, d, waves, split_tiles, mixed):
    """Tiny split lengths force several key ranges per prefill tile (cuts at or below each
    tile's first row), with 4- and 8-wave work-groups and in the mixed launch."""
    wl = small_workload(name, hq, hkv, d, "bf16")
    try:
        cb.cb_set_tuning("prefill_split_tiles", split_tiles)
        cb.cb_set_tuning("prefill_waves", waves)
        cb.cb_set_tuning("mixed_launch", mixed)
        run, step, batch, o = run_one_step(wl)
    finally:
        cb.cb_set_tuning("prefill_split_tiles", 0)
        cb.cb_set_tuning("prefill_waves", 0)
        cb.cb_set_tuning("mixed_launch", 0)
    check(o, oracle_full(wl, step), "bf16", f"prefill split {split_tiles} {name} Hq={hq} Hkv={hkv} D={d} w={waves}")


def test_prefill_split_off_matches_oracle_config2():
    """Config 2 with prefill splitting off (the default splits its c = 1024 chunk)."""
    wl = W.config(2, value_reading="unit")
    try:
        cb.cb_set_tuning("prefill_split", 0)
        run, step, batch, o = run_one_step(wl)
    finally:
        cb.cb_set_tuning("prefill_split", 1)
    rows, ref = oracle_rows(wl, step, [t for t in sample_rows(step, 24, np.random.default_rng(21)) if t >= 64])
    check(o[torch.from_numpy(rows).cuda()], ref, "bf16", "config 2 prefill unsplit")


def test_requests_with_no_rows_in_every_entry_point():
    """A request may take no rows in a step (q = 0 is legal). Its block ids are not staged
    (compact tables) and it gets no slots; every entry point must skip it, and all other
    rows match the two-call form bit for bit and the oracle."""
    wl = small_workload("mixed", 8, 2, 128, "bf16")
    run = DeviceRun(wl)
    step = run.sched.build()
    run.write_history(step)
    q, k, v = run.step_inputs(step)
    # insert empty requests before, between and after the real ones (same tables)
    R = step.num_reqs
    order = [None]
    for i in range(R):
        order += [i, None]
    cu, ctx, rows = [0], [], []
    for x in order:
        if x is None:
            ctx.append(5)
            rows.append(step.block_tables[0])
            cu.append(cu[-1])
        else:
            n = int(step.cu_q_lens[x + 1] - step.cu_q_lens[x])
            ctx.append(int(step.ctx_lens[x]))
            rows.append(step.block_tables[x])
            cu.append(cu[-1] + n)
    cu, ctx, bt = np.array(cu, np.int32), np.array(ctx, np.int32), np.stack(rows).astype(np.int32)
    assert cu[-1] == step.num_tokens
    shape, T, Rz, maxb = run.shape, step.num_tokens, len(ctx), bt.shape[1]
    # two-call form with the original batch (reference bits): append, then attend
    batch = cb.Batch.from_step(step, device=run.device)
    run.append(batch, k, v)
    o_ref = run.attention(batch, q)
    need = cb.cb_step_workspace_size(shape, Rz, T, maxb, cu, ctx)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o1 = torch.empty_like(q)
    cb.cb_step_forward(shape, Rz, T, maxb, cu, ctx, bt, q, k, v, run.k_cache, run.v_cache, wl.scale, o1, ws, need,
                       run.stream)
    o2 = torch.full_like(q, float("nan"))
    g = cb.cb_graph_create(shape, T, q, k, v, run.k_cache, run.v_cache, wl.scale, o2)
    try:
        cb.cb_graph_step(g, Rz, T, maxb, cu, ctx, bt, run.stream)
        torch.cuda.synchronize()
    finally:
        cb.cb_graph_destroy(g)
    assert torch.equal(o1, o_ref)
    assert torch.equal(o2, o_ref)
    check(o1, oracle_full(wl, step), "bf16", "empty requests")


@pytest.mark.parametrize("hq,hkv", [(8, 2), (16, 2), (4, 4)])
def test_decode_rows_longest_first_order(hq, hkv):
    """Decode splits in row order ("decode_order" = 0) instead of longest split first: the
    same values within tolerance, bit-identical since each split's math does not depend on
    its launch position."""
    wl = small_workload("long_decode", hq, hkv, 128, "bf16")
    outs = []
    try:
        for order in (1, 0):
            cb.cb_set_tuning("decode_order", order)
            run, step, batch, o = run_one_step(wl)
            outs.append(o)
    finally:
        cb.cb_set_tuning("decode_order", 1)
    assert torch.equal(outs[0], outs[1])
    check(outs[1], oracle_full(wl, step), "bf16", f"decode rows-first order Hq={hq} Hkv={hkv}")


def test_paged_read_probe_runs_and_writes_nothing():
    """The bench's measurement probe reads every page it is given (entries outside the pool
    skipped) and leaves its sink alone: constant pages fold to zero, never the sink's key."""
    n = 1000
    pages = torch.full((n * 4096,), 3, dtype=torch.uint8, device="cuda")
    order = torch.randperm(n, device="cuda", dtype=torch.int32)
    order[7] = n + 5                                  # skipped
    order[11] = -1                                    # skipped
    sink = torch.zeros(cb.cb_paged_read_probe_sink_words(n), dtype=torch.int32, device="cuda")
    cb.cb_paged_read_probe(pages, n, order, sink, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert int(sink.abs().sum().item()) == 0
