"""Captured steps (cb_graph_*) on the GPU: every replay against the eager entry point
(cb_step_forward, bit for bit) and sampled rows against the fp64 oracle.

A small scheduler trace drives both paths side by side, each with its own caches and step
builder, so the steps change size, mix and block tables from one replay to the next:
prefill-only steps at the start, mixed steps, decode-only steps once arrivals stop, and
steps whose grids change from one replay to the next, and steps that outgrow a graph's
workspace (a new capture). Between replays the test does its
own eager torch work and synchronises, and it checks every replay.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from ragged_continuous_batching_amd import cb
from ragged_continuous_batching_amd.runner import DeviceRun, GraphSteps

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-4, 1e-4)}


def small_trace(hq, hkv, d, dtype, steps=48, seed=77):
    """Poisson(3) arrivals for 30 steps, then none (the tail decodes until the trace drains)."""
    wl = W.trace_workload(seed=seed, steps=steps, rate=3.0, prompt_median=60, prompt_max=400, out_mean=8,
                          num_q_heads=hq, num_kv_heads=hkv, head_dim=d, token_budget=256, num_blocks=4096,
                          dtype=dtype, pool_rows=1 << 14)
    for k in range(30, steps):
        wl.arrivals[k] = []
    return wl


def eager_step(run, st, q, k, v):
    need = cb.cb_step_workspace_size(run.shape, st.num_reqs, st.num_tokens, st.max_blocks_per_req, st.cu_q_lens,
                                     st.ctx_lens)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    cb.cb_step_forward(run.shape, st.num_reqs, st.num_tokens, st.max_blocks_per_req, st.cu_q_lens, st.ctx_lens,
                       st.block_tables, q, k, v, run.k_cache, run.v_cache, run.wl.scale, o, ws, need, run.stream)
    return o


def oracle_rows(wl, st, rows):
    rows = np.asarray(sorted(set(int(t) for t in rows)))
    owner = st.token_to_req[rows]
    out = {}
    for i in np.unique(owner):
        sel = rows[owner == i]
        rid, c, s = int(st.req_ids[i]), int(st.ctx_lens[i]), int(st.cu_q_lens[i])
        pos = c + (sel - s)
        L = int(pos.max()) + 1
        ref = A.attend(wl.values(W.KIND_Q, rid, pos), wl.values(W.KIND_K, rid, np.arange(L)),
                       wl.values(W.KIND_V, rid, np.arange(L)), pos, wl.scale)
        for t, r in zip(sel, ref):
            out[int(t)] = r
    return rows, np.stack([out[int(t)] for t in rows])


def check(got, ref, dtype, what):
    g = got.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    mx, mean = TOL[dtype]
    print(f"{what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= mx and err.mean() <= mean, what


def replay_trace(wl, min_bucket, check_every=8):
    """Runs the trace eagerly and through GraphSteps side by side; returns the graph stats."""
    m = wl.token_budget
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    eager, graph = DeviceRun(wl), DeviceRun(wl)
    q_buf = torch.zeros(m, wl.num_q_heads, wl.head_dim, dtype=tdt, device="cuda")
    k_buf = torch.zeros(m, wl.num_kv_heads, wl.head_dim, dtype=tdt, device="cuda")
    v_buf = torch.zeros_like(k_buf)
    o_buf = torch.full_like(q_buf, float("nan"))
    gs = GraphSteps(graph, q_buf, k_buf, v_buf, o_buf, min_bucket=min_bucket)
    rng = np.random.default_rng(11)
    kinds = set()
    try:
        for k in range(wl.steps):
            for r in wl.arrivals[k]:
                eager.sched.add(r.req_id, r.prompt_len, r.out_len)
                graph.sched.add(r.req_id, r.prompt_len, r.out_len)
            st, sg = eager.sched.build(), graph.sched.build()
            for name in ("cu_q_lens", "ctx_lens", "block_tables"):
                assert np.array_equal(getattr(st, name), getattr(sg, name))
            T = st.num_tokens
            if T:
                print(f"[graph] step {k} T={T} R={st.num_reqs} decode={st.num_decode}", flush=True)
                kinds.add((st.num_decode > 0, st.num_decode < st.num_reqs))
                q, kn, vn = eager.step_inputs(st)
                o_e = eager_step(eager, st, q, kn, vn)
                q_buf[:T].copy_(q)
                k_buf[:T].copy_(kn)
                v_buf[:T].copy_(vn)
                gs.step(sg)
                o_g = o_buf[:T].clone()
                o_buf.fill_(float("nan"))          # eager work between replays
                torch.cuda.synchronize()
                assert torch.equal(o_g, o_e), f"step {k}: replay differs from cb_step_forward"
                if k % check_every == 0 or st.num_decode in (0, st.num_reqs):
                    cand = np.unique(np.concatenate([st.cu_q_lens[:-1], st.cu_q_lens[1:] - 1,
                                                     rng.integers(0, T, 24)]))
                    rows, ref = oracle_rows(wl, st, cand)
                    check(o_g[torch.from_numpy(rows).cuda()], ref, wl.dtype, f"graph step {k} (T={T})")
            eager.sched.commit()
            graph.sched.commit()
        stats = gs.stats()
    finally:
        gs.close()
    # prefill-only, mixed and decode-only steps all ran
    assert {(False, True), (True, True), (True, False)} <= kinds, kinds
    return stats


@pytest.mark.parametrize("hq,hkv,d,dtype", [(8, 2, 128, "bf16"), (8, 1, 128, "bf16"), (4, 4, 64, "bf16"),
                                            (2, 2, 64, "f32")])
def test_graph_replays_match_step_forward(hq, hkv, d, dtype):
    """Fixed prefill work-group size, so the eager plan and the captured one are the same."""
    wl = small_trace(hq, hkv, d, dtype)
    cb.cb_set_tuning("prefill_waves", 4)
    try:
        stats = replay_trace(wl, min_bucket=32)
    finally:
        cb.cb_set_tuning("prefill_waves", 0)
    print("graph stats", stats, flush=True)
    assert len(stats) >= 2                                   # several T buckets
    assert sum(s[0] for s in stats.values()) > 0


def test_graph_eight_wave_prefill():
    """256-row prefill work-groups in the captured step (forced), eager forced the same."""
    wl = small_trace(8, 2, 128, "bf16", seed=78)
    cb.cb_set_tuning("prefill_waves", 8)
    try:
        replay_trace(wl, min_bucket=256)
    finally:
        cb.cb_set_tuning("prefill_waves", 0)


def test_graph_rejects_rows_beyond_its_bucket():
    wl = small_trace(4, 2, 128, "bf16")
    run = DeviceRun(wl)
    q = torch.zeros(16, 4, 128, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(16, 2, 128, dtype=torch.bfloat16, device="cuda")
    g = cb.cb_graph_create(run.shape, 16, q, kv, kv, run.k_cache, run.v_cache, wl.scale, q)
    try:
        cu = np.array([0, 17], np.int32)
        with pytest.raises(cb.CbError) as e:
            cb.cb_graph_step(g, 1, 17, 2, cu, np.zeros(1, np.int32), np.array([0, 1], np.int32))
        assert e.value.status == cb.CB_ERR_INVALID_ARG
        with pytest.raises(cb.CbError):             # block id outside the pool
            cb.cb_graph_step(g, 1, 3, 1, np.array([0, 3], np.int32), np.zeros(1, np.int32),
                             np.array([wl.num_blocks], np.int32))
        assert cb.cb_graph_stats(g)[:2] == (0, 0)   # nothing captured or launched
    finally:
        cb.cb_graph_destroy(g)
