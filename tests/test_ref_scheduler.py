"""Pins for the reference step builder (CPU only): the pages' worked examples, the stated
rule (decode first, fill with chunks up to m, evict and admit on EOS), and invariants of a
long randomized trace."""
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle.scheduler import OutOfBlocks, RefScheduler

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_examples.json")))


def make(wl: W.Workload) -> RefScheduler:
    s = RefScheduler(wl.token_budget, wl.block_size, wl.num_blocks, wl.max_num_seqs, wl.free_list)
    for r in wl.requests:
        if r.cached is None:
            s.add(r.req_id, r.prompt_len, r.out_len)
        else:
            s.add_cached(r.req_id, r.prompt_len, r.out_len, r.cached, r.generated)
    return s


def test_tiny_config_step():
    """Three requests: decodes at contexts 12 and 20, a fresh 7-token prompt; decode rows first."""
    st = make(W.config(1)).build()
    assert st.cu_q_lens.tolist() == [0, 1, 2, 9]
    assert st.ctx_lens.tolist() == [12, 20, 0]
    assert st.block_tables.tolist() == [[0, -1], [1, 2], [3, -1]]
    assert st.slot_mapping.tolist() == [12, 36] + list(range(48, 55))
    assert st.token_to_req.tolist() == [0, 1] + [2] * 7
    assert st.num_decode == 2 and st.admitted == [2]


def test_pages_two_step_trace():
    """zhangchitc: A emits EOS, D (4 tokens) takes its slot, the next step runs D 4 + B 1 + C 1;
    one step later C finishes and the next waiting request takes its place."""
    g = GOLD["two_step_trace"]
    s = RefScheduler(token_budget=64, block_size=16, num_blocks=64)
    for rid, ctx in ((0, 9), (1, 4), (2, 2)):                       # A, B, C decoding
        s.add_cached(rid, ctx, 100, ctx, 1)
    st = s.build()
    assert st.num_tokens == 3
    s.commit(eos=[True, False, False])                              # A emits EOS
    s.add(3, 4, 100)                                                # D arrives, 4-token prompt
    st = s.build()
    assert st.evicted == [0] and st.admitted == [3]
    rows = dict(zip(["B", "C", "D"], np.diff(st.cu_q_lens).tolist()))
    assert rows == g["first_step_rows"] and st.num_tokens == g["first_step_tokens"]
    s.commit(eos=[False, True, False])                              # C finishes
    s.add(4, 3, 100)
    st = s.build()
    assert st.evicted == [2] and st.admitted == [4]
    assert st.req_ids.tolist() == [1, 3, 4]                         # B, D decode; E prefill


def test_pages_chunk_count():
    """Blog, "Chunked prefill": m = 4 and a 7-token prompt give ceil(7/4) = 2 chunks (4 + 3)."""
    g = GOLD["chunk_count"]
    s = RefScheduler(token_budget=g["m"], block_size=16, num_blocks=8)
    s.add(0, g["n"], 5)
    chunks = []
    while True:
        st = s.build()
        if st.ctx_lens[0] >= g["n"]:
            break
        chunks.append(int(st.cu_q_lens[-1]))
        s.commit()
    assert len(chunks) == g["chunks"] and chunks == [4, 3]


def test_decode_first_then_fill_to_budget():
    s = RefScheduler(token_budget=8, block_size=4, num_blocks=64)
    for rid in range(3):
        s.add_cached(rid, 5, 10, 5, 1)
    s.add(10, 20, 3)
    s.add(11, 2, 3)
    st = s.build()
    assert st.num_decode == 3 and st.num_tokens == 8
    assert np.diff(st.cu_q_lens).tolist() == [1, 1, 1, 5]          # the rest goes to the prompt
    assert st.admitted == [10]
    s.commit()
    st = s.build()
    assert np.diff(st.cu_q_lens).tolist() == [1, 1, 1, 5]          # partial prefill continues first
    assert st.ctx_lens.tolist()[3] == 5


def test_out_len_counts_the_prefill_token():
    s = RefScheduler(token_budget=16, block_size=4, num_blocks=16)
    s.add(0, 6, 1)              # done right after its prefill
    s.add(1, 3, 3)              # prefill, then 2 decodes
    steps = []
    while not s.idle():
        st = s.build()
        steps.append((st.req_ids.tolist(), np.diff(st.cu_q_lens).tolist()))
        s.commit()
    assert steps == [([0, 1], [6, 3]), ([1], [1]), ([1], [1]), ([], [])]


def test_eviction_returns_blocks_fifo():
    s = RefScheduler(token_budget=64, block_size=4, num_blocks=6)
    s.add(0, 9, 1)              # 3 blocks
    s.add(1, 4, 1)              # 1 block
    st = s.build()
    assert st.block_tables.tolist() == [[0, 1, 2], [3, -1, -1]]
    s.commit()
    s.add(2, 24, 1)             # needs 6 blocks: free list is now 4,5 then 0,1,2 then 3
    st = s.build()
    assert st.evicted == [0, 1]
    assert st.block_tables.tolist() == [[4, 5, 0, 1, 2, 3]]


def test_can_admit_blocks_fifo_head():
    s = RefScheduler(token_budget=64, block_size=4, num_blocks=3)
    s.add(0, 16, 2)             # needs 4 blocks: cannot be admitted
    s.add(1, 4, 2)              # would fit, but FIFO admission stops at the head
    st = s.build()
    assert st.num_reqs == 0 and st.admitted == []


def test_decode_out_of_blocks():
    s = RefScheduler(token_budget=64, block_size=4, num_blocks=1)
    s.add_cached(0, 4, 5, 4, 1)                                    # holds the only block
    with pytest.raises(OutOfBlocks):
        s.build()                                                   # position 4 needs block 2


def test_max_num_seqs():
    s = RefScheduler(token_budget=64, block_size=4, num_blocks=64, max_num_seqs=2)
    for rid in range(4):
        s.add(rid, 3, 2)
    assert s.build().admitted == [0, 1]


def check_trace_invariants(wl: W.Workload, steps: int):
    """Runs the trace; checks the rule and the allocator's bookkeeping at every step."""
    s = make(wl)
    bs, m = wl.block_size, wl.token_budget
    produced, processed = {}, {}
    meta = {}
    for k in range(steps):
        for r in wl.arrivals[k]:
            s.add(r.req_id, r.prompt_len, r.out_len)
            meta[r.req_id] = r
        st = s.build()
        T, R = st.num_tokens, st.num_reqs
        assert T <= m
        q = np.diff(st.cu_q_lens)
        assert (q[: st.num_decode] == 1).all() and (q >= 1).all()
        # decode-phase requests all run (they fit in m here) and come first
        dec = {r.req_id for r in s.running if r.ctx >= r.prompt_len}
        assert set(st.req_ids[: st.num_decode].tolist()) == dec
        # the step is full whenever work is waiting or unfinished prefills exist
        pending_prefill = any(r.ctx + q_i < r.prompt_len for r, q_i in s.pending)
        if s.waiting or pending_prefill:
            assert T == m
        # block tables: exactly ceil((c+q)/bs) valid entries, all distinct, disjoint from free
        used = []
        for i in range(R):
            nb = -(-(int(st.ctx_lens[i]) + int(q[i])) // bs)
            row = st.block_tables[i]
            assert (row[:nb] >= 0).all() and (row[nb:] == -1).all()
            used += row[:nb].tolist()
        allb = used + list(s.free) + [b for r in s.running for b in r.blocks if r.req_id not in set(st.req_ids.tolist())]
        assert len(set(used)) == len(used)
        assert sorted(allb) == list(range(wl.num_blocks))
        # slot mapping agrees with the table
        for t in range(T):
            i = int(st.token_to_req[t])
            p = int(st.ctx_lens[i]) + t - int(st.cu_q_lens[i])
            assert st.slot_mapping[t] == st.block_tables[i, p // bs] * bs + p % bs
        for i, rid in enumerate(st.req_ids.tolist()):
            processed[rid] = processed.get(rid, 0) + int(q[i])
        s.commit()
        for r in s.running:
            produced[r.req_id] = r.gen
    # every finished request processed prompt + out - 1 tokens and produced out tokens
    finished = [rid for rid, g in produced.items() if g == meta[rid].out_len]
    assert finished
    for rid in finished:
        assert processed[rid] == meta[rid].prompt_len + meta[rid].out_len - 1


def test_trace_invariants_small():
    wl = W.trace_workload(seed=11, steps=300, rate=2.0, prompt_median=40, prompt_max=300, out_mean=12,
                          token_budget=96, num_blocks=600)
    check_trace_invariants(wl, 300)


def test_trace_invariants_config5_head():
    wl = W.config(5)
    check_trace_invariants(wl, 60)


# ---- naive batching (the baseline the pages contrast continuous batching with) ----------
def run_to_completion(s, eos_at=None, max_steps=100000):
    """Builds and commits until idle; returns the non-empty steps (the last build only
    evicts the final batch and runs no rows)."""
    steps = []
    while not s.idle() and len(steps) < max_steps:
        st = s.build()
        eos = None
        if eos_at is not None:
            eos = np.array([eos_at(len(steps), int(rid)) for rid in st.req_ids], dtype=np.uint8)
        s.commit(eos)
        if st.num_reqs:
            steps.append(st)
    return steps


def test_static_batch_pads_to_longest_and_finishes_together():
    """zhangchitc "continuous-batching", "Naive batching": requests that start together
    are padded to the longest prompt, and the batch occupies its rows until its last
    member is done."""
    s = RefScheduler(token_budget=4, block_size=4, num_blocks=64)
    s.set_static(3)
    for rid, (p, o) in enumerate([(5, 2), (2, 4), (3, 3)]):
        s.add(rid, p, o)
    s.add(3, 2, 1)                                   # waits for the next batch
    steps = run_to_completion(s)
    first = steps[0]
    assert first.req_ids.tolist() == [0, 1, 2] and np.diff(first.cu_q_lens).tolist() == [5, 5, 5]
    assert first.num_tokens == 15 > 4                 # the token budget does not apply
    assert first.ctx_lens.tolist() == [0, 0, 0] and first.num_decode == 0
    # longest output is 4: three decode steps with all three members, done ones included
    for k, ctx in zip((1, 2, 3), ([5, 2, 3], [6, 3, 4], [7, 4, 5])):
        assert steps[k].req_ids.tolist() == [0, 1, 2] and steps[k].ctx_lens.tolist() == ctx
        assert steps[k].num_decode == 3 and steps[k].num_tokens == 3
    assert steps[4].evicted == [0, 1, 2] and steps[4].req_ids.tolist() == [3]
    assert len(steps) == 5                            # request 3: prefill only (out_len 1)


def test_static_request_at_a_time():
    """Batch size 1: no pads; each request takes 1 + (out_len - 1) steps on its own."""
    reqs = [(7, 3), (1, 5), (12, 1), (4, 2)]
    s = RefScheduler(token_budget=2, block_size=4, num_blocks=32)
    s.set_static(1)
    for rid, (p, o) in enumerate(reqs):
        s.add(rid, p, o)
    steps = run_to_completion(s)
    assert len(steps) == sum(o for _, o in reqs)
    assert all(st.num_reqs == 1 for st in steps)
    rows = {}
    for st in steps:
        rows[int(st.req_ids[0])] = rows.get(int(st.req_ids[0]), 0) + st.num_tokens
    assert rows == {rid: p + o - 1 for rid, (p, o) in enumerate(reqs)}


def test_static_eos_ends_the_batch_early():
    s = RefScheduler(token_budget=8, block_size=4, num_blocks=64)
    s.set_static(2)
    s.add(0, 3, 50)
    s.add(1, 4, 50)
    s.add(2, 2, 1)
    steps = run_to_completion(s, eos_at=lambda k, rid: k == 2)   # both flag EOS at step 2
    assert [st.req_ids.tolist() for st in steps] == [[0, 1], [0, 1], [0, 1], [2]]
    assert steps[3].evicted == [0, 1]


def test_static_closed_form_on_a_trace():
    """Rows processed = sum over batches of size x (P + O - 1), with P the longest prompt and
    O the longest output of the batch; rows useful = sum of prompt + out - 1; every block is
    accounted for at every step."""
    wl = W.trace_workload(seed=5, steps=40, rate=1.2, prompt_median=30, prompt_max=200, out_mean=15,
                          token_budget=64, num_blocks=4000)
    reqs = [r for k in range(wl.steps) for r in wl.arrivals[k]][:40]
    for B in (1, 3, 8):
        s = RefScheduler(wl.token_budget, wl.block_size, wl.num_blocks)
        s.set_static(B)
        for r in reqs:
            s.add(r.req_id, r.prompt_len, r.out_len)
        steps = run_to_completion(s)
        expect_rows, expect_steps = 0, 0
        for i in range(0, len(reqs), B):
            grp = reqs[i:i + B]
            P, O = max(r.prompt_len for r in grp), max(r.out_len for r in grp)
            expect_rows += len(grp) * (P + O - 1)
            expect_steps += O
        assert sum(st.num_tokens for st in steps) == expect_rows
        assert len(steps) == expect_steps
        assert s.num_free_blocks == wl.num_blocks
        useful = sum(r.prompt_len + r.out_len - 1 for r in reqs)
        assert expect_rows >= useful and (B > 1 or expect_rows == useful)


def test_static_padded_prompt_out_of_blocks():
    s = RefScheduler(token_budget=8, block_size=4, num_blocks=3)
    s.set_static(2)
    s.add(0, 20, 2)
    with pytest.raises(OutOfBlocks):
        s.build()


# ---- preemption by recompute (NEXT #2) ---------------------------------------------------
def test_preemption_victim_is_latest_and_resumes_its_output():
    """Three decoding requests on a pool that cannot hold their next tokens: the most recently
    admitted gives back its blocks, waits at the head of the queue, and on re-admission
    prefills prompt + generated tokens; the last of them yields its next token."""
    s = RefScheduler(token_budget=64, block_size=4, num_blocks=6)
    s.set_preemption(True)
    for rid in range(3):
        s.add(rid, 4, 10)
    st = s.build()                                   # three prompts of 4: 3 blocks
    assert st.admitted == [0, 1, 2]
    s.commit()                                        # each produced 1 token; ctx = 4
    st = s.build()                                    # decodes need one new block each: 3 = 3 free
    assert st.num_decode == 3 and st.preempted == []
    s.commit()
    for _ in range(3):                                # ctx 5..7 stay inside the second block
        st = s.build()
        s.commit()
    st = s.build()                                    # ctx 8: each needs a third block, none free
    assert st.preempted == [2] and st.req_ids.tolist() == [0, 1]
    assert [w.req_id for w in s.waiting] == [2]
    v = s.waiting[0]
    assert v.ctx == 0 and v.pre_len == 4 + v.gen and v.gen == 5 and v.blocks == []
    s.commit()


def recompute_trace(wl, steps_limit=20000, watermark=0):
    s = make(wl)
    s.set_preemption(True, watermark)
    meta = {r.req_id: r for k in range(wl.steps) for r in wl.arrivals[k]}
    rows, extra, preempts = {}, {}, 0
    ctx_of = {}
    k = 0
    while k < wl.steps or not s.idle():
        if k < wl.steps:
            for r in wl.arrivals[k]:
                s.add(r.req_id, r.prompt_len, r.out_len)
        before = {r.req_id: r.ctx for r in s.running}
        st = s.build()
        for rid in st.preempted:
            extra[rid] = extra.get(rid, 0) + before[rid]
            preempts += 1
        q = np.diff(st.cu_q_lens)
        for i, rid in enumerate(st.req_ids.tolist()):
            rows[rid] = rows.get(rid, 0) + int(q[i])
        s.commit()
        k += 1
        assert k < steps_limit
    return meta, rows, extra, preempts, s


def test_preemption_completes_every_request_with_recompute_rows():
    """Under block pressure every request finishes; each processed prompt + out - 1 rows plus,
    per preemption, the positions it had in the cache when it was preempted."""
    wl = W.trace_workload(seed=8, steps=150, rate=1.0, prompt_median=30, prompt_max=120, out_mean=40,
                          token_budget=128, num_blocks=40)
    meta, rows, extra, preempts, s = recompute_trace(wl)
    assert preempts > 0
    assert s.num_free_blocks == wl.num_blocks
    for rid, r in meta.items():
        assert rows[rid] == r.prompt_len + r.out_len - 1 + extra.get(rid, 0), rid


def test_preemption_watermark_keeps_blocks_free_at_admission():
    s = RefScheduler(token_budget=64, block_size=4, num_blocks=10)
    s.set_preemption(True, watermark_blocks=4)
    s.add(0, 16, 3)                                   # 4 blocks, leaves 6 >= 4
    s.add(1, 12, 3)                                   # 3 blocks would leave 3 < 4: waits
    st = s.build()
    assert st.admitted == [0] and s.num_free_blocks == 6
    wl = W.trace_workload(seed=9, steps=120, rate=1.0, prompt_median=30, prompt_max=120, out_mean=30,
                          token_budget=128, num_blocks=48)
    meta, rows, extra, preempts, s = recompute_trace(wl, watermark=6)
    for rid, r in meta.items():
        assert rows[rid] == r.prompt_len + r.out_len - 1 + extra.get(rid, 0)
