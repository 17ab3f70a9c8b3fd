"""Drives a synthetic workload through the C ABI on one GPU (tests, smoke and bench).

Plumbing only: torch allocates device memory and gathers synthetic input rows from the
seeded value pools. Every step of the attention path (batch build, block allocation, KV
append, attention, commit) runs in libcb.so.
"""
from __future__ import annotations

import numpy as np
import torch

from . import cb


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


class DeviceRun:
    """Caches, value pools and a cb_sched for one workload on `device`.

    Cached requests (``Request.cached``) get their history written through cb_kv_append on
    the first step. ``stale`` fills every cache slot with NaN first, so a kernel that reads a
    slot outside a request's visible range shows up as a NaN in the output.
    """

    def __init__(self, wl, device="cuda", stale=float("nan"), sched=None):
        import workloads as W
        self.W = W
        self.wl = wl
        self.device = torch.device(device)
        self.tdtype = torch_dtype(wl.dtype)
        self.shape = cb.make_shape(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks, wl.dtype,
                                   wl.block_size)
        nb, hkv, d, bs = wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.block_size
        fill = stale if stale is not None else 0.0
        self.k_cache = torch.full((nb, hkv, bs, d), fill, dtype=self.tdtype, device=self.device)
        self.v_cache = torch.full((nb, hkv, d, bs), fill, dtype=self.tdtype, device=self.device)
        self.pools = [self._pool(k) for k in (W.KIND_Q, W.KIND_K, W.KIND_V)]
        if sched is None:
            sched = cb.Scheduler(wl.token_budget, wl.block_size, wl.num_blocks, wl.max_num_seqs, wl.free_list)
            for r in wl.requests:
                if r.cached is None:
                    sched.add(r.req_id, r.prompt_len, r.out_len)
                else:
                    sched.add_cached(r.req_id, r.prompt_len, r.out_len, r.cached, r.generated)
        self.sched = sched
        self._pending_history = {r.req_id: r.cached for r in wl.requests if r.cached}
        self.stream = torch.cuda.current_stream(self.device)
        self.workspace = torch.empty(0, dtype=torch.uint8, device=self.device)

    def _pool(self, kind):
        raw = self.wl.raw_pool(kind).copy()          # the pools are read-only arrays
        if self.wl.dtype == "bf16":
            return torch.from_numpy(raw.view(np.int16)).to(self.device).view(torch.bfloat16)
        return torch.from_numpy(raw).to(self.device)

    # ---- inputs ---------------------------------------------------------------------
    def gather(self, kind, req_ids, positions):
        """Device tensor [N, H, D] of pool rows for tokens (req_ids[i], positions[i])."""
        idx = self.wl.index(kind, req_ids, positions)
        return self.pools[kind][torch.from_numpy(idx).to(self.device)]

    def step_tokens(self, step):
        """(req_ids, positions) of every packed row of a step."""
        owner = step.token_to_req
        rids = step.req_ids[owner]
        pos = step.ctx_lens[owner] + (np.arange(step.num_tokens) - step.cu_q_lens[owner])
        return rids, pos

    def step_inputs(self, step):
        W = self.W
        rids, pos = self.step_tokens(step)
        return (self.gather(W.KIND_Q, rids, pos), self.gather(W.KIND_K, rids, pos), self.gather(W.KIND_V, rids, pos))

    # ---- device calls ---------------------------------------------------------------
    def append(self, batch: cb.Batch, k_new, v_new):
        cb.cb_kv_append(self.shape, batch.struct, k_new, v_new, self.k_cache, self.v_cache, self.stream)

    def write_history(self, step):
        """Writes the cached prefix of requests added with ``cached`` positions (once)."""
        rows = [i for i, rid in enumerate(step.req_ids.tolist()) if rid in self._pending_history]
        if not rows:
            return
        W = self.W
        lens = np.array([self._pending_history.pop(int(step.req_ids[i])) for i in rows], dtype=np.int32)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        bt = step.block_tables[rows]
        rids = np.repeat(step.req_ids[rows], lens)
        pos = np.concatenate([np.arange(n) for n in lens])
        batch = cb.Batch(cu, np.zeros(len(rows), np.int32), bt, device=self.device)
        k = self.gather(W.KIND_K, rids, pos)
        v = self.gather(W.KIND_V, rids, pos)
        self.append(batch, k, v)

    def attention(self, batch: cb.Batch, q, out=None):
        need = cb.cb_ragged_attention_workspace_size(self.shape, batch.struct)
        if self.workspace.numel() < need:
            self.workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        o = out if out is not None else torch.empty_like(q)
        cb.cb_ragged_attention(self.shape, batch.struct, q, self.k_cache, self.v_cache, self.wl.scale, o,
                               self.workspace, self.workspace.numel(), self.stream)
        return o

    def run_step(self, step=None, inputs=None):
        """One step: build (unless given), write pending history, append, attend.
        Returns (step, batch, q, k_new, v_new, o); the caller commits."""
        if step is None:
            step = self.sched.build()
        self.write_history(step)
        batch = cb.Batch.from_step(step, device=self.device)
        q, k, v = inputs if inputs is not None else self.step_inputs(step)
        self.append(batch, k, v)
        o = self.attention(batch, q)
        return step, batch, q, k, v, o

    # ---- reading the cache back (tests) ---------------------------------------------
    def gather_cache(self, block_row, length):
        """K [length, Hkv, D] and V [length, Hkv, D] of one request, through its block row."""
        bs = self.wl.block_size
        pos = torch.arange(length, device=self.device)
        blocks = torch.from_numpy(np.asarray(block_row[: -(-length // bs)], dtype=np.int64)).to(self.device)
        blk = blocks[pos // bs]
        off = pos % bs
        k = self.k_cache[blk, :, off, :]                      # [L, Hkv, D]
        v = self.v_cache[blk, :, :, off]                      # [L, Hkv, D]
        return k, v


class GraphSteps:
    """Captured steps (cb_graph) keyed by a bucket of packed rows: the smallest power of two
    >= T, at least ``min_bucket`` and at most the buffers' row count. Every bucket's graph is
    bound to the first rows of the same fixed buffers q, k_new, v_new, o (the caller writes
    a step's rows there), so buckets differ only in their launch capacities.
    """

    def __init__(self, run: DeviceRun, q, k_new, v_new, o, min_bucket: int = 64):
        self.run, self.q, self.k_new, self.v_new, self.o = run, q, k_new, v_new, o
        self.max_rows = q.shape[0]
        self.min_bucket = min_bucket
        self.graphs = {}

    def bucket(self, num_tokens: int) -> int:
        b = self.min_bucket
        while b < num_tokens:
            b *= 2
        return min(b, self.max_rows)

    def step(self, st, stream=None) -> None:
        """One step from a built step (``Step`` or the raw ``cb_step`` of build_raw)."""
        T = int(st.num_tokens)
        if T == 0:
            return
        b = self.bucket(T)
        g = self.graphs.get(b)
        if g is None:
            g = cb.cb_graph_create(self.run.shape, b, self.q, self.k_new, self.v_new, self.run.k_cache,
                                   self.run.v_cache, self.run.wl.scale, self.o)
            self.graphs[b] = g
        cb.cb_graph_step(g, st.num_reqs, T, st.max_blocks_per_req, st.cu_q_lens, st.ctx_lens, st.block_tables,
                         stream if stream is not None else self.run.stream)

    def stats(self):
        """{bucket: (replays, captures, workspace_bytes)}."""
        return {b: cb.cb_graph_stats(g) for b, g in sorted(self.graphs.items())}

    def close(self) -> None:
        for g in self.graphs.values():
            cb.cb_graph_destroy(g)
        self.graphs.clear()
