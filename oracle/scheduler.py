"""Reference step builder for continuous batching. TEST INFRASTRUCTURE ONLY.

The rule being restated:

* Hugging Face blog "Continuous batching from first principles", section "Continuous
  batching": aim for m tokens per step, add every decoding prompt first (one token each),
  then fill what is left with prefill prompts, split by chunked prefill. Finished prompts
  leave at once and their slots go to waiting requests.
* zhangchitc "continuous-batching", section "Continuous batching: a new request joins as
  soon as one finishes": when A emits EOS, waiting request D (4 tokens) joins B and C, and
  the next step runs 4 + 1 + 1 rows.
* hassanahmed "How continuous batching speeds up LLM serving", the scheduler loop: each
  pass evicts finished requests (releasing their KV blocks), admits waiting requests while
  ``can_admit`` holds, then runs one forward step. Section on paged memory: the cache is
  kept in fixed-size blocks that are handed out and reclaimed on demand.

Readings where the pages are silent (both the C++ builder and this reference take them):

* Decodes come first in request-admission order, then chunks of partly prefilled requests
  (admission order), then new admissions (FIFO). If there are more decodes than m, the
  first m run.
* Chunks are greedy: min(remaining prompt, remaining budget, what the free blocks can hold).
* ``can_admit``: the free list holds the blocks for the first chunk, and, if
  ``max_num_seqs`` > 0, fewer than that many requests are running. The first waiting
  request that cannot be admitted stops admission (FIFO).
* Blocks are allocated lazily so request r holds ceil((c_r + q_r) / bs) blocks after the
  step is built. They come from the head of a FIFO free list. On eviction they go back to
  the tail, in block-table order.
* Preemption (``set_preemption``; hassanahmed, paged-memory section: when the card fills, a
  request is evicted for a while and brought back later), read as recompute: while the decode
  tokens need more blocks than are free, the most recently admitted running request returns
  all its blocks and goes to the head of the waiting queue; re-admitted, it prefills its
  prompt and the tokens it generated (chunked like any prompt), and the last of them yields
  its next token. A watermark keeps that many blocks free at admission.
* ``out_len`` counts the token produced by the last prefill chunk. A request is done once
  it has produced ``out_len`` tokens, or when the caller flags EOS for a step in which it
  produced a token. Done requests are evicted at the start of the next build.

``set_static(B)`` switches to the naive batching the pages contrast this with (zhangchitc
"continuous-batching", section "Naive batching: the whole batch finishes together";
hassanahmed, the batch loop that returns results when the batch finishes; B = 1 is
request-at-a-time): up to B waiting requests start together, every prompt is padded to the
longest one P and prefilled in one step, then every member decodes one row per step, done
ones included, until all are done, and only then do they all leave. Readings: pads are rows
after the prompt (positions prompt_len .. P-1, causally invisible to the prompt's rows) and
hold no context afterwards (the first decode row overwrites position prompt_len); admission
stops at the first request for which the free list cannot hold ceil(P / bs) blocks for every
member so far; the token budget m does not apply.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

import numpy as np


class OutOfBlocks(RuntimeError):
    pass


@dataclass
class _Req:
    req_id: int
    prompt_len: int
    out_len: int
    pre_len: int = 0          # positions to prefill before decoding (set on creation)
    ctx: int = 0
    gen: int = 0
    blocks: list = field(default_factory=list)
    done: bool = False


@dataclass
class Step:
    req_ids: np.ndarray
    cu_q_lens: np.ndarray
    ctx_lens: np.ndarray
    block_tables: np.ndarray          # [R, max_blocks_per_req], -1 padded
    slot_mapping: np.ndarray
    token_to_req: np.ndarray
    num_decode: int
    evicted: list
    admitted: list
    preempted: list = field(default_factory=list)

    @property
    def num_reqs(self) -> int:
        return len(self.req_ids)

    @property
    def num_tokens(self) -> int:
        return int(self.cu_q_lens[-1])


def _ceil(a: int, b: int) -> int:
    return -(-a // b)


class RefScheduler:
    def __init__(self, token_budget: int, block_size: int, num_blocks: int, max_num_seqs: int = 0,
                 free_list=None):
        assert token_budget >= 1 and block_size >= 1 and num_blocks >= 0
        self.m, self.bs, self.max_num_seqs = int(token_budget), int(block_size), int(max_num_seqs)
        order = range(num_blocks) if free_list is None else [int(b) for b in free_list]
        self.free = deque(order)
        self.waiting: deque[_Req] = deque()
        self.running: list[_Req] = []
        self.pending = None
        self.static_b = 0
        self.preempt, self.watermark = False, 0

    def set_preemption(self, enable: bool, watermark_blocks: int = 0) -> None:
        assert watermark_blocks >= 0 and not (enable and self.static_b)
        self.preempt, self.watermark = bool(enable), int(watermark_blocks)

    def set_static(self, batch_size: int) -> None:
        assert batch_size >= 1 and not self.running and self.pending is None and not self.preempt
        self.static_b = int(batch_size)

    # ---- requests ----------------------------------------------------------------------
    def add(self, req_id: int, prompt_len: int, out_len: int) -> None:
        assert prompt_len >= 1 and out_len >= 1
        self.waiting.append(_Req(int(req_id), int(prompt_len), int(out_len), int(prompt_len)))

    def add_cached(self, req_id: int, prompt_len: int, out_len: int, cached: int, generated: int) -> None:
        """A running request whose first ``cached`` positions are already in the cache."""
        r = _Req(int(req_id), int(prompt_len), int(out_len), int(prompt_len), int(cached), int(generated))
        prefill_ok = r.gen == 0 and 0 <= r.ctx < r.prompt_len
        decode_ok = 1 <= r.gen < r.out_len and r.ctx == r.prompt_len + r.gen - 1
        assert prefill_ok or decode_ok, "inconsistent cached state"
        need = _ceil(r.ctx, self.bs)
        if need > len(self.free):
            raise OutOfBlocks("add_cached")
        r.blocks = [self.free.popleft() for _ in range(need)]
        self.running.append(r)

    # ---- one step ----------------------------------------------------------------------
    def build(self) -> Step:
        assert self.pending is None, "commit the previous step first"
        if self.static_b:
            return self._build_static()
        bs = self.bs
        evicted = []
        for r in self.running:                              # 1. evict finished
            if r.done:
                self.free.extend(r.blocks)
                r.blocks = []
                evicted.append(r.req_id)
        self.running = [r for r in self.running if not r.done]

        def decode_rows():                                   # 2. decode first
            dec = [r for r in self.running if r.ctx >= r.pre_len][: self.m]
            return dec, sum(max(0, _ceil(r.ctx + 1, bs) - len(r.blocks)) for r in dec)
        decodes, need = decode_rows()
        preempted = []
        # preemption: the most recently admitted request returns its blocks and goes back to
        # the head of the queue; re-admitted, it prefills all tokens it has, the last of which
        # yields its next token
        while need > len(self.free) and self.preempt and self.running:
            v = self.running.pop()
            self.free.extend(v.blocks)
            v.blocks = []
            v.pre_len = v.prompt_len + v.gen
            v.ctx = 0
            preempted.append(v.req_id)
            self.waiting.appendleft(v)
            decodes, need = decode_rows()
        if need > len(self.free):
            raise OutOfBlocks("decode")
        for r in decodes:
            while len(r.blocks) < _ceil(r.ctx + 1, bs):
                r.blocks.append(self.free.popleft())
        budget = self.m - len(decodes)

        chunks = []
        for r in self.running:                              # 3. continue partial prefills
            if budget == 0:
                break
            if r.ctx >= r.pre_len:
                continue
            q = min(r.pre_len - r.ctx, budget, (len(r.blocks) + len(self.free)) * bs - r.ctx)
            if q <= 0:
                continue
            while len(r.blocks) < _ceil(r.ctx + q, bs):
                r.blocks.append(self.free.popleft())
            chunks.append((r, q))
            budget -= q

        admitted = []
        while self.waiting and budget > 0 and (self.max_num_seqs == 0 or len(self.running) < self.max_num_seqs):
            w = self.waiting[0]                             # 4. admit while can_admit
            q = min(w.pre_len, budget)
            if _ceil(q, bs) + self.watermark > len(self.free):
                break
            self.waiting.popleft()
            w.blocks = [self.free.popleft() for _ in range(_ceil(q, bs))]
            self.running.append(w)
            chunks.append((w, q))
            admitted.append(w.req_id)
            budget -= q

        batch = [(r, 1) for r in decodes] + chunks
        step = self._emit(batch, len(decodes), evicted, admitted)
        step.preempted = preempted
        return step

    def _build_static(self) -> Step:
        bs = self.bs
        evicted, admitted = [], []
        if self.running and all(r.done for r in self.running):      # the batch finished
            for r in self.running:
                self.free.extend(r.blocks)
                r.blocks = []
                evicted.append(r.req_id)
            self.running = []
        if not self.running:                                          # next batch: padded prefill
            members, P = [], 0
            for w in list(self.waiting)[: self.static_b]:
                P2 = max(P, w.prompt_len)
                if (len(members) + 1) * _ceil(P2, bs) > len(self.free):
                    break
                members.append(w)
                P = P2
            if not members and self.waiting:
                raise OutOfBlocks("padded prompt")
            for w in members:
                self.waiting.popleft()
                w.blocks = [self.free.popleft() for _ in range(_ceil(P, bs))]
                self.running.append(w)
                admitted.append(w.req_id)
            return self._emit([(w, P) for w in members], 0, evicted, admitted)
        need = sum(max(0, _ceil(r.ctx + 1, bs) - len(r.blocks)) for r in self.running)
        if need > len(self.free):
            raise OutOfBlocks("decode")
        for r in self.running:
            while len(r.blocks) < _ceil(r.ctx + 1, bs):
                r.blocks.append(self.free.popleft())
        return self._emit([(r, 1) for r in self.running], len(self.running), evicted, admitted)

    def _emit(self, batch, num_decode, evicted, admitted) -> Step:
        bs = self.bs
        R = len(batch)
        cu = np.zeros(R + 1, dtype=np.int32)
        ctx = np.zeros(R, dtype=np.int32)
        for i, (r, q) in enumerate(batch):
            cu[i + 1] = cu[i] + q
            ctx[i] = r.ctx
        maxb = max((_ceil(r.ctx + q, bs) for r, q in batch), default=0)
        bt = np.full((R, maxb), -1, dtype=np.int32)
        T = int(cu[-1])
        slots = np.zeros(T, dtype=np.int32)
        owner = np.zeros(T, dtype=np.int32)
        for i, (r, q) in enumerate(batch):
            nb = _ceil(r.ctx + q, bs)
            bt[i, :nb] = r.blocks[:nb]
            for k in range(q):
                p = r.ctx + k
                slots[cu[i] + k] = r.blocks[p // bs] * bs + p % bs
                owner[cu[i] + k] = i
        self.pending = batch
        return Step(np.array([r.req_id for r, _ in batch], dtype=np.int64), cu, ctx, bt, slots, owner,
                    num_decode, evicted, admitted)

    def commit(self, eos=None) -> None:
        assert self.pending is not None, "no step to commit"
        for i, (r, q) in enumerate(self.pending):
            # a padded prefill (naive batching) ends at the prompt: pad rows hold no context
            r.ctx = min(r.ctx + q, r.pre_len) if r.ctx < r.pre_len else r.ctx + q
            if r.ctx >= r.pre_len:                          # this step produced a token
                r.gen += 1
                if r.gen >= r.out_len or (eos is not None and bool(eos[i])):
                    r.done = True
        self.pending = None

    # ---- introspection -----------------------------------------------------------------
    @property
    def num_free_blocks(self) -> int:
        return len(self.free)

    def idle(self) -> bool:
        return not self.running and not self.waiting
