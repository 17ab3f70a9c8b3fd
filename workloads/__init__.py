"""Seeded synthetic workloads for ragged continuous-batching attention.

This module only draws random numbers and lays data out. It holds request lengths, arrival
traces, value pools, and the counter-based index that maps (kind, request, position, head)
to a pool row. It contains none of the attention, paging or scheduling arithmetic. Both the
fp64 oracle (``oracle/``) and the HIP path consume what it produces, and neither side feeds
anything back into it.

Recipe (every draw is seeded; ``seed = 1000 + config id`` for the five named workloads):

* Lengths come from ``numpy.random.default_rng(seed)``, drawn in a fixed order per workload.
* Values come from three pools (Q, K, V), each ``POOL_ROWS`` rows of ``head_dim``; a fourth
  (X, always bf16) holds layer inputs for the token-wise projections, a token's input row
  being d_model / head_dim pool rows side by side. Synthetic weights are N(0, 1/fan_in)
  from ``default_rng([seed, 100 + which])``, rounded to bf16. Pool
  ``kind`` is drawn from ``default_rng([seed, kind])`` as N(0,1) fp32, then multiplied by
  ``value_std``. For bf16 workloads it is then rounded to bf16 (round to nearest, ties to
  even).
* Row (kind, request, position, head) is ``splitmix64(key) mod POOL_ROWS``, where ``key``
  packs the four integers. The value of a token therefore depends only on its request and
  position, never on how the scheduler packs it. A request's cached history can be
  regenerated for any single request without replaying a trace.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from functools import lru_cache

import numpy as np

KIND_Q, KIND_K, KIND_V, KIND_X = 0, 1, 2, 3
_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)


# --------------------------------------------------------------------------------------
# counter-based pool index
# --------------------------------------------------------------------------------------
def _splitmix64(x: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser (Steele, Lea & Flood 2014), on uint64 arrays with wraparound."""
    x = x.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        x += np.uint64(0x9E3779B97F4A7C15)
        x = (x ^ (x >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        x = (x ^ (x >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        x = x ^ (x >> np.uint64(31))
    return x


def pool_index(seed: int, kind: int, req_ids, positions, num_heads: int, pool_rows: int) -> np.ndarray:
    """Pool rows for tokens (req_ids[i], positions[i]) and heads 0..num_heads-1 -> int64 [N, H]."""
    req = np.asarray(req_ids, dtype=np.uint64).reshape(-1, 1)
    pos = np.asarray(positions, dtype=np.uint64).reshape(-1, 1)
    head = np.arange(num_heads, dtype=np.uint64).reshape(1, -1)
    with np.errstate(over="ignore"):
        key = (np.uint64(seed) << np.uint64(44)) ^ (np.uint64(kind) << np.uint64(40))
        key = _splitmix64(np.full(1, key, dtype=np.uint64))[0]
        key = key ^ (req << np.uint64(32)) ^ (pos << np.uint64(8)) ^ head
        h = _splitmix64(key)
    return (h % np.uint64(pool_rows)).astype(np.int64)


# --------------------------------------------------------------------------------------
# bf16 storage
# --------------------------------------------------------------------------------------
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    with np.errstate(over="ignore"):
        r = (u + bias) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------------------
# workload description
# --------------------------------------------------------------------------------------
@dataclass
class Request:
    req_id: int
    prompt_len: int
    out_len: int
    cached: int | None = None      # tokens already in the KV cache when the run starts;
                                   # None means the request arrives in the waiting queue
    generated: int = 0             # output tokens already produced (for cached requests)


@dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                      # "f32" or "bf16"
    token_budget: int               # m, tokens per step
    num_blocks: int                 # physical blocks in the KV pool
    scale: float                    # softmax scale passed to the attention call
    seed: int
    value_std: float
    requests: list[Request]         # present before the first step
    arrivals: list[list[Request]] | None = None   # per-step arrivals (trace workloads)
    free_list: np.ndarray | None = None           # initial free-list order (None: 0..NB-1)
    pool_rows: int = 1 << 18
    max_num_seqs: int = 0
    note: str = ""

    @property
    def steps(self) -> int:
        return len(self.arrivals) if self.arrivals is not None else 1

    # ---- values ------------------------------------------------------------------------
    def _pools(self):
        return _pools(self.seed, self.pool_rows, self.head_dim, self.value_std, self.dtype)

    def index(self, kind: int, req_ids, positions) -> np.ndarray:
        heads = self.num_q_heads if kind == KIND_Q else self.num_kv_heads
        return pool_index(self.seed, kind, req_ids, positions, heads, self.pool_rows)

    def raw_pool(self, kind: int) -> np.ndarray:
        """Pool storage: uint16 bf16 bits [rows, D] for bf16, float32 [rows, D] for f32."""
        return self._pools()[kind]

    def values(self, kind: int, req_id: int, positions) -> np.ndarray:
        """float32 [len(positions), H, D] values (exactly representable in the workload dtype)."""
        positions = np.asarray(positions, dtype=np.int64)
        idx = self.index(kind, np.full(len(positions), req_id), positions)
        raw = self.raw_pool(kind)[idx]
        return f32_from_bf16_bits(raw) if self.dtype == "bf16" else raw.astype(np.float32)

    def token_values(self, kind: int, req_ids, positions) -> np.ndarray:
        idx = self.index(kind, req_ids, positions)
        raw = self.raw_pool(kind)[idx]
        return f32_from_bf16_bits(raw) if self.dtype == "bf16" else raw.astype(np.float32)

    # ---- layer inputs (token-wise projections around attention) ------------------------
    def x_index(self, req_ids, positions, d_model: int) -> np.ndarray:
        """Pool rows [N, d_model / head_dim] of the layer input of tokens (req, position)."""
        return pool_index(self.seed, KIND_X, req_ids, positions, d_model // self.head_dim, self.pool_rows)

    def x_raw_pool(self) -> np.ndarray:
        return _x_pool(self.seed, self.pool_rows, self.head_dim, self.value_std)

    def x_values(self, req_ids, positions, d_model: int) -> np.ndarray:
        """float32 [N, d_model] layer inputs (bf16-representable): each token's row is its
        d_model / head_dim pool rows side by side."""
        idx = self.x_index(req_ids, positions, d_model)
        return f32_from_bf16_bits(self.x_raw_pool()[idx]).reshape(len(idx), d_model)


def layer_weights(seed: int, which: int, rows: int, cols: int) -> np.ndarray:
    """bf16 bits [rows, cols] of a synthetic weight: N(0, 1/cols) from default_rng([seed,
    100 + which]), rounded to bf16 (which: 0 = QKV projection, 1 = output projection)."""
    g = np.random.default_rng([seed, 100 + which])
    w = g.standard_normal((rows, cols), dtype=np.float32) * np.float32(1.0 / math.sqrt(cols))
    return bf16_bits_from_f32(w.astype(np.float32))


@lru_cache(maxsize=2)
def _x_pool(seed: int, rows: int, head_dim: int, std: float):
    g = np.random.default_rng([seed, KIND_X])
    x = g.standard_normal((rows, head_dim), dtype=np.float32)
    if std != 1.0:
        x = (x * np.float32(std)).astype(np.float32)
    out = bf16_bits_from_f32(x)
    out.setflags(write=False)
    return out


@lru_cache(maxsize=4)
def _pools(seed: int, rows: int, head_dim: int, std: float, dtype: str):
    out = []
    for kind in (KIND_Q, KIND_K, KIND_V):
        g = np.random.default_rng([seed, kind])
        x = g.standard_normal((rows, head_dim), dtype=np.float32)
        if std != 1.0:
            x = (x * np.float32(std)).astype(np.float32)
        out.append(bf16_bits_from_f32(x) if dtype == "bf16" else x)
        out[-1].setflags(write=False)
    return tuple(out)


def _lognormal_lengths(rng, n: int, median: float, sigma: float, lo: int, hi: int) -> np.ndarray:
    z = rng.standard_normal(n)
    return np.clip(np.rint(median * np.exp(sigma * z)), lo, hi).astype(np.int64)


# --------------------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------------------
def _blocks(n: int, bs: int) -> int:
    return -(-n // bs)


def config(cid: int, *, value_reading: str = "literal") -> Workload:
    """Workload ``cid`` in 1..5 (see the module docstring for the recipe)."""
    seed = 1000 + cid
    rng = np.random.default_rng(seed)
    bs = 16
    if cid == 1:
        # Tiny ragged step: decodes at contexts 12 and 20, one fresh 7-token prompt.
        reqs = [Request(0, 12, 1 << 20, cached=12, generated=1),
                Request(1, 20, 1 << 20, cached=20, generated=1),
                Request(2, 7, 1 << 20)]
        return Workload("tiny ragged step", 2, 2, 64, bs, "f32", 9, 8, 1 / math.sqrt(64), seed,
                        1.0, reqs, pool_rows=4096)
    if cid == 2:
        # Llama-2-7B-shaped layer: 64 decodes (contexts U{512..4096}) plus two 992-token
        # chunks, one continuing a prompt with 1024 tokens cached, one starting a new prompt.
        ctx = rng.integers(512, 4097, size=64)
        reqs = [Request(i, int(c), 1 << 20, cached=int(c), generated=1) for i, c in enumerate(ctx)]
        reqs.append(Request(64, 1024 + 992, 1 << 20, cached=1024, generated=0))
        reqs.append(Request(65, 2048, 1 << 20))
        need = sum(_blocks(int(c) + 1, bs) for c in ctx) + _blocks(2016, bs) + _blocks(992, bs)
        std = 1 / math.sqrt(128) if value_reading == "literal" else 1.0
        return Workload("Llama-2-7B-shaped mixed step", 32, 32, 128, bs, "bf16", 2048, need + 64,
                        1 / math.sqrt(128), seed, std, reqs,
                        note=f"values N(0,1)*{std:.6g}")
    if cid == 3:
        # Decode-only GQA: 256 decodes, contexts lognormal(median 2048, sigma 1) in [64, 32768],
        # blocks dealt from a seeded permutation of the pool.
        ctx = _lognormal_lengths(rng, 256, 2048, 1.0, 64, 32768)
        reqs = [Request(i, int(c), 1 << 20, cached=int(c), generated=1) for i, c in enumerate(ctx)]
        nb = sum(_blocks(int(c) + 1, bs) for c in ctx)
        perm = rng.permutation(nb).astype(np.int32)
        return Workload("decode-only GQA", 32, 8, 128, bs, "bf16", 256, nb, 1 / math.sqrt(128),
                        seed, 1.0, reqs, free_list=perm)
    if cid == 4:
        # Chunked-prefill-heavy: four 2048-token chunks with 0, 2048, 6144, 14336 cached.
        reqs = [Request(i, c + 2048, 1 << 20, cached=c, generated=0)
                for i, c in enumerate((2048, 6144, 14336))]
        reqs.append(Request(3, 2048, 1 << 20))
        need = sum(_blocks(c + 2048, bs) for c in (2048, 6144, 14336)) + _blocks(2048, bs)
        return Workload("chunked-prefill-heavy", 32, 32, 128, bs, "bf16", 8192, need,
                        1 / math.sqrt(128), seed, 1.0, reqs)
    if cid == 5:
        return trace_workload(seed=seed)
    raise ValueError(f"unknown workload {cid}")


def trace_workload(*, seed: int = 1005, steps: int = 500, rate: float = 8.0, prompt_median: float = 512,
                   prompt_max: int = 8192, out_mean: float = 256, num_q_heads: int = 64,
                   num_kv_heads: int = 8, head_dim: int = 128, token_budget: int = 4096,
                   num_blocks: int = 131072, dtype: str = "bf16", pool_rows: int = 1 << 18) -> Workload:
    """Scheduler-trace replay: Poisson(rate) arrivals per step, lognormal prompts
    (sigma 1, clipped to [1, prompt_max]) and geometric output lengths (support >= 1)."""
    rng = np.random.default_rng(seed)
    counts = rng.poisson(rate, size=steps)
    total = int(counts.sum())
    prompts = _lognormal_lengths(rng, total, prompt_median, 1.0, 1, prompt_max)
    outs = rng.geometric(1.0 / out_mean, size=total).astype(np.int64)
    arrivals, k = [], 0
    for s in range(steps):
        arrivals.append([Request(k + j, int(prompts[k + j]), int(outs[k + j])) for j in range(int(counts[s]))])
        k += int(counts[s])
    return Workload("scheduler-trace replay", num_q_heads, num_kv_heads, head_dim, 16, dtype,
                    token_budget, num_blocks, 1 / math.sqrt(head_dim), seed, 1.0, [], arrivals,
                    pool_rows=pool_rows)


def custom(requests: list[Request], *, num_q_heads=2, num_kv_heads=2, head_dim=64, dtype="f32",
           token_budget=1 << 30, num_blocks=None, seed=7, value_std=1.0, scale=None,
           free_list=None, pool_rows=4096, block_size=16) -> Workload:
    """Small ad-hoc workload for edge cases."""
    if num_blocks is None:
        num_blocks = sum(_blocks((r.cached or 0) + r.prompt_len + 4, block_size) for r in requests) + 8
    return Workload("custom", num_q_heads, num_kv_heads, head_dim, block_size, dtype, token_budget,
                    num_blocks, scale if scale is not None else 1 / math.sqrt(head_dim), seed,
                    value_std, requests, free_list=free_list, pool_rows=pool_rows)
