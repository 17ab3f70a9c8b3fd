"""Token-wise layers around attention, in fp64. TEST INFRASTRUCTURE ONLY: nothing in the
product imports this module.

Hugging Face blog "Continuous batching from first principles", section "Attention":
normalisation and matrix multiplications are token-wise, each output row depends on its own
input row only, so on the packed stream they are plain row-by-row products; the QKV
projection produces the query, key and value states of every token. hassanahmed "How
continuous batching speeds up LLM serving": selective batching batches exactly these
operations. zhangchitc "continuous-batching", section "Inside the kernel": the new keys and
values are written into each request's cache entry before attention reads it back.

Readings: weights follow the torch Linear layout [out features, in features]; the QKV
weight stacks the Hq*D query rows, then Hkv*D key rows, then Hkv*D value rows, head-major
(feature h*D + d is dimension d of head h).
"""
from __future__ import annotations

import numpy as np


def linear(a, w) -> np.ndarray:
    """y[m, n] = sum_k a[m, k] w[n, k] in fp64 (a: [M, K], w: [N, K])."""
    return np.asarray(a, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def qkv_split(y, num_q_heads: int, num_kv_heads: int, head_dim: int):
    """Split projected rows [T, (Hq + 2 Hkv) D] into q [T, Hq, D], k and v [T, Hkv, D]."""
    y = np.asarray(y)
    T = y.shape[0]
    qd, kd = num_q_heads * head_dim, num_kv_heads * head_dim
    assert y.shape[1] == qd + 2 * kd
    q = y[:, :qd].reshape(T, num_q_heads, head_dim)
    k = y[:, qd:qd + kd].reshape(T, num_kv_heads, head_dim)
    v = y[:, qd + kd:].reshape(T, num_kv_heads, head_dim)
    return q, k, v
