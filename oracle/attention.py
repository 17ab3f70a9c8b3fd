"""fp64 oracle of one step of ragged attention. TEST INFRASTRUCTURE ONLY.

What is computed (in the pages' terms):

* Hugging Face blog "Continuous batching from first principles", section "Attention":
  for one prompt, scores are Q K^T. A boolean mask is applied point-wise and then a
  row-wise softmax. The result multiplies V. Q may have fewer rows than K ("Why this
  matters"), and K and V always have the same length.
* Same blog, sections "KV-cache" and "Chunked prefill": cached K/V states are prepended
  to the new ones. The mask is the matching rows of the full causal mask. A query at
  absolute position p sees keys 0..p ("bottom-right" alignment).
* Same blog, section "Continuous batching" (ragged batching), and zhangchitc
  "continuous-batching", section "Ragged batching: attention in per-request blocks":
  prompts are concatenated with no batch axis. The mask is block-diagonal, so a query
  never sees another request's keys, and masked pairs carry zero weight.
* zhangchitc "Inside the kernel: cu_seqlens splits six rows back into three":
  ``cu_q_lens`` is the prefix sum of per-request query counts, and request r owns packed
  rows ``cu_q_lens[r] .. cu_q_lens[r+1]-1``.

Readings where the pages are silent (each is listed with its reason in the design notes):

* Scale: the pages show softmax(mask(Q K^T)) V with no scale. An explicit ``scale``
  multiplies the scores.
* Masked scores become -inf, so they get exactly zero weight.
* Grouped-query heads: q-head h reads kv-head h // (Hq // Hkv).
* Softmax is the plain two-pass form (max-subtract, exp, normalise), not an online one.

Every function computes in float64 from whatever float inputs it is given.
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64


def attend(q, keys, values, positions, scale):
    """Masked softmax attention of one request.

    q: [n, Hq, D] query rows; keys, values: [L, Hkv, D] all of the request's keys and values
    (cached history followed by this step's new tokens); positions: [n] absolute position of
    each query row. Row i sees keys 0..positions[i] (causal, bottom-right aligned).
    Returns [n, Hq, D] float64.
    """
    q = np.asarray(q, dtype=F64)
    keys = np.asarray(keys, dtype=F64)
    values = np.asarray(values, dtype=F64)
    positions = np.asarray(positions, dtype=np.int64)
    n, hq, d = q.shape
    L, hkv, _ = keys.shape
    assert values.shape == keys.shape and hq % hkv == 0
    assert n == 0 or positions.max() < L
    group = hq // hkv
    visible = np.arange(L)[None, :] <= positions[:, None]          # [n, L] boolean mask
    out = np.zeros((n, hq, d), dtype=F64)
    for g in range(hkv):
        kg = np.ascontiguousarray(keys[:, g, :])                    # [L, D] kv head g, read by
        vg = np.ascontiguousarray(values[:, g, :])                  # query heads h // group == g
        for h in range(g * group, (g + 1) * group):
            s = scale * (q[:, h, :] @ kg.T)                         # [n, L] scores
            s = np.where(visible, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)                   # row-wise softmax
            out[:, h, :] = p @ vg
    return out


def ragged_attention(q, k_new, v_new, hist_k, hist_v, cu_q_lens, ctx_lens, scale):
    """One step over a packed batch.

    q: [T, Hq, D]; k_new, v_new: [T, Hkv, D] this step's keys/values in packed order;
    hist_k[r], hist_v[r]: [ctx_lens[r], Hkv, D] request r's cached history;
    cu_q_lens: [R+1]; ctx_lens: [R]. Returns O [T, Hq, D] float64.
    """
    q = np.asarray(q)
    cu = [int(x) for x in cu_q_lens]
    out = np.zeros(q.shape, dtype=F64)
    for r in range(len(cu) - 1):
        s, e, c = cu[r], cu[r + 1], int(ctx_lens[r])
        if e == s:
            continue
        assert len(hist_k[r]) == c and len(hist_v[r]) == c
        keys = np.concatenate([np.asarray(hist_k[r], F64).reshape(c, *k_new.shape[1:]),
                               np.asarray(k_new[s:e], F64)])
        vals = np.concatenate([np.asarray(hist_v[r], F64).reshape(c, *v_new.shape[1:]),
                               np.asarray(v_new[s:e], F64)])
        out[s:e] = attend(q[s:e], keys, vals, c + np.arange(e - s), scale)
    return out


# --------------------------------------------------------------------------------------
# independent restatements used to pin the oracle
# --------------------------------------------------------------------------------------
def attend_scalar(q, keys, values, positions, scale):
    """Brute force with Python scalars and math.exp: the same definition, no numpy algebra."""
    q = np.asarray(q, dtype=F64).tolist()
    keys = np.asarray(keys, dtype=F64).tolist()
    values = np.asarray(values, dtype=F64).tolist()
    n = len(q)
    hq = len(q[0]) if n else 0
    hkv = len(keys[0]) if keys else 1
    group = hq // hkv if hkv else 1
    out = []
    for i in range(n):
        row = []
        for h in range(hq):
            g = h // group
            lim = int(positions[i])
            sc = []
            for j in range(lim + 1):
                acc = 0.0
                for a, b in zip(q[i][h], keys[j][g]):
                    acc += a * b
                sc.append(scale * acc)
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            tot = sum(w)
            d = len(values[0][g])
            row.append([sum(w[j] * values[j][g][k] for j in range(lim + 1)) / tot for k in range(d)])
        out.append(row)
    return np.asarray(out, dtype=F64).reshape(n, hq, -1)


def stream_mask(cu_q_lens, ctx_lens):
    """The blog's single boolean mask over the concatenated stream.

    Keys are laid out request by request as [history_r ; new_r]. Returns (mask [T, Kt],
    key_owner [Kt], key_pos [Kt]), where mask[i, j] is True when key j belongs to query i's
    request and its position is not after the query's.
    """
    cu = [int(x) for x in cu_q_lens]
    q_owner, q_pos, k_owner, k_pos = [], [], [], []
    for r in range(len(cu) - 1):
        c, n = int(ctx_lens[r]), cu[r + 1] - cu[r]
        q_owner += [r] * n
        q_pos += list(range(c, c + n))
        k_owner += [r] * (c + n)
        k_pos += list(range(c + n))
    q_owner, q_pos = np.array(q_owner, dtype=np.int64), np.array(q_pos, dtype=np.int64)
    k_owner, k_pos = np.array(k_owner, dtype=np.int64), np.array(k_pos, dtype=np.int64)
    mask = (q_owner[:, None] == k_owner[None, :]) & (k_pos[None, :] <= q_pos[:, None])
    return mask, k_owner, k_pos


def ragged_attention_dense_mask(q, k_new, v_new, hist_k, hist_v, cu_q_lens, ctx_lens, scale):
    """Ragged attention as one dense masked softmax over the whole concatenated stream."""
    q = np.asarray(q, dtype=F64)
    cu = [int(x) for x in cu_q_lens]
    ks, vs = [], []
    for r in range(len(cu) - 1):
        ks += [np.asarray(hist_k[r], F64).reshape(-1, *k_new.shape[1:]), np.asarray(k_new[cu[r]:cu[r + 1]], F64)]
        vs += [np.asarray(hist_v[r], F64).reshape(-1, *v_new.shape[1:]), np.asarray(v_new[cu[r]:cu[r + 1]], F64)]
    K = np.concatenate(ks) if ks else np.zeros((0,) + k_new.shape[1:])
    V = np.concatenate(vs) if vs else np.zeros((0,) + v_new.shape[1:])
    mask, _, _ = stream_mask(cu, ctx_lens)
    T, hq, d = q.shape
    group = hq // K.shape[1]
    out = np.zeros((T, hq, d), dtype=F64)
    for h in range(hq):
        s = scale * (q[:, h, :] @ K[:, h // group, :].T)
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[:, h // group, :]
    return out


def padded_batch(q, k_new, v_new, hist_k, hist_v, cu_q_lens, ctx_lens):
    """Blog section "Continuous batching", batched generation: add a batch axis and left-pad.

    Returns (Qp [B, Qmax, Hq, D], Kp, Vp [B, Lmax, Hkv, D], mask [B, Qmax, Lmax],
    q_valid [B, Qmax], pad_query_tokens). Pad positions carry zeros and are masked out.
    """
    cu = [int(x) for x in cu_q_lens]
    B = len(cu) - 1
    nq = [cu[r + 1] - cu[r] for r in range(B)]
    L = [int(ctx_lens[r]) + nq[r] for r in range(B)]
    qmax, lmax = max(nq), max(L)
    T, hq, d = q.shape
    hkv = k_new.shape[1]
    Qp = np.zeros((B, qmax, hq, d), F64)
    Kp = np.zeros((B, lmax, hkv, d), F64)
    Vp = np.zeros((B, lmax, hkv, d), F64)
    mask = np.zeros((B, qmax, lmax), bool)
    q_valid = np.zeros((B, qmax), bool)
    for r in range(B):
        c = int(ctx_lens[r])
        qo, ko = qmax - nq[r], lmax - L[r]                       # left padding offsets
        Qp[r, qo:] = q[cu[r]:cu[r + 1]]
        Kp[r, ko:] = np.concatenate([np.asarray(hist_k[r], F64).reshape(c, hkv, d), k_new[cu[r]:cu[r + 1]]])
        Vp[r, ko:] = np.concatenate([np.asarray(hist_v[r], F64).reshape(c, hkv, d), v_new[cu[r]:cu[r + 1]]])
        q_valid[r, qo:] = True
        for i in range(nq[r]):
            # padded row qo+i holds position c+i; padded column ko+j holds position j
            mask[r, qo + i, ko:ko + c + i + 1] = True
    pad_tokens = int(B * qmax - sum(nq))
    return Qp, Kp, Vp, mask, q_valid, pad_tokens


def padded_batch_attention(q, k_new, v_new, hist_k, hist_v, cu_q_lens, ctx_lens, scale):
    """Attention on the left-padded batch, unpacked back to [T, Hq, D] (pad rows dropped)."""
    Qp, Kp, Vp, mask, q_valid, _ = padded_batch(q, k_new, v_new, hist_k, hist_v, cu_q_lens, ctx_lens)
    B, qmax, hq, d = Qp.shape
    group = hq // Kp.shape[2]
    out = np.zeros((B, qmax, hq, d), F64)
    for h in range(hq):
        s = scale * np.einsum("bqd,bkd->bqk", Qp[:, :, h], Kp[:, :, h // group])
        s = np.where(mask, s, -np.inf)
        with np.errstate(invalid="ignore"):
            s = s - s.max(axis=2, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=2, keepdims=True)                    # pad rows become NaN
        out[:, :, h] = np.einsum("bqk,bkd->bqd", p, Vp[:, :, h // group])
    return out[q_valid]                                              # request order, row order
