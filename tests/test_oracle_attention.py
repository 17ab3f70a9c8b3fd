"""Pins for the fp64 attention oracle (CPU only).

Each check ties ``oracle.attention`` to something other than itself: numbers printed on
the pages (tests/golden/pages_worked_examples.json), independent restatements (scalar brute
force, the blog's dense mask over the concatenated stream, the left-padded batch), a
library routine on a special case (torch SDPA in float64), closed forms, and invariants
that the pages state. ``test_planted_mistakes_are_caught`` checks that plausible bugs
planted in the oracle make at least one pin fail.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_examples.json")))


def _case(lens, ctxs, hq=2, hkv=2, d=16, seed=0, scale=None):
    """Random fp64 packed step: q, k_new, v_new, hist_k, hist_v, cu, ctx, scale."""
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    q = rng.standard_normal((T, hq, d))
    kn = rng.standard_normal((T, hkv, d))
    vn = rng.standard_normal((T, hkv, d))
    hk = [rng.standard_normal((c, hkv, d)) for c in ctxs]
    hv = [rng.standard_normal((c, hkv, d)) for c in ctxs]
    return q, kn, vn, hk, hv, cu, np.asarray(ctxs), (1 / math.sqrt(d) if scale is None else scale)


CASES = {
    "pages_D4_B1_C1": ([4, 1, 1], [0, 4, 2]),
    "tiny_config": ([1, 1, 7], [12, 20, 0]),
    "chunk_after_cache": ([5, 3, 1, 1], [9, 0, 31, 0]),
    "empty_request": ([2, 0, 3], [1, 5, 0]),
}


# --------------------------------------------------------------------------------------
# pins, each a function of the two oracle entry points so that planted bugs can be run
# through them
# --------------------------------------------------------------------------------------
def pin_dense_mask(ragged):
    for lens, ctxs in CASES.values():
        args = _case(lens, ctxs, hq=4, hkv=2)
        np.testing.assert_allclose(ragged(*args), A.ragged_attention_dense_mask(*args), rtol=0, atol=1e-12)


def pin_bruteforce(ragged):
    for lens, ctxs in CASES.values():
        q, kn, vn, hk, hv, cu, ctx, sc = _case(lens, ctxs, hq=4, hkv=2, d=8, seed=1)
        o = ragged(q, kn, vn, hk, hv, cu, ctx, sc)
        for r in range(len(lens)):
            s, e = int(cu[r]), int(cu[r + 1])
            if e == s:
                continue
            keys = np.concatenate([hk[r], kn[s:e]])
            vals = np.concatenate([hv[r], vn[s:e]])
            ref = A.attend_scalar(q[s:e], keys, vals, ctx[r] + np.arange(e - s), sc)
            np.testing.assert_allclose(o[s:e], ref, rtol=0, atol=1e-12)


def pin_padded_batch(ragged):
    for lens, ctxs in CASES.values():
        if 0 in lens:
            continue
        args = _case(lens, ctxs, hq=4, hkv=2, seed=2)
        np.testing.assert_allclose(ragged(*args), A.padded_batch_attention(*args), rtol=0, atol=1e-12)


def pin_sdpa(ragged):
    """Library special case: torch SDPA (float64, CPU) with GQA heads repeated."""
    for lens, ctxs in CASES.values():
        q, kn, vn, hk, hv, cu, ctx, sc = _case(lens, ctxs, hq=6, hkv=2, seed=3)
        o = ragged(q, kn, vn, hk, hv, cu, ctx, sc)
        for r in range(len(lens)):
            s, e, c = int(cu[r]), int(cu[r + 1]), int(ctx[r])
            if e == s:
                continue
            keys = torch.from_numpy(np.concatenate([hk[r], kn[s:e]])).permute(1, 0, 2)
            vals = torch.from_numpy(np.concatenate([hv[r], vn[s:e]])).permute(1, 0, 2)
            keys = keys.repeat_interleave(3, dim=0)
            vals = vals.repeat_interleave(3, dim=0)
            qq = torch.from_numpy(q[s:e]).permute(1, 0, 2)
            if c == 0:
                ref = torch.nn.functional.scaled_dot_product_attention(qq, keys, vals, is_causal=True, scale=sc)
            else:   # SDPA's is_causal is top-left aligned; give the bottom-right mask explicitly
                mask = torch.arange(c + e - s)[None, :] <= (c + torch.arange(e - s))[:, None]
                ref = torch.nn.functional.scaled_dot_product_attention(qq, keys, vals, attn_mask=mask, scale=sc)
            np.testing.assert_allclose(o[s:e], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def pin_closed_forms(ragged):
    # scale 0: every visible key has equal weight -> O is the running mean of visible V
    q, kn, vn, hk, hv, cu, ctx, _ = _case([3, 1, 6], [2, 7, 0], hq=2, hkv=1, seed=4)
    o = ragged(q, kn, vn, hk, hv, cu, ctx, 0.0)
    for r in range(3):
        s, e, c = int(cu[r]), int(cu[r + 1]), int(ctx[r])
        vals = np.concatenate([hv[r], vn[s:e]])[:, 0, :]
        for i in range(e - s):
            np.testing.assert_allclose(o[s + i, 0], vals[: c + i + 1].mean(axis=0), rtol=0, atol=1e-12)
            np.testing.assert_allclose(o[s + i, 1], vals[: c + i + 1].mean(axis=0), rtol=0, atol=1e-12)
    # constant V -> O is that constant
    q, kn, vn, hk, hv, cu, ctx, sc = _case([4, 1], [0, 5], seed=5)
    u = np.linspace(-1, 1, 16)
    vn[:] = u
    hv = [np.broadcast_to(u, h.shape).copy() for h in hv]
    o = ragged(q, kn, vn, hk, hv, cu, ctx, sc)
    np.testing.assert_allclose(o, np.broadcast_to(u, o.shape), rtol=0, atol=1e-12)
    # first row of a fresh prompt sees only itself -> O = v0 exactly
    q, kn, vn, hk, hv, cu, ctx, sc = _case([5], [0], seed=6)
    o = ragged(q, kn, vn, hk, hv, cu, ctx, sc)
    assert np.array_equal(o[0], vn[0])
    # one key with a dominant logit -> O is (to 1e-12) that key's value
    q, kn, vn, hk, hv, cu, ctx, sc = _case([1], [9], seed=7)
    hk[0][3] = 60.0 * q[0] / np.linalg.norm(q[0], axis=-1, keepdims=True)
    o = ragged(q, kn, vn, hk, hv, cu, ctx, 1.0)
    np.testing.assert_allclose(o[0], hv[0][3], rtol=0, atol=1e-12)


def pin_chunked_equals_unchunked(ragged):
    """Blog, "Chunked prefill": splitting a prompt into chunks that reuse the cached K/V
    gives the same result as one prefill, for any split (here ceil(7/4) = 4 + 3 and 1+2+4)."""
    q, kn, vn, hk, hv, cu, ctx, sc = _case([7], [0], seed=8)
    whole = ragged(q, kn, vn, hk, hv, cu, ctx, sc)
    for split in ([4, 3], [1, 2, 4]):
        start, parts = 0, []
        for n in split:
            sl = slice(start, start + n)
            parts.append(ragged(q[sl], kn[sl], vn[sl], [kn[:start]], [vn[:start]], [0, n], [start], sc))
            start += n
        np.testing.assert_allclose(np.concatenate(parts), whole, rtol=0, atol=1e-12)


def pin_decode_equals_prefill_row(ragged):
    """Blog, "KV-cache": decoding token n+1 with n cached equals the last row of a full
    (n+1)-token prefill, because later tokens do not change earlier rows under the causal mask."""
    n = 12
    q, kn, vn, hk, hv, cu, ctx, sc = _case([n + 1], [0], seed=9)
    full = ragged(q, kn, vn, hk, hv, cu, ctx, sc)
    dec = ragged(q[n:], kn[n:], vn[n:], [kn[:n]], [vn[:n]], [0, 1], [n], sc)
    np.testing.assert_allclose(dec[0], full[n], rtol=0, atol=1e-12)


def pin_permutation(ragged):
    lens, ctxs = [3, 1, 5, 2], [4, 9, 0, 1]
    q, kn, vn, hk, hv, cu, ctx, sc = _case(lens, ctxs, seed=10)
    o = ragged(q, kn, vn, hk, hv, cu, ctx, sc)
    perm = [2, 0, 3, 1]
    rows = np.concatenate([np.arange(cu[r], cu[r + 1]) for r in perm])
    lens2 = [lens[r] for r in perm]
    cu2 = np.concatenate([[0], np.cumsum(lens2)])
    o2 = ragged(q[rows], kn[rows], vn[rows], [hk[r] for r in perm], [hv[r] for r in perm], cu2,
                [ctxs[r] for r in perm], sc)
    np.testing.assert_allclose(o2, o[rows], rtol=0, atol=1e-12)


PINS = [pin_dense_mask, pin_bruteforce, pin_padded_batch, pin_sdpa, pin_closed_forms,
        pin_chunked_equals_unchunked, pin_decode_equals_prefill_row, pin_permutation]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pins(pin):
    pin(A.ragged_attention)


# --------------------------------------------------------------------------------------
# numbers printed on the pages
# --------------------------------------------------------------------------------------
def test_pages_cu_seqlens():
    g = GOLD["cu_seqlens"]
    assert list(np.concatenate([[0], np.cumsum(g["lengths"])])) == g["cu_seqlens"]


def test_pages_score_shapes():
    """zhangchitc: D (4 queries, empty cache) is 4x4 lower triangular, B is 1x5, C is 1x3."""
    reqs = GOLD["score_shapes"]["requests"]
    cu = np.concatenate([[0], np.cumsum([r["q"] for r in reqs])])
    mask, owner, _ = A.stream_mask(cu, [r["ctx"] for r in reqs])
    for i, r in enumerate(reqs):
        block = mask[cu[i]:cu[i + 1]][:, owner == i]
        assert list(block.shape) == r["shape"]
        assert block.all() if r["q"] == 1 else np.array_equal(block, np.tril(np.ones(r["shape"], bool)))
        # nothing outside the request's own block is visible (block-diagonal)
        assert not mask[cu[i]:cu[i + 1]][:, owner != i].any()


def test_pages_padding_count():
    """Blog, dynamic scheduling: adding an n-token prompt to B-1 decoding prompts costs (n-1)(B-1) pads."""
    g = GOLD["padding_tokens"]
    B, n = g["B"], g["n"]
    lens = [n] + [1] * (B - 1)
    q, kn, vn, hk, hv, cu, ctx, _ = _case(lens, [0] + [3] * (B - 1), hq=1, hkv=1, d=2)
    *_, pad = A.padded_batch(q, kn, vn, hk, hv, cu, ctx)
    assert pad == g["pad"] == (n - 1) * (B - 1)


def test_pages_kv_cache_size():
    """Blog, "KV-cache": one token of one Llama-2-7B layer holds 2*H*A values, 16 KB in fp16."""
    g = GOLD["kv_cache_size"]
    w = W.config(2)
    per_position = 2 * w.num_kv_heads * w.head_dim          # K and V rows of one position
    assert (w.num_kv_heads, w.head_dim) == (g["heads"], g["head_dim"])
    assert per_position == g["values_per_token_per_layer"]
    assert per_position * 2 == g["bytes_per_token_per_layer_fp16"]


def test_prompt_of_seven_tokens_is_causal():
    """Blog, "Attention": for the 7-token prompt the mask is lower triangular."""
    n = len(GOLD["prompt_7_tokens"]["tokens"])
    mask, _, _ = A.stream_mask([0, n], [0])
    assert np.array_equal(mask, np.tril(np.ones((n, n), bool)))


# --------------------------------------------------------------------------------------
# planted mistakes (run on the CPU only): each must fail at least one pin
# --------------------------------------------------------------------------------------
def _mutant_attend(kind):
    def attend(q, keys, values, positions, scale):
        q = np.asarray(q, np.float64); keys = np.asarray(keys, np.float64); values = np.asarray(values, np.float64)
        positions = np.asarray(positions)
        n, hq, d = q.shape
        L, hkv, _ = keys.shape
        g_of = (lambda h: h % hkv) if kind == "gqa_modulo" else (lambda h: h // (hq // hkv))
        if kind == "top_left_causal":
            visible = np.arange(L)[None, :] <= np.arange(n)[:, None]
        elif kind == "excludes_self":
            visible = np.arange(L)[None, :] < positions[:, None]
        else:
            visible = np.arange(L)[None, :] <= positions[:, None]
        out = np.zeros((n, hq, d))
        for h in range(hq):
            g = g_of(h)
            sc = 1.0 if kind == "no_scale" else scale
            s = sc * (q[:, h] @ keys[:, g].T)
            s = np.where(visible, s, -np.inf)
            ax = 0 if kind == "softmax_axis" else 1
            with np.errstate(invalid="ignore"):
                s = s - s.max(axis=ax, keepdims=True)
                p = np.exp(s)
                p = p / p.sum(axis=ax, keepdims=True)
            p = np.nan_to_num(p)
            vv = keys if kind == "keys_as_values" else values
            out[:, h] = p @ vv[:, g]
        return out
    return attend


MUTANTS = ["top_left_causal", "excludes_self", "gqa_modulo", "no_scale", "softmax_axis", "keys_as_values",
           "drop_history"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistakes_are_caught(kind, monkeypatch):
    if kind == "drop_history":
        orig = A.ragged_attention

        def ragged(q, kn, vn, hk, hv, cu, ctx, sc):
            o = np.zeros(np.asarray(q).shape)
            for r in range(len(cu) - 1):
                s, e = int(cu[r]), int(cu[r + 1])
                if e > s:
                    o[s:e] = A.attend(q[s:e], kn[s:e], vn[s:e], np.arange(e - s), sc)
            return o
        del orig
    else:
        monkeypatch.setattr(A, "attend", _mutant_attend(kind))
        ragged = A.ragged_attention
    failures = 0
    for pin in PINS:
        try:
            pin(ragged)
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures >= 1, f"planted mistake {kind} passed every pin"
