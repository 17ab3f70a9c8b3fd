"""Pins for the token-wise layer oracle (CPU only): brute force, closed forms and the
token-wise property the pages state."""
import numpy as np

import workloads as W
from oracle import layer as L


def test_linear_against_brute_force():
    rng = np.random.default_rng(0)
    a = rng.integers(-3, 4, size=(5, 7)).astype(np.float64)
    w = rng.integers(-3, 4, size=(4, 7)).astype(np.float64)
    y = L.linear(a, w)
    for m in range(5):
        for n in range(4):
            s = 0.0
            for k in range(7):
                s += a[m, k] * w[n, k]
            assert y[m, n] == s


def test_linear_identity_permutation_and_linearity():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((6, 8))
    assert np.array_equal(L.linear(a, np.eye(8)), a)
    perm = rng.permutation(8)
    assert np.array_equal(L.linear(a, np.eye(8)[perm]), a[:, perm])
    b = rng.integers(-4, 5, size=(6, 8)).astype(np.float64)
    c = rng.integers(-4, 5, size=(6, 8)).astype(np.float64)
    w = rng.integers(-4, 5, size=(3, 8)).astype(np.float64)
    assert np.array_equal(L.linear(2 * b + c, w), 2 * L.linear(b, w) + L.linear(c, w))


def test_token_wise_rows_do_not_interact():
    """Hugging Face blog, "Attention": token-wise operations see each token alone, so
    packing order does not matter: permuting the packed rows permutes the outputs."""
    rng = np.random.default_rng(2)
    a = rng.standard_normal((9, 16))
    w = rng.standard_normal((12, 16))
    perm = rng.permutation(9)
    assert np.allclose(L.linear(a[perm], w), L.linear(a, w)[perm], rtol=0, atol=1e-12)


def test_qkv_split_layout_head_major():
    """Selector weights: output feature f copies input feature sel[f]; the split must hand
    query head h dimension d the feature h*D + d, then keys, then values."""
    hq, hkv, d = 3, 1, 4
    n_out = (hq + 2 * hkv) * d
    x = np.arange(2 * n_out, dtype=np.float64).reshape(2, n_out)
    sel = np.eye(n_out)
    q, k, v = L.qkv_split(L.linear(x, sel), hq, hkv, d)
    assert q.shape == (2, hq, d) and k.shape == (2, hkv, d) and v.shape == (2, hkv, d)
    for t in range(2):
        for h in range(hq):
            assert np.array_equal(q[t, h], x[t, h * d:(h + 1) * d])
        assert np.array_equal(k[t, 0], x[t, hq * d:(hq + 1) * d])
        assert np.array_equal(v[t, 0], x[t, (hq + 1) * d:])


def test_layer_inputs_and_weights():
    wl = W.custom([W.Request(0, 10, 1)], num_q_heads=4, num_kv_heads=2, head_dim=64, dtype="bf16")
    x1 = wl.x_values([3, 3, 5], [7, 8, 7], 256)
    x2 = wl.x_values([5], [7], 256)
    assert x1.shape == (3, 256) and np.array_equal(x1[2], x2[0])       # value = f(request, position)
    assert not np.array_equal(x1[0], x1[1])
    bits = W.layer_weights(wl.seed, 0, 512, 1024)
    w = W.f32_from_bf16_bits(bits)
    assert abs(w.std() * np.sqrt(1024) - 1.0) < 0.02                    # N(0, 1/fan_in)
    assert np.array_equal(W.bf16_bits_from_f32(w), bits)                # exactly bf16
