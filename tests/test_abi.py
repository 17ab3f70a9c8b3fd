"""The C-ABI library (CPU only): it loads, exports every function that include/cb.h declares,
and rejects malformed arguments before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

from ragged_continuous_batching_amd import cb

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "cb.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cb_[a-z_0-9]+)\s*\(", text)))


def test_header_functions_are_exported():
    names = declared_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(cb.lib, n), f"{n} declared in cb.h but not exported"
    assert set(names) == set(cb.EXPORTED)


def test_device_checks_absent_from_the_normal_build():
    """Counting clamped block ids is a debug copy's feature; the normal library says so."""
    if cb.LIB_PATH.endswith(os.path.join("checks", "libcb.so")):
        pytest.skip("this process loaded the device-checks copy")
    with pytest.raises(cb.CbError) as e:
        cb.cb_debug_violations()
    assert e.value.status == cb.CB_ERR_UNSUPPORTED
    assert "--device-checks" in str(e.value)


def test_version_and_names():
    assert "gfx950" in cb.cb_version()
    assert cb.cb_kernel_name(cb.CB_KERNEL_DECODE) == "row_attn_kernel"
    assert cb.cb_kernel_name(99) == ""


def _shape(**kw):
    d = dict(num_q_heads=4, num_kv_heads=2, head_dim=128, num_blocks=16, dtype="bf16")
    d.update(kw)
    return cb.make_shape(**d)


def _batch(cu, ctx, maxb):
    """cb_batch with host mirrors only; device pointers are dummies that are never read."""
    cu = np.asarray(cu, np.int32)
    ctx = np.asarray(ctx, np.int32)
    b = cb.cb_batch(len(ctx), int(cu[-1]), maxb, 256, 256, 256, cu.ctypes.data, ctx.ctypes.data)
    b._keep = (cu, ctx)
    return b


FAKE = 1 << 20   # 16-byte aligned non-null address; validation fails before any use


@pytest.mark.parametrize("shape_kw,status", [
    (dict(num_q_heads=6, num_kv_heads=4), cb.CB_ERR_INVALID_ARG),
    (dict(num_q_heads=12, num_kv_heads=4), cb.CB_ERR_UNSUPPORTED),     # group of 3
    (dict(head_dim=96), cb.CB_ERR_UNSUPPORTED),
    (dict(block_size=8), cb.CB_ERR_UNSUPPORTED),
    (dict(num_blocks=0), cb.CB_ERR_INVALID_ARG),
])
def test_bad_shape_rejected(shape_kw, status):
    shape = _shape(**shape_kw)
    b = _batch([0, 1], [3], 1)
    rc = cb.lib.cb_ragged_attention(ctypes.byref(shape), ctypes.byref(b), FAKE, FAKE, FAKE, 1.0, FAKE, FAKE,
                                    1 << 20, None)
    assert rc == status, cb.cb_last_error()
    assert cb.cb_last_error()


@pytest.mark.parametrize("cu,ctx,maxb,why", [
    ([1, 2], [0], 4, "cu_q_lens[0]"),
    ([0, 3, 2], [0, 0], 4, "decreases"),
    ([0, 2], [-1], 4, "negative"),
    ([0, 2], [31], 1, "needs 3 blocks"),
])
def test_bad_metadata_rejected(cu, ctx, maxb, why):
    shape = _shape()
    b = _batch(cu, ctx, maxb)
    for rc in (
        cb.lib.cb_ragged_attention(ctypes.byref(shape), ctypes.byref(b), FAKE, FAKE, FAKE, 1.0, FAKE, FAKE, 1 << 30,
                                   None),
        cb.lib.cb_kv_append(ctypes.byref(shape), ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, None),
    ):
        assert rc == cb.CB_ERR_INVALID_ARG
        assert why in cb.cb_last_error()
    assert cb.cb_ragged_attention_workspace_size(shape, b) == 0


def test_num_tokens_mismatch_and_alignment():
    shape = _shape()
    b = _batch([0, 2], [0], 1)
    b.num_tokens = 3
    assert cb.lib.cb_kv_append(ctypes.byref(shape), ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, None) == cb.CB_ERR_INVALID_ARG
    b = _batch([0, 2], [0], 1)
    rc = cb.lib.cb_ragged_attention(ctypes.byref(shape), ctypes.byref(b), FAKE + 2, FAKE, FAKE, 1.0, FAKE, FAKE,
                                    1 << 30, None)
    assert rc == cb.CB_ERR_INVALID_ARG and "aligned" in cb.cb_last_error()


def test_workspace_checks():
    shape = _shape()
    b = _batch([0, 1, 2], [4000, 17], 256)
    need = cb.cb_ragged_attention_workspace_size(shape, b)
    assert need > 0
    rc = cb.lib.cb_ragged_attention(ctypes.byref(shape), ctypes.byref(b), FAKE, FAKE, FAKE, 1.0, FAKE, FAKE, need - 1,
                                    None)
    assert rc == cb.CB_ERR_WORKSPACE_TOO_SMALL
    rc = cb.lib.cb_ragged_attention(ctypes.byref(shape), ctypes.byref(b), FAKE, FAKE, FAKE, 1.0, FAKE, FAKE + 16,
                                    need, None)
    assert rc == cb.CB_ERR_INVALID_ARG and "256-byte" in cb.cb_last_error()


def test_empty_batch_is_a_no_op():
    shape = _shape()
    cu = np.zeros(1, np.int32)
    b = cb.cb_batch(0, 0, 0, None, None, None, cu.ctypes.data, cu.ctypes.data)
    assert cb.lib.cb_ragged_attention(ctypes.byref(shape), ctypes.byref(b), None, None, None, 1.0, None, None, 0,
                                      None) == 0
    assert cb.lib.cb_kv_append(ctypes.byref(shape), ctypes.byref(b), None, None, None, None, None) == 0
    assert cb.cb_ragged_attention_workspace_size(shape, b) == 0


def header_tuning_keys():
    """The keys listed in cb.h's cb_set_tuning comment, with their documented defaults."""
    text = open(HEADER).read()
    block = text[text.index("Tuning knobs"):text.index("int cb_set_tuning")]
    return re.findall(r'^\s*\*\s+"([a-z_]+)"', block, flags=re.M)


TUNING_DEFAULTS = {"split_blocks": 0, "target_waves": 0, "overlap_prefill": 0, "xcds": 8, "decode_mfma": 1,
                   "decode_group": 8, "stage_kernel": 1, "prefill_waves": 0, "prefill_snake": 1, "prefill_split": 1,
                   "prefill_split_tiles": 0, "decode_order": 1, "mixed_launch": 0, "mixed_order": 0,
                   "prefill_heads": 0}


def test_tuning_keys():
    keys = header_tuning_keys()
    assert sorted(keys) == sorted(TUNING_DEFAULTS), keys
    for k in keys:
        assert cb.cb_get_tuning(k) == TUNING_DEFAULTS[k], k
        with cb.tuned(**{k: 1 if k not in ("prefill_waves", "decode_group", "prefill_heads") else 4}):
            assert cb.cb_get_tuning(k) in (1, 4)
        assert cb.cb_get_tuning(k) == TUNING_DEFAULTS[k], k
    for bad in ("no_such_key", "prefill_touch"):
        with pytest.raises(cb.CbError):
            cb.cb_set_tuning(bad, 1)
        with pytest.raises(cb.CbError):
            cb.cb_get_tuning(bad)
    with pytest.raises(cb.CbError):
        cb.cb_set_tuning("split_blocks", -1)
    for k, v in (("prefill_waves", 6), ("decode_group", 3), ("prefill_heads", 3)):
        with pytest.raises(cb.CbError):
            cb.cb_set_tuning(k, v)
        assert cb.cb_get_tuning(k) == TUNING_DEFAULTS[k]
    assert cb.lib.cb_get_tuning(b"xcds", None) == cb.CB_ERR_INVALID_ARG


def test_every_tuning_key_has_a_gpu_test():
    """Each documented key is set to a non-default value by some GPU parity test."""
    tdir = os.path.dirname(os.path.abspath(__file__))
    text = ""
    for name in sorted(os.listdir(tdir)):
        if name.startswith("test_gpu") and name.endswith(".py"):
            text += open(os.path.join(tdir, name)).read()
    for k in header_tuning_keys():
        assert re.search(r'(cb_set_tuning\("%s"|\b%s=)' % (k, k), text), f"no GPU test sets {k}"


def test_kv_bytes_per_position_matches_pages():
    """Hugging Face blog, "KV-cache": one Llama-2-7B position of one layer = 8,192 values =
    16 KB in fp16. The two cache pages of a block hold exactly that per position."""
    shape = cb.make_shape(32, 32, 128, 1, "bf16")
    per_block_bytes = 2 * shape.num_kv_heads * shape.block_size * shape.head_dim * 2
    assert per_block_bytes // shape.block_size == 16384


def test_step_forward_checks_host_metadata():
    shape = _shape(num_blocks=8)
    cu = np.array([0, 3], np.int32)
    ctx = np.array([14], np.int32)
    bt = np.array([[0, 9]], np.int32)                       # block 9 is outside the pool of 8
    need = cb.cb_step_workspace_size(shape, 1, 3, 2, cu, ctx)
    assert need > 0
    with pytest.raises(cb.CbError) as e:
        cb.cb_step_forward(shape, 1, 3, 2, cu, ctx, bt, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, FAKE, FAKE, need, 0)
    assert e.value.status == cb.CB_ERR_INVALID_ARG and "out of range" in str(e.value)
    bt = np.array([[0, 1]], np.int32)
    with pytest.raises(cb.CbError) as e:
        cb.cb_step_forward(shape, 1, 3, 2, cu, ctx, bt, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, FAKE, FAKE, need - 1, 0)
    assert e.value.status == cb.CB_ERR_WORKSPACE_TOO_SMALL
    with pytest.raises(cb.CbError) as e:
        cb.cb_step_forward(shape, 1, 3, 2, cu, ctx, bt, FAKE, FAKE, FAKE, FAKE, FAKE, -1.0, FAKE, FAKE, need, 0)
    assert e.value.status == cb.CB_ERR_INVALID_ARG and "scale" in str(e.value)


def test_scale_must_be_positive():
    shape = _shape()
    b = _batch([0, 1], [3], 1)
    for sc in (0.0, -0.5, float("inf"), float("nan")):
        rc = cb.lib.cb_ragged_attention(ctypes.byref(shape), ctypes.byref(b), FAKE, FAKE, FAKE, sc, FAKE, FAKE,
                                        1 << 30, None)
        assert rc == cb.CB_ERR_INVALID_ARG, sc


def test_linear_checks_shapes_and_pointers():
    for (m, n, k) in [(4, 96, 64), (4, 128, 48), (4, 128, (1 << 20) + 64), (-1, 128, 64)]:
        assert cb.lib.cb_linear(m, n, k, FAKE, FAKE, FAKE, None) == cb.CB_ERR_UNSUPPORTED, (m, n, k)
    assert cb.lib.cb_linear(4, 128, 64, None, FAKE, FAKE, None) == cb.CB_ERR_INVALID_ARG
    assert cb.lib.cb_linear(4, 128, 64, FAKE + 2, FAKE, FAKE, None) == cb.CB_ERR_INVALID_ARG
    assert cb.lib.cb_linear(0, 128, 64, None, None, None, None) == cb.CB_OK


def test_qkv_project_checks_shapes_and_pointers():
    b = _batch([0, 2], [5], 1)
    fp32 = _shape(dtype="fp32")
    assert cb.lib.cb_qkv_project(ctypes.byref(fp32), ctypes.byref(b), 256, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 None) == cb.CB_ERR_UNSUPPORTED
    shape = _shape()
    for dm in (0, 100, (1 << 20) + 64):
        assert cb.lib.cb_qkv_project(ctypes.byref(shape), ctypes.byref(b), dm, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     None) == cb.CB_ERR_UNSUPPORTED, dm
    narrow = _shape(num_q_heads=1, num_kv_heads=1, head_dim=64)           # Hkv*D = 64
    assert cb.lib.cb_qkv_project(ctypes.byref(narrow), ctypes.byref(b), 256, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 None) == cb.CB_ERR_UNSUPPORTED
    assert cb.lib.cb_qkv_project(ctypes.byref(shape), ctypes.byref(b), 256, FAKE, None, FAKE, FAKE, FAKE,
                                 None) == cb.CB_ERR_INVALID_ARG
    empty = _batch([0], [], 0)
    assert cb.lib.cb_qkv_project(ctypes.byref(shape), ctypes.byref(empty), 256, None, None, None, None, None,
                                 None) == cb.CB_OK


def test_graph_entry_points_check_arguments():
    """cb_graph_create rejects bad arguments before it touches the device; the other graph
    calls reject a NULL graph."""
    shape = _shape()
    out = ctypes.c_void_p(123)
    for args, status in [
        ((0, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, FAKE), cb.CB_ERR_INVALID_ARG),          # max_tokens
        ((8, FAKE, None, FAKE, FAKE, FAKE, 1.0, FAKE), cb.CB_ERR_INVALID_ARG),          # k_new NULL
        ((8, FAKE, FAKE + 4, FAKE, FAKE, FAKE, 1.0, FAKE), cb.CB_ERR_INVALID_ARG),      # unaligned
        ((8, None, FAKE, FAKE, FAKE, FAKE, 1.0, FAKE), cb.CB_ERR_INVALID_ARG),          # q NULL
        ((8, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0, FAKE), cb.CB_ERR_INVALID_ARG),          # scale
    ]:
        rc = cb.lib.cb_graph_create(ctypes.byref(shape), *args, ctypes.byref(out))
        assert rc == status, cb.cb_last_error()
        assert out.value is None                                                         # nothing created
        out = ctypes.c_void_p(123)
    bad = _shape(head_dim=96)
    assert cb.lib.cb_graph_create(ctypes.byref(bad), 8, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, FAKE,
                                  ctypes.byref(out)) == cb.CB_ERR_UNSUPPORTED
    assert cb.lib.cb_graph_create(ctypes.byref(shape), 8, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, FAKE,
                                  None) == cb.CB_ERR_INVALID_ARG
    cu = np.array([0, 1], np.int32)
    assert cb.lib.cb_graph_step(None, 1, 1, 1, cu.ctypes.data, cu.ctypes.data, cu.ctypes.data, None) == \
        cb.CB_ERR_INVALID_ARG
    assert cb.lib.cb_graph_stats(None, None, None, None) == cb.CB_ERR_INVALID_ARG
    cb.lib.cb_graph_destroy(None)


def test_noalloc_rejects_a_plan_larger_than_its_array():
    """cb_ragged_attention_noalloc checks the batch's workspace against its fixed array before
    it touches the device: a 256-row chunk after 16k cached tokens split into one-tile key
    ranges needs about 1 GiB of partials."""
    shape = cb.make_shape(32, 32, 128, 4096, "bf16")
    b = _batch([0, 256], [16384], 1040)
    with cb.tuned(prefill_split_tiles=1):
        need = cb.cb_ragged_attention_workspace_size(shape, b)
        assert need > cb.NOALLOC_SCRATCH_BYTES
        st = cb.lib.cb_ragged_attention_noalloc(ctypes.byref(shape), ctypes.byref(b), FAKE, FAKE, FAKE, 0.1, FAKE,
                                                None)
    assert st == cb.CB_ERR_WORKSPACE_TOO_SMALL
    assert "fixed" in cb.cb_last_error()
    assert "CB_NOALLOC_SCRATCH_BYTES (32u << 20)" in open(HEADER).read()


def test_paged_read_probe_checks_arguments():
    """The measurement probe rejects an empty or NULL page set before any launch, and sizes
    its sink at one word per work-group of 64 pages."""
    assert cb.cb_paged_read_probe_sink_words(0) == 0
    assert cb.cb_paged_read_probe_sink_words(1) == 1
    assert cb.cb_paged_read_probe_sink_words(64) == 1
    assert cb.cb_paged_read_probe_sink_words(65) == 2
    with pytest.raises(cb.CbError):
        cb.cb_paged_read_probe(None, 16, None, None)
    with pytest.raises(cb.CbError):
        cb.cb_paged_read_probe(256, 0, 256, 256)
    with pytest.raises(cb.CbError):          # misaligned pages
        cb.cb_paged_read_probe(257, 4, 256, 256)
