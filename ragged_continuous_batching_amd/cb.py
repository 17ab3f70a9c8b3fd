"""ctypes binding of libcb.so (include/cb.h). Argument marshalling only.

Every function keeps the C name and argument order. Tensor arguments may be torch tensors
(their data pointers are passed) or integer addresses. Streams may be a torch Stream, an
integer hipStream_t, or None (the current torch stream when torch is imported, else 0).
Nothing here computes any part of the attention step: all of it runs in the library.
If libcb.so is missing the import fails; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

# CB_LIBRARY names another build of the same library to load instead (the host-sanitized
# test copy); by default the in-tree libcb.so.
LIB_PATH = os.environ.get("CB_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcb.so")

CB_OK = 0
CB_ERR_INVALID_ARG = -1
CB_ERR_UNSUPPORTED = -2
CB_ERR_HIP = -3
CB_ERR_OUT_OF_BLOCKS = -4
CB_ERR_WORKSPACE_TOO_SMALL = -5
CB_ERR_STATE = -6
CB_F32, CB_BF16 = 0, 1
CB_KERNEL_APPEND, CB_KERNEL_DECODE, CB_KERNEL_COMBINE, CB_KERNEL_PREFILL, CB_KERNEL_GEMM, CB_KERNEL_MIXED = 0, 1, 2, 3, 4, 5
KERNELS = {"append": 0, "decode": 1, "combine": 2, "prefill": 3, "gemm": 4, "mixed": 5}

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


class CbError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"cb status {status}: {msg}")
        self.status = status


class cb_shape(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class cb_batch(ctypes.Structure):
    _fields_ = [("num_reqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32), ("max_blocks_per_req", ctypes.c_int32),
                ("cu_q_lens", ctypes.c_void_p), ("ctx_lens", ctypes.c_void_p), ("block_tables", ctypes.c_void_p),
                ("h_cu_q_lens", ctypes.c_void_p), ("h_ctx_lens", ctypes.c_void_p)]


class cb_plan_info(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "prefill_rows", "prefill_items", "prefill_split_items", "decode_splits", "decode_items", "split_blocks",
        "split_min_blocks", "split_max_blocks", "longest_first", "matrix_core_decode", "combine_rows", "mixed",
        "prefill_heads")]


class cb_step(ctypes.Structure):
    _fields_ = [("num_reqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32), ("max_blocks_per_req", ctypes.c_int32),
                ("num_decode", ctypes.c_int32), ("req_ids", _i64p), ("cu_q_lens", _i32p), ("ctx_lens", _i32p),
                ("block_tables", _i32p), ("slot_mapping", _i32p), ("token_to_req", _i32p),
                ("num_evicted", ctypes.c_int32), ("num_admitted", ctypes.c_int32), ("evicted", _i64p),
                ("admitted", _i64p), ("num_preempted", ctypes.c_int32), ("preempted", _i64p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m ragged_continuous_batching_amd.build`")
    # torch ships its own HIP runtime (same soname, libamdhip64.so.7). Loading torch first
    # makes libcb.so bind to that copy, so that the process holds one HIP runtime and
    # device pointers and streams from torch are valid in the library.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    sig = {
        "cb_kv_append": (ctypes.c_int, [ctypes.POINTER(cb_shape), ctypes.POINTER(cb_batch), P, P, P, P, P]),
        "cb_ragged_attention_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(cb_shape), ctypes.POINTER(cb_batch)]),
        "cb_plan_describe": (ctypes.c_int, [ctypes.POINTER(cb_shape), ctypes.POINTER(cb_batch),
                                            ctypes.POINTER(cb_plan_info)]),
        "cb_ragged_attention": (ctypes.c_int, [ctypes.POINTER(cb_shape), ctypes.POINTER(cb_batch), P, P, P,
                                               ctypes.c_float, P, P, ctypes.c_size_t, P]),
        "cb_ragged_attention_noalloc": (ctypes.c_int, [ctypes.POINTER(cb_shape), ctypes.POINTER(cb_batch), P, P, P,
                                                       ctypes.c_float, P, P]),
        "cb_step_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(cb_shape), ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.c_int32, P, P]),
        "cb_step_forward": (ctypes.c_int, [ctypes.POINTER(cb_shape), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           P, P, P, P, P, P, P, P, ctypes.c_float, P, P, ctypes.c_size_t, P]),
        "cb_step_slots": (ctypes.c_int, [ctypes.POINTER(cb_shape), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         P, P, P, P]),
        "cb_last_error": (ctypes.c_char_p, []),
        "cb_version": (ctypes.c_char_p, []),
        "cb_debug_violations": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]),
        "cb_set_tuning": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_int32]),
        "cb_get_tuning": (ctypes.c_int, [ctypes.c_char_p, _i32p]),
        "cb_profile_enable": (ctypes.c_int, [ctypes.c_int]),
        "cb_profile_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_double), _i64p]),
        "cb_profile_launches": (ctypes.c_int, [ctypes.c_int, P, ctypes.c_int64, _i64p]),
        "cb_linear": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P, P]),
        "cb_qkv_project": (ctypes.c_int, [ctypes.POINTER(cb_shape), ctypes.POINTER(cb_batch), ctypes.c_int32, P, P,
                                          P, P, P, P]),
        "cb_profile_reset": (ctypes.c_int, []),
        "cb_profile_select": (ctypes.c_int, [ctypes.c_uint32]),
        "cb_kernel_name": (ctypes.c_char_p, [ctypes.c_int]),
        "cb_paged_read_probe_sink_words": (ctypes.c_int32, [ctypes.c_int32]),
        "cb_paged_read_probe": (ctypes.c_int, [P, ctypes.c_int32, P, P, P]),
        "cb_sched_create": (P, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P]),
        "cb_sched_add": (ctypes.c_int, [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]),
        "cb_sched_set_static": (ctypes.c_int, [P, ctypes.c_int32]),
        "cb_sched_set_preemption": (ctypes.c_int, [P, ctypes.c_int32, ctypes.c_int32]),
        "cb_sched_add_cached": (ctypes.c_int, [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32]),
        "cb_sched_build": (ctypes.c_int, [P, ctypes.POINTER(cb_step)]),
        "cb_sched_commit": (ctypes.c_int, [P, P]),
        "cb_sched_clone": (P, [P]),
        "cb_sched_destroy": (None, [P]),
        "cb_sched_stats": (ctypes.c_int, [P, _i32p, _i32p, _i32p]),
        "cb_graph_create": (ctypes.c_int, [ctypes.POINTER(cb_shape), ctypes.c_int32, P, P, P, P, P, ctypes.c_float,
                                           P, ctypes.POINTER(ctypes.c_void_p)]),
        "cb_graph_step": (ctypes.c_int, [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P, P]),
        "cb_graph_stats": (ctypes.c_int, [P, _i64p, _i64p, ctypes.POINTER(ctypes.c_size_t)]),
        "cb_graph_destroy": (None, [P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()
EXPORTED = ("cb_kv_append", "cb_ragged_attention_workspace_size", "cb_plan_describe", "cb_ragged_attention",
            "cb_ragged_attention_noalloc",
            "cb_step_workspace_size",
            "cb_step_forward", "cb_step_slots", "cb_last_error",
            "cb_version", "cb_debug_violations", "cb_set_tuning", "cb_get_tuning", "cb_profile_enable", "cb_profile_read", "cb_profile_launches",
            "cb_profile_reset", "cb_profile_select",
            "cb_kernel_name", "cb_paged_read_probe_sink_words", "cb_paged_read_probe", "cb_sched_create", "cb_sched_add", "cb_sched_add_cached", "cb_sched_build",
            "cb_sched_commit", "cb_sched_clone", "cb_sched_destroy", "cb_sched_stats", "cb_sched_set_static",
            "cb_sched_set_preemption", "cb_linear", "cb_qkv_project", "cb_graph_create", "cb_graph_step",
            "cb_graph_stats", "cb_graph_destroy")


def _check(status: int) -> int:
    if status != CB_OK:
        raise CbError(status, lib.cb_last_error().decode())
    return status


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()


def _stream(s):
    if s is None:
        try:
            import torch
            return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
        except Exception:
            return 0
    if isinstance(s, int):
        return s
    return s.cuda_stream


# ---- device entry points --------------------------------------------------------------
def cb_kv_append(shape: cb_shape, batch: cb_batch, k_new, v_new, k_cache, v_cache, stream=None) -> int:
    return _check(lib.cb_kv_append(ctypes.byref(shape), ctypes.byref(batch), _ptr(k_new), _ptr(v_new),
                                   _ptr(k_cache), _ptr(v_cache), _stream(stream)))


def cb_ragged_attention_workspace_size(shape: cb_shape, batch: cb_batch) -> int:
    return int(lib.cb_ragged_attention_workspace_size(ctypes.byref(shape), ctypes.byref(batch)))


def cb_plan_describe(shape: cb_shape, batch: cb_batch) -> dict:
    """The launch plan cb_ragged_attention would use for `batch` (host-side, no GPU)."""
    info = cb_plan_info()
    _check(lib.cb_plan_describe(ctypes.byref(shape), ctypes.byref(batch), ctypes.byref(info)))
    return {name: int(getattr(info, name)) for name, _ in cb_plan_info._fields_}


def cb_ragged_attention(shape: cb_shape, batch: cb_batch, q, k_cache, v_cache, scale: float, o, workspace,
                        workspace_bytes: int, stream=None) -> int:
    return _check(lib.cb_ragged_attention(ctypes.byref(shape), ctypes.byref(batch), _ptr(q), _ptr(k_cache),
                                          _ptr(v_cache), ctypes.c_float(scale), _ptr(o), _ptr(workspace),
                                          ctypes.c_size_t(workspace_bytes), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20        # CB_NOALLOC_SCRATCH_BYTES in cb.h


def cb_ragged_attention_noalloc(shape: cb_shape, batch: cb_batch, q, k_cache, v_cache, scale: float, o,
                                stream=None) -> int:
    """cb_ragged_attention without a workspace (the library's fixed device array)."""
    return _check(lib.cb_ragged_attention_noalloc(ctypes.byref(shape), ctypes.byref(batch), _ptr(q), _ptr(k_cache),
                                                  _ptr(v_cache), float(scale), _ptr(o), _stream(stream)))


def _host_i32(a):
    """Host int32 data as (address, owner): a ctypes int32 pointer (a built step's own arrays,
    passed through without a copy) or anything numpy turns into a contiguous int32 array."""
    if isinstance(a, _i32p):
        return ctypes.cast(a, ctypes.c_void_p).value, None
    arr = np.ascontiguousarray(a, dtype=np.int32)
    return arr.ctypes.data, arr


def cb_step_workspace_size(shape: cb_shape, num_reqs: int, num_tokens: int, max_blocks_per_req: int, h_cu_q_lens,
                           h_ctx_lens) -> int:
    (cu, _a), (ctx, _b) = _host_i32(h_cu_q_lens), _host_i32(h_ctx_lens)
    return int(lib.cb_step_workspace_size(ctypes.byref(shape), int(num_reqs), int(num_tokens), int(max_blocks_per_req),
                                          cu, ctx))


CB_SLOT_SOLE_WRITER = 1 << 30


def cb_step_slots(shape: cb_shape, num_reqs: int, num_tokens: int, max_blocks_per_req: int, h_cu_q_lens, h_ctx_lens,
                  h_block_tables) -> np.ndarray:
    """The cache slot of every packed row as the step entry points stage it (host only)."""
    (cu, _a), (ctx, _b), (bt, _c) = _host_i32(h_cu_q_lens), _host_i32(h_ctx_lens), _host_i32(h_block_tables)
    out = np.zeros(max(int(num_tokens), 0), np.int32)
    _check(lib.cb_step_slots(ctypes.byref(shape), int(num_reqs), int(num_tokens), int(max_blocks_per_req), cu, ctx,
                             bt, out.ctypes.data_as(ctypes.c_void_p)))
    return out


def cb_step_forward(shape: cb_shape, num_reqs: int, num_tokens: int, max_blocks_per_req: int, h_cu_q_lens,
                    h_ctx_lens, h_block_tables, q, k_new, v_new, k_cache, v_cache, scale: float, o, workspace,
                    workspace_bytes: int, stream=None) -> int:
    """Host metadata may be numpy arrays or the int32 pointers of a cb_step (Scheduler.build_raw)."""
    (cu, _a), (ctx, _b), (bt, _c) = _host_i32(h_cu_q_lens), _host_i32(h_ctx_lens), _host_i32(h_block_tables)
    return _check(lib.cb_step_forward(ctypes.byref(shape), int(num_reqs), int(num_tokens), int(max_blocks_per_req),
                                      cu, ctx, bt, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                      ctypes.c_float(scale), _ptr(o), _ptr(workspace),
                                      ctypes.c_size_t(workspace_bytes), _stream(stream)))


def cb_graph_create(shape: cb_shape, max_tokens: int, q, k_new, v_new, k_cache, v_cache, scale: float, o) -> int:
    """Returns the cb_graph handle (an address) bound to these buffers of max_tokens rows."""
    out = ctypes.c_void_p()
    _check(lib.cb_graph_create(ctypes.byref(shape), int(max_tokens), _ptr(q), _ptr(k_new), _ptr(v_new),
                               _ptr(k_cache), _ptr(v_cache), ctypes.c_float(scale), _ptr(o), ctypes.byref(out)))
    return out.value


def cb_graph_step(graph: int, num_reqs: int, num_tokens: int, max_blocks_per_req: int, h_cu_q_lens, h_ctx_lens,
                  h_block_tables, stream=None) -> int:
    """Host metadata as in cb_step_forward (numpy arrays or a cb_step's int32 pointers)."""
    (cu, _a), (ctx, _b), (bt, _c) = _host_i32(h_cu_q_lens), _host_i32(h_ctx_lens), _host_i32(h_block_tables)
    return _check(lib.cb_graph_step(graph, int(num_reqs), int(num_tokens), int(max_blocks_per_req), cu, ctx, bt,
                                    _stream(stream)))


def cb_graph_stats(graph: int):
    """(replays, captures, workspace_bytes)."""
    replays, captures, ws = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    _check(lib.cb_graph_stats(graph, ctypes.byref(replays), ctypes.byref(captures), ctypes.byref(ws)))
    return replays.value, captures.value, ws.value


def cb_graph_destroy(graph: int) -> None:
    lib.cb_graph_destroy(graph)


def cb_linear(M: int, N: int, K: int, a, w, c, stream=None) -> int:
    """c[M, N] = a[M, K] w[N, K]^T (bf16)."""
    return _check(lib.cb_linear(int(M), int(N), int(K), _ptr(a), _ptr(w), _ptr(c), _stream(stream)))


def cb_qkv_project(shape: cb_shape, batch: cb_batch, d_model: int, x, w_qkv, q, k_cache, v_cache,
                   stream=None) -> int:
    """QKV projection of the packed rows with the paged KV append fused in."""
    return _check(lib.cb_qkv_project(ctypes.byref(shape), ctypes.byref(batch), int(d_model), _ptr(x), _ptr(w_qkv),
                                     _ptr(q), _ptr(k_cache), _ptr(v_cache), _stream(stream)))


def cb_last_error() -> str:
    return lib.cb_last_error().decode()


def cb_version() -> str:
    return lib.cb_version().decode()


def cb_set_tuning(key: str, value: int) -> int:
    return _check(lib.cb_set_tuning(key.encode(), int(value)))


def cb_get_tuning(key: str) -> int:
    v = ctypes.c_int32(0)
    _check(lib.cb_get_tuning(key.encode(), ctypes.byref(v)))
    return int(v.value)


class tuned:
    """Context manager: sets tuning keys for the duration of a block and restores the values
    they had before (``with tuned(overlap_prefill=1): ...``)."""

    def __init__(self, **keys):
        self.keys = keys
        self.saved = {}

    def __enter__(self):
        for k, v in self.keys.items():
            self.saved[k] = cb_get_tuning(k)
            cb_set_tuning(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self.saved.items():
            cb_set_tuning(k, v)
        return False


def cb_debug_violations(reset: bool = False) -> int:
    """Out-of-pool block ids the kernels met since the last reset (debug copy built with
    --device-checks; raises CbError(CB_ERR_UNSUPPORTED) in the normal build)."""
    n = ctypes.c_uint32()
    _check(lib.cb_debug_violations(ctypes.byref(n), 1 if reset else 0))
    return n.value


def cb_profile_enable(on: bool) -> int:
    return _check(lib.cb_profile_enable(1 if on else 0))


def cb_profile_select(kernel_ids=None) -> int:
    """Times only the given kernel ids while profiling is on (None: every kernel)."""
    mask = 0
    for k in kernel_ids or ():
        mask |= 1 << int(k)
    return _check(lib.cb_profile_select(mask))


def cb_profile_launches(kernel_id: int) -> np.ndarray:
    """Per-launch durations (ms) of one kernel id, in launch order."""
    n = ctypes.c_int64()
    _check(lib.cb_profile_launches(int(kernel_id), None, 0, ctypes.byref(n)))
    out = np.zeros(n.value, dtype=np.float32)
    _check(lib.cb_profile_launches(int(kernel_id), out.ctypes.data, n.value, ctypes.byref(n)))
    return out


def cb_profile_read(kernel_id: int):
    ms = ctypes.c_double(0)
    n = ctypes.c_int64(0)
    _check(lib.cb_profile_read(int(kernel_id), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def cb_profile_reset() -> int:
    return _check(lib.cb_profile_reset())


def cb_kernel_name(kernel_id: int) -> str:
    return lib.cb_kernel_name(int(kernel_id)).decode()


def cb_paged_read_probe_sink_words(n_pages: int) -> int:
    return int(lib.cb_paged_read_probe_sink_words(int(n_pages)))


def cb_paged_read_probe(pages, n_pages: int, order, sink, stream=None) -> int:
    """Reads n_pages 4 KiB pages in the given order as the decode kernels read the cache
    (a measurement aid; device tensors in, nothing out)."""
    return _check(lib.cb_paged_read_probe(_ptr(pages), int(n_pages), _ptr(order), _ptr(sink), _stream(stream)))


# ---- host step builder ----------------------------------------------------------------
def _arr(p, n, dtype):
    if n == 0:
        return np.zeros(0, dtype=dtype)
    return np.ctypeslib.as_array(p, shape=(n,)).astype(dtype, copy=True)


class Step:
    """Copies of one built step's arrays (the library's own storage is reused next build)."""

    def __init__(self, st: cb_step):
        R, T, B = st.num_reqs, st.num_tokens, st.max_blocks_per_req
        self.num_reqs, self.num_tokens, self.max_blocks_per_req, self.num_decode = R, T, B, st.num_decode
        self.req_ids = _arr(st.req_ids, R, np.int64)
        self.cu_q_lens = _arr(st.cu_q_lens, R + 1, np.int32)
        self.ctx_lens = _arr(st.ctx_lens, R, np.int32)
        self.block_tables = _arr(st.block_tables, R * B, np.int32).reshape(R, B)
        self.slot_mapping = _arr(st.slot_mapping, T, np.int32)
        self.token_to_req = _arr(st.token_to_req, T, np.int32)
        self.evicted = _arr(st.evicted, st.num_evicted, np.int64).tolist()
        self.admitted = _arr(st.admitted, st.num_admitted, np.int64).tolist()
        self.preempted = _arr(st.preempted, st.num_preempted, np.int64).tolist()


class Scheduler:
    """Owning wrapper of a cb_sched (cb_sched_create ... cb_sched_destroy)."""

    def __init__(self, token_budget: int, block_size: int, num_blocks: int, max_num_seqs: int = 0,
                 free_list=None, _handle=None):
        if _handle is not None:
            self._h = _handle
        else:
            fl = None
            if free_list is not None:
                self._fl = np.ascontiguousarray(free_list, dtype=np.int32)
                fl = self._fl.ctypes.data
            self._h = lib.cb_sched_create(int(token_budget), int(block_size), int(num_blocks), int(max_num_seqs), fl)
            if not self._h:
                raise CbError(CB_ERR_INVALID_ARG, cb_last_error())
        self._step = cb_step()
        self.last = None

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and lib is not None:
            lib.cb_sched_destroy(h)
            self._h = None

    def add(self, req_id: int, prompt_len: int, out_len: int) -> None:
        _check(lib.cb_sched_add(self._h, int(req_id), int(prompt_len), int(out_len)))

    def set_preemption(self, enable: bool, watermark_blocks: int = 0) -> None:
        """Preemption by recompute when decode tokens do not fit the free list."""
        _check(lib.cb_sched_set_preemption(self._h, 1 if enable else 0, int(watermark_blocks)))

    def set_static(self, batch_size: int) -> None:
        """Naive padded batching of up to batch_size requests (1 = request-at-a-time)."""
        _check(lib.cb_sched_set_static(self._h, int(batch_size)))

    def add_cached(self, req_id: int, prompt_len: int, out_len: int, cached: int, generated: int) -> None:
        _check(lib.cb_sched_add_cached(self._h, int(req_id), int(prompt_len), int(out_len), int(cached),
                                       int(generated)))

    def build(self) -> Step:
        _check(lib.cb_sched_build(self._h, ctypes.byref(self._step)))
        self.last = Step(self._step)
        return self.last

    def build_raw(self) -> cb_step:
        """Builds and returns the library's own cb_step view (valid until the next call)."""
        _check(lib.cb_sched_build(self._h, ctypes.byref(self._step)))
        return self._step

    def commit(self, eos=None) -> None:
        if eos is None:
            _check(lib.cb_sched_commit(self._h, None))
        else:
            e = np.ascontiguousarray(eos, dtype=np.uint8)
            _check(lib.cb_sched_commit(self._h, e.ctypes.data))

    def clone(self) -> "Scheduler":
        h = lib.cb_sched_clone(self._h)
        if not h:
            raise CbError(CB_ERR_INVALID_ARG, "cb_sched_clone failed")
        return Scheduler(0, 0, 0, _handle=h)

    def stats(self):
        a, b, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib.cb_sched_stats(self._h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
        return a.value, b.value, c.value


# ---- helpers that assemble the ABI structs --------------------------------------------
def make_shape(num_q_heads: int, num_kv_heads: int, head_dim: int, num_blocks: int, dtype: str,
               block_size: int = 16) -> cb_shape:
    return cb_shape(num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, CB_BF16 if dtype == "bf16" else CB_F32)


class Batch:
    """A cb_batch plus the buffers it points to (kept alive here).

    Host mirrors are int32 numpy arrays; device arrays are torch int32 tensors (the torch
    copy to the device is plumbing, done with ``non_blocking`` from pinned host memory).
    """

    def __init__(self, cu_q_lens, ctx_lens, block_tables, device="cuda", stream=None):
        import torch
        self.h_cu = np.ascontiguousarray(cu_q_lens, dtype=np.int32)
        self.h_ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        if bt.ndim == 1:
            bt = bt.reshape(len(self.h_ctx), -1)
        self.h_bt = bt
        R = len(self.h_ctx)
        self.num_reqs, self.num_tokens = R, int(self.h_cu[-1]) if len(self.h_cu) else 0
        self.max_blocks = int(bt.shape[1]) if bt.ndim == 2 else 0
        pin = torch.cuda.is_available() and device != "cpu"
        host = [torch.from_numpy(a.reshape(-1).copy()) for a in (self.h_cu, self.h_ctx, self.h_bt)]
        if pin:
            host = [h.pin_memory() for h in host]
        self._host = host
        if device == "cpu":
            self.d_cu, self.d_ctx, self.d_bt = host
        else:
            self.d_cu, self.d_ctx, self.d_bt = (h.to(device, non_blocking=True) for h in host)
        self.struct = cb_batch(R, self.num_tokens, self.max_blocks, self.d_cu.data_ptr(), self.d_ctx.data_ptr(),
                               self.d_bt.data_ptr() if self.d_bt.numel() else self.d_cu.data_ptr(),
                               self.h_cu.ctypes.data, self.h_ctx.ctypes.data)

    @classmethod
    def from_step(cls, step: Step, device="cuda"):
        return cls(step.cu_q_lens, step.ctx_lens, step.block_tables, device=device)
