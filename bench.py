"""Benchmark: one step of the ragged continuous-batching hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline]

A step is the whole path over one batch: host batch build (a fresh copy of the scheduler
state, decode first, chunks up to m, block allocation), the metadata upload, cb_kv_append,
cb_ragged_attention (prefill MFMA tiles, split-K decode, combine), and the commit. Inputs
(Q, new K/V, the cached history) are resident in HBM before timing starts. The default
workload is the Llama-2-7B-shaped mixed step: Hq = Hkv = 32, D = 128, bf16, m = 2048,
64 decodes with contexts U{512..4096} plus two 992-token chunks (contexts 0 and 1024).

Prints one JSON line. ``roofline`` describes the dominant kernel: average duration from
hipEvents recorded by the library on the kernel's own stream during the timed steps, and
algorithmic bytes (each visible K/V position read once, Q read once, O written once) or
algorithmic flops (unmasked pairs only). ``traffic`` comes from the committed rocprofv3
counter summary of that kernel (profiles/*_pmc.json) and is null when the kernel's code
(comments aside) has changed since the counters were taken. ``cpu_baseline`` times the fp64 oracle on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6     # 256 CU x 4096 FLOP/clk x 2.4 GHz (dense)
PROFILE_STEPS = 10            # untimed steps that time every kernel of a fixed step


def algorithmic(wl, step):
    """Bytes and flops the method must move/compute for this step (per launch)."""
    import numpy as np
    e = 2 if wl.dtype == "bf16" else 4
    q = np.diff(step.cu_q_lens).astype(np.int64)
    c = step.ctx_lens.astype(np.int64)
    L = c + q
    hkv, hq, d = wl.num_kv_heads, wl.num_q_heads, wl.head_dim
    dec = q == 1
    out = {}
    for name, m in (("all", np.ones_like(dec)), ("decode", dec), ("prefill", ~dec)):
        out[name] = {
            "bytes": int(e * (2 * (L[m] * hkv * d).sum() + 2 * q[m].sum() * hq * d)),
            "flops": int(4 * d * hq * (q[m] * c[m] + q[m] * (q[m] + 1) // 2).sum()),
            "tokens": int(q[m].sum()),
        }
    out["append_bytes"] = int(4 * e * q.sum() * hkv * d)
    return out


def code_text(src):
    """C/C++ source without comments and blank lines: what the compiler sees of it."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(line.rstrip() for line in src.splitlines() if line.strip())


def source_sha(*names):
    """Hash of the code (comments ignored) of the named csrc files."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "ragged_continuous_batching_amd", "csrc", n), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


# a kernel's traffic depends on its code and on the work lists the planner gives it
KERNEL_SOURCES = {"row_attn_kernel": ("attn_rows.hip", "cb_device.h", "cb_plan.h", "plan.cpp"),
                  "row_attn_mfma_kernel": ("attn_decode_gqa.hip", "attn_decode_gqa.h", "cb_device.h", "cb_plan.h",
                                           "plan.cpp"),
                  "prefill_kernel": ("attn_prefill.hip", "attn_prefill.h", "cb_device.h", "cb_plan.h", "plan.cpp")}


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary
    profiles/<kernel>_<workload>_pmc.json, or None if it is absent or the kernel's sources
    have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_sha(*KERNEL_SOURCES[kernel]):
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def _oracle_sample(wl, step, budget_s):
    """(rows done, requests done, seconds): the fp64 oracle over the step's requests in
    packed order, one call per request including the gathering of its inputs, until the
    budget is spent."""
    import numpy as np
    import workloads as W
    from oracle import attention as A
    t_start = time.perf_counter()
    done_tokens, done_reqs = 0, 0
    for i in range(step.num_reqs):
        rid, c = int(step.req_ids[i]), int(step.ctx_lens[i])
        s, e = int(step.cu_q_lens[i]), int(step.cu_q_lens[i + 1])
        pos = c + np.arange(e - s)
        keys = wl.values(W.KIND_K, rid, np.arange(c + e - s))
        vals = wl.values(W.KIND_V, rid, np.arange(c + e - s))
        q = wl.values(W.KIND_Q, rid, pos)
        A.attend(q, keys, vals, pos, wl.scale)
        done_tokens += e - s
        done_reqs += 1
        if time.perf_counter() - t_start > budget_s:
            break
    return done_tokens, done_reqs, time.perf_counter() - t_start


def cpu_baseline(wl, step, budget_s=25.0, one_thread_budget_s=15.0):
    """Times the fp64 oracle on this step's rows (all of them if they fit the budget, else
    the largest prefix of requests in packed order that does), once with the BLAS threads
    numpy has (all host cores the process may use) and once on one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    wl.raw_pool(0)                               # the value pools are built before timing
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])

    def sample_text(tokens, reqs):
        return (f"all {step.num_reqs} requests ({step.num_tokens} rows) of the step" if reqs == step.num_reqs
                else f"first {reqs} of {step.num_reqs} requests ({tokens} of {step.num_tokens} rows)")
    tokens, reqs, dt = _oracle_sample(wl, step, budget_s)
    with threadpool_limits(1):
        tokens1, reqs1, dt1 = _oracle_sample(wl, step, one_thread_budget_s)
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": sample_text(tokens, reqs) + ", fp64 numpy, one call per request incl. gathering inputs",
            "seconds": round(dt, 3), "cpu_model": cpu_model(), "host_cores_visible": len(os.sched_getaffinity(0)),
            "one_thread": {"value": round(tokens1 / dt1, 1), "unit": "tokens/s", "cores": 1,
                           "sample": sample_text(tokens1, reqs1), "seconds": round(dt1, 3)}}


def launch_step(cb, run, st, q, k_new, v_new, o, ws, stream):
    """Append + attention of one built step through the single-call entry point."""
    T = st.num_tokens
    cb.cb_step_forward(run.shape, st.num_reqs, T, st.max_blocks_per_req, st.cu_q_lens, st.ctx_lens,
                       st.block_tables, q[:T], k_new[:T], v_new[:T], run.k_cache, run.v_cache, run.wl.scale,
                       o[:T], ws, ws.numel(), stream)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=None, choices=[2, 3, 4, 5],
                    help="one workload only: 2 mixed step, 3 decode-only GQA, 4 chunked prefill, 5 the 500-step "
                         "scheduler trace (steps = trace steps after the warm-up). Default: config 2 is the "
                         "headline and configs 3, 4 and 5 are reported under 'configs' in the same line")
    ap.add_argument("--no-subconfigs", action="store_true",
                    help="default run: report config 2 only (no 'configs' sub-results)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--api", choices=["fused", "split"], default="fused",
                    help="fused: one cb_step_forward call per step (one metadata upload); split: Batch upload + "
                         "cb_kv_append + cb_ragged_attention")
    ap.add_argument("--compare-policies", action="store_true",
                    help="offline throughput of the first --requests requests of the config-5 trace under "
                         "continuous batching, naive padded batching (batch 32 and 8) and request-at-a-time, "
                         "all through the same kernels")
    ap.add_argument("--requests", type=int, default=256)
    ap.add_argument("--compare-policies-trace", action="store_true",
                    help="the config-5 trace itself (500 steps, the same Poisson arrivals) under continuous "
                         "batching, naive padded batching (32, 8) and request-at-a-time: generated tokens/s "
                         "and the pad and idle rows each policy processes")
    ap.add_argument("--layer", action="store_true",
                    help="config 2 with the token-wise projections around attention (Llama-2-7B shapes, "
                         "d_model 4096, synthetic bf16 weights): fused QKV projection + paged append, "
                         "ragged attention, output projection")
    ap.add_argument("--pool-blocks", type=int, default=0,
                    help="config 5 only: a KV pool of this many blocks with preemption by recompute "
                         "(0 = the configured pool, which never fills)")
    ap.add_argument("--watermark", type=int, default=0, help="blocks kept free at admission with --pool-blocks")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step as a captured HIP graph (cb_graph_step, T-bucketed); value is the "
                         "graph's rate and the roofline kernel durations come from the eager pass of the same run "
                         "(configs 2-4); with --config 5 the whole trace replays through graphs")
    ap.add_argument("--long-chunk", type=int, default=0, metavar="N",
                    help="instead of a config: one 256-row prefill chunk after N cached tokens (a late chunk "
                         "of a long prompt; Hq = Hkv = 32, D = 128, bf16), the case where prefill tiles are "
                         "split over key ranges")
    ap.add_argument("--tune", action="append", default=[], metavar="KEY=VALUE",
                    help="cb_set_tuning(KEY, VALUE) before the run (repeatable)")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time the steps without the library's per-kernel timing events (config 5: no "
                         "per-kernel durations or roofline; fixed steps: the dominant kernel's duration "
                         "comes from the untimed profiled steps)")
    ap.add_argument("--all-kernel-events", action="store_true",
                    help="config 5: an event pair around every kernel of the timed steps (default: only "
                         "around the launches that stream the cache)")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip timing the paged read probe (the attainable rate reported beside HBM rooflines)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain elementwise copy of 512 MiB (read 512 MiB, write 512 MiB) three "
                         "times, so that counter runs can scale FETCH_SIZE/WRITE_SIZE by a known size")
    args = ap.parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the multi-GPU design is described but not built.", file=sys.stderr)
        return 2

    import torch

    from ragged_continuous_batching_amd import cb

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    for kv in args.tune:
        key, val = kv.split("=")
        cb.cb_set_tuning(key, int(val))
    if args.compare_policies:
        return bench_policies(args)
    if args.compare_policies_trace:
        return bench_policies_trace(args)
    if args.layer:
        return bench_layer(args)
    if args.copy_calibration:
        src = torch.ones(1 << 27, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    rate = None if args.no_read_probe else paged_read_rate()
    if args.config == 5:
        result = bench_trace(args)
    elif args.config is not None or args.long_chunk:
        result = bench_fixed(args, args.config or 0)
    else:
        result = bench_fixed(args, 2)
        if not args.no_subconfigs:
            result["configs"] = {}
            for c in (3, 4):
                release_device_memory()
                result["configs"][str(c)] = sub_result(bench_fixed(args, c, cpu_budget_s=5.0))
            release_device_memory()
            result["configs"]["5"] = sub_result(bench_trace(args, trace_window=True))
    if rate is not None:
        add_attainable(result, rate)
    print(json.dumps(result), flush=True)
    return 0


def paged_read_rate(n_pages=1 << 19, reps=5, per_rep=4):
    """GB/s at which this GPU reads 4 KiB pages in a random order with the decode kernels'
    loads (cb_paged_read_probe over 2 GiB, a seeded permutation). Each timed repetition is
    `per_rep` back-to-back launches between two torch events, enqueued behind a launch that
    keeps the GPU busy, so the host's launch overhead never shows as idle time between the
    events; the best of `reps` repetitions after a warm-up."""
    import torch

    from ragged_continuous_batching_amd import cb
    pages = torch.ones(n_pages * 4096, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(12345)
    order = torch.randperm(n_pages, generator=g, device="cuda", dtype=torch.int32)
    sink = torch.zeros(cb.cb_paged_read_probe_sink_words(n_pages), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def probe():
        cb.cb_paged_read_probe(pages, n_pages, order, sink, stream.cuda_stream)

    best = float("inf")
    for i in range(reps + 1):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        probe()                                   # keeps the GPU busy while the rest is enqueued
        t0.record(stream)
        for _ in range(per_rep):
            probe()
        t1.record(stream)
        t1.synchronize()
        if i >= 1:
            best = min(best, t0.elapsed_time(t1) / per_rep)
    del pages, order, sink
    release_device_memory()
    return n_pages * 4096 / (best * 1e-3) / 1e9


def add_attainable(result, rate):
    """Puts the decode kernels' bandwidth beside the probe's paged read rate."""
    for r in [result] + list(result.get("configs", {}).values()):
        roof = r.get("roofline")
        if isinstance(roof, dict) and roof.get("bound") == "hbm" and roof.get("achieved"):
            roof["attainable"] = round(rate, 1)
            roof["frac_of_attainable"] = round(roof["achieved"] / rate, 4)
    result["attainable_read"] = {"value": round(rate, 1), "unit": "GB/s",
                                 "probe": "cb_paged_read_probe: 2 GiB of 4 KiB pages in a seeded random order, "
                                          "non-temporal 16-byte loads as the decode kernels issue them; best of 5 "
                                          "repetitions of 4 back-to-back launches"}


def release_device_memory():
    import gc
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


SUB_KEYS = ("config", "steps", "warmup", "ms_per_step", "value", "unit", "device_ms_per_step", "roofline",
            "kernels", "cpu_baseline", "window", "kernels_all", "prefill_roofline")


def sub_result(r):
    """The fields of another workload's result that go into the headline line."""
    return {k: r[k] for k in SUB_KEYS if k in r}


def bench_fixed(args, cfg, cpu_budget_s=25.0):
    """One fixed step (configs 2-4, or the late chunk when cfg = 0), rebuilt from the same
    scheduler state every step. Returns the result dict."""
    import numpy as np
    import torch

    import workloads as W
    from ragged_continuous_batching_amd import cb
    from ragged_continuous_batching_amd.runner import DeviceRun

    names = {2: "llama2-7b-shaped mixed step (64 decodes + 2x992 prefill chunks)",
             3: "decode-only GQA (256 decodes, lognormal contexts)",
             4: "chunked-prefill-heavy (4x2048-token chunks)"}
    if cfg == 0:
        n = args.long_chunk
        wl = W.custom([W.Request(0, n + 256, 1 << 20, cached=n, generated=0)], num_q_heads=32, num_kv_heads=32,
                      head_dim=128, dtype="bf16", seed=1006, token_budget=256)
        names[0] = f"late chunk of a long prompt (256 rows after {n} cached tokens, Hq=Hkv=32, D=128)"
    else:
        wl = W.config(cfg)
    run = DeviceRun(wl, stale=None)
    base = run.sched
    # setup: write the cached history once (not timed)
    probe = base.clone()
    step0 = probe.build()
    run.write_history(step0)
    del probe
    q, k_new, v_new = run.step_inputs(step0)
    torch.cuda.synchronize()
    alg = algorithmic(wl, step0)
    T = step0.num_tokens
    o = torch.empty_like(q)
    ws_bytes = max(cb.cb_ragged_attention_workspace_size(run.shape, cb.Batch.from_step(step0).struct),
                   cb.cb_step_workspace_size(run.shape, step0.num_reqs, T, step0.max_blocks_per_req,
                                             step0.cu_q_lens, step0.ctx_lens))
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    host_ms = []

    def one_step():
        t0 = time.perf_counter()
        s = base.clone()
        if args.api == "fused":
            st = s.build_raw()           # the library's own arrays, no copies
            host_ms.append((time.perf_counter() - t0) * 1e3)
            launch_step(cb, run, st, q, k_new, v_new, o, ws, stream)
            s.commit()
            return s
        st = s.build()
        batch = cb.Batch.from_step(st)
        host_ms.append((time.perf_counter() - t0) * 1e3)
        cb.cb_kv_append(run.shape, batch.struct, k_new, v_new, run.k_cache, run.v_cache, stream)
        cb.cb_ragged_attention(run.shape, batch.struct, q, run.k_cache, run.v_cache, wl.scale, o, ws, ws.numel(),
                               stream)
        s.commit()
        return batch, st

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    # Every kernel's time, from untimed steps with an event pair around each launch. Inside
    # the timed steps only the dominant kernel carries events (each pair costs the stream
    # about a microsecond or two).
    cb.cb_profile_reset()
    cb.cb_profile_select(None)
    cb.cb_profile_enable(True)
    for _ in range(PROFILE_STEPS):
        one_step()
    torch.cuda.synchronize()
    cb.cb_profile_enable(False)
    kernels = {}
    for name, kid in cb.KERNELS.items():
        ms, n = cb.cb_profile_read(kid)
        if n:
            kernels[name] = {"avg_us": round(ms * 1e3 / n, 2), "launches": n, "timed_steps": False}
    cb.cb_profile_reset()
    dominant = "prefill" if cfg in (0, 4) else "decode"
    if dominant == "decode" and "mixed" in kernels:
        dominant = "mixed"                 # prefill tiles and decode waves in one launch

    host_ms.clear()
    cb.cb_profile_select([cb.KERNELS[dominant]])
    cb.cb_profile_enable(not args.no_kernel_events)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    keep = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        keep.append(one_step())
        if len(keep) > 4:
            keep.pop(0)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cb.cb_profile_enable(False)
    cb.cb_profile_select(None)
    ms_per_step = wall * 1e3 / args.steps
    device_ms = ev0.elapsed_time(ev1) / args.steps
    ms, n = cb.cb_profile_read(cb.KERNELS[dominant])
    if n:
        kernels[dominant] = {"avg_us": round(ms * 1e3 / n, 2), "launches": n, "timed_steps": True}
    cb.cb_profile_reset()

    avg_s = kernels[dominant]["avg_us"] * 1e-6
    if dominant == "mixed":
        achieved = alg["all"]["bytes"] / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "mfma_frac": round(alg["prefill"]["flops"] / avg_s / 1e12 / BF16_PEAK_TFLOPS, 4)}
    elif dominant == "decode":
        achieved = alg["decode"]["bytes"] / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = alg["prefill"]["flops"] / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    roof["kernel"] = cb.cb_kernel_name(cb.KERNELS[dominant])
    if dominant == "decode" and wl.dtype == "bf16" and wl.num_q_heads // wl.num_kv_heads >= 4:
        roof["kernel"] = "row_attn_mfma_kernel"        # grouped-query decode runs on the matrix cores
    roof["traffic"] = measured_traffic(roof["kernel"], f"config{cfg}")

    result = {
        "metric": "ragged-attention tokens/s per step",
        "value": round(T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": names[cfg], "num_tokens": T, "num_reqs": step0.num_reqs,
                   "num_decode": step0.num_decode, "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "block_size": wl.block_size, "token_budget": wl.token_budget,
                   "seed": wl.seed, "api": args.api},
        "roofline": roof,
        "device_ms_per_step": round(device_ms, 4),
        "host_build_ms_per_step": round(float(np.mean(host_ms)), 4),
        "kernels": kernels,
        "kernel_events": (f"{dominant}: event pairs inside the timed steps; other kernels: "
                          f"{PROFILE_STEPS} untimed steps with an event pair around every launch"),
        "algorithmic": alg,
        "attention_tokens_per_s": round(T / (sum(kernels[k]["avg_us"] for k in kernels if k != "append") * 1e-6), 1),
    }
    if dominant == "decode" and "prefill" in kernels and alg["prefill"]["flops"] > 0:
        # the prefill rows of a decode-dominated step, timed alone: their own MFMA fraction
        pre_s = kernels["prefill"]["avg_us"] * 1e-6
        pre_tf = alg["prefill"]["flops"] / pre_s / 1e12
        result["prefill_roofline"] = {"bound": "mfma", "achieved": round(pre_tf, 1), "peak": BF16_PEAK_TFLOPS,
                                      "unit": "TFLOP/s", "frac": round(pre_tf / BF16_PEAK_TFLOPS, 4),
                                      "kernel": "prefill_kernel", "timed_steps": kernels["prefill"]["timed_steps"]}
    if args.graph:
        result["eager"] = {"value": result["value"], "ms_per_step": result["ms_per_step"],
                           "device_ms_per_step": result["device_ms_per_step"]}
        result.update(bench_graph_step(args, cb, run, base, q, k_new, v_new, o, stream))
        result["config"]["api"] = "graph"
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, step0, budget_s=cpu_budget_s,
                                              one_thread_budget_s=min(15.0, cpu_budget_s))
    del run, q, k_new, v_new, o, ws
    return result


def bench_graph_step(args, cb, run, base, q, k_new, v_new, o, stream):
    """The same step through a captured graph (bucket = T): warm-up, then K timed steps of
    clone + build + cb_graph_step + commit, after the same loop through cb_step_forward with
    kernel timing off (the fair eager comparison). Returns the fields that replace the eager
    ones."""
    import torch
    from ragged_continuous_batching_amd.runner import GraphSteps

    gs = GraphSteps(run, q, k_new, v_new, o, min_bucket=q.shape[0])
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")

    def one_graph():
        s = base.clone()
        st = s.build_raw()
        gs.step(st, stream)
        s.commit()
        return s

    def one_eager():
        s = base.clone()
        st = s.build_raw()
        need = cb.cb_step_workspace_size(run.shape, st.num_reqs, st.num_tokens, st.max_blocks_per_req,
                                         st.cu_q_lens, st.ctx_lens)
        nonlocal ws
        if ws.numel() < need:
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        launch_step(cb, run, st, q, k_new, v_new, o, ws, stream)
        s.commit()
        return s

    def timed(one):
        for _ in range(max(args.warmup, 2)):
            one()
        torch.cuda.synchronize()
        keep = []
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            keep.append(one())
            if len(keep) > 4:
                keep.pop(0)
        ev1.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps, ev0.elapsed_time(ev1) / args.steps

    try:
        eager_ms, _ = timed(one_eager)           # the same entry point with kernel timing off
        ms, dev_ms = timed(one_graph)
        stats = gs.stats()
    finally:
        gs.close()
    T = q.shape[0]
    return {"value": round(T / (ms * 1e-3), 1), "ms_per_step": round(ms, 4), "device_ms_per_step": round(dev_ms, 4),
            "graph": {"api": "graph", "buckets": {str(b): {"replays": r, "captures": c, "workspace_bytes": w}
                                                   for b, (r, c, w) in stats.items()},
                      "eager_ms_per_step_without_kernel_events": round(eager_ms, 4),
                      "roofline_from": "kernel events of the eager pass of this run (same kernels, same plan)"}}


TRACE_WINDOW_WARMUP = 5          # the trace's timed window as a sub-result: steps 5..499


def bench_trace(args, trace_window=False):
    """Scheduler-trace replay (Hq=64, Hkv=8, m=4096, Poisson(8) arrivals, 500 steps): every
    step is built by the step builder, appended and attended. Step inputs come from fixed
    synthetic Q/K/V buffers of m rows resident in HBM (values do not change the work).
    trace_window: time steps 5..499 whatever --steps/--warmup say (the sub-result of the
    default run). Returns the result dict."""
    import numpy as np
    import torch

    import workloads as W
    from ragged_continuous_batching_amd import cb
    from ragged_continuous_batching_amd.runner import DeviceRun

    wl = W.config(5)
    total_steps = wl.steps
    if trace_window:
        warm, steps = TRACE_WINDOW_WARMUP, total_steps - TRACE_WINDOW_WARMUP
    else:
        warm = min(args.warmup, total_steps - 1)
        steps = min(args.steps if args.steps != 50 else total_steps - warm, total_steps - warm)
    cpu_step_index = warm + steps // 2          # the oracle is timed on this step's batch
    sched = None
    if args.pool_blocks:
        sched = cb.Scheduler(wl.token_budget, wl.block_size, args.pool_blocks, wl.max_num_seqs)
        sched.set_preemption(True, args.watermark)
    run = DeviceRun(wl, stale=None, sched=sched)
    g = torch.Generator(device="cuda").manual_seed(wl.seed)
    m = wl.token_budget
    q = torch.randn(m, wl.num_q_heads, wl.head_dim, device="cuda", generator=g).to(torch.bfloat16)
    k_new = torch.randn(m, wl.num_kv_heads, wl.head_dim, device="cuda", generator=g).to(torch.bfloat16)
    v_new = torch.randn(m, wl.num_kv_heads, wl.head_dim, device="cuda", generator=g).to(torch.bfloat16)
    o = torch.empty_like(q)
    # dry run of the schedule on a copy: the largest workspace any step needs
    dry = run.sched.clone()
    need, alg_dec_bytes, alg_pre_bytes, both, tokens, preempted, alg_pre_flops = 0, [], [], [], [], [], []
    for kstep in range(total_steps):
        for r in wl.arrivals[kstep]:
            dry.add(r.req_id, r.prompt_len, r.out_len)
        st = dry.build()
        preempted.append(len(st.preempted))
        b = cb.cb_batch(st.num_reqs, st.num_tokens, st.max_blocks_per_req, 256, 256, 256,
                        st.cu_q_lens.ctypes.data, st.ctx_lens.ctypes.data)
        need = max(need, cb.cb_ragged_attention_workspace_size(run.shape, b),
                   cb.cb_step_workspace_size(run.shape, st.num_reqs, st.num_tokens, st.max_blocks_per_req,
                                             st.cu_q_lens, st.ctx_lens))
        alg = algorithmic(wl, st)
        alg_dec_bytes.append(alg["decode"]["bytes"])
        alg_pre_bytes.append(alg["prefill"]["bytes"])
        alg_pre_flops.append(alg["prefill"]["flops"])
        both.append(alg["decode"]["tokens"] > 0 and alg["prefill"]["tokens"] > 0)
        tokens.append(st.num_tokens)
        if kstep == cpu_step_index:
            cpu_step = st
        dry.commit()
    del dry
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sched = run.sched
    gs = None
    if args.graph:
        from ragged_continuous_batching_amd.runner import GraphSteps
        gs = GraphSteps(run, q, k_new, v_new, o, min_bucket=256)

    def one(kstep, sched=sched):
        for r in wl.arrivals[kstep]:
            sched.add(r.req_id, r.prompt_len, r.out_len)
        if gs is not None:
            st = sched.build_raw()
            T = st.num_tokens
            gs.step(st, stream)
            sched.commit()
            return None, T
        if args.api == "fused":
            st = sched.build_raw()
            T = st.num_tokens
            launch_step(cb, run, st, q, k_new, v_new, o, ws, stream)
            sched.commit()
            return None, T
        st = sched.build()
        T = st.num_tokens
        batch = cb.Batch.from_step(st)
        cb.cb_kv_append(run.shape, batch.struct, k_new, v_new, run.k_cache, run.v_cache, stream)
        cb.cb_ragged_attention(run.shape, batch.struct, q, run.k_cache, run.v_cache, wl.scale, o, ws, ws.numel(),
                               stream)
        sched.commit()
        return batch, T

    for kstep in range(warm):
        one(kstep)
    torch.cuda.synchronize()
    # the scheduler state at the start of the window, for a second (profiled) pass over it
    profile_pass = not (args.no_kernel_events or args.all_kernel_events or gs is not None or args.api != "fused")
    window_start = sched.clone() if profile_pass else None
    cb.cb_profile_reset()
    # Only the launches that stream the cache carry events in the timed steps (each event
    # pair costs the stream about a microsecond or two), unless every kernel is asked for.
    cb.cb_profile_select(None if args.all_kernel_events else [cb.KERNELS["decode"], cb.KERNELS["mixed"]])
    cb.cb_profile_enable(not args.no_kernel_events)
    keep = []
    t0 = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for kstep in range(warm, warm + steps):
        keep.append(one(kstep))
        if len(keep) > 4:
            keep.pop(0)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cb.cb_profile_enable(False)
    cb.cb_profile_select(None)
    kernels = {}
    for name, kid in cb.KERNELS.items():
        ms, n = cb.cb_profile_read(kid)
        if n:
            kernels[name] = {"avg_us": round(ms * 1e3 / n, 2), "launches": n, "total_ms": round(ms, 3)}
    # Per-step efficiency of the launch that streams the cache: the decode kernel, or the
    # mixed launch (prefill tiles and decode waves together; its bytes are both parts') when
    # the step has both kinds of rows and the mixed launch is on.
    mixed = "mixed" in kernels
    dec_ms = [float(x) for x in cb.cb_profile_launches(cb.KERNELS["decode"])]
    mix_ms = [float(x) for x in cb.cb_profile_launches(cb.KERNELS["mixed"])]
    step_bytes, step_ms = [], []
    per_step = None
    for k in range(warm, warm + steps):
        if mixed and both[k]:
            if mix_ms:
                step_bytes.append(alg_dec_bytes[k] + alg_pre_bytes[k])
                step_ms.append(mix_ms.pop(0))
        elif alg_dec_bytes[k] > 0 and dec_ms:
            step_bytes.append(alg_dec_bytes[k])
            step_ms.append(dec_ms.pop(0))
    if step_ms and not dec_ms and not mix_ms:
        eff = np.array(step_bytes, dtype=np.float64) / (np.array(step_ms, dtype=np.float64) * 1e-3) / (HBM_PEAK_GBS * 1e9)
        per_step = {"p10": round(float(np.percentile(eff, 10)), 4), "p50": round(float(np.percentile(eff, 50)), 4),
                    "p90": round(float(np.percentile(eff, 90)), 4),
                    "share_of_steps_at_or_above_0.70": round(float((eff >= 0.70).mean()), 4),
                    "steps": int(len(eff))}
    cb.cb_profile_reset()
    if profile_pass:
        # The same window again from the same scheduler state, with an event pair around every
        # kernel (not part of the timed rate): each kernel's share of the step and the prefill
        # kernel's MFMA fraction over the window.
        cb.cb_profile_select(None)
        cb.cb_profile_enable(True)
        for kstep in range(warm, warm + steps):
            one(kstep, window_start)
        torch.cuda.synchronize()
        cb.cb_profile_enable(False)
        all_kernels = {}
        for name, kid in cb.KERNELS.items():
            ms, n = cb.cb_profile_read(kid)
            if n:
                all_kernels[name] = {"avg_us": round(ms * 1e3 / n, 2), "launches": n, "total_ms": round(ms, 3)}
        cb.cb_profile_reset()
    else:
        all_kernels = kernels if args.all_kernel_events else None
    prefill_roof = None
    if all_kernels and "prefill" in all_kernels:
        pre_tflops = sum(alg_pre_flops[warm:warm + steps]) / (all_kernels["prefill"]["total_ms"] * 1e-3) / 1e12
        prefill_roof = {"bound": "mfma", "achieved": round(pre_tflops, 1), "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(pre_tflops / BF16_PEAK_TFLOPS, 4), "kernel": "prefill_kernel",
                        "flops_over_window": int(sum(alg_pre_flops[warm:warm + steps]))}
    T_total = int(sum(tokens[warm:warm + steps]))
    dec_bytes = int(sum(alg_dec_bytes[warm:warm + steps]))
    graph_stats = None
    if gs is not None:
        graph_stats = {str(b): {"replays": r, "captures": c, "workspace_bytes": w} for b, (r, c, w) in gs.stats().items()}
        gs.close()
    roofline = None
    if step_ms:
        achieved = sum(step_bytes) / (sum(step_ms) * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "kernel": "mixed_attn_kernel + row_attn_mfma_kernel" if mixed else "row_attn_mfma_kernel",
                    "traffic": None, "per_step_frac": per_step}
    result = {
        "metric": "ragged-attention tokens/s per step",
        "value": round(T_total / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(wall * 1e3 / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "scheduler-trace replay (500 steps, Poisson(8) arrivals, lognormal prompts, "
                               "geometric outputs)", "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "token_budget": m,
                   "num_blocks": args.pool_blocks or wl.num_blocks, "seed": wl.seed,
                   "tokens_timed": T_total, "api": "graph" if gs is not None else args.api,
                   "preemptions_timed": int(sum(preempted[warm:warm + steps])),
                   "watermark": args.watermark if args.pool_blocks else None},
        "roofline": roofline,
        "device_ms_per_step": round(ev0.elapsed_time(ev1) / steps, 4),
        "kernels": kernels,
    }
    result["window"] = f"trace steps {warm}..{warm + steps - 1} timed (steps 0..{warm - 1} warm up)"
    if all_kernels is not None and profile_pass:
        result["kernels_all"] = all_kernels
        result["kernels_all_note"] = ("a second pass over the same window with an event pair around every "
                                      "kernel (not timed for the rate)")
    if prefill_roof is not None:
        result["prefill_roofline"] = prefill_roof
    if roofline is not None:
        roofline["traffic"] = measured_traffic(roofline["kernel"], f"config5_steps{warm}-{warm + steps - 1}")
    if graph_stats is not None:
        result["graph"] = {"buckets": graph_stats,
                           "roofline": "null: kernels inside a graph carry no per-kernel events"}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, cpu_step, budget_s=5.0, one_thread_budget_s=5.0)
        result["cpu_baseline"]["sample"] += f" (trace step {cpu_step_index})"
    del run, q, k_new, v_new, o, ws
    return result


def bench_layer(args):
    """One attention layer step on config 2's batch: x [T, 4096] -> cb_qkv_project (Q, and
    K/V straight into the paged cache) -> cb_ragged_attention -> cb_linear (output
    projection). The cached history is written beforehand (not timed). Throughput = rows / s;
    the roofline line is the QKV projection (the dominant GEMM), bf16 MFMA bound."""
    import numpy as np
    import torch

    import workloads as W
    from ragged_continuous_batching_amd import cb
    from ragged_continuous_batching_amd.runner import DeviceRun

    d_model = 4096
    wl = W.config(2)
    run = DeviceRun(wl, stale=None)
    base = run.sched
    probe = base.clone()
    step0 = probe.build()
    run.write_history(step0)
    del probe
    T = step0.num_tokens
    hq, hkv, d = wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    n_qkv = (hq + 2 * hkv) * d

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

    w_qkv = dev_bf16(W.layer_weights(wl.seed, 0, n_qkv, d_model))
    w_o = dev_bf16(W.layer_weights(wl.seed, 1, d_model, hq * d))
    owner = step0.token_to_req
    rids = step0.req_ids[owner]
    pos = step0.ctx_lens[owner] + (np.arange(T) - step0.cu_q_lens[owner])
    x = dev_bf16(W.bf16_bits_from_f32(wl.x_values(rids, pos, d_model)))
    q = torch.empty(T, hq, d, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    y = torch.empty(T, d_model, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(cb.cb_ragged_attention_workspace_size(run.shape, cb.Batch.from_step(step0).struct), 256),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    keep = []

    def one_step():
        s = base.clone()
        st = s.build()
        batch = cb.Batch.from_step(st)
        cb.cb_qkv_project(run.shape, batch.struct, d_model, x, w_qkv, q, run.k_cache, run.v_cache, stream)
        cb.cb_ragged_attention(run.shape, batch.struct, q, run.k_cache, run.v_cache, wl.scale, o, ws, ws.numel(),
                               stream)
        cb.cb_linear(T, d_model, hq * d, o.reshape(T, -1), w_o, y, stream)
        s.commit()
        keep.append(batch)
        if len(keep) > 4:
            keep.pop(0)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    cb.cb_profile_reset()
    cb.cb_profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cb.cb_profile_enable(False)
    gemm_ms = cb.cb_profile_launches(cb.KERNELS["gemm"])
    qkv_us = float(np.mean(gemm_ms[0::2])) * 1e3
    out_us = float(np.mean(gemm_ms[1::2])) * 1e3
    kernels = {}
    for name, kid in cb.KERNELS.items():
        ms, n = cb.cb_profile_read(kid)
        if n:
            kernels[name] = {"avg_us": round(ms * 1e3 / n, 2), "launches": n}
    cb.cb_profile_reset()
    qkv_flops = 2.0 * T * d_model * n_qkv
    out_flops = 2.0 * T * (hq * d) * d_model
    achieved = qkv_flops / (qkv_us * 1e-6) / 1e12
    ms_per_step = wall * 1e3 / args.steps
    result = {
        "metric": "attention-layer tokens/s per step (QKV projection + attention + output projection)",
        "value": round(T / (ms_per_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (random bf16 weights, N(0, 1/fan_in))",
        "config": {"workload": "llama2-7b-shaped attention layer on the mixed step (64 decodes + 2x992 chunks)",
                   "num_tokens": T, "d_model": d_model, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "kernel": "gemm_bt_kernel (QKV projection)",
                     "traffic": None},
        "gemm_us": {"qkv_projection": round(qkv_us, 2), "output_projection": round(out_us, 2),
                    "output_projection_tflops": round(out_flops / (out_us * 1e-6) / 1e12, 1)},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        from oracle import layer as LY
        rows = 64                                        # a bounded sample of the step's rows
        xs = W.f32_from_bf16_bits(W.bf16_bits_from_f32(wl.x_values(rids[:rows], pos[:rows], d_model)))
        wq = W.f32_from_bf16_bits(W.layer_weights(wl.seed, 0, n_qkv, d_model))
        t1 = time.perf_counter()
        LY.linear(xs, wq)
        dt = time.perf_counter() - t1
        result["cpu_baseline"] = {"value": round(rows / dt, 1), "unit": "tokens/s (QKV projection only)",
                                  "cores": os.cpu_count(), "kind": "oracle",
                                  "sample": f"fp64 QKV projection of the first {rows} rows"}
    print(json.dumps(result), flush=True)
    return 0


def bench_policies(args):
    """The baselines the pages compare continuous batching with, on one request set: the
    first N requests of the config-5 trace, all waiting at the start, each policy run until
    every request has finished. Same kernels, same entry point, same cache; only the step
    builder's policy differs (cb_sched_set_static). Throughput = generated tokens (sum of
    out_len) / wall time; rows = packed rows the kernels processed."""
    import numpy as np
    import torch

    import workloads as W
    from ragged_continuous_batching_amd import cb
    from ragged_continuous_batching_amd.runner import DeviceRun

    wl = W.config(5)
    reqs = [r for k in range(wl.steps) for r in wl.arrivals[k]][: args.requests]
    run = DeviceRun(wl, stale=None)
    stream = torch.cuda.current_stream()
    policies = [("continuous", 0), ("naive-batch-32", 32), ("naive-batch-8", 8), ("request-at-a-time", 1)]

    def fresh(b):
        s = cb.Scheduler(wl.token_budget, wl.block_size, wl.num_blocks, wl.max_num_seqs, wl.free_list)
        if b:
            s.set_static(b)
        for r in reqs:
            s.add(r.req_id, r.prompt_len, r.out_len)
        return s

    # size the buffers from a dry run of every policy (host only)
    max_t, max_ws, dry = 1, 256, {}
    for name, b in policies:
        s, steps, rows = fresh(b), 0, 0
        while True:
            st = s.build_raw()
            if st.num_reqs == 0 and s.stats()[:2] == (0, 0):
                break
            if st.num_reqs == 0 and st.num_evicted == 0:
                raise RuntimeError("a step with no rows while requests are left")
            if st.num_reqs:
                max_t = max(max_t, st.num_tokens)
                max_ws = max(max_ws, cb.cb_step_workspace_size(run.shape, st.num_reqs, st.num_tokens,
                                                               st.max_blocks_per_req, st.cu_q_lens, st.ctx_lens))
                steps += 1
                rows += st.num_tokens
            s.commit()
        dry[name] = (steps, rows)
    g = torch.Generator(device="cuda").manual_seed(wl.seed)
    q = torch.randn(max_t, wl.num_q_heads, wl.head_dim, device="cuda", generator=g).to(torch.bfloat16)
    k_new = torch.randn(max_t, wl.num_kv_heads, wl.head_dim, device="cuda", generator=g).to(torch.bfloat16)
    v_new = torch.randn(max_t, wl.num_kv_heads, wl.head_dim, device="cuda", generator=g).to(torch.bfloat16)
    o = torch.empty_like(q)
    ws = torch.empty(max_ws, dtype=torch.uint8, device="cuda")

    def drive(s, limit=None):
        n = 0
        while limit is None or n < limit:
            st = s.build_raw()
            if st.num_reqs == 0 and s.stats()[:2] == (0, 0):
                break
            if st.num_reqs == 0 and st.num_evicted == 0:
                raise RuntimeError("a step with no rows while requests are left")
            if st.num_reqs:
                launch_step(cb, run, st, q, k_new, v_new, o, ws, stream)
            s.commit()
            n += 1

    drive(fresh(0), limit=200)                      # warm-up (clocks, code objects)
    torch.cuda.synchronize()
    gen = int(sum(r.out_len for r in reqs))
    useful = int(sum(r.prompt_len + r.out_len - 1 for r in reqs))
    out = {}
    for name, b in policies:
        s = fresh(b)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        drive(s)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        steps, rows = dry[name]
        out[name] = {"generated_tokens_per_s": round(gen / wall, 1), "seconds": round(wall, 4), "steps": steps,
                     "rows": rows, "useful_row_fraction": round(useful / rows, 4)}
    base = out["continuous"]["generated_tokens_per_s"]
    result = {
        "metric": "generated tokens/s, offline, per scheduling policy",
        "value": base, "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"first {len(reqs)} requests of the scheduler trace (lognormal prompts, geometric "
                               "outputs), all waiting at the start", "num_q_heads": wl.num_q_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "token_budget": wl.token_budget,
                   "generated_tokens": gen, "useful_rows": useful},
        "policies": out,
        "continuous_over": {n: round(base / v["generated_tokens_per_s"], 2) for n, v in out.items() if n != "continuous"},
    }
    print(json.dumps(result), flush=True)
    return 0


def classify_rows(step, prompt, out, gen):
    """(real rows, pad rows, idle rows, emitted tokens) of one built step; `gen` (request id ->
    tokens generated so far) is advanced. Request r's known sequence is its prompt and the
    tokens generated so far (positions < prompt + gen); a step's rows beyond it are pads of a
    padded prefill (more than one row) or idle rows of a batch member that has finished. A step
    emits a token for r when it processes the sequence's last known position and r still owes
    tokens."""
    real = pad = idle = emitted = 0
    cu = step.cu_q_lens
    for i in range(step.num_reqs):
        rid = int(step.req_ids[i])
        c, q = int(step.ctx_lens[i]), int(cu[i + 1] - cu[i])
        P, O, g = prompt[rid], out[rid], gen.get(rid, 0)
        n_real = max(0, min(c + q, P + g) - c)
        real += n_real
        if q > 1:
            pad += q - n_real
        else:
            idle += q - n_real
        if g < O and c <= P - 1 + g < c + q:
            gen[rid] = g + 1
            emitted += 1
    return real, pad, idle, emitted


def bench_policies_trace(args):
    """The config-5 scheduler trace itself, 500 steps with the same Poisson arrivals, under
    each policy the pages compare continuous batching with (zhangchitc "Naive batching";
    hassanahmed's request-at-a-time serving): continuous batching (m = 4096), naive padded
    batches of 32 and 8, and request-at-a-time. Same kernels, entry point and cache; only the
    step builder's policy differs. A host-only dry run of each schedule classifies its rows
    (real, pad, idle) and counts the tokens it emits; the timed run then replays the same
    schedule through cb_step_forward. Throughput = tokens emitted in the 500 steps / wall
    time."""
    import torch

    import workloads as W
    from ragged_continuous_batching_amd import cb
    from ragged_continuous_batching_amd.runner import DeviceRun

    wl = W.config(5)
    prompt = {r.req_id: r.prompt_len for k in range(wl.steps) for r in wl.arrivals[k]}
    out = {r.req_id: r.out_len for k in range(wl.steps) for r in wl.arrivals[k]}
    run = DeviceRun(wl, stale=None)
    stream = torch.cuda.current_stream()
    policies = [("continuous", 0), ("naive-batch-32", 32), ("naive-batch-8", 8), ("request-at-a-time", 1)]

    def fresh(b):
        s = cb.Scheduler(wl.token_budget, wl.block_size, wl.num_blocks, wl.max_num_seqs, wl.free_list)
        if b:
            s.set_static(b)
        return s

    stats, max_t, max_ws = {}, 1, 256
    for name, b in policies:
        s, gen = fresh(b), {}
        tot = {"steps": 0, "empty_steps": 0, "rows": 0, "real_rows": 0, "pad_rows": 0, "idle_rows": 0,
               "generated_tokens": 0}
        for k in range(wl.steps):
            for r in wl.arrivals[k]:
                s.add(r.req_id, r.prompt_len, r.out_len)
            st = s.build()
            if st.num_reqs:
                max_t = max(max_t, st.num_tokens)
                max_ws = max(max_ws, cb.cb_step_workspace_size(run.shape, st.num_reqs, st.num_tokens,
                                                               st.max_blocks_per_req, st.cu_q_lens, st.ctx_lens))
                real, pad, idle, emitted = classify_rows(st, prompt, out, gen)
                tot["rows"] += st.num_tokens
                tot["real_rows"] += real
                tot["pad_rows"] += pad
                tot["idle_rows"] += idle
                tot["generated_tokens"] += emitted
            else:
                tot["empty_steps"] += 1
            tot["steps"] += 1
            s.commit()
        tot["requests_finished"] = sum(1 for rid, g in gen.items() if g >= out[rid])
        tot["requests_arrived"] = len(prompt)
        stats[name] = tot
    g = torch.Generator(device="cuda").manual_seed(wl.seed)
    q = torch.randn(max_t, wl.num_q_heads, wl.head_dim, device="cuda", generator=g).to(torch.bfloat16)
    k_new = torch.randn(max_t, wl.num_kv_heads, wl.head_dim, device="cuda", generator=g).to(torch.bfloat16)
    v_new = torch.randn(max_t, wl.num_kv_heads, wl.head_dim, device="cuda", generator=g).to(torch.bfloat16)
    o = torch.empty_like(q)
    ws = torch.empty(max_ws, dtype=torch.uint8, device="cuda")

    def drive(s, steps):
        for k in range(steps):
            for r in wl.arrivals[k]:
                s.add(r.req_id, r.prompt_len, r.out_len)
            st = s.build_raw()
            if st.num_reqs:
                launch_step(cb, run, st, q, k_new, v_new, o, ws, stream)
            s.commit()

    drive(fresh(0), 100)                          # warm-up (clocks, code objects)
    torch.cuda.synchronize()
    results = {}
    for name, b in policies:
        s = fresh(b)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        drive(s, wl.steps)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        st = stats[name]
        results[name] = dict(st, seconds=round(wall, 4),
                             generated_tokens_per_s=round(st["generated_tokens"] / wall, 1),
                             real_row_fraction=round(st["real_rows"] / max(1, st["rows"]), 4),
                             ms_per_step=round(wall * 1e3 / wl.steps, 4))
    base = results["continuous"]["generated_tokens_per_s"]
    result = {
        "metric": "generated tokens/s over the 500-step trace, per scheduling policy",
        "value": base, "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "scheduler-trace replay (500 steps, Poisson(8) arrivals per step, lognormal "
                               "prompts, geometric outputs), the same arrivals for every policy",
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "token_budget": wl.token_budget},
        "policies": results,
        "continuous_over": {n: round(base / v["generated_tokens_per_s"], 2) for n, v in results.items()
                            if n != "continuous" and v["generated_tokens_per_s"] > 0},
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
