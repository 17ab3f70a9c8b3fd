"""The debug copy of the library built with device checks (build.py --device-checks).

In that copy every kernel that clamps a block id read from the device block table (an id
outside the cache pool is read as block 0, an append to such a block is dropped) also
counts the event in a device counter, and cb_debug_violations reads the sum. The block
table is device memory the host never reads, so these checks are the only guard against a
caller's corrupt table. A clean step counts nothing; a step whose device block table holds
one id past the pool counts it and still finishes with finite outputs (no fault).
The copy is loaded in a child process through CB_LIBRARY, as the sanitized host copy is.
"""
import os
import subprocess
import sys

import pytest

from ragged_continuous_batching_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
import numpy as np
import torch
import workloads as W
from ragged_continuous_batching_amd import cb
from ragged_continuous_batching_amd.runner import DeviceRun

assert cb.LIB_PATH.endswith("checks/libcb.so"), cb.LIB_PATH
hq, hkv, d = int(sys.argv[1]), int(sys.argv[2]), int(sys.argv[3])
reqs = [W.Request(0, 37, 1 << 20, cached=37, generated=1), W.Request(1, 130, 1 << 20),
        W.Request(2, 300, 1 << 20, cached=200), W.Request(3, 1, 1 << 20)]
wl = W.custom(reqs, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype="bf16", seed=5)
run = DeviceRun(wl, stale=0.0)
cb.cb_debug_violations(reset=True)
step, batch, q, k, v, o = run.run_step()
torch.cuda.synchronize()
clean = cb.cb_debug_violations(reset=True)
print("case", hq, hkv, d, "clean", clean, flush=True)
assert clean == 0, clean
assert torch.isfinite(o.float()).all()

nb = wl.num_blocks
bt = batch.d_bt.view(step.num_reqs, -1)
# block 0 of every request is read by each of its rows (causal attention covers position 0)
for r in range(step.num_reqs):
    bt[r, 0] = nb + 3
o2 = run.attention(batch, q)
torch.cuda.synchronize()
bad_attn = cb.cb_debug_violations(reset=True)
print("case", hq, hkv, d, "attention", bad_attn, flush=True)
assert bad_attn > 0
assert torch.isfinite(o2.float()).all()

# the block of each request's first new row: the append must drop those rows
for r in range(step.num_reqs):
    bt[r, int(step.ctx_lens[r]) // 16] = nb + 7
run.append(batch, k, v)
torch.cuda.synchronize()
bad_append = cb.cb_debug_violations(reset=True)
print("case", hq, hkv, d, "append", bad_append, flush=True)
assert bad_append > 0
print("ok", flush=True)
"""


@pytest.fixture(scope="module")
def checks_lib():
    if not os.path.exists(B.CHECKS_LIB):
        pytest.skip("no device-checks build (python -m ragged_continuous_batching_amd.build --device-checks)")
    return B.CHECKS_LIB


@pytest.mark.gpu
@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (4, 4, 128), (4, 2, 64)])
def test_block_ids_past_the_pool_are_counted(checks_lib, hq, hkv, d):
    env = dict(os.environ, CB_LIBRARY=checks_lib)
    r = subprocess.run([sys.executable, "-c", CHILD, str(hq), str(hkv), str(d)], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=240)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ok" in r.stdout, out[-3000:]
