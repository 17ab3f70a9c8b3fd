"""CPU oracle for ragged continuous-batching attention. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import anything from here. The product (``ragged_continuous_batching_amd``) never
imports, calls or links it, and this package shares no code with the product.

Contents:
* ``attention``: plain fp64 per-request masked softmax attention. It is written as the
  definition on the pages (Hugging Face blog "Continuous batching from first principles",
  sections "Attention", "KV-cache", "Chunked prefill" and "Continuous batching"; and
  zhangchitc "continuous-batching", section "Ragged batching: attention in per-request
  blocks"). Three independent restatements sit beside it: a scalar brute-force loop, the
  dense block-diagonal mask over the concatenated stream, and the left-padded batch.
* ``scheduler``: a reference of the step-building rule (decode first, then prefill chunks
  up to the budget m, evict and admit on EOS) with a FIFO block allocator.

Pins for each function live in ``tests/test_oracle_*.py`` and ``tests/test_ref_scheduler.py``.
"""
from . import attention, scheduler  # noqa: F401
