"""CPU oracle for the MoE expert layer's grouped-GEMM path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything under ``oracle/``: only the tests, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` do.  The
oracle shares no code with the HIP library (no kernels, headers, helpers or
tables); the only thing both sides share are the seeded inputs from
``workloads/``.

What it computes (the plain definition, slowly, in float64 unless a step
fixes another precision):

1. route      -- per token the k largest router logits (ties to the lower
                 expert id), weights = softmax over the selected logits; flat
                 rows past the valid-row count become sentinel (id = E).
2. offsets    -- per-expert histogram with the sentinel bin left out, and its
                 exclusive scan; ``offsets[E]`` = number of valid rows.
3. permute    -- stable sort of flat rows by expert id, sentinel last.
4. per-expert loop -- gate/up projection, SiLU(gate)*up, down projection,
                 on each expert's contiguous segment; sentinel rows zero.
5. combine    -- routing-weight-scaled sum back to token order.
6. backward   -- (``backward.py``) the gradients of steps 4-5 with the
                 routing held fixed: dx, dW13, dW2 and the routing-weight
                 gradients, by the chain rule through the same per-expert loop.

Sources: the transformers PR #45621 write-up ("MoE 및 FP8 커널 최적화"),
section 2 (sentinel tokens are excluded from the histogram / sorted as the
largest key; ``offsets[-1]`` is the valid-row count) and section 3 (sentinel
outputs must be initialised); the LlamaFactory PR #10481 write-up ("Triton
기반 Fused MoE 커널"), section 1 (the per-expert loop it replaces, and the
scatter -> grouped GEMM -> SiLU*up -> grouped GEMM -> gather pipeline); the
"트랜스포머에서 전문가 혼합 (MoEs)" write-up, sections on MoE basics (router
picks a small subset of experts per token) and expert backends (``eager``
loops over experts as the correctness reference; ``grouped_mm`` sorts tokens
by expert id).

Pins: every function here is checked, in the ``-m "not gpu"`` tests, against
something other than itself (brute-force dense evaluation, closed forms,
textbook SwiGLU via torch, torch's e4m3 cast, the valid-row counts the
transformers write-up prints, invariants).  Nothing here is "parity unpinned".
"""

from . import e4m3, routing, layer, gemm, brute  # noqa: F401
