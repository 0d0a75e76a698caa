"""Float64 CPU oracle for block-sparse attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this package: only the tests, the smoke entry point and the benchmark's CPU
baseline leg use it. It shares no code, table or helper with the HIP library.

Modules:
  attention  -- the plain definition of the sparse attention output and its
                log-sum-exp, computed with an explicit full-row softmax in float64
                (GenericBlockSparseAttention article, "sparse attention mechanism"
                formula; FlashAttention article, "three steps" exactness claim).
  scheduler  -- the reference task split written into the fixed 1024-int32
                metadata buffer (GBSA article, "two-stage call" section).
  formats    -- exact decoders for fp16 / bf16 / OCP e4m3fn storage.
"""
from . import attention, formats, scheduler  # noqa: F401
