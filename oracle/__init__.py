"""Plain fp64 CPU oracle for PagedAttention decode.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library or
its Python binding) imports, links or calls anything in this package.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.

The oracle computes, slowly and directly, what the paged decode path must
produce:

* ``formats``    -- exact decoding of the stored element types (fp32, bf16,
                    OCP fp8 E4M3FN) and the fp8 quantise-on-write rule.
* ``layout``     -- where element (block, kv head, slot, dim) lives in the
                    key and value block pools; scatter of new tokens through a
                    slot mapping; gather of a sequence through its block table.
* ``attention``  -- dense single-query softmax attention in fp64 over the
                    gathered cache.
* ``alloc_model``-- the block allocator's specification: FIFO free list,
                    refcounted blocks, fork, append with fill-before-allocate
                    and copy-on-write, free.

Sources (the pages this follows):
  * "Day 6/90 of Inference Engineering" (X thread on PagedAttention) --
    block-at-a-time allocation, fill before allocate, prefix sharing with a
    fresh block where prompts diverge, the block table that makes a
    scattered cache look contiguous.
  * "PagedAttention Kernel：大模型推理优化的显存管理革新" §1 (fixed-size
    pages scattered through device memory), §3.1 (QK^T per block, softmax,
    PV accumulated block by block), §6 (fp32 accumulation).

Parity status of every function is listed in each module header.  All of them
are pinned (see tests/test_oracle_*.py); none is "parity unpinned".
"""

from . import formats, layout, attention, alloc_model, replay  # noqa: F401
