"""CPU oracle for differentiated KV compaction and mixed-precision paged decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its Python
binding) imports, links or calls this package.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may use it.

This is a plain, slow, deliberately obvious implementation written from the DiffKV review
page (pith.science, "DiffKV: Differentiated Memory Management for Large Language Models
with Parallel KV Compaction"): its reading notes ("What carries the argument", "Core
claim") and the referee report (major comment 2 on Section 4 / Algorithm 1, minor
comment 4, the "free parameters" ledger).  It shares no code with the GPU path: it has its
own layout constants, its own packers and its own allocator.  numpy supplies IEEE float32
and float16 arithmetic (round-to-nearest-even) and float64 accumulation; nothing else is
borrowed.

Modules
  score      -- significance score, GQA max, three-tier thresholds, recent window
  quant      -- per-token asymmetric min/max quantizer (K8V4 / K4V2) and dequantizer
  layout     -- the unified page format: byte/bit position of every code and parameter
  pool       -- circular free-page ring, bidirectional page table, prefix-sum allocator
  place      -- page images of one head (what quantize_and_place must write)
  attention  -- decode attention over the dequantized live tokens, float64 accumulation

Parity status: every function here is pinned by CPU tests (tests/test_oracle_*.py) against
closed forms, special cases, invariants and hand-worked fixtures.  Parity with DiffKV's own
code is unpinned: the pages print no token-level example.
"""
