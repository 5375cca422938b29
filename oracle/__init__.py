"""CPU oracle for the paged decode path — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct model of what the paged KV cache computes:
  attention.py   generation-phase attention, gathered through block tables (fp64)
  prefill.py     prompt-phase causal attention over the same paged cache (fp64)
  fp8.py         the 8-bit (E4M3) storage format of an 8-bit key/value cache
  cache_ops.py   the new token's key/value write and the copy-on-write block copy
  allocator.py   the block allocator: free list, reference counts, copy-on-write
  sizing.py      the pages' cache-size arithmetic
  replay.py      replays a workload's operation script through the pieces above

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package. It shares no code with the HIP library (no kernels, headers,
helpers or constants) and the library never imports it; both sides only read
the same seeded inputs from the separate `workloads` module.

Every function cites the passage of the source pages it follows:
  «The KV Cache and PagedAttention» (world.lapla.si/en/kvcache) by section title,
  «KV cache» (tellworld.net/learn/kv-cache) by section title.
Parity status: every function here is pinned by CPU tests (tests/test_oracle_*.py,
tests/test_alloc_model.py, tests/test_sizing.py); none is "parity unpinned".
"""
