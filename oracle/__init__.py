"""Plain, slow, float64 CPU oracle for paged GQA decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, helpers, tables or constant
generators) and imports nothing from ``paged_kv_cache_105_amd``.

What it computes, and where the pages define it:

* ``kvbytes``   -- ideal cache payload and per-token growth (page 1,
  "KV cache: Generation state, latency, and allocation", section 21.1,
  Eq. 21.2 and Eq. 21.3; page 2, "KV Cache Explained", section "How much GPU
  memory does the KV cache use?").
* ``codecs``    -- bf16 and OCP E4M3FN (fp8) stored-scalar codecs.  The pages
  only say "FP8 KV ... needs scales" (page 2, section "What changes when you
  use FP8 KV"); the bit format is the OCP 8-bit floating point
  specification's E4M3 (no infinities, one NaN pattern per sign).
* ``blockpool`` -- the block allocator: free queue, reference counts,
  immediate release (page 1, section 21.5, Table 21.1 and the five-step
  walk after it; page 2, section "Why PagedAttention allocates KV in blocks").
* ``paged``     -- slot mapping, append (page 1, section 21.6, Eq. 21.6),
  gathering paged blocks back into the dense layout of Eq. 21.1, and exact
  softmax attention of one decode query per query head with grouped KV heads
  (page 1, section 21.1).

Every function here is pinned by a ``-m "not gpu"`` test to something other
than itself: numbers the pages print, closed forms, brute force on tiny
inputs, library routines on special cases, and paging invariants.
"""
