"""CPU oracle for the paged KV-cache hot path — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously correct model that the HIP path is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It imports nothing from
``paged_kv_cache_244_amd`` and shares no code, header, table or helper with
the HIP library; it takes plain numpy arrays as input.

Sources (the three web pages on PagedAttention, cited by title and section):

* "800 kilobytes per token" (shashforge.dev log) — sections "The old answer,
  imported honestly" and the lede.
* "Only 20.4% of your KV cache held actual tokens: how PagedAttention put a
  page table inside the attention kernel" (blog.teqners.com) — sections
  "Why the KV cache is the thing that limits your batch", "The page table,
  relocated into attention", "The block size tradeoff", "The part everyone
  forgets: pages enable sharing, not just packing".
* "The KV cache is a systems problem" (rsw.lol notes) — sections "Calculate
  bytes per token before choosing a batch", "Use blocks to bound waste, then
  price the boundary", "Shared prefixes need ownership rules", "Eviction and
  reuse can move costs elsewhere".

Modules:

* ``closed_forms`` — bytes per token, blocks per sequence, tail waste.
* ``cache``        — slot-mapped K/V write, block copy (within a pool and
  between the device and host pools), logical gather.
* ``attention``    — decode and causal prefill attention over a block table,
  and over contiguous rows, fp64.
* ``alloc_model``  — reference model of the block allocator (refcounts,
  demand allocation, fork, copy-on-write, free, deferred free, swap to and
  from a host tier).

Every function here is pinned by ``tests/test_oracle_*.py`` against values
printed on the pages, closed forms, library routines or brute force; none is
"parity unpinned".
"""

from . import alloc_model, attention, cache, closed_forms  # noqa: F401
