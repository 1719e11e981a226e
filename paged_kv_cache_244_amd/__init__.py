"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The hot path of PagedAttention as a C-ABI library of hand-written HIP kernels
(``libpagedkv.so``, declared in ``include/pagedkv.h``) plus this thin binding:

* ``pa_decode``       — single-query decode attention through per-request block
                        tables, with an optional split-context pass + reduce.
* ``kv_cache_write``  — slot-mapped append of new tokens' K/V.
* ``kv_copy_blocks``  — whole-block copy used by copy-on-write.
* ``BlockAllocator``  — host allocator: block tables, refcounts, demand
                        allocation, fork, copy-on-write, free.

PyTorch supplies device memory and streams only.  The library is loaded on the
first call and its absence is an error (there is no fallback path).
"""

from ._lib import (  # noqa: F401
    BadSequence,
    BlockAllocator,
    OutOfBlocks,
    PagedKVError,
    kv_cache_write,
    kv_copy_blocks,
    lib,
    pa_decode,
    pa_decode_workspace_size,
    set_kernel_policy,
)
