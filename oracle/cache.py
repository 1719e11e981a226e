"""Paged K/V storage: slot-mapped write, block copy, logical gather (oracle).

Test infrastructure only.  Layout of one cache pool (one for K, one for V):
``pool[num_blocks, kv_heads, block_size, head_dim]`` of float16.  Physical
block ``b`` holds, for every KV head, ``block_size`` token slots.

* A request's logical blocks are filled left to right and a per-request block
  table maps logical block ``j`` to a physical block anywhere in the pool
  (teqners explainer, section "The page table, relocated into attention").
  A slot number ``s`` names physical block ``s // B`` and offset ``s % B``.
* Copy-on-write copies one whole block — all heads, all ``B`` slots, for K
  and V and for every layer — from the shared source to a fresh destination
  (teqners explainer, section "The part everyone forgets: pages enable
  sharing, not just packing"; "800 kilobytes per token", "The old answer,
  imported honestly").

* Swap copies whole blocks between two pools of the same geometry (the
  device pool and a pool in host memory): block ``src`` of the source becomes
  block ``dst`` of the destination, for K and V and every layer (rsw.lol,
  section "Eviction and reuse can move costs elsewhere": evicted state moved
  to another memory tier).

* A table check (a debug aid, not part of attention): a request's table row
  must hold its context, and every entry covering the context must name a
  block of the pool (rsw.lol, section "Shared prefixes need ownership rules":
  a block is followed from allocation to reuse, and a table naming blocks
  outside the pool betrays a lifecycle mistake).

Every function copies bytes; nothing is rounded or converted.
"""

import numpy as np


def write_slots(k_pool, v_pool, k_new, v_new, slot_mapping, block_size):
    """Store token j's K/V vectors ``[kv_heads, head_dim]`` in slot ``slot_mapping[j]``.

    Tokens are stored one after another in order; a negative slot means "skip
    this token".  The pools are modified in place and also returned.
    """
    k_new = np.asarray(k_new)
    v_new = np.asarray(v_new)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    for j in range(slots.shape[0]):
        s = int(slots[j])
        if s < 0:
            continue
        block, offset = s // block_size, s % block_size
        k_pool[block, :, offset, :] = k_new[j]
        v_pool[block, :, offset, :] = v_new[j]
    return k_pool, v_pool


def copy_blocks(layer_pools, block_pairs):
    """For each (src, dst) pair in order and each layer: pool[dst] = pool[src].

    ``layer_pools`` is a list of ``(k_pool, v_pool)`` tuples, one per layer.
    The whole block is copied, filled and unfilled slots alike.
    """
    for src, dst in np.asarray(block_pairs, dtype=np.int64).reshape(-1, 2):
        for k_pool, v_pool in layer_pools:
            k_pool[dst] = k_pool[src]
            v_pool[dst] = v_pool[src]
    return layer_pools


def copy_blocks_between(src_layers, dst_layers, block_pairs):
    """For each (src, dst) pair and each layer: dst_pool[dst] = src_pool[src].

    ``src_layers`` and ``dst_layers`` are lists of ``(k_pool, v_pool)``, one per
    layer, of the same block geometry.  The whole block is copied.
    """
    for src, dst in np.asarray(block_pairs, dtype=np.int64).reshape(-1, 2):
        for (sk, sv), (dk, dv) in zip(src_layers, dst_layers):
            dk[dst] = sk[src]
            dv[dst] = sv[src]
    return dst_layers


def gather_logical(pool, table_row, num_tokens, block_size):
    """Return the ``[num_tokens, kv_heads, head_dim]`` view a sequence sees.

    Logical token t lives in physical block ``table_row[t // B]`` at offset
    ``t % B``.  Entries of ``table_row`` past the last used block are never read.
    """
    t = np.arange(num_tokens)
    phys = np.asarray(table_row)[t // block_size]
    return pool[phys, :, t % block_size, :]


def check_tables(tables, lens, block_size, num_blocks):
    """Count the faults of block tables against a pool of ``num_blocks`` blocks.

    ``tables[s]`` is request s's row of ``max_blocks`` entries and ``lens[s]`` its
    context length.  Request s needs ceil(len / block_size) blocks; a negative
    length, or one needing more blocks than the row holds, is a length fault.
    The entries covering the context (the first min(needed, max_blocks) of the
    row; none for a negative length) must lie in [0, num_blocks); each one that
    does not is an id fault.  Returns (id faults, length faults, first request,
    first entry), the first offender taken in (request, entry) order with a
    request's length fault (entry -1) before its entries, or (-1, -1) if none.
    """
    tables = np.asarray(tables)
    max_blocks = tables.shape[1] if tables.ndim == 2 else 0
    bad_ids = bad_lens = 0
    first = None
    for s, length in enumerate(int(x) for x in lens):
        needed = 0 if length < 0 else -(-length // block_size)
        if length < 0 or needed > max_blocks:
            bad_lens += 1
            if first is None:
                first = (s, -1)
        for j in range(min(needed, max_blocks)):
            block = int(tables[s, j])
            if block < 0 or block >= num_blocks:
                bad_ids += 1
                if first is None:
                    first = (s, j)
    if first is None:
        first = (-1, -1)
    return bad_ids, bad_lens, first[0], first[1]
