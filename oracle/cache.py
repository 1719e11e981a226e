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
