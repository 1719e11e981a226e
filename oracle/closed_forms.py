"""Closed-form sizes of a paged KV cache (oracle; test infrastructure only).

* Bytes per token: a cache keeps one key and one value vector per layer and
  per KV head, each ``head_dim`` elements wide ("The KV cache is a systems
  problem", section "Calculate bytes per token before choosing a batch").  For
  multi-head attention the KV heads times head_dim is the hidden size, which
  gives the OPT-13B figure in "800 kilobytes per token" (lede) and in the
  teqners explainer, section "Why the KV cache is the thing that limits your
  batch".
* Blocks per sequence: a block is taken only once the previous ones are full,
  so a sequence of L tokens holds ceil(L / B) blocks of B slots (teqners
  explainer, "The page table, relocated into attention"; rsw.lol, "Use blocks
  to bound waste, then price the boundary").
* Tail waste: the unused slots of the last block, ceil(L/B)*B - L, which is
  always below one block.
"""


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Key + value bytes one token occupies across all layers."""
    return 2 * layers * kv_heads * head_dim * elem_bytes


def mha_kv_bytes_per_token(hidden: int, layers: int, elem_bytes: int) -> int:
    """Multi-head form: every query head has its own KV head, so heads*dim = hidden."""
    return 2 * hidden * layers * elem_bytes


def blocks_for_tokens(num_tokens: int, block_size: int) -> int:
    """Number of fixed-size blocks a sequence of ``num_tokens`` holds (ceil)."""
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("num_tokens >= 0 and block_size > 0 required")
    return (num_tokens + block_size - 1) // block_size


def tail_waste_slots(num_tokens: int, block_size: int) -> int:
    """Unused slots in the last, partly filled block."""
    return blocks_for_tokens(num_tokens, block_size) * block_size - num_tokens
