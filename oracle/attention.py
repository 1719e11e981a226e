"""Single-query decode attention over a block table, in float64 (oracle).

Test infrastructure only.  What it computes:

A decode step attends one new query per request over every token the request
has cached; per request this is a matrix-vector product (teqners explainer,
section "Why the KV cache is the thing that limits your batch").  PagedAttention
computes exactly that attention, but fetches each key and value through the
request's block table from wherever its physical block lies ("800 kilobytes per
token", section "The old answer, imported honestly"; teqners explainer, section
"The page table, relocated into attention").  Query heads may be grouped so a
group shares one KV head ("The KV cache is a systems problem", section
"Calculate bytes per token before choosing a batch"); query head ``h`` reads KV
head ``h // (Hq // Hkv)``, consecutive query heads sharing one KV head.

For request i, query head h, with L = context_lens[i] and t in [0, L):

    K_t = Kpool[bt[i, t // B], g, t % B, :]      (and V_t likewise)
    s_t = scale * sum_d q[i, h, d] * K_t[d]
    p_t = exp(s_t - max_u s_u) / sum_u exp(s_u - max_u s_u)
    out[i, h, :] = sum_t p_t * V_t

Everything is widened to float64 first (fp16 and fp32 widen exactly), and the
scale is taken as float64(float32(scale)), the value a kernel receives.  A
request with L = 0 yields zeros.  Pool slots past L and table entries past
ceil(L/B) are never read.
"""

import numpy as np

from .cache import gather_logical


def attend_one(q_heads, keys, values, scale):
    """Attention of ``q_heads [Hq, D]`` over ``keys, values [L, Hkv, D]``, float64.

    Returns ``[Hq, D]`` float64.  Written head by head and token by token in
    vector form; the softmax subtracts the maximum score before exponentiating.
    """
    q_heads = np.asarray(q_heads, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    num_q_heads, head_dim = q_heads.shape
    num_tokens, num_kv_heads, _ = keys.shape
    out = np.zeros((num_q_heads, head_dim), dtype=np.float64)
    if num_tokens == 0:
        return out
    group = num_q_heads // num_kv_heads
    s64 = np.float64(np.float32(scale))
    for h in range(num_q_heads):
        g = h // group
        scores = s64 * (keys[:, g, :] @ q_heads[h])          # [L]
        weights = np.exp(scores - scores.max())
        probs = weights / weights.sum()
        out[h] = probs @ values[:, g, :]
    return out


def attend_paged(q, k_pool, v_pool, block_tables, context_lens, block_size, scale, seqs=None):
    """Decode attention for every request (or the listed ``seqs``) via its block table.

    q: ``[S, Hq, D]`` (float16 or float32); pools: ``[NB, Hkv, B, D]`` float16;
    block_tables: ``[S, max_blocks]`` int; context_lens: ``[S]`` int.
    Returns ``[S, Hq, D]`` float64 (rows not in ``seqs`` are left zero).
    """
    q = np.asarray(q)
    num_seqs, num_q_heads, head_dim = q.shape
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    rows = range(num_seqs) if seqs is None else seqs
    for i in rows:
        length = int(context_lens[i])
        keys = gather_logical(k_pool, block_tables[i], length, block_size)
        values = gather_logical(v_pool, block_tables[i], length, block_size)
        out[i] = attend_one(q[i], keys, values, scale)
    return out


def attend_contiguous(q, k_rows, v_rows, context_lens, scale, seqs=None):
    """Decode attention over the layout without a block table (float64).

    The pre-paging arrangement the pages compare against ("800 kilobytes per
    token", section "The old answer, imported honestly"): request i's keys for
    KV head g are one contiguous row ``k_rows[i, g, :L_i, :]``.  ``k_rows,
    v_rows``: ``[S, Hkv, Lmax, D]`` float16; q ``[S, Hq, D]``.  Returns
    ``[S, Hq, D]`` float64 (rows not in ``seqs`` are left zero).
    """
    q = np.asarray(q)
    num_seqs, num_q_heads, head_dim = q.shape
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    rows = range(num_seqs) if seqs is None else seqs
    for i in rows:
        length = int(context_lens[i])
        keys = np.swapaxes(k_rows[i, :, :length, :], 0, 1)     # [L, Hkv, D]
        values = np.swapaxes(v_rows[i, :, :length, :], 0, 1)
        out[i] = attend_one(q[i], keys, values, scale)
    return out


def attend_prefill_paged(q, k_pool, v_pool, block_tables, context_lens, q_starts, block_size,
                         scale):
    """Causal attention of each request's new tokens over its block table (float64).

    The prompt phase ("The KV cache is a systems problem", section "Memory
    savings change the scheduling question", where it is set against
    incremental decoding):
    request i holds L_i tokens, the last Q_i = q_starts[i+1] - q_starts[i] of
    which are its new queries; query j sits at position L_i - Q_i + j and sees
    tokens 0..that position, gathered through the table as in ``attend_paged``.
    q: ``[T, Hq, D]``; returns ``[T, Hq, D]`` float64 (a query at a negative
    position, or rows outside every request, stay zero).
    """
    q = np.asarray(q)
    total, num_q_heads, head_dim = q.shape
    out = np.zeros((total, num_q_heads, head_dim), dtype=np.float64)
    for i in range(len(context_lens)):
        length = int(context_lens[i])
        first, last = int(q_starts[i]), int(q_starts[i + 1])
        count = last - first
        keys = gather_logical(k_pool, block_tables[i], length, block_size)
        values = gather_logical(v_pool, block_tables[i], length, block_size)
        for j in range(count):
            pos = length - count + j
            if pos < 0:
                continue
            out[first + j] = attend_one(q[first + j], keys[:pos + 1], values[:pos + 1], scale)
    return out
