"""Seeded synthetic inputs for the paged decode path.

This module only draws random numbers and fixes shapes; it does none of the
method's arithmetic (no slot, table, attention or copy computation).  Both the
HIP path (tests, bench) and the CPU oracle (tests) take their inputs from here,
each then building its own block tables and caches.

The five workloads follow the shapes of the pages' examples:

* ``tiny``           — 1 layer, 2 heads x 64, fp16 K/V and fp32 q, 16-token
                       blocks, context lengths {7, 16, 33, 100}, a 64-block pool.
* ``opt13b``         — OPT-13B's attention layer: 40 heads x 128 (hidden 5120),
                       64 requests, lengths uniform in [1, 2048] ("800 kilobytes
                       per token", lede; teqners explainer, section "Why the KV
                       cache is the thing that limits your batch").
* ``gqa``            — 32 query heads sharing 8 KV heads x 128, 128 requests,
                       lengths log-uniform in [16, 4096] ("The KV cache is a
                       systems problem", section "Calculate bytes per token
                       before choosing a batch").
* ``parallel_sampling`` — 16 prompts of 64..512 tokens, 8 samples each sharing
                       the prompt blocks, 128 decode steps (teqners explainer,
                       section "The part everyone forgets: pages enable
                       sharing, not just packing").
* ``long_context``   — 16 requests of 8192..32768 tokens, 32/8 heads x 128,
                       block sizes 8..128 (teqners explainer, section "The
                       block size tradeoff").

Recipe: a ``numpy`` PCG64 generator seeded with the workload's index draws,
in this order, the lengths, the free-list permutation of the pool, the keys,
the values and the queries; values are N(0, 1) drawn in float32 and rounded
once to float16 (queries stay float32 in ``tiny``).  Large arrays are drawn in
a fixed number of chunks from spawned child generators, so the values do not
depend on the number of threads.  Each request's context length counts the
token of the current decode step: its first ``L - 1`` tokens are the prompt
already in the cache, token ``L - 1`` is written by the step and then attended.
"""

from __future__ import annotations

import math
import zlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_CHUNKS = 32


def _normal(seed_seq: np.random.SeedSequence, shape, dtype) -> np.ndarray:
    """N(0,1) float32 samples rounded to ``dtype``; deterministic for a seed."""
    total = int(np.prod(shape))
    out32 = np.empty(total, dtype=np.float32)
    children = seed_seq.spawn(_CHUNKS)
    bounds = np.linspace(0, total, _CHUNKS + 1).astype(np.int64)

    def fill(c):
        lo, hi = bounds[c], bounds[c + 1]
        if hi > lo:
            np.random.Generator(np.random.PCG64(children[c])).standard_normal(
                hi - lo, dtype=np.float32, out=out32[lo:hi])

    with ThreadPoolExecutor(max_workers=8) as pool:
        list(pool.map(fill, range(_CHUNKS)))
    return out32.astype(dtype, copy=False).reshape(shape)


@dataclass
class DecodeWorkload:
    """One decode step over a batch of requests whose prompts are already cached."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: type
    scale: float
    lengths: np.ndarray          # int32 [S], tokens attended, current token included
    num_blocks: int              # physical pool size
    initial_order: np.ndarray    # int32 [num_blocks], free-list permutation
    k_tokens: np.ndarray         # float16 [sum(L), Hkv, D], logical order, request by request
    v_tokens: np.ndarray         # float16 [sum(L), Hkv, D]
    q: np.ndarray                # q_dtype [S, Hq, D]
    offsets: np.ndarray = field(default=None)  # int64 [S + 1], start of each request in *_tokens
    partition_size: int = 512

    def __post_init__(self):
        if self.offsets is None:
            self.offsets = np.concatenate([[0], np.cumsum(self.lengths, dtype=np.int64)])

    @property
    def num_seqs(self) -> int:
        return int(self.lengths.shape[0])

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one decode step reads: logical tokens only."""
        return int(self.lengths.sum()) * 2 * self.num_kv_heads * self.head_dim * 2

    def tokens(self, i: int):
        lo, hi = self.offsets[i], self.offsets[i + 1]
        return self.k_tokens[lo:hi], self.v_tokens[lo:hi]


def step_inputs(w: DecodeWorkload, step: int):
    """New-token K, V ``[S, Hkv, D]`` and q ``[S, Hq, D]`` for decode step ``step`` >= 1
    after the workload's own step (step 0 uses the workload's last tokens and q)."""
    child = np.random.SeedSequence([zlib.crc32(w.name.encode()), step])
    sk, sv, sq = child.spawn(3)
    S = w.num_seqs
    k = _normal(sk, (S, w.num_kv_heads, w.head_dim), np.float16)
    v = _normal(sv, (S, w.num_kv_heads, w.head_dim), np.float16)
    q = _normal(sq, (S, w.num_q_heads, w.head_dim), w.q_dtype)
    return k, v, q


def _pool_blocks(lengths, block_size, slack):
    need = int(sum((int(L) + block_size - 1) // block_size for L in lengths))
    return int(math.ceil(slack * need))


def _decode(name, seed, lengths_fn, num_q_heads, num_kv_heads, head_dim, block_size,
            q_dtype=np.float16, num_blocks=None, slack=1.2, partition_size=512):
    root = np.random.SeedSequence(seed)
    s_len, s_perm, s_k, s_v, s_q = root.spawn(5)
    lengths = np.asarray(lengths_fn(np.random.Generator(np.random.PCG64(s_len))), dtype=np.int32)
    if num_blocks is None:
        num_blocks = _pool_blocks(lengths, block_size, slack)
    order = np.random.Generator(np.random.PCG64(s_perm)).permutation(num_blocks).astype(np.int32)
    total = int(lengths.sum())
    k = _normal(s_k, (total, num_kv_heads, head_dim), np.float16)
    v = _normal(s_v, (total, num_kv_heads, head_dim), np.float16)
    q = _normal(s_q, (lengths.shape[0], num_q_heads, head_dim), q_dtype)
    return DecodeWorkload(name, num_q_heads, num_kv_heads, head_dim, block_size, q_dtype,
                          1.0 / math.sqrt(head_dim), lengths, num_blocks, order, k, v, q,
                          partition_size=partition_size)


def tiny(seed: int = 0) -> DecodeWorkload:
    return _decode("tiny", seed, lambda g: [7, 16, 33, 100], 2, 2, 64, 16,
                   q_dtype=np.float32, num_blocks=64)


def opt13b(seed: int = 1, batch: int = 64) -> DecodeWorkload:
    return _decode("opt13b", seed, lambda g: g.integers(1, 2048 + 1, size=batch), 40, 40, 128, 16)


def _log_uniform(g, lo, hi, n):
    x = np.floor(np.exp(g.uniform(math.log(lo), math.log(hi + 1), size=n))).astype(np.int64)
    return np.clip(x, lo, hi)


def gqa(seed: int = 2, batch: int = 128) -> DecodeWorkload:
    return _decode("gqa", seed, lambda g: _log_uniform(g, 16, 4096, batch), 32, 8, 128, 16)


def long_context(block_size: int = 16, seed: int = 4, batch: int = 16) -> DecodeWorkload:
    """Same lengths and values for every block size: only the pool geometry changes."""
    return _decode(f"long_context_b{block_size}", seed,
                   lambda g: g.integers(8192, 32768 + 1, size=batch), 32, 8, 128, block_size)


def custom(name: str, seed: int, lengths, num_q_heads, num_kv_heads, head_dim, block_size,
           q_dtype=np.float16, slack: float = 1.2, num_blocks=None) -> DecodeWorkload:
    """A workload with explicit lengths (used for edge cases and small parity runs)."""
    return _decode(name, seed, lambda g: list(lengths), num_q_heads, num_kv_heads, head_dim,
                   block_size, q_dtype=q_dtype, num_blocks=num_blocks, slack=slack)


@dataclass
class SamplingWorkload:
    """Parallel sampling: prompts forked into ``samples`` continuations sharing blocks."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    prompt_lengths: np.ndarray   # int32 [num_prompts]
    samples: int
    steps: int
    num_blocks: int
    initial_order: np.ndarray
    prompt_k: np.ndarray         # float16 [sum(P), Hkv, D]
    prompt_v: np.ndarray
    step_seed: np.random.SeedSequence

    @property
    def num_prompts(self) -> int:
        return int(self.prompt_lengths.shape[0])

    @property
    def prompt_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.prompt_lengths, dtype=np.int64)])

    def step_inputs(self, step: int):
        """New-token K, V ``[S, Hkv, D]`` fp16 and q ``[S, Hq, D]`` fp16 for one step.

        ``S = num_prompts * samples``; sample ``j`` of prompt ``p`` is row ``p * samples + j``.
        """
        s = self.num_prompts * self.samples
        child = np.random.SeedSequence(self.step_seed.entropy,
                                       spawn_key=tuple(self.step_seed.spawn_key) + (step,))
        sk, sv, sq = child.spawn(3)
        k = _normal(sk, (s, self.num_kv_heads, self.head_dim), np.float16)
        v = _normal(sv, (s, self.num_kv_heads, self.head_dim), np.float16)
        q = _normal(sq, (s, self.num_q_heads, self.head_dim), np.float16)
        return k, v, q


def parallel_sampling(seed: int = 3, num_prompts: int = 16, samples: int = 8, steps: int = 128,
                      block_size: int = 16) -> SamplingWorkload:
    root = np.random.SeedSequence(seed)
    s_len, s_perm, s_k, s_v, s_steps = root.spawn(5)
    plen = np.random.Generator(np.random.PCG64(s_len)).integers(64, 512 + 1, size=num_prompts)
    plen = plen.astype(np.int32)
    # Pool: 1.2x what every sample would hold after the last step with no sharing at all.
    unshared = samples * sum((int(p) + steps + block_size - 1) // block_size for p in plen)
    num_blocks = int(math.ceil(1.2 * unshared))
    order = np.random.Generator(np.random.PCG64(s_perm)).permutation(num_blocks).astype(np.int32)
    total = int(plen.sum())
    k = _normal(s_k, (total, 40, 128), np.float16)
    v = _normal(s_v, (total, 40, 128), np.float16)
    return SamplingWorkload("parallel_sampling", 40, 40, 128, block_size, 1.0 / math.sqrt(128),
                            plen, samples, steps, num_blocks, order, k, v, s_steps)


def with_block_size(w: DecodeWorkload, block_size: int, seed: int = 4) -> DecodeWorkload:
    """The same requests and values stored with another block size: a new pool size
    (1.2x the blocks needed) and a new free-list permutation drawn for that size."""
    num_blocks = _pool_blocks(w.lengths, block_size, 1.2)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, block_size])))
    order = g.permutation(num_blocks).astype(np.int32)
    return DecodeWorkload(f"{w.name.split('_b')[0]}_b{block_size}", w.num_q_heads, w.num_kv_heads,
                          w.head_dim, block_size, w.q_dtype, w.scale, w.lengths, num_blocks, order,
                          w.k_tokens, w.v_tokens, w.q, w.offsets, w.partition_size)


@dataclass
class PrefillWorkload:
    """A batch of prompts processed at once: every prompt token is a query."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    lengths: np.ndarray          # int32 [S] prompt tokens
    num_blocks: int
    initial_order: np.ndarray
    k_tokens: np.ndarray         # float16 [sum(L), Hkv, D]
    v_tokens: np.ndarray
    q: np.ndarray                # float16 [sum(L), Hq, D], the prompt tokens' queries

    @property
    def num_seqs(self) -> int:
        return int(self.lengths.shape[0])

    def flops(self) -> int:
        """Causal attention work: a query at position p meets p + 1 keys; each
        (query, key, head) costs 2*D for the score and 2*D for the value sum."""
        pairs = sum(int(L) * (int(L) + 1) // 2 for L in self.lengths)
        return 4 * self.num_q_heads * self.head_dim * pairs


def prefill(seed: int = 6, batch: int = 16) -> PrefillWorkload:
    """16 prompts of U{512..4096} tokens, 32 query / 8 KV heads x 128, B = 16."""
    root = np.random.SeedSequence(seed)
    s_len, s_perm, s_k, s_v, s_q = root.spawn(5)
    lengths = np.random.Generator(np.random.PCG64(s_len)).integers(512, 4096 + 1, size=batch)
    lengths = lengths.astype(np.int32)
    hq, hkv, d, bs = 32, 8, 128, 16
    num_blocks = _pool_blocks(lengths, bs, 1.2)
    order = np.random.Generator(np.random.PCG64(s_perm)).permutation(num_blocks).astype(np.int32)
    total = int(lengths.sum())
    return PrefillWorkload("prefill", hq, hkv, d, bs, 1.0 / math.sqrt(d), lengths, num_blocks,
                           order, _normal(s_k, (total, hkv, d), np.float16),
                           _normal(s_v, (total, hkv, d), np.float16),
                           _normal(s_q, (total, hq, d), np.float16))


@dataclass
class BeamWorkload:
    """Beam-search-like churn: each prompt forks into ``beams`` requests sharing its
    blocks; every ``prune_every`` steps each prompt cancels ``prune`` beams and forks
    as many survivors, so copy-on-write copies and the reuse of freed blocks recur
    while kernels are queued ("Only 20.4% of your KV cache held actual tokens",
    section "The part everyone forgets: pages enable sharing, not just packing":
    beams kept or killed every step, dead ones giving their references back).  The
    schedule and every input are drawn from seeds."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    prompt_lengths: np.ndarray   # int32 [P]
    beams: int
    prune_every: int
    prune: int
    num_blocks: int
    initial_order: np.ndarray
    prompt_k: np.ndarray         # float16 [sum(P), Hkv, D]
    prompt_v: np.ndarray
    step_seed: np.random.SeedSequence
    schedule_seed: np.random.SeedSequence

    @property
    def num_prompts(self) -> int:
        return int(self.prompt_lengths.shape[0])

    def step_inputs(self, step: int):
        """New-token K, V ``[P*beams, Hkv, D]`` and q ``[P*beams, Hq, D]`` fp16 for one step."""
        s = self.num_prompts * self.beams
        child = np.random.SeedSequence(self.step_seed.entropy,
                                       spawn_key=tuple(self.step_seed.spawn_key) + (step,))
        sk, sv, sq = child.spawn(3)
        return (_normal(sk, (s, self.num_kv_heads, self.head_dim), np.float16),
                _normal(sv, (s, self.num_kv_heads, self.head_dim), np.float16),
                _normal(sq, (s, self.num_q_heads, self.head_dim), np.float16))

    def prune_plan(self, step: int):
        """None, or per prompt (beam positions to cancel, beam positions to fork), the
        positions indexing that prompt's current beam list."""
        if step == 0 or step % self.prune_every:
            return None
        child = np.random.SeedSequence(self.schedule_seed.entropy,
                                       spawn_key=tuple(self.schedule_seed.spawn_key) + (step,))
        g = np.random.Generator(np.random.PCG64(child))
        plan = []
        for _ in range(self.num_prompts):
            drop = g.choice(self.beams, size=self.prune, replace=False)
            keep = np.setdiff1d(np.arange(self.beams), drop)
            plan.append((sorted(int(x) for x in drop), [int(x) for x in g.choice(keep, size=self.prune)]))
        return plan


def beams(seed: int = 7, num_prompts: int = 8, beams: int = 8, prune_every: int = 4,
          prune: int = 4, max_steps: int = 256, block_size: int = 16) -> BeamWorkload:
    """8 prompts of U{256..1024} tokens x 8 beams, OPT-13B attention shape (40 x 128)."""
    root = np.random.SeedSequence(seed)
    s_len, s_perm, s_k, s_v, s_steps, s_sched = root.spawn(6)
    plen = np.random.Generator(np.random.PCG64(s_len)).integers(256, 1024 + 1, size=num_prompts)
    plen = plen.astype(np.int32)
    hq = hkv = 40
    d = 128
    # Pool: every beam holding a private copy of everything it could write, plus the prompts.
    private = num_prompts * beams * ((max_steps + block_size - 1) // block_size + 1)
    num_blocks = int(math.ceil(1.2 * (private + sum(-(-int(p) // block_size) for p in plen))))
    order = np.random.Generator(np.random.PCG64(s_perm)).permutation(num_blocks).astype(np.int32)
    total = int(plen.sum())
    return BeamWorkload("beams", hq, hkv, d, block_size, 1.0 / math.sqrt(d), plen, beams,
                        prune_every, prune, num_blocks, order,
                        _normal(s_k, (total, hkv, d), np.float16),
                        _normal(s_v, (total, hkv, d), np.float16), s_steps, s_sched)


WORKLOADS = {
    "tiny": tiny,
    "opt13b": opt13b,
    "gqa": gqa,
    "long_context": long_context,
}
