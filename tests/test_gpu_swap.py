"""Swap to the host tier on the GPU: kv_swap_blocks and PagedKVCache.swap_out/in.

"The KV cache is a systems problem" (rsw.lol), section "Eviction and reuse can
move costs elsewhere": evicted state may move to another memory tier.  The
checks:
* kv_swap_blocks against the oracle's copy between pools (bit-exact, raw
  random bit patterns including NaN and Inf, several layers and geometries,
  both directions, pairs outside a pool skipped);
* memory the kernel must not touch (pageable host memory) refused before a
  launch;
* a cache round trip: requests, among them a forked group sharing blocks,
  swapped out; their device blocks taken and overwritten by another request;
  swapped back in: decode output bit-identical to before, and within the
  tolerance of the oracle; sharing survives (the group's blocks copied once);
* a deferred swap-out with a second stream that does not wait: the parked
  device blocks are not handed to the other request before the copy is done;
* the benchmark's set at full size (32 OPT-13B requests, 1,734 blocks) out and
  back twice: every request's logical K/V bitwise unchanged;
* random histories (create, append, fork, free, swap out and in of random
  subsets, deferred or not) on one stream, checked against the oracle on each
  request's token list.
"""

import ctypes

import numpy as np
import pytest

from oracle import attention
from oracle import cache as oc
from paged_kv_cache_244_amd import _lib
from tests import paths

pytestmark = pytest.mark.gpu

GEOMS = [  # kv heads, head_dim, block_size, layers
    (8, 128, 16, 1),
    (2, 64, 8, 3),
    (40, 128, 16, 1),
    (4, 128, 128, 2),
    (1, 64, 32, 33),          # more layers than one launch carries
]


def _bits(rng, shape):
    return rng.integers(0, 1 << 16, size=shape, dtype=np.uint16).view(np.float16)


@pytest.mark.parametrize("hkv,d,bs,layers", GEOMS, ids=[f"h{g[0]}_d{g[1]}_b{g[2]}_l{g[3]}" for g in GEOMS])
def test_swap_blocks_matches_oracle(hkv, d, bs, layers):
    import torch

    print(f"\n[case] kv_swap_blocks hkv={hkv} d={d} bs={bs} layers={layers}", flush=True)
    rng = np.random.default_rng(hkv * 1000 + d + bs + layers)
    nb, nh = 37, 29
    dev_np = [(_bits(rng, (nb, hkv, bs, d)), _bits(rng, (nb, hkv, bs, d))) for _ in range(layers)]
    host_np = [(_bits(rng, (nh, hkv, bs, d)), _bits(rng, (nh, hkv, bs, d))) for _ in range(layers)]
    dev_k = [torch.from_numpy(k).cuda() for k, _ in dev_np]
    dev_v = [torch.from_numpy(v).cuda() for _, v in dev_np]
    host_k = [torch.from_numpy(k.copy()).pin_memory() for k, _ in host_np]
    host_v = [torch.from_numpy(v.copy()).pin_memory() for _, v in host_np]

    # Out: device -> host, distinct host destinations, a device source used twice.
    dst = rng.permutation(nh)[:20]
    src = rng.integers(0, nb, size=20)
    src[5] = src[2]
    pairs_out = np.stack([src, dst], axis=1).astype(np.int32)
    bad = np.array([[nb, 0], [-1, 1], [0, nh]], dtype=np.int32)      # skipped by the kernel
    _lib.kv_swap_blocks(host_k, host_v, dev_k, dev_v,
                        torch.from_numpy(np.concatenate([pairs_out, bad])).cuda())
    torch.cuda.synchronize()
    oc.copy_blocks_between(dev_np, host_np, pairs_out)
    for l in range(layers):
        assert np.array_equal(host_k[l].numpy().view(np.uint16), host_np[l][0].view(np.uint16))
        assert np.array_equal(host_v[l].numpy().view(np.uint16), host_np[l][1].view(np.uint16))

    # In: host -> device.
    dst = rng.permutation(nb)[:25]
    src = rng.integers(0, nh, size=25)
    pairs_in = np.stack([src, dst], axis=1).astype(np.int32)
    _lib.kv_swap_blocks(dev_k, dev_v, host_k, host_v, torch.from_numpy(pairs_in).cuda())
    torch.cuda.synchronize()
    oc.copy_blocks_between(host_np, dev_np, pairs_in)
    for l in range(layers):
        assert np.array_equal(dev_k[l].cpu().numpy().view(np.uint16), dev_np[l][0].view(np.uint16))
        assert np.array_equal(dev_v[l].cpu().numpy().view(np.uint16), dev_np[l][1].view(np.uint16))


def test_swap_blocks_refuses_memory_it_cannot_address():
    import torch

    print("\n[case] kv_swap_blocks argument checks", flush=True)
    dev = torch.zeros((4, 2, 16, 64), dtype=torch.float16, device="cuda")
    pageable = np.zeros((4, 2, 16, 64), dtype=np.float16)
    pairs = torch.tensor([[0, 1]], dtype=torch.int32, device="cuda")
    lib = _lib.lib()
    arr = lambda p: (ctypes.c_void_p * 1)(p)  # noqa: E731
    s = torch.cuda.current_stream().cuda_stream
    before = dev.clone()
    rc = lib.kv_swap_blocks(arr(pageable.ctypes.data), arr(pageable.ctypes.data), 4,
                            arr(dev.data_ptr()), arr(dev.data_ptr()), 4, 1, pairs.data_ptr(), 1, 2,
                            64, 16, s)
    assert rc == _lib.PKV_ERR_INVALID_ARG
    rc = lib.kv_swap_blocks(arr(dev.data_ptr()), arr(dev.data_ptr()), 4, arr(dev.data_ptr() + 2),
                            arr(dev.data_ptr()), 4, 1, pairs.data_ptr(), 1, 2, 64, 16, s)
    assert rc == _lib.PKV_ERR_INVALID_ARG                              # misaligned
    rc = lib.kv_swap_blocks(arr(dev.data_ptr()), arr(dev.data_ptr()), 4, arr(dev.data_ptr()),
                            arr(dev.data_ptr()), 4, 1, pairs.data_ptr(), 1, 2, 96, 16, s)
    assert rc == _lib.PKV_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(dev, before)
    with pytest.raises(TypeError):
        _lib.kv_swap_blocks([torch.from_numpy(pageable)], [torch.from_numpy(pageable)], [dev], [dev],
                            pairs)


def _fill(c, seqs, counts, rng):
    """Reserve and write random K/V for counts[i] more tokens of seqs[i]; returns the
    tokens per request (host arrays)."""
    import torch

    slots = c.reserve_many(seqs, counts)
    tot = int(sum(counts))
    k = rng.standard_normal((tot, c.num_kv_heads, c.head_dim)).astype(np.float16)
    v = rng.standard_normal((tot, c.num_kv_heads, c.head_dim)).astype(np.float16)
    for layer in range(len(c.k)):
        c.write(slots, torch.from_numpy(k + layer).cuda(), torch.from_numpy(v - layer).cuda(),
                layer=layer)
    out, o = {}, 0
    for s, n in zip(seqs, counts):
        out[s] = (k[o:o + n], v[o:o + n])
        o += n
    return out


def _decode_all(c, seqs, q, scale, layers):
    batch = c.batch(seqs)
    return [c.attend(q, batch, scale, layer=l).cpu().numpy() for l in range(layers)]


@pytest.mark.parametrize("deferred", [False, True])
def test_cache_round_trip_keeps_every_request(deferred):
    import torch

    from paged_kv_cache_244_amd.cache import PagedKVCache

    print(f"\n[case] cache swap round trip deferred={deferred}", flush=True)
    rng = np.random.default_rng(17)
    hq, hkv, d, bs, layers = 32, 8, 128, 16, 2
    nb, nh = 400, 300
    c = PagedKVCache(nb, hkv, d, bs, num_layers=layers, initial_order=rng.permutation(nb),
                     num_q_heads=hq, host_blocks=nh, host_order=rng.permutation(nh))
    # A: alone; P forked into three samples that then diverge; C: long.
    a, p, cc = c.new_sequence(), c.new_sequence(), c.new_sequence()
    toks = {}
    toks.update(_fill(c, [a, p, cc], [300, 100, 1000], rng))
    samples = [c.fork(p) for _ in range(3)]
    for s in samples:
        toks[s] = tuple(x.copy() for x in toks[p])
    c.free(p)
    more = _fill(c, samples, [5, 17, 1], rng)
    for s in samples:
        toks[s] = (np.concatenate([toks[s][0], more[s][0]]), np.concatenate([toks[s][1], more[s][1]]))
    live = [a, cc] + samples
    q = torch.from_numpy(rng.standard_normal((len(live), hq, d)).astype(np.float16)).cuda()
    scale = 1.0 / np.sqrt(d)
    before = _decode_all(c, live, q, scale, layers)

    moved = [cc] + samples
    shared_prompt_blocks = 100 // bs                     # the 6 full prompt blocks
    distinct = -(-1000 // bs) + sum(-(-(100 + n) // bs) for n in (5, 17, 1)) - 2 * shared_prompt_blocks
    used_before = c.alloc.stats()["used_blocks"]
    copied = c.swap_out(moved, deferred=deferred)
    st = c.alloc.stats()
    assert copied == distinct and st["host_used_blocks"] == distinct
    assert st["swapped_seqs"] == 4 and st["used_blocks"] == used_before - distinct
    with pytest.raises(_lib.Swapped):
        c.batch([cc])

    # Another request takes the freed device blocks and overwrites them.
    if deferred:
        c.retire(wait=True)
    x = c.new_sequence()
    junk = nb - c.alloc.stats()["used_blocks"] - 1
    slots = c.reserve(x, junk * bs)
    fill = torch.full((junk * bs, hkv, d), 1e4, dtype=torch.float16, device="cuda")
    for layer in range(layers):
        c.write(slots, fill, fill, layer=layer)
    c.free(x)

    assert c.swap_in(moved, deferred=deferred) == distinct
    assert c.alloc.stats()["host_used_blocks"] == 0
    after = _decode_all(c, live, q, scale, layers)
    torch.cuda.synchronize()
    for l in range(layers):
        assert np.array_equal(before[l].view(np.uint32), after[l].view(np.uint32)), f"layer {l}"
        for i, s in enumerate(live):
            k, v = toks[s]
            want = attention.attend_one(q[i].cpu().numpy(), k + l, v - l, scale)
            paths.assert_attention_close(after[l][i], want)
    c.retire(wait=True)


def test_deferred_swap_out_with_a_second_stream():
    import torch

    from paged_kv_cache_244_amd.cache import PagedKVCache

    print("\n[case] deferred swap-out, two streams", flush=True)
    rng = np.random.default_rng(29)
    hq, hkv, d, bs = 8, 2, 128, 16
    lx, ly = 2000, 800
    nbx, nby = -(-lx // bs), -(-ly // bs)
    nb = nbx + nby + 3
    c = PagedKVCache(nb, hkv, d, bs, initial_order=np.arange(nb), num_q_heads=hq,
                     host_blocks=nbx)
    x = c.new_sequence()
    toks = _fill(c, [x], [lx], rng)[x]
    x_blocks = set(c.alloc.export([x], nbx, -1)[0][0].tolist())
    c.swap_out([x], deferred=True)                      # the host does not wait
    assert c.alloc.stats()["pending_blocks"] == nbx
    y = c.new_sequence()
    y_slots, pairs = c.alloc.append(y, ly)
    assert not pairs
    assert not (set(c.alloc.export([y], nby, -1)[0][0].tolist()) & x_blocks), \
        "a block still being copied out was handed out"
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        junk = torch.full((ly, hkv, d), 1e4, dtype=torch.float16, device="cuda")
        _lib.kv_cache_write(c.k[0], c.v[0], junk, junk, torch.from_numpy(y_slots).cuda(),
                            stream=side)
    torch.cuda.synchronize()
    c.free(y)
    assert c.retire(wait=True) == nbx
    c.swap_in([x])
    q = torch.from_numpy(rng.standard_normal((1, hq, d)).astype(np.float16)).cuda()
    got = _decode_all(c, [x], q, 1.0 / np.sqrt(d), 1)[0][0]
    want = attention.attend_one(q[0].cpu().numpy(), toks[0], toks[1], 1.0 / np.sqrt(d))
    paths.assert_attention_close(got, want)


def test_swap_workload_full_size_round_trip():
    """The benchmark's swap set (every other request of the OPT-13B decode batch,
    40 x 128 heads, B = 16) out to the host tier and back, twice: every moved
    request's logical K and V, gathered through its table, are bitwise what they
    were, and the requests that stayed are untouched."""
    import torch

    from paged_kv_cache_244_amd import workloads
    from paged_kv_cache_244_amd.cache import PagedKVCache

    print("\n[case] swap full-size OPT-13B set", flush=True)
    w = workloads.opt13b()
    lens = [int(L) for L in w.lengths]
    bs = w.block_size
    moved_idx = list(range(0, len(lens), 2))
    moved_blocks = sum(-(-lens[i] // bs) for i in moved_idx)
    dev = torch.device("cuda")
    c = PagedKVCache(w.num_blocks, w.num_kv_heads, w.head_dim, bs, initial_order=w.initial_order,
                     num_q_heads=w.num_q_heads, host_blocks=moved_blocks)
    seqs = [c.new_sequence() for _ in lens]
    c.write(c.reserve_many(seqs, lens), torch.from_numpy(w.k_tokens).to(dev),
            torch.from_numpy(w.v_tokens).to(dev))

    def logical(seq):
        tables, _ = c.alloc.export([seq], c.alloc.num_blocks, 0)
        n = c.length(seq)
        t = torch.arange(n, device=dev)
        blocks = torch.from_numpy(tables[0]).to(dev).long()[t // bs]
        return c.k[0][blocks, :, t % bs, :], c.v[0][blocks, :, t % bs, :]

    before = {s: logical(s) for s in seqs}
    moved = [seqs[i] for i in moved_idx]
    for _ in range(2):
        assert c.swap_out(moved) == moved_blocks
        assert c.swap_in(moved) == moved_blocks
    torch.cuda.synchronize()
    for s in seqs:
        k, v = logical(s)
        assert torch.equal(k.view(torch.int16), before[s][0].view(torch.int16)), f"request {s}: K"
        assert torch.equal(v.view(torch.int16), before[s][1].view(torch.int16)), f"request {s}: V"
    st = c.alloc.stats()
    assert st["swapped_out_blocks"] == st["swapped_in_blocks"] == 2 * moved_blocks


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_histories_with_swaps(seed):
    """Random histories on a PagedKVCache with a host tier: new requests, appends of
    real tokens, forks, frees, swap-outs and swap-ins of random subsets (some
    deferred, retired later), all queued on one stream.  The test keeps each
    request's token list itself.  Every few operations every live request is
    checked: a swapped one through its host-tier table (bitwise), a resident one by
    decode attention against the oracle on its token list.  Swapped requests are
    checked once they are back (at later checkpoints, and all of them at the end)."""
    import torch

    from paged_kv_cache_244_amd.cache import PagedKVCache

    print(f"\n[case] random swap histories seed={seed}", flush=True)
    rng = np.random.default_rng(300 + seed)
    hq, hkv, d, bs, nb, nh = 8, 2, 64, 8, 160, 120
    c = PagedKVCache(nb, hkv, d, bs, initial_order=rng.permutation(nb), num_q_heads=hq,
                     host_blocks=nh, host_order=rng.permutation(nh))
    truth = {}

    def append(s, n):
        k = rng.standard_normal((n, hkv, d)).astype(np.float16)
        v = rng.standard_normal((n, hkv, d)).astype(np.float16)
        c.write(c.reserve(s, n), torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
        truth[s] = (np.concatenate([truth[s][0], k]), np.concatenate([truth[s][1], v]))

    def check():
        resident = [s for s in truth if not c.is_swapped(s) and len(truth[s][0])]
        if resident:
            q = torch.from_numpy(rng.standard_normal((len(resident), hq, d)).astype(np.float16)).cuda()
            got = c.attend(q, c.batch(resident), 1.0 / np.sqrt(d)).cpu().numpy()
            for i, s in enumerate(resident):
                want = attention.attend_one(q[i].cpu().numpy(), truth[s][0], truth[s][1],
                                            1.0 / np.sqrt(d))
                paths.assert_attention_close(got[i], want)

    for step in range(120):
        live = list(truth)
        resident = [s for s in live if not c.is_swapped(s)]
        swapped = [s for s in live if c.is_swapped(s)]
        op = int(rng.integers(8))
        try:
            if op == 0 or not live:
                s = c.new_sequence()
                truth[s] = (np.zeros((0, hkv, d), np.float16), np.zeros((0, hkv, d), np.float16))
                append(s, int(rng.integers(1, 40)))
            elif op in (1, 2) and resident:
                append(resident[rng.integers(len(resident))], int(rng.integers(1, 12)))
            elif op == 3 and resident:
                src = resident[rng.integers(len(resident))]
                child = c.fork(src)
                truth[child] = tuple(x.copy() for x in truth[src])
            elif op == 4:
                s = live[rng.integers(len(live))]
                c.free(s, deferred=bool(rng.random() < 0.5))
                del truth[s]
            elif op == 5 and resident:
                k = int(rng.integers(1, len(resident) + 1))
                pick = [resident[i] for i in rng.choice(len(resident), size=k, replace=False)]
                c.swap_out(pick, deferred=bool(rng.random() < 0.5))
            elif op == 6 and swapped:
                k = int(rng.integers(1, len(swapped) + 1))
                pick = [swapped[i] for i in rng.choice(len(swapped), size=k, replace=False)]
                c.swap_in(pick, deferred=bool(rng.random() < 0.5))
            else:
                c.retire(wait=bool(rng.random() < 0.3))
        except (_lib.OutOfBlocks, _lib.Swapped):
            pass
        if step % 15 == 14:
            check()
    while True:                              # everything back on the device, room permitting
        try:
            c.swap_in([s for s in truth if c.is_swapped(s)])
            break
        except _lib.OutOfBlocks:
            victim = next(s for s in truth if not c.is_swapped(s))
            c.free(victim)
            del truth[victim]
    check()
    torch.cuda.synchronize()
    st = c.alloc.stats()
    assert st["swapped_seqs"] == 0 and st["host_used_blocks"] == 0
    assert st["swapped_out_blocks"] > 20 and st["swapped_in_blocks"] > 20, st   # it did swap
