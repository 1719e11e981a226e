"""Pins for the CPU oracle: checks against facts that do not come from the oracle.

Each ``pin_*`` takes an ``impl`` namespace exposing ``attend_one``,
``attend_paged``, ``gather_logical``, ``write_slots`` and ``copy_blocks`` (the
oracle's functions, or a deliberately broken copy in the mutant test) and
raises ``AssertionError`` when the implementation disagrees with:

* closed forms of the attention definition (one token, zero query, equal keys,
  two tokens, the hard-max limit, a constant shift of every score);
* a library routine (torch float64 ``scaled_dot_product_attention`` on the
  contiguous layout, with its own grouped-query head mapping);
* pure-Python brute force with ``math.fsum`` on tiny inputs;
* invariants: paged == contiguous under any physical placement, invariance
  under permuting the logical token order, head grouping;
* the pool geometry fixed by a reshape of an identity placement.
"""

import math

import numpy as np
import torch


def _rand_case(rng, L, Hq, Hkv, D):
    q = rng.standard_normal((Hq, D))
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    return q, k, v


def pin_single_token(impl, rng):
    """L = 1: the only probability is 1, so the output is that token's value, exactly."""
    q, k, v = _rand_case(rng, 1, 4, 2, 16)
    out = impl.attend_one(q, k, v, 0.25)
    for h in range(4):
        assert np.array_equal(out[h], v[0, h // 2]), "L=1 must return v0"


def pin_zero_query_is_mean(impl, rng):
    """q = 0 makes every score equal, so the output is the mean of the values."""
    _, k, v = _rand_case(rng, 11, 2, 2, 8)
    out = impl.attend_one(np.zeros((2, 8)), k, v, 0.5)
    np.testing.assert_allclose(out, v.mean(axis=0), rtol=0, atol=1e-14)


def pin_equal_keys_is_mean(impl, rng):
    """Identical keys give identical scores, whatever q is: output = mean(V)."""
    q, k, v = _rand_case(rng, 9, 3, 3, 8)
    k[:] = k[0]
    out = impl.attend_one(q, k, v, 0.3)
    np.testing.assert_allclose(out, v.mean(axis=0), rtol=0, atol=1e-13)


def pin_two_tokens_logistic(impl, rng):
    """L = 2: softmax reduces to the logistic function of the score difference."""
    q, k, v = _rand_case(rng, 2, 2, 1, 8)
    scale = 0.7
    out = impl.attend_one(q, k, v, scale)
    s = np.float64(np.float32(scale))
    for h in range(2):
        d = s * (q[h] @ k[0, 0]) - s * (q[h] @ k[1, 0])
        w0 = 1.0 / (1.0 + math.exp(-d))
        want = w0 * v[0, 0] + (1.0 - w0) * v[1, 0]
        np.testing.assert_allclose(out[h], want, rtol=0, atol=1e-14)


def pin_hard_max_limit(impl, rng):
    """With scores far apart the softmax becomes one-hot on the largest score.

    Token t gets key t * e_0 and q = e_0, so score t * scale; with scale 1000
    the last token wins by 1000 per step and every other weight underflows to 0.
    """
    L, D = 6, 4
    k = np.zeros((L, 1, D))
    k[:, 0, 0] = np.arange(L)
    v = rng.standard_normal((L, 1, D))
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    out = impl.attend_one(q, k, v, 1000.0)
    assert np.array_equal(out[0], v[L - 1, 0]), "largest score must win"
    out_neg = impl.attend_one(-q, k, v, 1000.0)
    assert np.array_equal(out_neg[0], v[0, 0]), "negated query picks the smallest key"


def pin_score_shift_invariance(impl, rng):
    """Adding c*q/|q|^2 to every key shifts every score by scale*c: output unchanged."""
    q, k, v = _rand_case(rng, 13, 1, 1, 8)
    base = impl.attend_one(q, k, v, 0.5)
    k2 = k + 40.0 * q[0] / (q[0] @ q[0])
    shifted = impl.attend_one(q, k2, v, 0.5)
    np.testing.assert_allclose(shifted, base, rtol=0, atol=1e-12)


def pin_scale_applied(impl, rng):
    """attend(q, scale=s) == attend(s*q, scale=1) for s exact in float32."""
    q, k, v = _rand_case(rng, 10, 2, 2, 8)
    a = impl.attend_one(q, k, v, 0.375)
    b = impl.attend_one(0.375 * q, k, v, 1.0)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    c = impl.attend_one(q, k, v, 1.0)
    assert np.abs(a - c).max() > 1e-3, "scale must change the result"


def pin_torch_sdpa(impl, rng):
    """Library routine: torch fp64 SDPA over the contiguous layout, GQA by the library."""
    for (L, Hq, Hkv, D) in [(1, 2, 2, 8), (37, 8, 2, 16), (100, 4, 4, 64), (5, 4, 1, 8)]:
        q, k, v = _rand_case(rng, L, Hq, Hkv, D)
        scale = float(np.float32(1.0 / math.sqrt(D)))
        out = impl.attend_one(q, k, v, scale)
        tq = torch.from_numpy(q)[None, :, None, :]                      # [1, Hq, 1, D]
        tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]  # [1, Hkv, L, D]
        tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, scale=scale, enable_gqa=True)[0, :, 0, :].numpy()
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def pin_head_grouping(impl, rng):
    """KV head g holds the constant value g+1, so query head h must return h//G + 1."""
    L, Hq, Hkv, D = 7, 8, 2, 4
    q, k, _ = _rand_case(rng, L, Hq, Hkv, D)
    v = np.zeros((L, Hkv, D))
    for g in range(Hkv):
        v[:, g, :] = g + 1
    out = impl.attend_one(q, k, v, 0.5)
    for h in range(Hq):
        np.testing.assert_allclose(out[h], h // (Hq // Hkv) + 1, rtol=0, atol=1e-14)


def _brute(q, k, v, scale):
    s64 = float(np.float32(scale))
    L, Hkv, D = k.shape
    Hq = q.shape[0]
    out = [[0.0] * D for _ in range(Hq)]
    for h in range(Hq):
        g = h // (Hq // Hkv)
        sc = [s64 * math.fsum(float(q[h, d]) * float(k[t, g, d]) for d in range(D)) for t in range(L)]
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        z = math.fsum(w)
        for d in range(D):
            out[h][d] = math.fsum(w[t] * float(v[t, g, d]) for t in range(L)) / z
    return np.array(out)


def pin_brute_force(impl, rng):
    """Pure-Python loops with math.fsum on tiny inputs."""
    for (L, Hq, Hkv, D) in [(1, 1, 1, 1), (3, 2, 1, 4), (8, 4, 2, 8), (5, 2, 2, 3)]:
        q, k, v = _rand_case(rng, L, Hq, Hkv, D)
        np.testing.assert_allclose(impl.attend_one(q, k, v, 0.6), _brute(q, k, v, 0.6),
                                   rtol=0, atol=1e-14)


def pin_logical_permutation(impl, rng):
    """Attention is a sum over tokens: reordering K and V together changes nothing."""
    q, k, v = _rand_case(rng, 29, 4, 2, 16)
    perm = rng.permutation(29)
    a = impl.attend_one(q, k, v, 0.25)
    b = impl.attend_one(q, k[perm], v[perm], 0.25)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def _scatter(impl, k_tok, v_tok, placement, B, NB):
    """Place one request's tokens with the write oracle: logical block j -> placement[j]."""
    L, Hkv, D = k_tok.shape
    kp = np.full((NB, Hkv, B, D), np.nan, dtype=np.float16)
    vp = np.full((NB, Hkv, B, D), np.nan, dtype=np.float16)
    slots = [int(placement[t // B]) * B + t % B for t in range(L)]
    impl.write_slots(kp, vp, k_tok, v_tok, slots, B)
    return kp, vp


def pin_identity_placement_is_reshape(impl, rng):
    """With block j at physical j, the pool transposed to [NB, B, Hkv, D] and flattened
    over (NB, B) is the logical sequence — a library reshape, not the oracle's indexing."""
    L, Hkv, D, B, NB = 45, 3, 8, 8, 6
    k = rng.standard_normal((L, Hkv, D)).astype(np.float16)
    v = rng.standard_normal((L, Hkv, D)).astype(np.float16)
    kp, vp = _scatter(impl, k, v, np.arange(NB), B, NB)
    flat_k = kp.transpose(0, 2, 1, 3).reshape(NB * B, Hkv, D)[:L]
    flat_v = vp.transpose(0, 2, 1, 3).reshape(NB * B, Hkv, D)[:L]
    assert np.array_equal(flat_k, k) and np.array_equal(flat_v, v)
    g = impl.gather_logical(kp, np.arange(NB), L, B)
    assert np.array_equal(g, k)


def pin_paged_equals_contiguous(impl, rng):
    """Any physical placement gives bitwise the same output as the contiguous layout;
    unused slots (NaN) and table padding (an out-of-range id) are never read."""
    B, NB, Hq, Hkv, D = 16, 40, 4, 2, 32
    for L in (1, 15, 16, 17, 33, 100):
        k = rng.standard_normal((L, Hkv, D)).astype(np.float16)
        v = rng.standard_normal((L, Hkv, D)).astype(np.float16)
        q = rng.standard_normal((1, Hq, D)).astype(np.float32)
        want = impl.attend_one(q[0], k, v, 0.125)
        for _ in range(3):
            placement = rng.permutation(NB)
            kp, vp = _scatter(impl, k, v, placement, B, NB)
            nb = (L + B - 1) // B
            table = np.full((1, 10), 10 ** 6, dtype=np.int64)
            table[0, :nb] = placement[:nb]
            got = impl.attend_paged(q, kp, vp, table, [L], B, 0.125)
            assert np.array_equal(got[0], want), f"paged != contiguous at L={L}"


def pin_contiguous_rows(impl, rng):
    """The layout without a block table: rows built from the logical tokens by a
    library transpose, padded with NaN past each length (never read), give bitwise
    the output of attend_one on the logical tokens, request by request."""
    S, Hq, Hkv, D, Lmax = 4, 6, 3, 8, 48
    lens = [1, 17, 48, 0]
    q = rng.standard_normal((S, Hq, D)).astype(np.float32)
    k_rows = np.full((S, Hkv, Lmax, D), np.nan, dtype=np.float16)
    v_rows = np.full((S, Hkv, Lmax, D), np.nan, dtype=np.float16)
    toks = []
    for i, L in enumerate(lens):
        k = rng.standard_normal((L, Hkv, D)).astype(np.float16)
        v = rng.standard_normal((L, Hkv, D)).astype(np.float16)
        k_rows[i, :, :L, :] = k.transpose(1, 0, 2)
        v_rows[i, :, :L, :] = v.transpose(1, 0, 2)
        toks.append((k, v))
    got = impl.attend_contiguous(q, k_rows, v_rows, lens, 0.25)
    for i, (k, v) in enumerate(toks):
        assert np.array_equal(got[i], impl.attend_one(q[i], k, v, 0.25)), f"row {i}"
    assert np.array_equal(got[3], np.zeros((Hq, D)))


def _prefill_case(impl, rng, lens, qlens, Hq, Hkv, D, B):
    """Requests scattered through random placements; q rows are each request's
    last qlens[i] positions."""
    NB = sum(-(-L // B) for L in lens) + 3
    kp = np.full((NB, Hkv, B, D), np.nan, dtype=np.float16)
    vp = np.full((NB, Hkv, B, D), np.nan, dtype=np.float16)
    perm = rng.permutation(NB)
    tables = np.full((len(lens), NB), 10 ** 6, dtype=np.int64)
    toks, used = [], 0
    for i, L in enumerate(lens):
        k = rng.standard_normal((L, Hkv, D)).astype(np.float16)
        v = rng.standard_normal((L, Hkv, D)).astype(np.float16)
        nb = -(-L // B)
        place = perm[used:used + nb]
        used += nb
        tables[i, :nb] = place
        slots = [int(place[t // B]) * B + t % B for t in range(L)]
        impl.write_slots(kp, vp, k, v, slots, B)
        toks.append((k, v))
    starts = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int64)
    q = rng.standard_normal((int(starts[-1]), Hq, D)).astype(np.float16)
    return kp, vp, tables, starts, q, toks


def pin_prefill_torch_causal_sdpa(impl, rng):
    """Library routine: torch fp64 SDPA with is_causal over the logical tokens (a full
    prompt, Q = L), GQA by the library."""
    for (L, Hq, Hkv, D, B) in [(1, 2, 2, 8, 4), (37, 8, 2, 16, 8), (50, 4, 4, 32, 16)]:
        kp, vp, tables, starts, q, toks = _prefill_case(impl, rng, [L], [L], Hq, Hkv, D, B)
        scale = float(np.float32(1.0 / math.sqrt(D)))
        out = impl.attend_prefill_paged(q, kp, vp, tables, [L], starts, B, scale)
        k, v = toks[0]
        tq = torch.from_numpy(np.ascontiguousarray(q.astype(np.float64).transpose(1, 0, 2)))[None]
        tk = torch.from_numpy(np.ascontiguousarray(k.astype(np.float64).transpose(1, 0, 2)))[None]
        tv = torch.from_numpy(np.ascontiguousarray(v.astype(np.float64).transpose(1, 0, 2)))[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, scale=scale, is_causal=True, enable_gqa=True)[0].numpy().transpose(1, 0, 2)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def pin_prefill_rows_are_decodes(impl, rng):
    """A query at position p sees exactly tokens 0..p: it equals a decode over the
    first p + 1 tokens (bitwise), and a continued chunk (Q < L) equals the matching
    rows of the full prompt's prefill."""
    lens, Hq, Hkv, D, B = [9, 33, 1], 4, 2, 8, 8
    kp, vp, tables, starts, q, toks = _prefill_case(impl, rng, lens, lens, Hq, Hkv, D, B)
    full = impl.attend_prefill_paged(q, kp, vp, tables, lens, starts, B, 0.3)
    for i, L in enumerate(lens):
        for j in range(L):
            row = int(starts[i]) + j
            want = impl.attend_paged(q[row][None], kp, vp, tables[i:i + 1], [j + 1], B, 0.3)[0]
            assert np.array_equal(full[row], want), f"request {i} query {j}"
    # continued prefill of the last 5 tokens of request 1
    chunk = np.array([0, 5], dtype=np.int64)
    part = impl.attend_prefill_paged(q[int(starts[1]) + 28:int(starts[1]) + 33], kp, vp,
                                     tables[1:2], [33], chunk, B, 0.3)
    assert np.array_equal(part, full[int(starts[1]) + 28:int(starts[1]) + 33])


def pin_zero_length(impl, rng):
    q = rng.standard_normal((1, 2, 8))
    kp = np.full((2, 2, 4, 8), np.nan, dtype=np.float16)
    out = impl.attend_paged(q, kp, kp, np.zeros((1, 2), dtype=np.int64), [0], 4, 1.0)
    assert np.array_equal(out, np.zeros((1, 2, 8)))


def pin_copy_blocks(impl, rng):
    """After copying (src, dst) every layer's dst block equals src; nothing else moves."""
    NB, Hkv, B, D = 8, 2, 4, 8
    layers = [(rng.standard_normal((NB, Hkv, B, D)).astype(np.float16),
               rng.standard_normal((NB, Hkv, B, D)).astype(np.float16)) for _ in range(3)]
    before = [(k.copy(), v.copy()) for k, v in layers]
    impl.copy_blocks(layers, [(1, 5), (2, 7)])
    for (k, v), (k0, v0) in zip(layers, before):
        for src, dst in [(1, 5), (2, 7)]:
            assert np.array_equal(k[dst], k0[src]) and np.array_equal(v[dst], v0[src])
        untouched = [b for b in range(NB) if b not in (5, 7)]
        assert np.array_equal(k[untouched], k0[untouched])
        assert np.array_equal(v[untouched], v0[untouched])


def pin_negative_slot_skipped(impl, rng):
    kp = np.zeros((2, 1, 4, 2), dtype=np.float16)
    vp = np.zeros((2, 1, 4, 2), dtype=np.float16)
    new = np.ones((2, 1, 2), dtype=np.float16)
    impl.write_slots(kp, vp, new, new, [-1, 6], 4)
    assert kp.sum() == 2 and kp[1, 0, 2].tolist() == [1, 1]


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
