"""CPU model of the prefill indexer's per-query candidate buffer.

The kernel appends, tile by tile, the keys above its running threshold to a
buffer of 3072 entries.  When the next tile's candidates would not fit, a
radix select keeps the k best, but it may stop early and keep up to
k + 256 entries (its slack), after which the tile's at most 64 candidates are
appended.  This model runs the same stopping rule (8-bit digits of
key - min(key) from the highest bit in which the entries differ) on
adversarial key streams and checks that the buffer never overflows for the
largest k the library accepts, 2752.  It also shows that the earlier limit
(3008) could overflow.
"""
import ctypes

import numpy as np
import pytest

from sparse_attention_04_amd import binding as B

CAP, SLACK, TILE = 3072, 256, 64
M32 = 0xFFFFFFFF


def select(keys, need, exact):
    """Indices (list order) the kernel's select keeps, and the smallest kept key."""
    mn, mx = min(keys), max(keys)
    y = [k - mn for k in keys]
    rng = mx - mn
    hi = rng.bit_length() - 1 if rng else -1
    prefix = 0
    pmask = (~(((2 << hi) - 1) & M32)) & M32 if hi >= 0 else M32
    rem, keep_all = need, False
    while hi >= 0:
        lo = max(hi - 7, 0)
        dmask = (2 << (hi - lo)) - 1
        hist = [0] * 256
        for v in y:
            if (v & pmask) == prefix:
                hist[(v >> lo) & dmask] += 1
        run = 0
        for b in range(255, -1, -1):
            if run + hist[b] >= rem:
                binabove, bc, bin_ = run, hist[b], b
                break
            run += hist[b]
        rem -= binabove
        prefix |= bin_ << lo
        pmask |= dmask << lo
        hi = lo - 1
        if bc == rem or (not exact and bc - rem <= SLACK):
            keep_all = True
            break
    kept, ties = [], 0
    for i, v in enumerate(y):
        ym = v & pmask
        if ym > prefix or (ym == prefix and (keep_all or ties < rem)):
            kept.append(i)
        if ym == prefix:
            ties += 1
    return kept, min(keys[i] for i in kept)


def max_fill(stream, k):
    """Largest buffer occupancy over a stream of positive keys (position order)."""
    cand, thr, worst = [], 0, 0
    for t0 in range(0, len(stream), TILE):
        tile = stream[t0:t0 + TILE]
        new = [x for x in tile if x > thr]
        if len(cand) + len(new) > CAP:
            kept, thr = select(cand, k, exact=False)
            cand = [cand[i] for i in kept]
            new = [x for x in tile if x > thr]
        cand += new
        worst = max(worst, len(cand))
    return worst


def streams(n, seed):
    r = np.random.default_rng(seed)
    yield list(range(1, n + 1))                                   # rising: every key a candidate
    yield [int(x) for x in r.integers(1, 1 << 31, n)]              # random
    # rising blocks whose low bits collide: the select's boundary bin stays
    # crowded for several digits before it can stop
    yield [(1 << 20) + (i // 300) * 512 + int(r.integers(0, 300)) for i in range(n)]
    yield [(1 << 24) + i // 16 for i in range(n)]                  # runs of 16 equal keys
    yield [(1 << 24) + (i // 290) * 290 + int(r.integers(0, 290)) for i in range(n)]


@pytest.mark.parametrize("seed", [0, 1])
def test_buffer_never_overflows_at_largest_k(seed):
    k = CAP - SLACK - TILE
    assert k == 2752
    for s in streams(12000, seed):
        assert max_fill(s, k) <= CAP


def test_earlier_limit_could_overflow():
    worst = max(max_fill(s, 3008) for s in streams(12000, 0))
    assert worst > CAP


def test_select_keeps_the_best_within_the_slack():
    r = np.random.default_rng(3)
    for _ in range(20):
        keys = [int(x) for x in r.integers(1, 5000, 3000)]
        need = int(r.integers(1, 2900))
        for exact in (True, False):
            kept, thr = select(keys, need, exact)
            order = sorted(range(len(keys)), key=lambda i: (-keys[i], i))
            best = set(order[:need])
            assert best <= set(kept)
            assert len(kept) == need if exact else need <= len(kept) <= need + SLACK


def test_abi_refuses_prefill_topk_above_bound():
    fake = 0x1000
    batch = B.dsa_batch(1, fake, fake, fake, 64, 100, 100, 4096)
    kc = B.dsa_paged_cache(fake, None, B.DSA_BF16, 64, 64, 128)
    ia = B.dsa_indexer_args(fake, B.DSA_BF16, None, fake, 64, 128, 2753, ctypes.pointer(kc))
    vc = B.dsa_paged_cache(fake, None, B.DSA_BF16, 64, 64, 576)
    sa = B.dsa_sfa_args(fake, B.DSA_BF16, 128, 576, 512, 0.07, ctypes.pointer(vc))
    need = B.dsa_workspace_size(B.DSA_OP_FUSED_PREFILL, batch, ia, sa)
    st = B.lib().dsa_fused_prefill(ctypes.pointer(batch), ctypes.pointer(ia), ctypes.pointer(sa), 64,
                                   ctypes.c_void_p(0x2000), None, None, ctypes.c_void_p(0x3000), need, None)
    assert st == B.DSA_ERR_UNSUPPORTED, B.lib().dsa_last_error()
    assert b"2752" in B.lib().dsa_last_error()


def test_abi_refuses_mx_prefill_with_unaligned_key_scales():
    """The MXFP8 prefill indexer reads each row's four e8m0 bytes as one 4-byte
    word: a scale pool that is not 4-byte aligned is refused before any launch."""
    fake = 0x1000
    batch = B.dsa_batch(1, fake, fake, fake, 100, 100, 100, 4096)
    kc = B.dsa_paged_cache(fake, ctypes.c_void_p(0x2001), B.DSA_MXFP8_E4M3, 64, 64, 128)
    ia = B.dsa_indexer_args(fake, B.DSA_MXFP8_E4M3, ctypes.c_void_p(0x3000), fake, 64, 128, 2048, ctypes.pointer(kc))
    vc = B.dsa_paged_cache(fake, None, B.DSA_BF16, 64, 64, 576)
    sa = B.dsa_sfa_args(fake, B.DSA_BF16, 128, 576, 512, 0.07, ctypes.pointer(vc))
    need = B.dsa_workspace_size(B.DSA_OP_FUSED_PREFILL, batch, ia, sa)
    st = B.lib().dsa_fused_prefill(ctypes.pointer(batch), ctypes.pointer(ia), ctypes.pointer(sa), 64,
                                   ctypes.c_void_p(0x2000), None, None, ctypes.c_void_p(0x3000), need, None)
    assert st == B.DSA_ERR_INVALID_ARG, B.lib().dsa_last_error()
    assert b"4-byte" in B.lib().dsa_last_error()
