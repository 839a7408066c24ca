"""CPU model of the decode indexer's boundary-bin choice (the last workgroup's
selection after the first radix pass), checked against a full sort.

The kernel turns each candidate (32-bit orderable key whose top 11 bits all
candidates share, position) into the 52-bit composite

    (key & 0x1FFFFF) << 31  |  (2^31 - 1 - position)

and runs a radix select over it with digits of 11, 11, 11, 11 and 8 bits from
the top, stopping once the boundary digit's candidates are all needed.  This
model follows the same digits and stopping rule in Python, so a wrong shift,
width or stopping condition in the scheme shows up here: the chosen set must
be the m largest keys, and among equal keys the m smallest positions (the
oracle's order), for any m in 1 .. n - 1.
"""
import numpy as np
import pytest

DIGITS = [(41, 0x7FF), (30, 0x7FF), (19, 0x7FF), (8, 0x7FF), (0, 0xFF)]


def composite(keys, pos):
    return ((keys.astype(np.uint64) & np.uint64(0x1FFFFF)) << np.uint64(31)) | \
        (np.uint64(0x7FFFFFFF) - pos.astype(np.uint64))


def model_select(keys, pos, m):
    c = composite(keys, pos)
    pre, pm, need = np.uint64(0), np.uint64(0), m
    for shift, dmask in DIGITS:
        inreg = (c & pm) == pre
        d = ((c[inreg] >> np.uint64(shift)) & np.uint64(dmask)).astype(np.int64)
        h = np.bincount(d, minlength=2048)
        above = np.cumsum(h[::-1])[::-1] - h          # counts in the bins above each bin
        b = int(np.nonzero((above < need) & (need <= above + h))[0][0])
        need -= int(above[b])
        pre |= np.uint64(b) << np.uint64(shift)
        pm |= np.uint64(dmask) << np.uint64(shift)
        if h[b] == need:
            break
    chosen = (c & pm) >= pre
    return np.sort(pos[chosen])


def reference(keys, pos, m):
    order = np.lexsort((pos, -keys.astype(np.int64)))   # key descending, then position ascending
    return np.sort(pos[order[:m]])


def _case(rng, n, kind):
    top = np.uint32(rng.integers(0, 2048)) << np.uint32(21)
    if kind == "random":
        low = rng.integers(0, 1 << 21, n)
    elif kind == "equal":
        low = np.full(n, rng.integers(0, 1 << 21))
    elif kind == "few":
        low = rng.choice(rng.integers(0, 1 << 21, 3), n)
    else:   # low bits only
        low = rng.integers(0, 4, n)
    keys = top | low.astype(np.uint32)
    pos = rng.choice(1 << 31, n, replace=False) if kind != "low" else rng.permutation(n).astype(np.int64) + (1 << 31) - n
    return keys.astype(np.uint32), pos.astype(np.int64)


@pytest.mark.parametrize("kind", ["random", "equal", "few", "low"])
def test_composite_select_matches_sort(kind):
    rng = np.random.default_rng(7)
    for n in (2, 3, 65, 1000, 3072):
        keys, pos = _case(rng, n, kind)
        for m in sorted({1, n // 2, n - 1, int(rng.integers(1, n))}):
            if not 1 <= m < n:
                continue
            assert np.array_equal(model_select(keys, pos, m), reference(keys, pos, m)), (kind, n, m)


def test_digits_cover_the_composite():
    """The five digits are disjoint and cover bits 0..51, the composite's width."""
    covered = 0
    for shift, dmask in DIGITS:
        bits = dmask << shift
        assert covered & bits == 0
        covered |= bits
    assert covered == (1 << 52) - 1
