"""Pins for the oracle: each check compares one oracle function with something
other than itself (brute-force loops, a library routine, a closed form or an
invariant) and raises AssertionError on disagreement.  They take the function
under test as an argument so that the mutation tests can feed them planted
mistakes and see them fail."""
from __future__ import annotations

import itertools
import math

import numpy as np
import torch


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- scores ---

def brute_scores(q, w, keys):
    """Triple loop in pure Python: score[s] = sum_h w[h] * sum_d q[h][d] * k[s][d]."""
    H, D = len(q), len(q[0])
    out = []
    for s in range(len(keys)):
        tot = 0.0
        for h in range(H):
            dot = 0.0
            for d in range(D):
                dot += float(q[h][d]) * float(keys[s][d])
            tot += float(w[h]) * dot
        out.append(tot)
    return np.array(out)


def pin_indexer_scores(fn):
    for seed, (H, D, n) in enumerate([(1, 1, 1), (3, 5, 7), (4, 8, 13), (2, 16, 3)]):
        r = _rng(100 + seed)
        q = r.standard_normal((H, D))
        w = r.standard_normal(H)            # any sign: no w >= 0 assumption
        keys = r.standard_normal((n, D))
        got = np.asarray(fn(q, w, keys), np.float64)
        ref = brute_scores(q.tolist(), w.tolist(), keys.tolist())
        assert got.shape == (n,), got.shape
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), (got, ref)
    # closed form: one-hot query rows pick key coordinates
    q = np.zeros((2, 4)); q[0, 1] = 1.0; q[1, 3] = 1.0
    w = np.array([2.0, -3.0])
    keys = np.arange(12, dtype=np.float64).reshape(3, 4)
    got = np.asarray(fn(q, w, keys))
    assert np.allclose(got, 2.0 * keys[:, 1] - 3.0 * keys[:, 3]), got


# ------------------------------------------------------------------ top-k ---

def brute_topk(scores, k):
    """Rank definition: position p is kept iff fewer than n positions beat it,
    where s beats p when its score is larger, or equal with a smaller position."""
    n = min(k, len(scores))
    keep = []
    for p in range(len(scores)):
        better = sum(1 for s in range(len(scores))
                     if scores[s] > scores[p] or (scores[s] == scores[p] and s < p))
        if better < n:
            keep.append(p)
    return keep


def pin_topk(fn):
    r = _rng(7)
    cases = []
    for n_pos in [1, 2, 5, 17, 64, 65, 100]:
        for k in [1, 3, 16, 64, 200]:
            cases.append((r.standard_normal(n_pos), k))
    # heavy ties: small integer scores, all-equal and monotone rows
    cases += [(r.integers(0, 3, 50).astype(float), 10),
              (np.zeros(40), 7),
              (np.arange(30, dtype=float), 5),
              (-np.arange(30, dtype=float), 5),
              (np.array([1.0, -0.0, 0.0, -1.0]), 2)]
    for scores, k in cases:
        got = list(np.asarray(fn(scores, k)).tolist())
        ref = brute_topk(list(scores), k)
        assert sorted(got) == ref, (scores, k, got, ref)
        n = min(k, len(scores))
        assert len(got) == n and len(set(got)) == n
        sel = np.zeros(len(scores), bool); sel[got] = True
        if 0 < n < len(scores):
            assert scores[sel].min() >= scores[~sel].max()


# -------------------------------------------------------------- attention ---

def dense_masked_attention(q, all_rows, keep, d_v, scale):
    """Dense attention over every visible row with -inf logits outside ``keep``
    (a different computation from gathering the kept rows first)."""
    z = scale * (q @ all_rows.T)
    mask = np.full(z.shape[1], -np.inf)
    mask[np.asarray(keep, int)] = 0.0
    z = z + mask
    zmax = np.max(z, axis=1, keepdims=True)
    p = np.exp(z - zmax)
    p /= p.sum(axis=1, keepdims=True)
    return p @ all_rows[:, :d_v]


def sdpa_masked(q, all_rows, keep, d_v, scale):
    """torch's scaled_dot_product_attention on the CPU, boolean mask, float64."""
    qt = torch.from_numpy(q)[None, :, None, :]                 # [1][H][1][Dqk]
    kt = torch.from_numpy(all_rows)[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(np.ascontiguousarray(all_rows[:, :d_v]))[None, None].expand(1, q.shape[0], -1, -1)
    m = torch.zeros(all_rows.shape[0], dtype=torch.bool)
    m[torch.as_tensor(np.asarray(keep, int))] = True
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.contiguous(), vt.contiguous(), attn_mask=m[None, None, None, :], scale=scale)
    return out[0, :, 0, :].numpy()


def pin_sparse_attention(fn):
    r = _rng(11)
    for (H, dqk, dv, n_all, n_keep) in [(1, 3, 2, 5, 1), (4, 10, 6, 20, 7), (8, 80, 64, 64, 33)]:
        q = r.standard_normal((H, dqk))
        rows = r.standard_normal((n_all, dqk))
        keep = np.sort(r.choice(n_all, n_keep, replace=False))
        scale = 1.0 / math.sqrt(dqk)
        o, lse = fn(q, rows[keep], dv, scale)
        o = np.asarray(o); lse = np.asarray(lse)
        assert o.shape == (H, dv) and lse.shape == (H,)
        assert np.allclose(o, dense_masked_attention(q, rows, keep, dv, scale), atol=1e-12)
        assert np.allclose(o, sdpa_masked(q, rows, keep, dv, scale), atol=1e-10)
        # softmax weights sum to one: sum_j exp(z_j - lse) == 1
        z = scale * (q @ rows[keep].T)
        assert np.allclose(np.exp(z - lse[:, None]).sum(1), 1.0, atol=1e-12)
        # the order of the gathered rows does not matter
        perm = r.permutation(n_keep)
        o2, lse2 = fn(q, rows[keep][perm], dv, scale)
        assert np.allclose(o2, o, atol=1e-12) and np.allclose(lse2, lse, atol=1e-12)
    # one row: the output is that row's V part and lse its logit
    q = r.standard_normal((3, 6)); row = r.standard_normal((1, 6))
    o, lse = fn(q, row, 4, 0.5)
    assert np.allclose(o, np.repeat(row[:, :4], 3, 0)) and np.allclose(lse, 0.5 * (q @ row[0]))
    # identical rows: the output is the row, lse = z + log n
    rows = np.repeat(row, 9, 0)
    o, lse = fn(q, rows, 4, 0.5)
    assert np.allclose(o, np.repeat(row[:, :4], 3, 0)) and np.allclose(lse, 0.5 * (q @ row[0]) + math.log(9))
    # zero query: uniform weights, the output is the mean of the V rows
    rows = r.standard_normal((5, 6))
    o, lse = fn(np.zeros((2, 6)), rows, 4, 1.0)
    assert np.allclose(o, np.repeat(rows[:, :4].mean(0, keepdims=True), 2, 0)) and np.allclose(lse, math.log(5))
    # huge logits stay finite (max subtraction)
    o, lse = fn(np.full((1, 2), 300.0), np.array([[3.0, 0.0], [1.0, 0.0]]), 1, 1.0)
    assert np.isfinite(o).all() and np.allclose(o, [[3.0]]) and np.allclose(lse, 900.0)


# ---------------------------------------------------------------- codecs ---

def pin_e4m3_table(table):
    table = np.asarray(table)
    lib = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_t, nan_l = np.isnan(table), np.isnan(lib)
    assert (nan_t == nan_l).all(), np.nonzero(nan_t != nan_l)
    assert np.array_equal(table[~nan_t], lib[~nan_l])
    # values stated by the OCP FP8 definition
    assert table[0x38] == 1.0 and table[0x7E] == 448.0 and table[0xFE] == -448.0
    assert table[0x01] == 2.0 ** -9 and table[0x08] == 2.0 ** -6 and table[0x80] == 0.0
    assert np.isnan(table[0x7F]) and np.isnan(table[0xFF])


def pin_e8m0(fn):
    b = np.arange(256, dtype=np.uint8)
    got = np.asarray(fn(b))
    lib = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(lib))
    ok = ~np.isnan(got)
    assert np.array_equal(got[ok], lib[ok])
    assert got[127] == 1.0 and got[128] == 2.0 and got[0] == 2.0 ** -127


def pin_bf16(fn):
    r = _rng(3)
    x = torch.from_numpy(r.standard_normal(1000).astype(np.float32) * 100).to(torch.bfloat16)
    x = torch.cat([x, torch.tensor([0.0, -0.0, 1.0, -2.5, 3.0e38], dtype=torch.bfloat16)])
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(np.asarray(fn(bits)), x.to(torch.float64).numpy())


# ------------------------------------------------------ FP8 tile-128 rows ---

def read_golden_tile_row(path):
    """The hand-worked FP8 tile-128 row: (bytes uint8 [D], scales [T], expected [D])."""
    dim, scales, elems = None, None, []
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        f = line.split()
        if f[0] == "dim":
            dim = int(f[1])
        elif f[0] == "scales":
            scales = np.array([float(x) for x in f[1:]])
        elif f[0] == "elem":
            elems.append((int(f[1]), int(f[2], 16), float(f[3])))
    raw = np.zeros(dim, np.uint8)
    want = np.zeros(dim)
    for i, byte, val in elems:
        raw[i] = byte
        want[i] = val
    return raw, scales, want


def pin_tile_decode(decode, golden_path):
    """decode(raw, 'fp8_t128', scale) against (1) the hand-worked golden row and
    (2) torch's float8_e4m3fn cast with each tile's scale spread by
    repeat_interleave, on rows whose tiles differ in magnitude by 10^4 steps
    (576 = 512 + 64: five tiles, the last short; 80: one short tile)."""
    raw, sc, want = read_golden_tile_row(golden_path)
    got = np.asarray(decode(raw[None], "fp8_t128", sc[None]))[0]
    assert got.shape == want.shape and np.array_equal(got, want), (got, want)
    r = _rng(77)
    for D in (576, 80, 256):
        T = -(-D // 128)
        b = r.integers(0, 256, (5, D)).astype(np.uint8)
        b[(b & 0x7F) == 0x7F] = 0x38                       # no NaN patterns
        s = (10.0 ** (4 * np.arange(T)))[None] * r.uniform(0.5, 2.0, (5, T))
        lib = torch.from_numpy(b).view(torch.float8_e4m3fn).double()
        spread = torch.repeat_interleave(torch.from_numpy(s), 128, dim=1)[:, :D]
        want = (lib * spread).numpy()
        got = np.asarray(decode(b, "fp8_t128", s))
        assert np.array_equal(got, want), D


# ------------------------------------------------ whole indexer per query ---

def _torch_e4m3(raw_bytes):
    """e4m3 bytes -> float64 through torch's float8_e4m3fn cast (a library route)."""
    t = torch.as_tensor(np.ascontiguousarray(raw_bytes, np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_e8m0(raw_byte):
    """One e8m0 scale byte -> float through torch's float8_e8m0fnu cast."""
    t = torch.tensor([int(raw_byte)], dtype=torch.uint8)
    return float(t.view(torch.float8_e8m0fnu).to(torch.float64)[0])


def _host(x):
    t = x.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.to(torch.float64).numpy()
    return t.numpy()


def loop_indexer_query(case, b, i):
    """The indexer for one query by explicit loops: every key position s <= t
    is looked up in the block table one at a time, its bytes and scale(s) are
    decoded with torch's FP8 / E8M0 casts, the query's scales are taken from
    its own token's row, and the scores come from the pure-Python triple loop.
    Returns (t, scores, kept positions, n-th largest score)."""
    P = case.page_size
    L, T = int(case.seq_lens_host[b]), int(case.q_lens_host[b])
    t = L - T + i
    tok = int(case.q_lens_host[:b].sum()) + i
    dt = case.idx_dtype
    bt = _host(case.block_table)[b]
    kpool = case.k_pool.detach().cpu()
    qraw = case.q_i.detach().cpu()[tok]
    H, D = qraw.shape
    if dt in ("fp8", "mxfp8"):
        q = _torch_e4m3(qraw.numpy())
        qs = _host(case.q_i_scale)[tok]
        for h in range(H):
            for d in range(D):
                q[h, d] *= float(qs[h]) if dt == "fp8" else _torch_e8m0(qs[h, d // 32])
    else:
        q = _host(qraw).astype(np.float64)
    keys = []
    for s in range(t + 1):
        page, off = int(bt[s // P]), s % P
        row = kpool[page, off]
        if dt in ("fp8", "mxfp8"):
            k = _torch_e4m3(row.numpy())
            sc = case.k_scale.detach().cpu()[page, off].numpy()
            for d in range(D):
                k[d] *= float(sc) if dt == "fp8" else _torch_e8m0(sc[d // 32])
        else:
            k = _host(row).astype(np.float64)
        keys.append(k.tolist())
    w = _host(case.w)[tok].astype(np.float64)
    scores = brute_scores(q.tolist(), w.tolist(), keys)
    keep = brute_topk(list(scores), case.topk)
    kth = min(scores[p] for p in keep)        # the n-th largest: the smallest kept score
    return t, scores, keep, kth


def pin_indexer_query(fn, cases):
    """fn(case, b, i) -> (t, scores, idx, kth) against the loop route above,
    for every query of every case."""
    for case in cases:
        for b in range(case.batch):
            for i in range(int(case.q_lens_host[b])):
                t, scores, idx, kth = fn(case, b, i)
                rt, rscores, rkeep, rkth = loop_indexer_query(case, b, i)
                assert t == rt, (t, rt)
                assert np.allclose(scores, rscores, rtol=1e-12, atol=1e-12), (case.name, b, i)
                assert list(np.asarray(idx).tolist()) == rkeep, (case.name, b, i)
                # kth is the n-th largest of fn's own scores (exactly: the
                # smallest kept one), and the loop route's up to rounding
                sc = np.asarray(scores)
                assert kth == sc[np.asarray(idx)].min(), (case.name, b, i, kth)
                assert np.isclose(kth, rkth, rtol=1e-12, atol=1e-12), (case.name, b, i, kth, rkth)
