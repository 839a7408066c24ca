"""The oracle against its pins (CPU only).

Each oracle function is checked against something other than itself: brute
force on tiny inputs, library routines (torch's FP8 / E8M0 / bf16 casts,
scaled_dot_product_attention), closed forms, invariants and the one worked
example the pages give (the two-device zigzag split).  The mutation tests at the
end plant plausible mistakes in copies of the oracle's functions and check that
the pins catch them."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import pins
from sparse_attention_04_amd.inputs import make_case, quant_fp8_rows, quant_fp8_tiles, quant_mx_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------- decoding ---

def test_e4m3_table_matches_library_and_spec():
    pins.pin_e4m3_table(oracle.e4m3fn_table())


def test_e8m0_matches_library():
    pins.pin_e8m0(oracle.decode_e8m0)


def test_bf16_decode_matches_library():
    pins.pin_bf16(oracle.decode_bf16_bits)


def test_fp8_per_row_scale_factors_out():
    """sum_d (a_d s_a)(b_d s_b) = s_a s_b sum_d a_d b_d: the oracle's decoded
    FP8 rows score the same as unscaled rows times the two scales."""
    r = np.random.default_rng(5)
    qb = r.integers(0, 256, (4, 32)).astype(np.uint8); qb[(qb & 0x7F) == 0x7F] = 0x38
    kb = r.integers(0, 256, (6, 32)).astype(np.uint8); kb[(kb & 0x7F) == 0x7F] = 0x38
    sq = r.uniform(0.1, 2.0, 4); sk = r.uniform(0.1, 2.0, 6)
    w = r.standard_normal(4)
    q = oracle.decode_values(qb, "fp8", sq)
    k = oracle.decode_values(kb, "fp8", sk)
    got = oracle.indexer_scores(q, w, k)
    raw = oracle.indexer_scores(oracle.decode_e4m3(qb), w * sq, oracle.decode_e4m3(kb)) * sk
    assert np.allclose(got, raw, rtol=1e-13)


def test_mx_groups_scale_independently():
    """Each group of 32 elements carries its own power-of-two scale."""
    bits = np.full((1, 64), 0x38, np.uint8)            # every element 1.0
    sc = np.array([[127 + 3, 127 - 2]], np.uint8)       # 2^3 and 2^-2
    v = oracle.decode_values(bits, "mxfp8", sc)
    assert np.all(v[0, :32] == 8.0) and np.all(v[0, 32:] == 0.25)


def test_input_quantisers_within_e4m3_error():
    """The input module's encoders (not the oracle) round within half an e4m3
    ulp of the scaled value; the oracle decodes them back."""
    r = np.random.default_rng(9)
    x = torch.from_numpy(r.standard_normal((50, 128)).astype(np.float32))
    x[3, 5] = 20.0
    bits, sc = quant_fp8_rows(x)
    back = oracle.decode_values(bits.numpy(), "fp8", sc.numpy())
    rel = np.abs(back - x.numpy()) / np.maximum(np.abs(x.numpy()), sc.numpy()[:, None] * 2 ** -6)
    assert rel.max() <= 2 ** -4 + 1e-9
    bits, e = quant_mx_rows(x)
    back = oracle.decode_values(bits.numpy(), "mxfp8", e.numpy())
    scale = np.repeat(2.0 ** (e.numpy().astype(np.int64) - 127), 32, axis=1)
    err = np.abs(back - x.numpy())
    inside = np.abs(x.numpy()) <= 448.0 * scale
    assert np.all(err[inside] <= np.maximum(np.abs(x.numpy()) * 2 ** -4, scale * 2 ** -9)[inside] + 1e-12)
    # beyond the element range the OCP rule saturates to the largest normal
    assert np.all(np.abs(back[~inside]) == 448.0 * scale[~inside])
    # group amax lands in [256, 512) before saturation at 448 (OCP MX rule)
    g = np.abs(x.numpy()).reshape(50, 4, 32).max(-1) / 2.0 ** (e.numpy().astype(np.int64) - 127)
    assert np.all((g >= 256) & (g < 512))


def test_fp8_tile128_decode_pins():
    """The SFA KV cache's FP8 rows: one scale per tile of 128 elements."""
    pins.pin_tile_decode(oracle.decode_values, os.path.join(GOLDEN, "kv_fp8_tile128.txt"))


def test_tile_quantiser_within_e4m3_error():
    """The input module's tile encoder: every tile's largest magnitude maps to
    448 (so decodes to itself up to fp32 rounding of the scale) and every
    element is within half an e4m3 ulp, whatever the other tiles hold."""
    r = np.random.default_rng(11)
    x = r.standard_normal((40, 576)).astype(np.float32)
    x *= (10.0 ** (np.arange(576) // 128 - 2)).astype(np.float32)   # tiles 1e-2 .. 1e2
    x[7, 130] = 0.0
    x[8, 512:] = 0.0                                                # an all-zero tile
    bits, sc = quant_fp8_tiles(torch.from_numpy(x))
    assert bits.shape == (40, 576) and sc.shape == (40, 5)
    back = oracle.decode_values(bits.numpy(), "fp8_t128", sc.numpy())
    tile_sc = np.repeat(sc.numpy().astype(np.float64), 128, axis=1)[:, :576]
    err = np.abs(back - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2 ** -4, tile_sc * 2 ** -10) + 1e-30)
    amax = np.abs(x[:, :512]).reshape(40, 4, 128).max(-1)
    assert np.allclose(np.abs(back[:, :512]).reshape(40, 4, 128).max(-1), amax, rtol=1e-6)
    assert np.allclose(np.abs(back[:, 512:]).max(-1), np.abs(x[:, 512:]).max(-1), rtol=1e-6)
    assert np.all(back[8, 512:] == 0.0) and sc[8, 4] == 1.0


# -------------------------------------------------------------- scores ---

def test_indexer_scores_brute_force():
    pins.pin_indexer_scores(oracle.indexer_scores)


def test_indexer_scores_collapse_identity():
    """With no activation, sum_h w_h (q_h . k) == (sum_h w_h q_h) . k."""
    r = np.random.default_rng(1)
    q, w, k = r.standard_normal((64, 128)), r.random(64) / 64, r.standard_normal((300, 128))
    collapsed = k @ (w @ q)
    assert np.allclose(oracle.indexer_scores(q, w, k), collapsed, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------- top-k ---

def test_topk_brute_force_rank_definition():
    pins.pin_topk(oracle.topk_select)


def test_topk_matches_argpartition_on_distinct_scores():
    r = np.random.default_rng(2)
    s = r.standard_normal(5000)
    got = oracle.topk_select(s, 2048)
    ref = np.sort(np.argpartition(-s, 2047)[:2048])
    assert np.array_equal(got, ref)


# ----------------------------------------------------------- attention ---

def test_sparse_attention_pins():
    pins.pin_sparse_attention(oracle.sparse_attention)


# -------------------------------------------------------------- paging ---

def test_paged_rows_identity_and_permutation_invariance():
    r = np.random.default_rng(4)
    P, npg, D = 4, 6, 3
    logical = r.standard_normal((npg * P, D))
    table = r.permutation(npg)
    pool = np.empty((npg, P, D))
    for lp in range(npg):
        pool[table[lp]] = logical[lp * P:(lp + 1) * P]
    pos = r.integers(0, npg * P, 40)
    assert np.array_equal(oracle.paged_rows(pool, table, P, pos), logical[pos])
    # move every physical page elsewhere and update the table: same rows
    perm = r.permutation(npg)
    pool2 = np.empty_like(pool); pool2[perm] = pool
    assert np.array_equal(oracle.paged_rows(pool2, perm[table], P, pos), logical[pos])


def test_query_position_reading():
    # decode: the single new token is the last one
    assert oracle.query_position(256, 1, 0) == 255
    # 4-token decode after 131072 cached keys: 131068..131071
    assert [oracle.query_position(131072, 4, i) for i in range(4)] == [131068, 131069, 131070, 131071]
    # 8192-token chunk after 122880 cached tokens
    assert oracle.query_position(131072, 8192, 0) == 122880
    # full causal prefill: t = i
    assert oracle.query_position(32768, 32768, 17) == 17


def test_case_poison_never_reached():
    c = make_case("c1_tiny_f32", 3, seq_len_range=(250, 250))   # ragged last page
    r = oracle.run_query(c, 0, 0)
    assert np.isfinite(r["scores"]).all() and np.isfinite(r["out"]).all()
    # the poisoned tail exists
    last = c.block_table[0, (250 - 1) // 16]
    assert torch.isnan(c.k_pool[last, 250 % 16:]).all()


def test_fp8_kv_case_wiring():
    """SFA over an FP8 tile-128 KV cache: the oracle's paged gather of rows and
    of their tile scales agrees with a route through torch's e4m3 cast and a
    per-element scale spread by repeat_interleave; poisoned pool entries
    (NaN scales, 0x7F bytes) are never reached."""
    c = make_case("c2_decode_fp8kv", 4, batch=2, seq_len_range=(300, 700), topk=64)
    assert c.kv_dtype == "fp8_t128" and c.kv_pool.dtype == torch.uint8
    assert c.kv_scale.shape == (c.num_pages, c.page_size, 5)
    for b in range(2):
        idx = np.sort(np.random.default_rng(b).choice(int(c.seq_lens_host[b]), 64, replace=False))
        out, lse = oracle.sfa_query(c, b, 0, idx)
        assert np.isfinite(out).all() and np.isfinite(lse).all()
        bt = c.block_table[b].long()
        pos = torch.from_numpy(idx)
        pg, off = bt[pos // c.page_size], pos % c.page_size
        raw = c.kv_pool[pg, off].view(torch.float8_e4m3fn).double()
        spread = torch.repeat_interleave(c.kv_scale[pg, off].double(), 128, dim=1)[:, :576]
        rows = (raw * spread).numpy()
        q = c.q_s[c.token(b, 0)].float().double().numpy()
        o2, l2 = oracle.sparse_attention(q, rows, c.d_v, c.softmax_scale)
        assert np.array_equal(out, o2) and np.array_equal(lse, l2)
    # the pool's unused rows are poisoned
    last = c.block_table[0, (int(c.seq_lens_host[0]) - 1) // 64]
    tail = int(c.seq_lens_host[0]) % 64
    if tail:
        assert (c.kv_pool[last, tail:] == 0x7F).all() and torch.isnan(c.kv_scale[last, tail:]).all()


# -------------------------------------------------------------- zigzag ---

def _read_golden_zigzag():
    units, n = [], None
    with open(os.path.join(GOLDEN, "zigzag_two_devices.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("n_blocks"):
                n = int(line.split()[1])
            else:
                units.append([int(x) for x in line.split(":")[1].split()])
    return n, units


def test_zigzag_two_device_example():
    n, units = _read_golden_zigzag()
    assert [sorted(u) for u in oracle.zigzag_units(n)] == units


@pytest.mark.parametrize("nb", [1, 2, 3, 7, 8, 512])
def test_zigzag_bijection_and_balance(nb):
    units = oracle.zigzag_units(nb)
    flat = sorted(b for u in units for b in u)
    assert flat == list(range(nb))                     # every block once
    # a cost linear in the block index is equal over the paired units
    costs = [sum(2 * b + 1 for b in u) for u in units if len(u) == 2]
    assert len(set(costs)) <= 1


# ---------------------------------------------------- whole-path brute force ---

def test_run_query_brute_force_tiny():
    """Full path on a tiny case by explicit loops: paged reads, scores, rank
    selection and dense masked attention."""
    c = make_case("c1_tiny_f32", 8, seq_len_range=(45, 45), q_len=3, page_size=4,
                  h_i=2, d_i=4, topk=16, h_s=3, d_qk=6, d_v=4, scale_dim=6)
    for i in range(3):
        r = oracle.run_query(c, 0, i)
        t = 45 - 3 + i
        assert r["t"] == t
        tok = c.token(0, i)
        kpool = c.k_pool.numpy().astype(np.float64)
        bt = c.block_table[0].numpy()
        keys = [kpool[bt[s // 4], s % 4] for s in range(t + 1)]
        sc = pins.brute_scores(c.q_i[tok].double().tolist(), c.w[tok].double().tolist(), keys)
        assert np.allclose(r["scores"], sc, rtol=1e-12)
        assert list(r["idx"]) == pins.brute_topk(list(sc), 16)
        kvpool = c.kv_pool.numpy().astype(np.float64)
        rows = np.array([kvpool[bt[s // 4], s % 4] for s in range(t + 1)])
        o = pins.dense_masked_attention(c.q_s[tok].double().numpy(), rows, r["idx"], 4, 1 / math.sqrt(6))
        assert np.allclose(r["out"], o, atol=1e-12)


# -------------------------------------------------------------- mutations ---

def _mutant_scores_no_weights(q, w, keys):
    return (keys @ q.T).sum(1)


def _mutant_scores_transposed(q, w, keys):
    return (keys @ q.T) @ w[::-1]


def _mutant_topk_tie_larger(scores, k):
    n = min(k, len(scores))
    pos = np.arange(len(scores))
    return np.sort(np.lexsort((-pos, -np.asarray(scores)))[:n])


def _mutant_topk_off_by_one(scores, k):
    return oracle.topk_select(scores, k + 1)


def _mutant_attn_no_scale(q, rows, d_v, scale):
    return oracle.sparse_attention(q, rows, d_v, 1.0)


def _mutant_attn_v_from_tail(q, rows, d_v, scale):
    o, lse = oracle.sparse_attention(q, rows, rows.shape[1], scale)
    return o[:, -d_v:], lse


def _mutant_attn_sign(q, rows, d_v, scale):
    return oracle.sparse_attention(q, rows, d_v, -scale)


def _mutant_tile_divides(raw, dtype, scale=None, group=32):
    v = oracle.decode_e4m3(raw)
    sc = np.asarray(scale, np.float64)
    return v / sc[..., np.arange(v.shape[-1]) // 128]


def _mutant_tile_64(raw, dtype, scale=None, group=32):
    v = oracle.decode_e4m3(raw)
    sc = np.asarray(scale, np.float64)
    t = np.minimum(np.arange(v.shape[-1]) // 64, sc.shape[-1] - 1)
    return v * sc[..., t]


def _mutant_tile_first_scale(raw, dtype, scale=None, group=32):
    return oracle.decode_e4m3(raw) * np.asarray(scale, np.float64)[..., :1]


@pytest.mark.parametrize("mutant", [_mutant_tile_divides, _mutant_tile_64, _mutant_tile_first_scale])
def test_tile_pin_catches_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        pins.pin_tile_decode(mutant, os.path.join(GOLDEN, "kv_fp8_tile128.txt"))


def _mutant_e4m3_bias(t=None):
    t = oracle.e4m3fn_table().copy()
    return t * 2.0


@pytest.mark.parametrize("pin,mutant", [
    (pins.pin_indexer_scores, _mutant_scores_no_weights),
    (pins.pin_indexer_scores, _mutant_scores_transposed),
    (pins.pin_topk, _mutant_topk_tie_larger),
    (pins.pin_topk, _mutant_topk_off_by_one),
    (pins.pin_sparse_attention, _mutant_attn_no_scale),
    (pins.pin_sparse_attention, _mutant_attn_v_from_tail),
    (pins.pin_sparse_attention, _mutant_attn_sign),
])
def test_pins_catch_planted_mistakes(pin, mutant):
    with pytest.raises(AssertionError):
        pin(mutant)


def test_codec_pin_catches_wrong_bias():
    with pytest.raises(AssertionError):
        pins.pin_e4m3_table(_mutant_e4m3_bias())


# ------------------------------------------- quantised indexer per query ---

def _small_quant_cases():
    """Small FP8 and MXFP8 indexer cases (and a bf16 one): ragged contexts over
    16-token pages in a permuted pool, 1 % outliers at +-20 before quantising,
    signed head weights, several query tokens per sequence (so a wrong token's
    scale row is a different row)."""
    kw = dict(batch=2, seq_len_range=(40, 75), q_len=2, page_size=16, h_i=3, d_i=64, topk=16,
              h_s=2, d_qk=16, d_v=8, scale_dim=16, w_signed=True)
    return [make_case("c4_decode_fp8", 21, **kw), make_case("c4_decode_mxfp8", 22, **kw),
            make_case("c2_decode_bf16", 23, **kw)]


def test_indexer_query_quantised_against_loop_route():
    """oracle.indexer_query (scores, Top-K and the n-th largest score) on FP8,
    MXFP8 and bf16 cases against explicit per-position block-table lookups,
    torch's float8_e4m3fn / float8_e8m0fnu casts and the pure-Python score
    loop ([P2] sec. 4.2: MXFP8 with 32-element groups; [P1] sec. 3)."""
    pins.pin_indexer_query(oracle.indexer_query, _small_quant_cases())


def _mutant_query(scale_unpaged=False, q_scale_token=0, kth_shift=0):
    """Copies of oracle.indexer_query with one planted mistake."""
    od = oracle.dsa_oracle

    def fn(case, b, i):
        P = case.page_size
        L, T = int(case.seq_lens_host[b]), int(case.q_lens_host[b])
        t = od.query_position(L, T, i)
        tok = case.token(b, i)
        bt = od._np(case.block_table[b])
        pos = np.arange(t + 1)
        qs_tok = min(tok + q_scale_token, case.total_q - 1)
        q = od.decode_values(od._np(case.q_i[tok]), case.idx_dtype,
                             None if case.q_i_scale is None else od._np(case.q_i_scale[qs_tok]))
        k_raw = od.paged_rows(od._np(case.k_pool), bt, P, pos)
        if case.k_scale is None:
            k_sc = None
        elif scale_unpaged:       # logical position used as a pool row
            flat = od._np(case.k_scale).reshape(-1, *case.k_scale.shape[2:])
            k_sc = flat[pos]
        else:
            k_sc = od.paged_rows(od._np(case.k_scale), bt, P, pos)
        keys = od.decode_values(k_raw, case.idx_dtype, k_sc)
        scores = od.indexer_scores(q, od._np(case.w[tok]).astype(np.float64), keys)
        idx = od.topk_select(scores, case.topk)
        kth = np.sort(scores)[::-1][len(idx) - 1 + kth_shift]
        return t, scores, idx, kth
    return fn


@pytest.mark.parametrize("mutant", [_mutant_query(scale_unpaged=True), _mutant_query(q_scale_token=1),
                                    _mutant_query(kth_shift=1)],
                         ids=["unpaged-key-scale", "next-token-q-scale", "kth-off-by-one"])
def test_indexer_query_pin_catches_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        pins.pin_indexer_query(mutant, _small_quant_cases())
