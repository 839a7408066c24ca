"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case is seeded; sizes are chosen so that the oracle finishes in seconds
while the kernels still see several workgroups per sequence, several tiles and
ragged last pages.  Full-size workloads are checked on sampled queries.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from checker import check_sfa, check_topk_row
from sparse_attention_04_amd import binding as B
from sparse_attention_04_amd.inputs import case_to, make_case

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    B.lib()  # fail loudly if the HIP library is missing


def _host_out(t):
    return t.float().cpu().numpy()


def _queries(case, limit=None):
    qs = [(b, i) for b in range(case.batch) for i in range(int(case.q_lens_host[b]))]
    if limit is not None and len(qs) > limit:
        r = np.random.default_rng(1234)
        sel = sorted(r.choice(len(qs), limit, replace=False))
        qs = [qs[s] for s in sel]
    return qs


def _check_indexer(case, call, idx, queries):
    idx_h = idx.cpu().numpy()
    diffs = 0
    refs = {}
    for (b, i) in queries:
        ref = oracle.run_query(case, b, i)
        refs[(b, i)] = ref
        diffs += check_topk_row(idx_h[case.token(b, i)], ref, case.topk)
    return refs, diffs


def _bar(case):
    """Tolerance class of a case's SFA output: the fp8 bar for an FP8 KV cache."""
    return "fp8" if case.kv_dtype == "fp8_t128" else case.sfa_dtype


def _check_sfa_on(case, out, queries, idx_rows):
    """out rows vs the oracle's SFA run on the given index rows."""
    out_h = _host_out(out)
    worst = (0.0, 0.0)
    for (b, i) in queries:
        tok = case.token(b, i)
        sel = idx_rows[tok]
        sel = sel[sel >= 0]
        ref_o, _ = oracle.sfa_query(case, b, i, sel)
        mx, rel = check_sfa(out_h[tok], ref_o, _bar(case))
        worst = (max(worst[0], mx), max(worst[1], rel))
    return worst


def _run_all_paths(case, queries=None, fused=True):
    queries = queries or _queries(case)
    call = B.Call(case)
    _say(f"{case.name} seed={case.seed} B={case.batch} L={list(case.seq_lens_host[:4])} "
         f"T={case.total_q} k={case.topk} P={case.page_size} dtype={case.idx_dtype}: indexer_topk")
    idx = call.indexer_topk().clone()
    torch.cuda.synchronize()
    refs, diffs = _check_indexer(case, call, idx, queries)
    # SFA on the oracle's index sets
    _say(f"{case.name}: sparse_attn on oracle indices")
    oidx = torch.full((case.total_q, case.topk), -1, dtype=torch.int32)
    for (b, i), ref in refs.items():
        row = ref["idx"]
        oidx[case.token(b, i), :len(row)] = torch.from_numpy(row.astype(np.int32))
    oidx_d = oidx.to(case.q_s.device)
    out, lse = call.sparse_attn(oidx_d)
    torch.cuda.synchronize()
    out_h, lse_h = _host_out(out), lse.cpu().numpy()
    for (b, i), ref in refs.items():
        tok = case.token(b, i)
        check_sfa(out_h[tok], ref["out"], _bar(case))
        assert np.allclose(lse_h[tok], ref["lse"], atol=2e-3, rtol=1e-4), (lse_h[tok][:4], ref["lse"][:4])
    if fused:
        _say(f"{case.name}: fused_decode")
        out, lse, fidx = call.fused_decode()
        torch.cuda.synchronize()
        fidx_h = fidx.cpu().numpy()
        for (b, i), ref in refs.items():
            check_topk_row(fidx_h[case.token(b, i)], ref, case.topk)
        _check_sfa_on(case, out, list(refs.keys()), fidx_h)
    return diffs


def test_c1_tiny_f32():
    case = case_to(make_case("c1_tiny_f32", 1), "cuda")
    _run_all_paths(case)


def test_c1_tiny_f32_ragged_pages():
    case = case_to(make_case("c1_tiny_f32", 11, batch=3, seq_len_range=(60, 250)), "cuda")
    _run_all_paths(case)


def test_c2_bf16_small():
    case = case_to(make_case("c2_decode_bf16", 2, batch=4, seq_len_range=(2500, 9000)), "cuda")
    _run_all_paths(case)


def test_c2_bf16_page16_ragged():
    case = case_to(make_case("c2_decode_bf16", 12, batch=3, seq_len_range=(2049, 5000), page_size=16), "cuda")
    _run_all_paths(case)


def test_short_contexts_keep_every_position():
    # t + 1 <= k: the index set is {0..t}, padded with -1
    case = case_to(make_case("c2_decode_bf16", 3, batch=3, seq_lens=[1, 777, 2048]), "cuda")
    _run_all_paths(case)


def test_context_just_above_k():
    case = case_to(make_case("c2_decode_bf16", 4, batch=2, seq_lens=[2049, 2050]), "cuda")
    _run_all_paths(case)


def test_equal_scores_go_to_smaller_positions():
    case = make_case("c2_decode_bf16", 5, batch=2, seq_lens=[3000, 6000])
    case.k_pool[:] = case.k_pool[0, 0]  # every key identical (poison included, but never read)
    case = case_to(case, "cuda")
    call = B.Call(case)
    _say("equal scores: indexer_topk")
    idx = call.indexer_topk().cpu().numpy()
    for b in range(2):
        row = np.sort(idx[b])
        assert np.array_equal(row, np.arange(case.topk)), row[:10]


@pytest.mark.parametrize("name", ["c4_decode_fp8", "c4_decode_mxfp8"])
def test_c4_quantised_small(name):
    case = case_to(make_case(name, 6, batch=3, seq_len_range=(3000, 7000)), "cuda")
    _run_all_paths(case)


def test_c5_multi_token_decode_small():
    case = case_to(make_case("c5_decode4", 7, batch=2, seq_len_range=(3000, 6000)), "cuda")
    _run_all_paths(case)


@pytest.mark.parametrize("name", ["c4_decode_fp8", "c4_decode_mxfp8"])
def test_multi_token_decode_quantised(name):
    # several query tokens per sequence with the FP8 / MXFP8 indexer
    case = case_to(make_case(name, 14, batch=2, seq_len_range=(3000, 6000), q_len=4), "cuda")
    _run_all_paths(case)


def test_multi_token_decode_mixed_counts():
    # 4, 2, 3 and 1 query tokens per sequence in one launch (one, two and
    # four wave groups per sequence), with contexts just above k so that some
    # queries of a sequence keep every visible position while others are scored
    case = case_to(make_case("c5_decode4", 15, batch=4, seq_lens=[2050, 5000, 2049, 6000],
                             q_lens=[4, 2, 3, 1]), "cuda")
    _run_all_paths(case)


def test_multi_token_decode_small_pages():
    # bf16 keys, three and four query tokens over 16-token pages: every
    # 64-key step of the shared-step scorer spans four pages, and contexts end
    # inside a step
    case = case_to(make_case("c5_decode4", 16, batch=3, seq_lens=[2100, 3333, 5001],
                             q_lens=[4, 3, 4], page_size=16), "cuda")
    _run_all_paths(case)


def test_multi_token_decode_f32_ragged():
    # three query tokens per sequence on the f32 path, ragged pages
    case = case_to(make_case("c1_tiny_f32", 13, batch=2, seq_len_range=(100, 250), q_len=3), "cuda")
    _run_all_paths(case)


def test_c1_tiny_fp8kv():
    # f32 queries over FP8 tile-128 rows of 80 elements (one short tile)
    case = case_to(make_case("c1_tiny_f32", 14, batch=3, seq_len_range=(60, 250), kv_dtype="fp8_t128"), "cuda")
    _run_all_paths(case)


def test_c2_fp8kv_small():
    # decode over an FP8 KV cache: head-split workgroups, split slot ranges
    case = case_to(make_case("c2_decode_fp8kv", 31, batch=4, seq_len_range=(2500, 9000)), "cuda")
    _run_all_paths(case)


def test_c2_fp8kv_short_contexts_and_small_pages():
    # index rows padded with -1 (masked rows, fallback loads), a context of one
    # token, and 16-token pages
    case = case_to(make_case("c2_decode_fp8kv", 32, batch=3, seq_lens=[1, 777, 2048], page_size=16), "cuda")
    _run_all_paths(case)


def test_c2_fp8kv_outliers():
    # 20-sigma outliers: tiles whose scale is set by one large element
    case = case_to(make_case("c2_decode_fp8kv", 33, batch=2, seq_len_range=(3000, 5000), outliers=0.01,
                             sfa_mult=1.0), "cuda")
    _run_all_paths(case)


@pytest.mark.parametrize("name", ["c2_decode_bf16", "c2_decode_bf16_32k"])
def test_c2_full_size_every_query(name):
    """The full decode workloads (32 sequences, contexts U[4096, 32768], and
    every context at 32768) in the launch configuration the benchmark times,
    every query checked against the oracle."""
    _say(f"{name} full size: generating on device")
    case = make_case(name, 2, device="cuda")
    call = B.Call(case)
    _say(f"{name} full size: fused_decode")
    out, lse, idx = call.fused_decode()
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    qs = _queries(case)
    for (b, i) in qs:
        ref = oracle.run_query(case, b, i)
        check_topk_row(idx_h[case.token(b, i)], ref, case.topk)
    mx, rel = _check_sfa_on(case, out, qs, idx_h)
    _say(f"{name} full size: max abs excess {mx:.3g}, rel L2 {rel:.3g}")
    _check_rows_valid(case, idx_h)


def _check_rows_valid(case, idx_h):
    """Every row holds n = min(k, t + 1) distinct positions in [0, t], then -1."""
    for b in range(case.batch):
        L, T = int(case.seq_lens_host[b]), int(case.q_lens_host[b])
        for i in range(T):
            t = L - T + i
            n = min(case.topk, t + 1)
            row = idx_h[case.token(b, i)]
            g = row[:n]
            assert np.all(row[n:] == -1), (b, i)
            assert g.min() >= 0 and g.max() <= t, (b, i)
            assert len(np.unique(g)) == n, (b, i)


@pytest.mark.parametrize("name", ["c4_decode_fp8", "c4_decode_mxfp8"])
def test_c4_full_size_sampled(name):
    """The quantised-indexer decode at full size (64 sequences, contexts
    U[16384, 65536], 1 % outliers at +-20) in the launch configuration the
    benchmark uses, checked on sampled queries and on the properties of every
    row."""
    _say(f"{name} full size: generating on device")
    case = make_case(name, 4, device="cuda")
    call = B.Call(case)
    _say(f"{name} full size: fused_decode")
    out, lse, idx = call.fused_decode()
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    qs = _queries(case, limit=16)
    for (b, i) in qs:
        _say(f"{name} full size: oracle query b={b} i={i}")
        check_topk_row(idx_h[case.token(b, i)], oracle.run_query(case, b, i), case.topk)
    _check_sfa_on(case, out, qs, idx_h)
    _check_rows_valid(case, idx_h)


def test_c5_chunked_prefill_full_size_sampled():
    """8 sequences of 131072 cached tokens, the last 8192 of each a new chunk
    (t = 122880 + i), at full size, checked on sampled queries (first and last
    chunk tokens among them) and on the properties of every row."""
    _say("c5 chunked prefill full size: generating on device")
    case = make_case("c5_chunk_prefill", 5, device="cuda")
    call = B.Call(case)
    _say("c5 chunked prefill full size: fused_prefill")
    out, lse, idx = call.fused_prefill()
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    T = int(case.q_lens_host[0])
    qs = [(0, 0), (7, T - 1)] + [q for q in _queries(case, limit=2) if q not in ((0, 0), (7, T - 1))]
    for (b, i) in qs:
        _say(f"c5 chunked prefill full size: oracle query b={b} i={i}")
        check_topk_row(idx_h[case.token(b, i)], oracle.run_query(case, b, i), case.topk)
    _check_sfa_on(case, out, qs, idx_h)
    _check_rows_valid(case, idx_h)


def test_c5_decode4_full_size_sampled():
    """4-token decode at 131072 tokens (8 sequences, causal among the 4 new
    tokens) at full size, checked on sampled queries and every row."""
    _say("c5 decode4 full size: generating on device")
    case = make_case("c5_decode4", 5, device="cuda")
    call = B.Call(case)
    _say("c5 decode4 full size: fused_decode")
    out, lse, idx = call.fused_decode()
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    qs = [(0, 0), (3, 3)] + [q for q in _queries(case, limit=2) if q not in ((0, 0), (3, 3))]
    for (b, i) in qs:
        _say(f"c5 decode4 full size: oracle query b={b} i={i}")
        check_topk_row(idx_h[case.token(b, i)], oracle.run_query(case, b, i), case.topk)
    _check_sfa_on(case, out, qs, idx_h)
    _check_rows_valid(case, idx_h)


def test_multi_token_decode_sub_batches():
    """Four query tokens for 32 sequences of about 56k tokens (bf16).  With all
    32 in one launch a workgroup would hold about 8000 keys x 4 queries of
    scores, four histograms and the 32 KiB key-exchange area, more than the
    LDS; the decode planner then launches sub-batches of 16 sequences.
    Sampled queries of both halves, the SFA on them, and every row's
    properties."""
    _say("multi-token sub-batches: generating on device")
    case = make_case("c5_decode4", 17, device="cuda", batch=32, seq_len_range=(54000, 57000))
    call = B.Call(case)
    _say("multi-token sub-batches: fused_decode")
    out, lse, idx = call.fused_decode()
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    qs = [(0, 0), (15, 3), (16, 0), (31, 3)]
    for (b, i) in qs:
        _say(f"multi-token sub-batches: oracle query b={b} i={i}")
        check_topk_row(idx_h[case.token(b, i)], oracle.run_query(case, b, i), case.topk)
    _check_sfa_on(case, out, qs, idx_h)
    _check_rows_valid(case, idx_h)


def test_fused_equals_composition():
    case = case_to(make_case("c2_decode_bf16", 8, batch=3, seq_len_range=(3000, 5000)), "cuda")
    call = B.Call(case)
    _say("composition: fused vs indexer+sparse_attn")
    out_f, _, idx_f = call.fused_decode()
    out_f = out_f.clone()
    idx_f = idx_f.clone()
    idx = call.indexer_topk().clone()
    assert torch.equal(torch.sort(idx, 1).values, torch.sort(idx_f, 1).values)
    out, _ = call.sparse_attn(idx_f)
    assert torch.allclose(out.float(), out_f.float(), atol=1e-6)


# ------------------------------------------------------------------ prefill ---

def _sample_prefill_queries(case, per_seq=40, seed=0):
    """Block edges, the k boundary, the first and last tokens, plus random ones."""
    r = np.random.default_rng(seed)
    qs = []
    for b in range(case.batch):
        T = int(case.q_lens_host[b])
        L = int(case.seq_lens_host[b])
        cand = {0, T - 1, min(T - 1, 63), min(T - 1, 64), T // 2}
        for i in range(T):
            t = L - T + i
            if t in (case.topk - 2, case.topk - 1, case.topk, case.topk + 1, 3071, 3072, 3073):
                cand.add(i)
        cand |= set(r.integers(0, T, per_seq).tolist())
        qs += [(b, i) for i in sorted(cand) if 0 <= i < T]
    return qs


def _run_prefill(case, queries):
    call = B.Call(case)
    _say(f"{case.name} seed={case.seed} B={case.batch} L={list(case.seq_lens_host[:4])} "
         f"T={list(case.q_lens_host[:4])} k={case.topk}: fused_prefill")
    out, lse, idx = call.fused_prefill()
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    for (b, i) in queries:
        ref = oracle.run_query(case, b, i)
        check_topk_row(idx_h[case.token(b, i)], ref, case.topk)
    _check_sfa_on(case, out, queries, idx_h)
    return idx_h


def test_prefill_compaction_small_k():
    # 5000 keys with k = 256: candidate buffers overflow and are compacted
    case = case_to(make_case("c3_prefill_bf16", 21, seq_len_range=(5000, 5000), q_len=5000, topk=256), "cuda")
    _run_prefill(case, _sample_prefill_queries(case, per_seq=60))


def test_prefill_full_k_ragged_tail():
    # k = 2048 over 4133 keys: ragged last query block and last page
    case = case_to(make_case("c3_prefill_bf16", 22, seq_len_range=(4133, 4133), q_len=4133), "cuda")
    _run_prefill(case, _sample_prefill_queries(case, per_seq=40))


def test_chunked_prefill_after_cache():
    # a 700-token chunk appended after 5300 cached tokens (every t >= 5300)
    case = case_to(make_case("c5_chunk_prefill", 23, seq_len_range=(6000, 6000), q_len=700, batch=2), "cuda")
    _run_prefill(case, _sample_prefill_queries(case, per_seq=25))


def test_prefill_small_pages():
    # 16-token pages: a 64-key tile spans four pages, each row looked up on its own
    case = case_to(make_case("c3_prefill_bf16", 26, seq_len_range=(3100, 3100), q_len=900, page_size=16,
                             topk=1024), "cuda")
    _run_prefill(case, _sample_prefill_queries(case, per_seq=30))


@pytest.mark.parametrize("page_size", [1, 1024])
def test_prefill_extreme_page_sizes(page_size):
    # one-token pages (every key and latent row through its own block-table
    # entry) and 1024-token pages (a tile never crosses a page)
    case = case_to(make_case("c3_prefill_bf16", 28, seq_len_range=(2600, 2600), q_len=300, page_size=page_size,
                             topk=512), "cuda")
    _run_prefill(case, _sample_prefill_queries(case, per_seq=20))


def test_prefill_mixed_batch_zigzag_units():
    # sequences with different numbers of query blocks (odd, even, one) share a launch
    case = case_to(make_case("c3_prefill_bf16", 24, batch=3, seq_lens=[3000, 2100, 4100], q_lens=[130, 64, 257],
                             topk=512), "cuda")
    _run_prefill(case, _sample_prefill_queries(case, per_seq=20))


def test_prefill_fp8kv():
    # causal prefill over an FP8 KV cache: the 128-head workgroups of large
    # launches, ragged last query block and page
    case = case_to(make_case("c3_prefill_bf16", 27, seq_len_range=(4133, 4133), q_len=4133,
                             kv_dtype="fp8_t128"), "cuda")
    _run_prefill(case, _sample_prefill_queries(case, per_seq=30))


@pytest.mark.parametrize("name", ["c3_prefill_fp8", "c3_prefill_mxfp8"])
def test_prefill_quantised_indexer(name):
    # the quantised indexer in causal prefill: e4m3 key rows and their scale
    # words staged per tile, 1% outliers at 20 sigma in q and K, ragged last
    # query block and page
    case = case_to(make_case(name, 61, seq_len_range=(4133, 4133), q_len=4133), "cuda")
    _run_prefill(case, _sample_prefill_queries(case, per_seq=30))


@pytest.mark.parametrize("name", ["c3_prefill_fp8", "c3_prefill_mxfp8"])
def test_chunked_prefill_quantised_small_pages(name):
    # a 700-token chunk after 5300 cached tokens over 16-token pages: every key
    # row and its scale word are looked up through their own page
    case = case_to(make_case(name, 62, batch=2, seq_len_range=(6000, 6000), q_len=700, page_size=16,
                             topk=1024), "cuda")
    _run_prefill(case, _sample_prefill_queries(case, per_seq=25))


@pytest.mark.parametrize("name", ["c3_prefill_fp8", "c3_prefill_mxfp8"])
def test_quantised_prefill_mixed_batch(name):
    # sequences with different numbers of query blocks share a launch
    case = case_to(make_case(name, 63, batch=3, seq_lens=[3000, 2100, 4100], q_lens=[130, 64, 257],
                             topk=512), "cuda")
    _run_prefill(case, _sample_prefill_queries(case, per_seq=20))


def test_prefill_equal_scores():
    case = make_case("c3_prefill_bf16", 25, seq_len_range=(3500, 3500), q_len=300, topk=1024)
    case.k_pool[:] = case.k_pool[0, 0]
    case = case_to(case, "cuda")
    call = B.Call(case)
    _say("prefill equal scores")
    _, _, idx = call.fused_prefill()
    idx = idx.cpu().numpy()
    for i in range(300):
        assert np.array_equal(np.sort(idx[i]), np.arange(1024)), i


def test_c3_full_size_sampled():
    """The 32768-token causal prefill at full size, checked on sampled queries
    and, for every query, on the properties of its index row."""
    _say("c3 full size: generating on device")
    case = make_case("c3_prefill_bf16", 3, device="cuda")
    qs = [(0, i) for i in (0, 2047, 2048, 2049, 9000, 20000, 32767)]
    idx_h = _run_prefill(case, qs)
    t = np.arange(case.total_q)
    n = np.minimum(case.topk, t + 1)
    valid = idx_h >= 0
    assert np.array_equal(valid.sum(1), n)
    assert np.all(np.where(valid, idx_h <= t[:, None], True))


@pytest.mark.parametrize("name", ["c3_prefill_fp8", "c3_prefill_mxfp8"])
def test_quantised_prefill_full_size_sampled(name):
    """The 32768-token causal prefill with the quantised indexer, checked on
    sampled queries and, for every query, on the properties of its index row."""
    _say(f"{name} full size: generating on device")
    case = make_case(name, 3, device="cuda")
    qs = [(0, i) for i in (0, 2048, 2049, 15000, 32767)]
    idx_h = _run_prefill(case, qs)
    t = np.arange(case.total_q)
    n = np.minimum(case.topk, t + 1)
    valid = idx_h >= 0
    assert np.array_equal(valid.sum(1), n)
    assert np.all(np.where(valid, idx_h <= t[:, None], True))


def test_c2_fp8kv_full_size_every_query():
    """The decode workload at full size (32 sequences, contexts U[4096, 32768])
    with the SFA KV cache in FP8, in the configuration the benchmark times,
    every query checked against the oracle."""
    _say("c2 fp8 KV full size: generating on device")
    case = make_case("c2_decode_fp8kv", 6, device="cuda")
    call = B.Call(case)
    _say("c2 fp8 KV full size: fused_decode")
    out, lse, idx = call.fused_decode()
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    qs = _queries(case)
    for (b, i) in qs:
        ref = oracle.run_query(case, b, i)
        check_topk_row(idx_h[case.token(b, i)], ref, case.topk)
    mx, rel = _check_sfa_on(case, out, qs, idx_h)
    _say(f"c2 fp8 KV full size: max abs excess {mx:.3g}, rel L2 {rel:.3g}")
    _check_rows_valid(case, idx_h)


# ------------------------------------------------------- signed head weights ---

@pytest.mark.parametrize("name", ["c2_decode_bf16", "c4_decode_fp8", "c4_decode_mxfp8", "c5_decode4"])
def test_signed_head_weights_decode(name):
    """Head weights of either sign (U(-1,1)/64): the weighted sum may cancel
    and the scores take both signs."""
    kw = dict(batch=3, seq_len_range=(2500, 6000), w_signed=True)
    if name == "c5_decode4":
        kw["batch"] = 2
    case = case_to(make_case(name, 41, **kw), "cuda")
    _run_all_paths(case)


def test_signed_head_weights_prefill():
    case = case_to(make_case("c3_prefill_bf16", 42, seq_len_range=(3000, 3000), q_len=3000, w_signed=True),
                   "cuda")
    _run_prefill(case, _sample_prefill_queries(case, per_seq=30))


# ---------------------------------------------------- largest prefill Top-K ---

def test_prefill_largest_topk():
    """k = 2752, the largest the prefill indexer takes, with positions on both
    sides of its 3072-entry candidate buffer (t from 3000 to 3399): the
    mid-query selects then keep up to k + 256 candidates before the next
    64-key tile is appended."""
    case = case_to(make_case("c5_chunk_prefill", 43, batch=1, seq_len_range=(3400, 3400), q_len=400,
                             topk=2752), "cuda")
    qs = [(0, i) for i in range(0, 400, 7)] + [(0, i) for i in range(68, 78)] + [(0, 399)]
    idx_h = _run_prefill(case, sorted(set(qs)))
    _check_rows_valid(case, idx_h)


# ---------------------------------------------- a dominant row in a late tile ---

def _plant_dominant_row(case, b, pos, value):
    """Make latent row `pos` of sequence b equal `value` in every column and
    the query of b all ones: its logit is scale * 576 * value above the
    others' (about 166 nats for value 4 at scale 1/sqrt(192))."""
    P = case.page_size
    page = int(case.block_table[b, pos // P])
    if case.kv_dtype == "fp8_t128":
        case.kv_pool[page, pos % P] = 0x38                 # e4m3 1.0
        case.kv_scale[page, pos % P] = value
    else:
        case.kv_pool[page, pos % P] = value
    case.q_s[case.token(b, 0)] = 1.0


@pytest.mark.parametrize("kv", ["bf16", "fp8_t128"])
def test_sfa_dominant_row_in_late_tile(kv):
    """A logit ~166 nats above every other, at a slot that is not in the first
    tile a workgroup reads (the last slot of one row, slot 1000 of another):
    the softmax reference moves up and the output equals that row's V part."""
    name = "c2_decode_fp8kv" if kv == "fp8_t128" else "c2_decode_bf16"
    case = make_case(name, 44, batch=2, seq_lens=[3000, 3500])
    r = np.random.default_rng(44)
    rows = np.full((2, case.topk), -1, np.int32)
    planted = [2500, 3100]
    for b, slot in ((0, case.topk - 1), (1, 1000)):
        t = int(case.seq_lens_host[b]) - 1
        _plant_dominant_row(case, b, planted[b], 4.0)
        others = r.choice(np.setdiff1d(np.arange(t + 1), [planted[b]]), case.topk - 1, replace=False)
        row = np.insert(others, slot, planted[b])
        rows[b] = row
    case = case_to(case, "cuda")
    call = B.Call(case)
    _say(f"dominant late row ({kv}): sparse_attn")
    out, lse = call.sparse_attn(torch.from_numpy(rows).cuda())
    torch.cuda.synchronize()
    out_h, lse_h = _host_out(out), lse.cpu().numpy()
    assert np.isfinite(out_h).all() and np.isfinite(lse_h).all()
    for b in range(2):
        ref_o, ref_lse = oracle.sfa_query(case, b, 0, rows[b])
        check_sfa(out_h[b], ref_o, _bar(case))
        assert np.allclose(out_h[b], 4.0, atol=1e-2)
        assert np.allclose(lse_h[b], ref_lse, atol=2e-3, rtol=1e-4), (lse_h[b][:4], ref_lse[:4])
