"""The fused decode kernel (indexer and attention in one launch) against the
two-kernel path of the same call (DSA_FUSED_KERNEL=0) and against the oracle.

Both paths select the same index sets (exact Top-K); the order of positions
within a row depends on which workgroup scored which pages, so rows are
compared as sets, and the attention outputs, which sum the same rows split
into differently ordered ranges, within the bf16 bar.  The per-sequence ready
words the fused kernel uses must be left zero, so one workspace keeps serving
calls of any shape."""
import contextlib
import os
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
    B.lib()


@contextlib.contextmanager
def _env(**kv):
    old = {k: os.environ.get(k) for k in kv}
    os.environ.update(kv)
    try:
        yield
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _fused(call):
    out, lse, idx = call.fused_decode()
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()


def _max_abs_v(case):
    """Largest |V| element of the latent rows (the NaN page tails aside)."""
    v = case.kv_pool[..., :case.d_v].float().cpu().numpy()   # bf16 -> f32 is exact
    return float(np.nanmax(np.abs(v)))


def _compare_paths(case, sample=None):
    call = B.Call(case)
    _say(f"{case.name} B={case.batch} T={case.total_q}: two-kernel path")
    with _env(DSA_FUSED_KERNEL="0"):
        out0, lse0, idx0 = _fused(call)
    _say(f"{case.name}: fused kernel")
    out1, lse1, idx1 = _fused(call)
    assert np.array_equal(np.sort(idx0, 1), np.sort(idx1, 1))
    # the same rows in other ranges: each path's fp16 partials are within
    # 2^-11 of max|V| (a partial is a convex combination of V rows) and its
    # bf16 output within 2^-8 relative, so the two differ by at most
    # 2^-10 max|V| + 2^-7 |out|; each path is held to the oracle's bar below
    mag = np.maximum(np.abs(out0), np.abs(out1))
    tol = 2.0 ** -7 * mag + 2.0 ** -10 * _max_abs_v(case) + 2.0 ** -16
    assert np.all(np.abs(out0 - out1) <= tol), float(np.max(np.abs(out0 - out1) - tol))
    assert np.allclose(lse0, lse1, atol=1e-4, rtol=1e-5)
    toks = range(case.total_q) if sample is None else sample
    where = {case.token(b, i): (b, i) for b in range(case.batch) for i in range(int(case.q_lens_host[b]))}
    for g in toks:
        b, i = where[g]
        ref = oracle.run_query(case, b, i)
        check_topk_row(idx1[g], ref, case.topk)
        sel = idx1[g][idx1[g] >= 0]
        ref_o, _ = oracle.sfa_query(case, b, i, sel)
        check_sfa(out1[g], ref_o, case.sfa_dtype)
    return call


def test_fused_kernel_matches_two_kernel_path_small():
    case = case_to(make_case("c2_decode_bf16", 81, batch=5, seq_len_range=(2500, 9000)), "cuda")
    _compare_paths(case)


def test_fused_kernel_short_and_ragged_contexts():
    # sequences that keep every position (no scores: published without a
    # barrier), one just above k, ragged last pages, 16-token pages
    case = case_to(make_case("c2_decode_bf16", 82, batch=4, seq_lens=[1, 2048, 2049, 5001], page_size=16),
                   "cuda")
    _compare_paths(case)


def test_fused_kernel_multi_token():
    # 4, 2, 3 and 1 query tokens per sequence (causal among them), two of them
    # close to k
    case = case_to(make_case("c5_decode4", 86, batch=4, seq_lens=[2050, 5000, 2049, 6000],
                             q_lens=[4, 2, 3, 1]), "cuda")
    _compare_paths(case)


@pytest.mark.parametrize("name", ["c4_decode_fp8", "c4_decode_mxfp8"])
def test_fused_kernel_quantised_indexer(name):
    case = case_to(make_case(name, 87, batch=3, seq_len_range=(3000, 7000)), "cuda")
    _compare_paths(case)


@pytest.mark.parametrize("page_size", [1, 2, 1024, 4096])
def test_fused_kernel_extreme_page_sizes(page_size):
    # the smallest and largest page sizes the boundary takes: one key per
    # block-table entry, and pages larger than a whole context
    case = case_to(make_case("c2_decode_bf16", 93, batch=3, seq_lens=[700, 3000, 5000], page_size=page_size),
                   "cuda")
    _compare_paths(case)


@pytest.mark.parametrize("topk", [1, 64, 4096])
def test_fused_kernel_other_topk(topk):
    # a single selected row (one range of one tile per token) and a small k,
    # both through the fused kernel, and k twice the usual (64 ranges per
    # token, more tasks than workgroups: the two-kernel path); contexts both
    # below and above k
    case = case_to(make_case("c2_decode_bf16", 92, batch=4, seq_lens=[700, 3000, 5000, 9000], topk=topk), "cuda")
    _compare_paths(case)


@pytest.mark.parametrize("name", ["c4_decode_fp8", "c4_decode_mxfp8"])
def test_fused_kernel_quantised_indexer_multi_token(name):
    # the quantised indexers with 4, 2, 3 and 1 query tokens per sequence
    case = case_to(make_case(name, 91, batch=4, seq_lens=[2050, 5000, 2049, 6000], q_lens=[4, 2, 3, 1]), "cuda")
    _compare_paths(case)


@pytest.mark.parametrize("q_lens", [[2, 0, 3], [1, 0, 1]])
def test_fused_kernel_sequence_without_query_tokens(q_lens):
    # a sequence with cached keys but no new token: its indexer workgroups
    # publish nothing, no attention task waits for it, and its state words
    # end zero like the others'
    case = case_to(make_case("c5_decode4", 88, batch=3, seq_lens=[3000, 2500, 4000], q_lens=q_lens), "cuda")
    call = _compare_paths(case)
    ws, _ = call.workspace(B.DSA_OP_FUSED_DECODE)
    state = B.dsa_workspace_size(B.DSA_OP_INDEXER_TOPK, call.batch, call.iargs, call.sargs)
    assert int(ws[256:state].count_nonzero()) == 0


def test_fused_kernel_full_size_32k():
    _say("c2_decode_bf16_32k: generating on device")
    case = make_case("c2_decode_bf16_32k", 83, device="cuda")
    _compare_paths(case, sample=[0, 13, 31])


def test_fused_kernel_leaves_ready_words_zero():
    """Calls of different batch sizes on one workspace: the per-sequence state
    (counters, ready words) is zero after each call and every call is right."""
    small = case_to(make_case("c2_decode_bf16", 84, batch=2, seq_len_range=(3000, 5000)), "cuda")
    big = case_to(make_case("c2_decode_bf16", 85, batch=7, seq_len_range=(3000, 9000)), "cuda")
    calls = {c.batch: B.Call(c) for c in (small, big)}
    need = max(call.workspace(B.DSA_OP_FUSED_DECODE)[1] for call in calls.values())
    state = max(B.dsa_workspace_size(B.DSA_OP_INDEXER_TOPK, call.batch, call.iargs, call.sargs)
                for call in calls.values())
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for k, case in enumerate((small, big, small, big)):
        call = calls[case.batch]
        _say(f"shared workspace, call {k}: B={case.batch}")
        call.use_workspace(B.DSA_OP_FUSED_DECODE, ws)
        out, lse, idx = _fused(call)
        assert int(ws[256:state].count_nonzero()) == 0, k
        for b in range(case.batch):
            check_topk_row(idx[case.token(b, 0)], oracle.run_query(case, b, 0), case.topk)


def test_fused_kernel_graph_replays_take_fresh_epochs():
    """A captured fused decode replayed several times: each replay derives its
    ready-word epoch from the workspace's call counter, which the launch after
    the fused kernel advances, so a ready word that a late writer of the
    previous call could leave behind (planted here before every replay: the
    previous call's epoch in every sequence's word) is never taken for the
    next call's.  The index buffer is set to -1 before each replay, so rows
    read before they were written would show.  Every replay must match the
    eager call."""
    case = case_to(make_case("c2_decode_bf16", 89, batch=3, seq_len_range=(3000, 6000)), "cuda")
    call = B.Call(case)
    _say(f"graph: {case.name} B={case.batch}: eager call")
    out0, lse0, idx0 = _fused(call)
    ws, _ = call.workspace(B.DSA_OP_FUSED_DECODE)
    words = ws.view(torch.int32)
    _say("graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call.fused_decode()
    torch.cuda.synchronize()
    for r in range(4):
        c0 = int(words[8].item()) & 0xFFFFFFFF
        for b in range(case.batch):
            words[64 + 32 * b + 3] = c0 - (1 << 32) if c0 >= (1 << 31) else c0
        call.idx.fill_(-1)
        torch.cuda.synchronize()
        _say(f"graph: replay {r} (counter {c0})")
        g.replay()
        torch.cuda.synchronize()
        c1 = int(words[8].item()) & 0xFFFFFFFF
        assert c1 == (c0 + 1 if c0 + 1 < (1 << 32) else 1), (c0, c1)
        assert int(words[64:64 + 32 * case.batch].count_nonzero()) == 0, "state words left set"
        out1 = call.out.float().cpu().numpy()
        lse1 = call.lse.cpu().numpy()
        idx1 = call.idx.cpu().numpy()
        assert np.array_equal(np.sort(idx0, 1), np.sort(idx1, 1)), r
        mag = np.maximum(np.abs(out0), np.abs(out1))
        assert np.all(np.abs(out0 - out1) <= 2.0 ** -6 * mag + 2.0 ** -10), r
        assert np.allclose(lse0, lse1, atol=1e-4, rtol=1e-5), r
        # eager work between replays
        call.indexer_topk()
        torch.cuda.synchronize()


def test_fused_kernel_withheld_handoff_gives_empty_ranges():
    """The tasks' failure path, forced from the host (DSA_TEST_WITHHOLD_READY:
    no sequence's rows are ever published and each task gives up after a few
    sleeps): every task writes an empty range, so the output is zero with
    lse = -inf, the index rows are still complete, the error bit is set, the
    state words come back zero and the next call is exact."""
    case = case_to(make_case("c2_decode_bf16", 90, batch=3, seq_len_range=(3000, 6000)), "cuda")
    call = B.Call(case)
    _say(f"withheld handoff: {case.name} B={case.batch}: normal call")
    out0, lse0, idx0 = _fused(call)
    ws, _ = call.workspace(B.DSA_OP_FUSED_DECODE)
    state = B.dsa_workspace_size(B.DSA_OP_INDEXER_TOPK, call.batch, call.iargs, call.sargs)
    B.dsa_take_device_errors(ws)
    _say("withheld handoff: every task gives up")
    with _env(DSA_TEST_WITHHOLD_READY="1"):
        out1, lse1, idx1 = _fused(call)
    assert np.array_equal(np.sort(idx0, 1), np.sort(idx1, 1))
    assert np.all(out1 == 0.0)
    assert np.all(np.isneginf(lse1))
    with pytest.raises(B.DsaError) as ei:
        B.dsa_take_device_errors(ws)
    assert ei.value.status == B.DSA_ERR_HIP
    assert int(ws[256:state].count_nonzero()) == 0
    _say("withheld handoff: a normal call afterwards")
    out2, lse2, idx2 = _fused(call)
    assert np.array_equal(np.sort(idx0, 1), np.sort(idx2, 1))
    mag = np.maximum(np.abs(out0), np.abs(out2))
    assert np.all(np.abs(out0 - out2) <= 2.0 ** -6 * mag + 2.0 ** -10)
    B.dsa_take_device_errors(ws)
