"""The allocation-free decode entry point against the workspace one, on the GPU.

Two calls in a row through the C ABI, the second with a smaller batch (the
static scratch keeps the first call's contents): the index sets must be
identical and the SFA output within the bf16 bar of the workspace path's, and
both are checked against the oracle on every query."""
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


def test_noalloc_matches_workspace_entry_point():
    assert torch.cuda.is_available()
    B.lib()
    cases = [case_to(make_case("c2_decode_bf16", 61, batch=6, seq_len_range=(3000, 9000)), "cuda"),
             case_to(make_case("c5_decode4", 62, batch=2, seq_len_range=(2500, 4000)), "cuda")]
    for case in cases:
        call = B.Call(case)
        _say(f"no-alloc: {case.name} B={case.batch} T={case.total_q}: workspace path")
        out_w, lse_w, idx_w = (t.clone() for t in call.fused_decode())
        out = torch.empty_like(out_w)
        lse = torch.empty_like(lse_w)
        idx = torch.empty_like(idx_w)
        _say(f"no-alloc: {case.name}: static-scratch path")
        call.fused_decode_noalloc(out, lse, idx)
        torch.cuda.synchronize()
        assert torch.equal(torch.sort(idx, 1).values, torch.sort(idx_w, 1).values)
        out_h, outw_h = out.float().cpu().numpy(), out_w.float().cpu().numpy()
        idx_h = idx.cpu().numpy()
        for b in range(case.batch):
            for i in range(int(case.q_lens_host[b])):
                tok = case.token(b, i)
                check_sfa(out_h[tok], outw_h[tok], "bf16")
                ref = oracle.run_query(case, b, i)
                check_topk_row(idx_h[tok], ref, case.topk)
                sel = idx_h[tok][idx_h[tok] >= 0]
                check_sfa(out_h[tok], oracle.sfa_query(case, b, i, sel)[0], "bf16")
        assert np.allclose(lse.cpu().numpy(), lse_w.cpu().numpy(), atol=1e-4, rtol=1e-5)


def test_noalloc_calls_of_growing_shapes():
    """A small call, then a larger one whose indexer state reaches past where
    the small call left its index rows: the static array keeps state and
    scratch apart, so the larger call is still exact."""
    B.lib()
    for case in (case_to(make_case("c2_decode_bf16", 64, batch=2, seq_len_range=(2200, 3000)), "cuda"),
                 case_to(make_case("c5_decode4", 65, batch=6, seq_len_range=(3000, 5000)), "cuda")):
        call = B.Call(case)
        out = torch.empty_like(call.out)
        lse = torch.empty_like(call.lse)
        idx = torch.empty_like(call.idx)
        _say(f"no-alloc growing: {case.name} B={case.batch} T={case.total_q}")
        call.fused_decode_noalloc(out, lse, idx)
        torch.cuda.synchronize()
        idx_h, out_h = idx.cpu().numpy(), out.float().cpu().numpy()
        for b in range(case.batch):
            for i in range(int(case.q_lens_host[b])):
                tok = case.token(b, i)
                check_topk_row(idx_h[tok], oracle.run_query(case, b, i), case.topk)
        tok = case.token(case.batch - 1, 0)
        check_sfa(out_h[tok], oracle.sfa_query(case, case.batch - 1, 0, idx_h[tok][idx_h[tok] >= 0])[0], "bf16")


def test_noalloc_rejects_calls_beyond_its_scratch():
    B.lib()
    case = case_to(make_case("c2_decode_bf16", 63, batch=2, seq_len_range=(3000, 4000)), "cuda")
    call = B.Call(case)
    call.batch.total_q = 4096          # a decode batch whose scratch exceeds the static array
    call.batch.batch = 2
    call.batch.max_q_len = 2048
    need = B.dsa_workspace_size(B.DSA_OP_FUSED_DECODE, call.batch, call.iargs, call.sargs)
    assert need > B.dsa_noalloc_scratch_bytes()
    st = B.lib().dsa_fused_decode_noalloc(*(B.ctypes.pointer(x) for x in (call.batch, call.iargs, call.sargs)),
                                          call.out.data_ptr(), call.lse.data_ptr(), None, None)
    assert st == B.DSA_ERR_UNSUPPORTED and b"static scratch" in B.lib().dsa_last_error()


def test_noalloc_empty_call_then_real_call():
    """No new token in any sequence (total_q = 0): the call returns without
    computing; the next call on the same static scratch is exact."""
    assert torch.cuda.is_available()
    B.lib()
    empty = case_to(make_case("c5_decode4", 65, batch=2, seq_lens=[3000, 4000], q_lens=[0, 0]), "cuda")
    real = case_to(make_case("c2_decode_bf16", 66, batch=3, seq_len_range=(2500, 6000)), "cuda")
    ce, cr = B.Call(empty), B.Call(real)
    _say("no-alloc: empty call")
    ce.fused_decode_noalloc(ce.out, ce.lse, ce.idx)
    _say(f"no-alloc: {real.name} B={real.batch} T={real.total_q} after it")
    out, lse, idx = torch.empty_like(cr.out), torch.empty_like(cr.lse), torch.empty_like(cr.idx)
    cr.fused_decode_noalloc(out, lse, idx)
    torch.cuda.synchronize()
    idx_h, out_h = idx.cpu().numpy(), out.float().cpu().numpy()
    for b in range(real.batch):
        g = real.token(b, 0)
        ref = oracle.run_query(real, b, 0)
        check_topk_row(idx_h[g], ref, real.topk)
        sel = idx_h[g][idx_h[g] >= 0]
        ref_o, _ = oracle.sfa_query(real, b, 0, sel)
        check_sfa(out_h[g], ref_o, real.sfa_dtype)
    # no bounded wait gave up in these calls: the static scratch's error bits are clear
    B.dsa_take_device_errors(None)


def test_noalloc_graph_replays_match_the_eager_call():
    """A captured allocation-free call (captured after an eager one, which
    makes the one-time clear) replayed three times, with eager work between
    the replays: each replay's rows and outputs match the eager call's."""
    assert torch.cuda.is_available()
    B.lib()
    case = case_to(make_case("c2_decode_bf16", 67, batch=3, seq_len_range=(3000, 6000)), "cuda")
    call = B.Call(case)
    out, lse, idx = torch.empty_like(call.out), torch.empty_like(call.lse), torch.empty_like(call.idx)
    _say("no-alloc graph: eager call")
    call.fused_decode_noalloc(out, lse, idx)
    torch.cuda.synchronize()
    out0, lse0, idx0 = out.float().cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call.fused_decode_noalloc(out, lse, idx)
    torch.cuda.synchronize()
    for r in range(3):
        idx.fill_(-1)
        torch.cuda.synchronize()
        _say(f"no-alloc graph: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        out1, lse1, idx1 = out.float().cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()
        assert np.array_equal(np.sort(idx0, 1), np.sort(idx1, 1)), r
        mag = np.maximum(np.abs(out0), np.abs(out1))
        assert np.all(np.abs(out0 - out1) <= 2.0 ** -6 * mag + 2.0 ** -10), r
        assert np.allclose(lse0, lse1, atol=1e-4, rtol=1e-5), r
        call.fused_decode()     # eager work between replays (the workspace path)
        torch.cuda.synchronize()
    B.dsa_take_device_errors(None)
