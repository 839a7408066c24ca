"""DSA_DEBUG=1: the device-side checks of the batch contents refuse a call
whose lengths, query offsets, block-table entries or index rows break the
preconditions, before any other kernel of the call runs (so the bad values
never reach a kernel that would follow them), and pass a valid call."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from checker import check_topk_row
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


@pytest.fixture()
def debug_env():
    old = os.environ.get("DSA_DEBUG")
    os.environ["DSA_DEBUG"] = "1"
    yield
    if old is None:
        os.environ.pop("DSA_DEBUG", None)
    else:
        os.environ["DSA_DEBUG"] = old


def _case():
    return case_to(make_case("c2_decode_bf16", 71, batch=3, seq_len_range=(2500, 4000)), "cuda")


def _refused(fn, what):
    with pytest.raises(B.DsaError) as ei:
        fn()
    assert ei.value.status == B.DSA_ERR_INVALID_ARG, ei.value
    assert what in str(ei.value), str(ei.value)


def test_valid_calls_pass(debug_env):
    case = _case()
    call = B.Call(case)
    _say("debug checks: valid fused decode")
    out, lse, idx = call.fused_decode()
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    for b in range(case.batch):
        check_topk_row(idx_h[case.token(b, 0)], oracle.run_query(case, b, 0), case.topk)
    _say("debug checks: valid sparse_attn on those rows")
    call.sparse_attn(idx)
    torch.cuda.synchronize()


def test_block_table_entry_out_of_range_is_refused(debug_env):
    case = _case()
    call = B.Call(case)
    # declare the pools one page shorter than the highest page in use, so a
    # block-table entry is out of range while every page it names exists
    bt = case.block_table.cpu().numpy()
    P = case.page_size
    used = max(int(bt[b, :(int(case.seq_lens_host[b]) + P - 1) // P].max()) for b in range(case.batch))
    call.k_cache.num_pages = used
    call.kv_cache.num_pages = used
    _say(f"debug checks: num_pages {used} with page {used} in use, indexer_topk and fused_decode")
    _refused(call.indexer_topk, "block_table entry")
    _refused(call.fused_decode, "block_table entry")


def test_length_beyond_capacity_is_refused(debug_env):
    case = _case()
    # one key more than the block table can address (the check refuses the
    # call before any kernel would follow the length)
    case.seq_lens[0] = case.block_table.shape[1] * case.page_size + 1
    call = B.Call(case)
    _say("debug checks: seq_len beyond max_pages_per_seq * page_size")
    _refused(call.indexer_topk, "seq_lens entry")


def test_index_row_outside_the_sequence_is_refused(debug_env):
    case = _case()
    call = B.Call(case)
    idx = torch.full((case.total_q, case.topk), -1, dtype=torch.int32, device="cuda")
    idx[:, 0] = 0
    idx[1, 5] = int(case.seq_lens_host[1])     # one past the last key of sequence 1
    _say("debug checks: index row position >= seq_len")
    _refused(lambda: call.sparse_attn(idx), "index row")
