"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects bad arguments with the documented status before touching the GPU."""
import ctypes
import os
import re

import pytest

from sparse_attention_04_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dsa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|size_t|dsa_status)\s+(dsa_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 7
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.EXPORTED)


def test_status_strings():
    lib = B.lib()
    assert lib.dsa_status_string(0) == b"ok"
    assert lib.dsa_status_string(3) == b"workspace too small"
    assert lib.dsa_status_string(99) == b"unknown status"


def _structs(h_i=64, d_i=128, dt=B.DSA_BF16, topk=2048, page=64, h_s=128, dqk=576, dv=512, sdt=B.DSA_BF16):
    # fake non-null device pointers: validation fails before any dereference
    fake = 0x1000
    batch = B.dsa_batch(2, fake, fake, fake, 8, 2, 1, 512)
    kc = B.dsa_paged_cache(fake, fake, dt, 16, page, d_i)
    ia = B.dsa_indexer_args(fake, dt, fake, fake, h_i, d_i, topk, ctypes.pointer(kc))
    vc = B.dsa_paged_cache(fake, None, sdt, 16, page, dqk)
    sa = B.dsa_sfa_args(fake, sdt, h_s, dqk, dv, 0.07, ctypes.pointer(vc))
    return batch, ia, sa, (kc, vc)


def _status(fn, *a):
    try:
        fn(*a)
    except B.DsaError as e:
        return e.status
    return 0


def test_workspace_size_positive_and_monotone():
    batch, ia, sa, keep = _structs()
    n1 = B.dsa_workspace_size(B.DSA_OP_FUSED_DECODE, batch, ia, sa)
    batch.total_q = 64
    batch.max_q_len = 32
    n2 = B.dsa_workspace_size(B.DSA_OP_FUSED_DECODE, batch, ia, sa)
    assert 0 < n1 < n2
    assert B.dsa_workspace_size(99, batch, ia, sa) == 0


@pytest.mark.parametrize("mutate,expected", [
    (lambda b, i, s: setattr(b, "batch", 0), B.DSA_ERR_INVALID_ARG),
    (lambda b, i, s: setattr(b, "seq_lens", None), B.DSA_ERR_INVALID_ARG),
    (lambda b, i, s: setattr(b, "max_q_len", 1000), B.DSA_ERR_INVALID_ARG),
    (lambda b, i, s: setattr(i, "topk", 0), B.DSA_ERR_INVALID_ARG),
    (lambda b, i, s: setattr(i, "q", None), B.DSA_ERR_INVALID_ARG),
    (lambda b, i, s: setattr(i, "q_scale", None) or setattr(i, "q_dtype", B.DSA_FP8_E4M3), B.DSA_ERR_INVALID_ARG),
    (lambda b, i, s: setattr(i, "n_heads", 32), B.DSA_ERR_UNSUPPORTED),
    (lambda b, i, s: setattr(i, "head_dim", 64), B.DSA_ERR_UNSUPPORTED),
    (lambda b, i, s: setattr(i.k_cache.contents, "dtype", B.DSA_F32), B.DSA_ERR_INVALID_ARG),
    (lambda b, i, s: setattr(i.k_cache.contents, "page_size", 0), B.DSA_ERR_UNSUPPORTED),
    (lambda b, i, s: setattr(i.k_cache.contents, "page_size", 48), B.DSA_ERR_UNSUPPORTED),
    (lambda b, i, s: setattr(b, "max_pages_per_seq", 1), B.DSA_ERR_INVALID_ARG),
    (lambda b, i, s: setattr(s, "v_dim", 256), B.DSA_ERR_UNSUPPORTED),
    (lambda b, i, s: setattr(s, "q_dtype", B.DSA_FP8_E4M3), B.DSA_ERR_UNSUPPORTED),
    (lambda b, i, s: setattr(s, "softmax_scale", 0.0), B.DSA_ERR_INVALID_ARG),
    # FP8 tile-128 rows are an SFA KV cache format only, and carry their scales
    (lambda b, i, s: setattr(s.kv_cache.contents, "dtype", B.DSA_FP8_E4M3_TILE128), B.DSA_ERR_INVALID_ARG),
    (lambda b, i, s: setattr(s, "q_dtype", B.DSA_FP8_E4M3_TILE128), B.DSA_ERR_UNSUPPORTED),
    (lambda b, i, s: setattr(i, "q_dtype", B.DSA_FP8_E4M3_TILE128), B.DSA_ERR_INVALID_ARG),
    (lambda b, i, s: setattr(s.kv_cache.contents, "dtype", B.DSA_FP8_E4M3), B.DSA_ERR_INVALID_ARG),
])
def test_fused_decode_rejects_bad_arguments(mutate, expected):
    batch, ia, sa, keep = _structs()
    mutate(batch, ia, sa)
    out = ctypes.c_void_p(0x2000)
    st = B.lib().dsa_fused_decode(ctypes.pointer(batch), ctypes.pointer(ia), ctypes.pointer(sa), out, None, None,
                                  None, 0, None)
    assert st == expected, B.lib().dsa_last_error()
    assert B.lib().dsa_last_error() != b""


def test_workspace_too_small_is_reported_before_any_launch():
    batch, ia, sa, keep = _structs()
    need = B.dsa_workspace_size(B.DSA_OP_FUSED_DECODE, batch, ia, sa)
    st = B.lib().dsa_fused_decode(ctypes.pointer(batch), ctypes.pointer(ia), ctypes.pointer(sa),
                                  ctypes.c_void_p(0x2000), None, None, ctypes.c_void_p(0x3000), need - 1, None)
    assert st == B.DSA_ERR_WORKSPACE_TOO_SMALL
    st = B.lib().dsa_indexer_topk(ctypes.pointer(batch), ctypes.pointer(ia), ctypes.c_void_p(0x2000), None, 0, None)
    assert st == B.DSA_ERR_WORKSPACE_TOO_SMALL


def test_indexer_requires_output():
    batch, ia, sa, keep = _structs()
    st = B.lib().dsa_indexer_topk(ctypes.pointer(batch), ctypes.pointer(ia), None, None, 0, None)
    assert st == B.DSA_ERR_INVALID_ARG


def test_prefill_rejects_other_block_sizes():
    batch, ia, sa, keep = _structs()
    st = B.lib().dsa_fused_prefill(ctypes.pointer(batch), ctypes.pointer(ia), ctypes.pointer(sa), 32,
                                   ctypes.c_void_p(0x2000), None, None, None, 0, None)
    assert st == B.DSA_ERR_UNSUPPORTED


def test_sparse_attn_argument_checks():
    batch, ia, sa, keep = _structs()
    st = B.lib().dsa_sparse_attn(ctypes.pointer(batch), ctypes.pointer(sa), None, 2048,
                                 ctypes.c_void_p(0x2000), None, None, 0, None)
    assert st == B.DSA_ERR_INVALID_ARG
    st = B.lib().dsa_sparse_attn(ctypes.pointer(batch), ctypes.pointer(sa), ctypes.c_void_p(0x4000), 0,
                                 ctypes.c_void_p(0x2000), None, None, 0, None)
    assert st == B.DSA_ERR_INVALID_ARG


def test_fp8_kv_cache_passes_validation():
    """An FP8 tile-128 KV cache with its scale pool is accepted for bf16 and
    f32 queries: the call gets as far as the workspace check."""
    for kw in (dict(), dict(h_s=8, dqk=80, dv=64, sdt=B.DSA_F32, h_i=4, d_i=32, dt=B.DSA_F32, topk=64)):
        batch, ia, sa, (kc, vc) = _structs(**kw)
        vc.dtype = B.DSA_FP8_E4M3_TILE128
        vc.scale = 0x5000
        need = B.dsa_workspace_size(B.DSA_OP_FUSED_DECODE, batch, ia, sa)
        st = B.lib().dsa_fused_decode(ctypes.pointer(batch), ctypes.pointer(ia), ctypes.pointer(sa),
                                      ctypes.c_void_p(0x2000), None, None, ctypes.c_void_p(0x3000), need - 1, None)
        assert st == B.DSA_ERR_WORKSPACE_TOO_SMALL, B.lib().dsa_last_error()


@pytest.mark.parametrize("what", ["out", "ws", "q", "kv", "bt"])
def test_misaligned_pointers_are_rejected(what):
    """The kernels move q, cache rows, outputs and the workspace 16 bytes at a
    time; a misaligned pointer is refused before anything is enqueued."""
    batch, ia, sa, (kc, vc) = _structs()
    out, ws = 0x2000, 0x3000
    if what == "out":
        out = 0x2008
    elif what == "ws":
        ws = 0x3004
    elif what == "q":
        sa.q = 0x1008
    elif what == "kv":
        vc.data = 0x1004
    else:
        batch.block_table = 0x1002
    need = B.dsa_workspace_size(B.DSA_OP_FUSED_DECODE, batch, ia, sa)
    st = B.lib().dsa_fused_decode(ctypes.pointer(batch), ctypes.pointer(ia), ctypes.pointer(sa),
                                  ctypes.c_void_p(out), None, None, ctypes.c_void_p(ws), need, None)
    assert st == B.DSA_ERR_INVALID_ARG, B.lib().dsa_last_error()
    assert b"align" in B.lib().dsa_last_error()


def test_empty_calls_return_ok_without_per_token_arrays():
    """total_q = 0: every entry point validates and returns DSA_OK without
    computing, and the per-token arrays may be NULL (nothing is enqueued, so
    the fake batch and workspace pointers are never used)."""
    batch, ia, sa, keep = _structs()
    batch.total_q = 0
    batch.max_q_len = 0
    ia.q = ia.q_scale = ia.head_weights = None
    sa.q = None
    lib = B.lib()
    bp, ip, sp = ctypes.pointer(batch), ctypes.pointer(ia), ctypes.pointer(sa)
    ws = ctypes.c_void_p(0x4000)
    n = B.dsa_workspace_size(B.DSA_OP_FUSED_DECODE, batch, ia, sa)
    assert lib.dsa_fused_decode(bp, ip, sp, None, None, None, ws, n, None) == B.DSA_OK, lib.dsa_last_error()
    n = B.dsa_workspace_size(B.DSA_OP_INDEXER_TOPK, batch, ia, sa)
    assert lib.dsa_indexer_topk(bp, ip, None, ws, n, None) == B.DSA_OK, lib.dsa_last_error()
    n = B.dsa_workspace_size(B.DSA_OP_SPARSE_ATTN, batch, ia, sa)
    assert lib.dsa_sparse_attn(bp, sp, None, 2048, None, None, ws, n, None) == B.DSA_OK, lib.dsa_last_error()
    n = B.dsa_workspace_size(B.DSA_OP_FUSED_PREFILL, batch, ia, sa)
    assert lib.dsa_fused_prefill(bp, ip, sp, 64, None, None, None, ws, n, None) == B.DSA_OK, lib.dsa_last_error()
    fake = 0x1000
    pa = B.dsa_prolog_args(None, 7168, fake, fake, fake, fake, fake, 1e-6, 64, 128, B.DSA_FP8_E4M3)
    kc = B.dsa_paged_cache(fake, fake, B.DSA_FP8_E4M3, 16, 64, 128)
    n = lib.dsa_prolog_workspace_size(bp, ctypes.pointer(pa))
    assert lib.dsa_indexer_prolog(bp, ctypes.pointer(pa), None, None, None, ctypes.pointer(kc), None, None, ws, n,
                                  None) == B.DSA_OK, lib.dsa_last_error()
    # with a token the same NULL arrays are refused
    batch.total_q = 1
    batch.max_q_len = 1
    assert lib.dsa_fused_decode(bp, ip, sp, None, None, None, ws, 1 << 30, None) == B.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_topk(bp, ip, None, ws, 1 << 30, None) == B.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_prolog(bp, ctypes.pointer(pa), None, None, None, ctypes.pointer(kc), None, None, ws,
                                  1 << 30, None) == B.DSA_ERR_INVALID_ARG


def test_take_device_errors_checks_its_pointer_first():
    # a misaligned workspace is refused before anything touches the device
    assert B.lib().dsa_take_device_errors(ctypes.c_void_p(0x1004), None) == B.DSA_ERR_INVALID_ARG
    assert b"aligned" in B.lib().dsa_last_error()
