"""Thin ctypes binding of the C ABI in include/dsa.h.

Argument marshalling only: every step of the computation runs in the HIP
library ``libdsa.so``.  PyTorch is used for device memory and the stream.  The
library must have been built (``python -m sparse_attention_04_amd.build`` or
``__graft_entry__.build()``); there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE_TOO_SMALL, DSA_ERR_HIP = range(5)
DSA_F32, DSA_BF16, DSA_FP8_E4M3, DSA_MXFP8_E4M3, DSA_FP8_E4M3_TILE128 = range(5)
DSA_OP_INDEXER_TOPK, DSA_OP_SPARSE_ATTN, DSA_OP_FUSED_DECODE, DSA_OP_FUSED_PREFILL = range(4)

DTYPE_CODE = {"f32": DSA_F32, "bf16": DSA_BF16, "fp8": DSA_FP8_E4M3, "mxfp8": DSA_MXFP8_E4M3,
              "fp8_t128": DSA_FP8_E4M3_TILE128}

EXPORTED = ("dsa_workspace_size", "dsa_indexer_topk", "dsa_sparse_attn", "dsa_fused_decode",
            "dsa_fused_prefill", "dsa_status_string", "dsa_last_error", "dsa_fused_decode_noalloc",
            "dsa_noalloc_scratch_bytes", "dsa_indexer_prolog", "dsa_prolog_workspace_size",
            "dsa_take_device_errors")


class DsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"dsa status {status}: {message}")
        self.status = status


class dsa_paged_cache(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32), ("dim", ctypes.c_int32)]


class dsa_batch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_lens", ctypes.c_void_p), ("cu_q", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("max_pages_per_seq", ctypes.c_int32),
                ("total_q", ctypes.c_int32), ("max_q_len", ctypes.c_int32), ("max_seq_len", ctypes.c_int32)]


class dsa_indexer_args(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("q_dtype", ctypes.c_int32), ("q_scale", ctypes.c_void_p),
                ("head_weights", ctypes.c_void_p), ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("k_cache", ctypes.POINTER(dsa_paged_cache))]


class dsa_sfa_args(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("q_dtype", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("qk_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("kv_cache", ctypes.POINTER(dsa_paged_cache))]


class dsa_prolog_args(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("d_model", ctypes.c_int32), ("w_q", ctypes.c_void_p),
                ("w_k", ctypes.c_void_p), ("w_w", ctypes.c_void_p), ("ln_gamma", ctypes.c_void_p),
                ("ln_beta", ctypes.c_void_p), ("ln_eps", ctypes.c_float), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libdsa.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.dsa_workspace_size.restype = ctypes.c_size_t
        L.dsa_workspace_size.argtypes = [ctypes.c_int32, P(dsa_batch), P(dsa_indexer_args), P(dsa_sfa_args)]
        L.dsa_indexer_topk.restype = ctypes.c_int
        L.dsa_indexer_topk.argtypes = [P(dsa_batch), P(dsa_indexer_args), ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p]
        L.dsa_sparse_attn.restype = ctypes.c_int
        L.dsa_sparse_attn.argtypes = [P(dsa_batch), P(dsa_sfa_args), ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p]
        L.dsa_fused_decode.restype = ctypes.c_int
        L.dsa_fused_decode.argtypes = [P(dsa_batch), P(dsa_indexer_args), P(dsa_sfa_args), ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
        L.dsa_fused_prefill.restype = ctypes.c_int
        L.dsa_fused_prefill.argtypes = [P(dsa_batch), P(dsa_indexer_args), P(dsa_sfa_args), ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]
        L.dsa_fused_decode_noalloc.restype = ctypes.c_int
        L.dsa_fused_decode_noalloc.argtypes = [P(dsa_batch), P(dsa_indexer_args), P(dsa_sfa_args), ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.dsa_noalloc_scratch_bytes.restype = ctypes.c_size_t
        L.dsa_noalloc_scratch_bytes.argtypes = []
        L.dsa_indexer_prolog.restype = ctypes.c_int
        L.dsa_indexer_prolog.argtypes = [P(dsa_batch), P(dsa_prolog_args), ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, P(dsa_paged_cache), ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.dsa_prolog_workspace_size.restype = ctypes.c_size_t
        L.dsa_prolog_workspace_size.argtypes = [P(dsa_batch), P(dsa_prolog_args)]
        L.dsa_status_string.restype = ctypes.c_char_p
        L.dsa_status_string.argtypes = [ctypes.c_int32]
        L.dsa_last_error.restype = ctypes.c_char_p
        L.dsa_last_error.argtypes = []
        L.dsa_take_device_errors.restype = ctypes.c_int
        L.dsa_take_device_errors.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _LIB = L
    return _LIB


def _check(status: int):
    if status != DSA_OK:
        raise DsaError(status, lib().dsa_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ------------------------------------------------------ raw ABI functions ---

def dsa_workspace_size(op, batch, iargs=None, sargs=None) -> int:
    P = ctypes.pointer
    return int(lib().dsa_workspace_size(op, P(batch), P(iargs) if iargs is not None else None,
                                        P(sargs) if sargs is not None else None))


def dsa_indexer_topk(batch, iargs, idx_out, ws, ws_bytes, stream=None):
    _check(lib().dsa_indexer_topk(ctypes.pointer(batch), ctypes.pointer(iargs), _ptr(idx_out), _ptr(ws),
                                  ws_bytes, _stream(stream)))


def dsa_sparse_attn(batch, sargs, idx, topk, out, lse, ws, ws_bytes, stream=None):
    _check(lib().dsa_sparse_attn(ctypes.pointer(batch), ctypes.pointer(sargs), _ptr(idx), topk, _ptr(out),
                                 _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def dsa_fused_decode(batch, iargs, sargs, out, lse, idx_out, ws, ws_bytes, stream=None):
    _check(lib().dsa_fused_decode(ctypes.pointer(batch), ctypes.pointer(iargs), ctypes.pointer(sargs),
                                  _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(ws), ws_bytes, _stream(stream)))


def dsa_fused_prefill(batch, iargs, sargs, q_block, out, lse, idx_out, ws, ws_bytes, stream=None):
    _check(lib().dsa_fused_prefill(ctypes.pointer(batch), ctypes.pointer(iargs), ctypes.pointer(sargs),
                                   q_block, _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(ws), ws_bytes,
                                   _stream(stream)))


def dsa_fused_decode_noalloc(batch, iargs, sargs, out, lse, idx_out, stream=None):
    _check(lib().dsa_fused_decode_noalloc(ctypes.pointer(batch), ctypes.pointer(iargs), ctypes.pointer(sargs),
                                          _ptr(out), _ptr(lse), _ptr(idx_out), _stream(stream)))


def dsa_noalloc_scratch_bytes() -> int:
    return int(lib().dsa_noalloc_scratch_bytes())


def dsa_take_device_errors(ws=None, stream=None):
    """Raise DsaError(DSA_ERR_HIP) if a bounded wait of the decode indexer gave
    up in a call on workspace `ws` (None: the static scratch of the
    allocation-free entry point) since the last check; clears the bits."""
    _check(lib().dsa_take_device_errors(_ptr(ws), _stream(stream)))


def dsa_indexer_prolog(batch, pargs, q_out, q_scale_out, w_out, k_cache, q_bf16_out, k_bf16_out, ws, ws_bytes,
                       stream=None):
    _check(lib().dsa_indexer_prolog(ctypes.pointer(batch), ctypes.pointer(pargs), _ptr(q_out), _ptr(q_scale_out),
                                    _ptr(w_out), ctypes.pointer(k_cache), _ptr(q_bf16_out), _ptr(k_bf16_out),
                                    _ptr(ws), ws_bytes, _stream(stream)))


def dsa_prolog_workspace_size(batch, pargs) -> int:
    return int(lib().dsa_prolog_workspace_size(ctypes.pointer(batch), ctypes.pointer(pargs)))


# ------------------------------------------- struct builders from tensors ---

class Call:
    """Holds the ctypes structs for one workload (and references to its
    tensors), plus output and workspace tensors allocated with torch."""

    def __init__(self, case):
        c = case
        self.case = c
        self.batch = dsa_batch(c.batch, _ptr(c.seq_lens), _ptr(c.cu_q), _ptr(c.block_table),
                               c.max_pages_per_seq, c.total_q, c.max_q_len, c.max_seq_len)
        idt = DTYPE_CODE[c.idx_dtype]
        self.k_cache = dsa_paged_cache(_ptr(c.k_pool), _ptr(c.k_scale), idt, c.num_pages, c.page_size, c.d_i)
        self.iargs = dsa_indexer_args(_ptr(c.q_i), idt, _ptr(c.q_i_scale), _ptr(c.w), c.h_i, c.d_i, c.topk,
                                      ctypes.pointer(self.k_cache))
        sdt = DTYPE_CODE[c.sfa_dtype]
        kdt = DTYPE_CODE[getattr(c, "kv_dtype", None) or c.sfa_dtype]
        self.kv_cache = dsa_paged_cache(_ptr(c.kv_pool), _ptr(getattr(c, "kv_scale", None)), kdt,
                                        c.num_pages, c.page_size, c.d_qk)
        self.sargs = dsa_sfa_args(_ptr(c.q_s), sdt, c.h_s, c.d_qk, c.d_v, float(c.softmax_scale),
                                  ctypes.pointer(self.kv_cache))
        dev = c.q_s.device
        self.idx = torch.empty((c.total_q, c.topk), dtype=torch.int32, device=dev)
        self.out = torch.empty((c.total_q, c.h_s, c.d_v), dtype=c.q_s.dtype, device=dev)
        self.lse = torch.empty((c.total_q, c.h_s), dtype=torch.float32, device=dev)
        self._ws = {}

    def workspace(self, op):
        """The call's workspace and its size in bytes (which the calls pass on:
        the library keeps scratch at the end of the buffer it is given).
        Zero-filled when allocated, as the ABI asks of a workspace before its
        first use (calls leave it ready for the next)."""
        n = dsa_workspace_size(op, self.batch, self.iargs, self.sargs)
        if op not in self._ws or self._ws[op].numel() < n:
            self._ws[op] = torch.zeros(max(n, 1), dtype=torch.uint8, device=self.case.q_s.device)
        return self._ws[op], self._ws[op].numel()

    def use_workspace(self, op, ws):
        """Run `op` with a caller-supplied (zero-filled before first use) workspace."""
        self._ws[op] = ws

    def indexer_topk(self, stream=None):
        ws, n = self.workspace(DSA_OP_INDEXER_TOPK)
        dsa_indexer_topk(self.batch, self.iargs, self.idx, ws, n, stream)
        return self.idx

    def sparse_attn(self, idx, stream=None):
        ws, n = self.workspace(DSA_OP_SPARSE_ATTN)
        dsa_sparse_attn(self.batch, self.sargs, idx, idx.shape[1], self.out, self.lse, ws, n, stream)
        return self.out, self.lse

    def fused_decode(self, with_idx=True, stream=None):
        ws, n = self.workspace(DSA_OP_FUSED_DECODE)
        dsa_fused_decode(self.batch, self.iargs, self.sargs, self.out, self.lse,
                         self.idx if with_idx else None, ws, n, stream)
        return self.out, self.lse, self.idx

    def prolog(self, pro, q_bf16_out=None, k_bf16_out=None, stream=None):
        """Run the indexer prolog on the prolog inputs `pro` (make_prolog): it
        writes this case's indexer q, q scales and head weights and appends the
        new tokens' keys to its K cache.  Returns the tensors it wrote."""
        c = self.case
        args = dsa_prolog_args(_ptr(pro["x"]), pro["d_model"], _ptr(pro["w_q"]), _ptr(pro["w_k"]),
                               _ptr(pro["w_w"]), _ptr(pro["ln_gamma"]), _ptr(pro["ln_beta"]), pro["ln_eps"],
                               c.h_i, c.d_i, DTYPE_CODE[c.idx_dtype])
        n = dsa_prolog_workspace_size(self.batch, args)
        if "prolog" not in self._ws or self._ws["prolog"].numel() < n:
            self._ws["prolog"] = torch.zeros(max(n, 1), dtype=torch.uint8, device=c.q_s.device)
        dsa_indexer_prolog(self.batch, args, c.q_i, c.q_i_scale, c.w, self.k_cache, q_bf16_out, k_bf16_out,
                           self._ws["prolog"], n, stream)
        return c.q_i, c.q_i_scale, c.w

    def fused_decode_noalloc(self, out, lse, idx=None, stream=None):
        dsa_fused_decode_noalloc(self.batch, self.iargs, self.sargs, out, lse, idx, stream)
        return out, lse, idx

    def fused_prefill(self, with_idx=True, stream=None, q_block=64):
        ws, n = self.workspace(DSA_OP_FUSED_PREFILL)
        dsa_fused_prefill(self.batch, self.iargs, self.sargs, q_block, self.out, self.lse,
                          self.idx if with_idx else None, ws, n, stream)
        return self.out, self.lse, self.idx
