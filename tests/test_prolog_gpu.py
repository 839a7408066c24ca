"""The indexer prolog on the GPU against the oracle, through the C ABI.

q and k before quantisation are floating point (float32 accumulation on the
GPU, float64 in the oracle), so they must agree within one bf16 unit in the
last place; the quantised bytes and scales are integers decided from those
bf16 values, so the oracle's quantiser is applied to the GPU's own bf16 q and
k and must reproduce the stored bytes and scales exactly.  Keys are appended
only at the new tokens' cache rows.  Then the quantised decode step runs on
the inputs the prolog produced on the device and is checked against the
oracle reading the same tensors."""
import sys

import numpy as np
import pytest
import torch

import oracle
from checker import check_sfa, check_topk_row
from sparse_attention_04_amd import binding as B
from sparse_attention_04_amd.inputs import case_to, make_case, make_prolog

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    B.lib()


def _bits(t):
    t = t.detach().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _within_one_ulp(got_bits, ref_bits, slack):
    """bf16 values within one unit in the last place of the oracle's, plus
    `slack`: the float32 accumulation's own error (about 2^-24 per unit of
    sum |terms|), which matters where the terms cancel to a small result."""
    g = oracle.decode_bf16_bits(got_bits)
    r = oracle.decode_bf16_bits(ref_bits)
    ulp = np.maximum(np.abs(r), 2.0 ** -126) * 2.0 ** -7
    assert np.all(np.abs(g - r) <= ulp + slack), np.abs(g - r).max()
    return float(np.mean(g != r))


def _run_prolog(case, d_model, seed, tokens=None):
    pro = make_prolog(case, seed, d_model=d_model)
    k_before = case.k_pool.clone()
    ks_before = None if case.k_scale is None else case.k_scale.clone()
    call = B.Call(case)
    q_bf16 = torch.empty((case.total_q, case.h_i * case.d_i), dtype=torch.bfloat16, device=case.q_s.device)
    k_bf16 = torch.empty((case.total_q, case.d_i), dtype=torch.bfloat16, device=case.q_s.device)
    _say(f"prolog {case.name} T={case.total_q} d_model={d_model} dtype={case.idx_dtype}")
    call.prolog(pro, q_bf16, k_bf16)
    torch.cuda.synchronize()
    if case.idx_dtype == "bf16":
        q_bf16 = case.q_i.reshape(case.total_q, -1)
    x, wq, wk, ww = (_bits(pro[k]) for k in ("x", "w_q", "w_k", "w_w"))
    gamma, beta = pro["ln_gamma"].cpu().numpy(), pro["ln_beta"].cpu().numpy()
    qg, kg = _bits(q_bf16), _bits(k_bf16)
    q_store, w_out = _bits(case.q_i), case.w.cpu().numpy()
    q_sc = None if case.q_i_scale is None else case.q_i_scale.cpu().numpy()
    kpool, kscale = _bits(case.k_pool), None if case.k_scale is None else case.k_scale.cpu().numpy()
    bt = case.block_table.cpu().numpy()
    touched = set()
    flips = []
    toks = [(b, i) for b in range(case.batch) for i in range(int(case.q_lens_host[b]))]
    for (b, i) in toks:
        g = case.token(b, i)
        page, row = oracle.append_position(int(case.seq_lens_host[b]), int(case.q_lens_host[b]), i, bt[b],
                                           case.page_size)
        touched.add(page * case.page_size + row)
        if tokens is not None and g not in tokens:
            continue
        q_ref, k_ref, w_ref = oracle.prolog_token(x[g], wq, wk, ww, gamma, beta, case.h_i, case.d_i, pro["ln_eps"])
        ax = np.abs(oracle.decode_bf16_bits(x[g]))
        qmag = np.abs(oracle.decode_bf16_bits(wq)) @ ax
        kmag = np.abs(oracle.decode_bf16_bits(wk)) @ ax
        # k: the projection's error, scaled by LayerNorm's 1 / std and gamma
        kp = oracle.decode_bf16_bits(wk) @ oracle.decode_bf16_bits(x[g])
        kslack = 2.0 ** -20 * kmag.max() / np.sqrt(kp.var() + pro["ln_eps"]) * np.abs(gamma) + 2.0 ** -20
        flips.append(_within_one_ulp(qg[g], q_ref.reshape(-1), 2.0 ** -20 * qmag))
        flips.append(_within_one_ulp(kg[g], k_ref, kslack))
        mag = np.abs(oracle.decode_bf16_bits(ww)) @ ax
        assert np.all(np.abs(w_out[g] - w_ref) <= 1e-4 * mag + 1e-30), np.abs(w_out[g] - w_ref).max()
        # stored q and its scales: the oracle's quantiser on the GPU's bf16 q
        qs, qsc = oracle.quantise_query(qg[g].reshape(case.h_i, case.d_i), case.idx_dtype)
        assert np.array_equal(np.asarray(q_store[g]).reshape(qs.shape), qs), g
        if qsc is not None:
            assert np.array_equal(q_sc[g].reshape(qsc.shape), qsc), g
        # the appended key and its scale(s)
        ks, ksc = oracle.quantise_key(kg[g], case.idx_dtype)
        assert np.array_equal(np.asarray(kpool[page, row]), ks), (g, page, row)
        if ksc is not None:
            assert np.array_equal(np.asarray(kscale[page, row]).reshape(np.shape(ksc)), ksc), (g, page, row)
    # every other cache row is untouched
    flat_b = k_before.reshape(-1, case.d_i)
    flat_a = case.k_pool.reshape(-1, case.d_i)
    keep = torch.ones(flat_a.shape[0], dtype=torch.bool, device=flat_a.device)
    keep[torch.tensor(sorted(touched), device=flat_a.device)] = False
    same = (flat_a[keep] == flat_b[keep]) | (flat_a[keep] != flat_a[keep])     # NaN poison compares unequal
    assert bool(same.all())
    if ks_before is not None:
        sa, sb = case.k_scale.reshape(flat_a.shape[0], -1)[keep], ks_before.reshape(flat_a.shape[0], -1)[keep]
        assert bool(((sa == sb) | (sa != sa)).all())
    _say(f"prolog {case.name}: bf16 rounding flips {max(flips):.4f} of elements at most")
    return call


def _check_decode(case, call, limit=None):
    out, lse, idx = call.fused_decode()
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    out_h = out.float().cpu().numpy()
    qs = [(b, i) for b in range(case.batch) for i in range(int(case.q_lens_host[b]))]
    if limit:
        qs = [qs[j] for j in np.random.default_rng(3).choice(len(qs), limit, replace=False)]
    for (b, i) in qs:
        ref = oracle.run_query(case, b, i)
        row = idx_h[case.token(b, i)]
        check_topk_row(row, ref, case.topk)
        check_sfa(out_h[case.token(b, i)], oracle.sfa_query(case, b, i, row[row >= 0])[0], case.sfa_dtype)


@pytest.mark.parametrize("name", ["c4_decode_fp8", "c4_decode_mxfp8"])
def test_prolog_quantised_decode_small(name):
    case = case_to(make_case(name, 71, batch=3, seq_len_range=(3000, 6000)), "cuda")
    call = _run_prolog(case, 1024, 71)
    _check_decode(case, call)


def test_prolog_bf16_multi_token():
    # four new tokens per sequence over 16-token pages: keys appended at the
    # last four positions, some in a fresh page
    case = case_to(make_case("c5_decode4", 72, batch=2, seq_lens=[3001, 4100], page_size=16), "cuda")
    call = _run_prolog(case, 1024, 72)
    _check_decode(case, call)


def test_prolog_many_tokens_ragged():
    # 150 new tokens: three 64-token blocks, the last ragged; MXFP8 keys
    case = case_to(make_case("c4_decode_mxfp8", 73, batch=2, seq_lens=[2600, 3100], q_lens=[70, 80]), "cuda")
    _run_prolog(case, 2048, 73)


def test_prolog_full_size_fp8():
    """The quantised decode workload at full size (64 sequences, contexts
    U[16384, 65536]) with its inputs produced by the prolog from hidden rows of
    width 7168: every token's prolog outputs, then sampled decode queries."""
    _say("prolog full size: generating on device")
    case = make_case("c4_decode_fp8", 74, device="cuda")
    call = _run_prolog(case, 7168, 74)
    _check_decode(case, call, limit=8)


@pytest.mark.parametrize("name,heads,d_model", [("c4_decode_fp8", 32, 640), ("c4_decode_mxfp8", 128, 384),
                                                ("c5_decode4", 96, 1024)])
def test_prolog_other_head_counts_and_widths(name, heads, d_model):
    """Head counts other than 64 and hidden widths that split d_model unevenly
    (640: ranges of 2 and 3 chunks of 128) or not at all (384): the GEMM's
    tiles of 144 concatenated weight rows end partway through W_w, and with
    96 heads the workgroups take more than one round."""
    case = case_to(make_case(name, 76, batch=2, seq_lens=[3000, 4100], h_i=heads), "cuda")
    _run_prolog(case, d_model, 76)
