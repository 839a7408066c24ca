"""The oracle's indexer-prolog functions against their pins (CPU only).

Each is checked against something other than itself: hand-worked golden rows
(tests/golden/prolog_quant_rows.txt), torch's bfloat16 / float8_e4m3fn casts
and layer_norm, exact rational arithmetic, pure-Python loops, and the
properties the OCP FP8 / MX definitions fix.  Planted mistakes must fail."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prolog_quant_rows.txt")


def _golden():
    fp8_vals, fp8_codes, fp8_scale = [], [], None
    mx = np.zeros(64, np.float32)
    mx_codes, mx_scales = {}, {}
    for line in open(GOLDEN):
        f = line.split("#")[0].split()
        if not f:
            continue
        if f[0] == "fp8" and f[1] == "scale":
            fp8_scale = float(f[2])
        elif f[0] == "fp8":
            fp8_vals.append(float(f[1]))
            fp8_codes.append(int(f[2], 16))
        elif f[0] == "mx" and f[1] == "group":
            mx_scales[int(f[2])] = int(f[4], 16)
        elif f[0] == "mx":
            mx[int(f[1])] = float(f[2])
            mx_codes[int(f[1])] = int(f[3], 16)
    return (np.array(fp8_vals, np.float32), fp8_codes, fp8_scale), (mx, mx_codes, mx_scales)


# ---------------------------------------------------------------- pins ---

def pin_fp8_quantise(fn):
    (v, codes, scale), _ = _golden()
    b, s = fn(v)
    assert [int(x) for x in b] == codes, [hex(int(x)) for x in b]
    assert float(s) == scale
    # torch's e4m3 cast of v / scale (float32 division), and the row's amax
    # always lands on 448
    r = np.random.default_rng(5)
    for row in [r.standard_normal(128).astype(np.float32) * 3, np.zeros(32, np.float32),
                (r.standard_normal(64) * 1e-3).astype(np.float32)]:
        b, s = fn(row)
        amax = np.float32(np.abs(row).max())
        want_s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
        assert np.float32(s) == want_s
        y = torch.from_numpy((row / want_s).astype(np.float32)).clamp(-448, 448)
        lib = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(np.asarray(b, np.uint8), lib)
        if amax > 0:
            assert np.abs(oracle.decode_e4m3(np.asarray(b))).max() == 448.0


def pin_mx_quantise(fn):
    _, (v, codes, scales) = _golden()
    b, e = fn(v)
    b = np.asarray(b)
    for i in range(64):
        assert int(b[i]) == codes.get(i, 0), (i, hex(int(b[i])))
    assert [int(x) for x in e] == [scales[0], scales[1]]
    # OCP MX v1.0 rule: each nonzero group's amax * 2^-E lies in [256, 512)
    # (e4m3's largest power of two is 2^8); elements beyond 448 saturate
    r = np.random.default_rng(6)
    x = (r.standard_normal(4096) * np.repeat(10.0 ** r.uniform(-3, 3, 128), 32)).astype(np.float32)
    b, e = fn(x)
    E = np.asarray(e, np.int64) - 127
    g = np.abs(x.astype(np.float64)).reshape(-1, 32).max(1) * 2.0 ** -E
    assert np.all((g >= 256) & (g < 512))
    y = np.clip(x.astype(np.float64) * np.repeat(2.0 ** -E, 32), -448, 448).astype(np.float32)
    lib = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(np.asarray(b, np.uint8), lib)


def _exact_bf16(v: float) -> int:
    """Nearest bf16 to v by exact rational arithmetic (ties to even), for
    normal-range finite v."""
    if v == 0:
        return 0x8000 if math.copysign(1, v) < 0 else 0
    sign = 0x8000 if v < 0 else 0
    a = Fraction(abs(v))
    e = math.floor(math.log2(abs(v)))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 7)
    m = a / ulp
    lo = math.floor(m)
    rem = m - lo
    mm = lo + 1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1) else lo
    val = float(mm * ulp)
    return sign | int(np.float32(val).view(np.uint32) >> 16)


def pin_round_bf16(fn):
    r = np.random.default_rng(8)
    # float32-exact inputs: torch's bfloat16 cast is a single rounding
    x32 = (r.standard_normal(3000) * 10.0 ** r.uniform(-30, 30, 3000)).astype(np.float32)
    lib = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(np.asarray(fn(x32.astype(np.float64))), lib)
    # float64 inputs, against exact rational rounding (catches rounding
    # through float32 first: 1 + 2^-8 + 2^-30 must round up, not to the tie)
    x64 = np.concatenate([r.standard_normal(500) * 10.0 ** r.uniform(-20, 20, 500),
                          [1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8 + 2.0 ** -40)]])
    got = np.asarray(fn(x64))
    for v, g in zip(x64, got):
        assert int(g) == _exact_bf16(float(v)), (v, hex(int(g)), hex(_exact_bf16(float(v))))


def pin_layer_norm(fn):
    r = np.random.default_rng(9)
    v = r.standard_normal((7, 128)) * 3 + 1
    gamma, beta = r.standard_normal(128), r.standard_normal(128)
    lib = torch.nn.functional.layer_norm(torch.from_numpy(v), (128,), torch.from_numpy(gamma),
                                         torch.from_numpy(beta), eps=1e-6).numpy()
    assert np.allclose(fn(v, gamma, beta, 1e-6), lib, rtol=1e-12, atol=1e-12)
    # closed form: a row of two values -1, +1 (mean 0, var 1)
    row = np.array([[-1.0, 1.0]])
    assert np.allclose(fn(row, np.ones(2), np.zeros(2), 0.0), row)


def pin_prolog_token(fn):
    """Tiny dims, pure-Python loops for the projections, torch's layer_norm."""
    r = np.random.default_rng(10)
    H, D, dm = 3, 8, 16
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    x, wq, wk, ww = bf(r.standard_normal(dm)), bf(r.standard_normal((H * D, dm))), bf(r.standard_normal((D, dm))), \
        bf(r.standard_normal((H, dm)))
    gamma, beta = r.standard_normal(D), r.standard_normal(D)
    q, k, w = fn(x, wq, wk, ww, gamma, beta, H, D)
    dec = lambda b: oracle.decode_bf16_bits(b).tolist()
    xv, wqv, wkv, wwv = dec(x), dec(wq), dec(wk), dec(ww)
    qref = [sum(wqv[o][i] * xv[i] for i in range(dm)) for o in range(H * D)]
    kp = [sum(wkv[o][i] * xv[i] for i in range(dm)) for o in range(D)]
    wref = [sum(wwv[o][i] * xv[i] for i in range(dm)) for o in range(H)]
    kref = torch.nn.functional.layer_norm(torch.tensor(kp, dtype=torch.float64), (D,),
                                          torch.from_numpy(gamma), torch.from_numpy(beta), eps=1e-6).numpy()
    assert np.allclose(w, wref, rtol=1e-12)
    assert [int(b) for b in np.asarray(q).reshape(-1)] == [_exact_bf16(v) for v in qref]
    assert [int(b) for b in np.asarray(k)] == [_exact_bf16(float(v)) for v in kref]


def pin_append(fn):
    r = np.random.default_rng(12)
    for _ in range(50):
        P = int(r.choice([1, 4, 16, 64]))
        L = int(r.integers(1, 300))
        T = int(r.integers(1, L + 1))
        i = int(r.integers(0, T))
        bt = r.permutation(L // P + 2) + 3
        t = L - T + i
        page, row = fn(L, T, i, bt, P)
        # walk the logical positions page by page until t is reached
        s, lp = 0, 0
        while s + P <= t:
            s += P
            lp += 1
        assert (page, row) == (int(bt[lp]), t - s)


# -------------------------------------------------------------- tests ---

def test_fp8_quantise_pins():
    pin_fp8_quantise(oracle.fp8_quantise)


def test_mx_quantise_pins():
    pin_mx_quantise(oracle.mx_quantise)


def test_round_bf16_pins():
    pin_round_bf16(oracle.round_bf16_bits)


def test_layer_norm_pins():
    pin_layer_norm(oracle.layer_norm)


def test_prolog_token_pins():
    pin_prolog_token(oracle.prolog_token)


def test_append_position_pins():
    pin_append(oracle.append_position)


def test_e4m3_encode_ties_and_boundaries():
    """Every midpoint between neighbouring e4m3 values goes to the even code;
    values at and past 448 saturate; signed zeros keep their sign."""
    t = oracle.e4m3fn_table()[:0x7F]
    mids = (t[:-1] + t[1:]) / 2
    codes = oracle.e4m3_encode(mids.astype(np.float32))
    want = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F))
    assert np.array_equal(codes, want)
    assert list(oracle.e4m3_encode(np.array([448.0, 463.9, 1e30, -1e30, 0.0, -0.0], np.float32))) == \
        [0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x80]


# ----------------------------------------------------------- mutations ---

def _m_fp8_wrong_max(v):
    v = np.asarray(v, np.float32)
    s = np.float32(np.abs(v).max() / np.float32(240.0))
    return oracle.e4m3_encode(v / s), s


def _m_fp8_truncate(v):
    v = np.asarray(v, np.float32)
    amax = np.float32(np.abs(v).max())
    s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    y = (v / s).astype(np.float32)
    t = oracle.e4m3fn_table()[:0x7F]
    code = np.searchsorted(t, np.minimum(np.abs(y), 448), side="right") - 1      # toward zero
    return np.where(np.signbit(y), code | 0x80, code).astype(np.uint8), s


def _m_mx_ceil(v, group=32):
    v = np.asarray(v, np.float32).reshape(-1, group)
    codes, scales = [], []
    for g in v:
        amax = float(np.abs(g).max())
        E = (math.ceil(math.log2(amax)) - 8) if amax > 0 else -127
        codes.append(oracle.e4m3_encode(np.ldexp(g.astype(np.float64), -E)))
        scales.append(E + 127)
    return np.concatenate(codes), np.asarray(scales, np.uint8)


def _m_round_via_f32(x):
    x = np.asarray(x, np.float64).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _m_ln_unbiased(v, gamma, beta, eps=1e-6):
    v = np.asarray(v, np.float64)
    mu = v.mean(-1, keepdims=True)
    var = v.var(-1, ddof=1, keepdims=True)
    return (v - mu) / np.sqrt(var + eps) * gamma + beta


def _m_append_off_by_one(L, T, i, bt, P):
    t = L - T + i - 1 if L - T + i > 0 else 0
    return int(np.asarray(bt)[t // P]), t % P


def _m_prolog_k_unnormalised(x, wq, wk, ww, gamma, beta, H, D, eps=1e-6):
    q, _, w = oracle.prolog_token(x, wq, wk, ww, gamma, beta, H, D, eps)
    k = oracle.decode_bf16_bits(wk) @ oracle.decode_bf16_bits(x)
    return q, oracle.round_bf16_bits(k), w


@pytest.mark.parametrize("pin,mutant", [
    (pin_fp8_quantise, _m_fp8_wrong_max),
    (pin_fp8_quantise, _m_fp8_truncate),
    (pin_mx_quantise, _m_mx_ceil),
    (pin_round_bf16, _m_round_via_f32),
    (pin_layer_norm, _m_ln_unbiased),
    (pin_append, _m_append_off_by_one),
    (pin_prolog_token, _m_prolog_k_unnormalised),
])
def test_prolog_pins_catch_planted_mistakes(pin, mutant):
    with pytest.raises(AssertionError):
        pin(mutant)
