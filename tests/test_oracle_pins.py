"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test checks one oracle function against an independent authority:
torch's CPU bf16 conversion and eager bf16 ops (library routines), exact
rational arithmetic (``fractions`` / ``decimal``), closed forms, torch's own
float64 LayerNorm / RMSNorm, and exact metamorphic invariants.  The cases are
chosen so that a plausible slip in the oracle (a dropped term, N-1 instead of
N, a fused single-rounding modulate, a wrong operand order, a transposed
batch index) fails at least one of them.
"""
from decimal import Decimal, getcontext
from fractions import Fraction
import json
import math
import os

import numpy as np
import pytest
import torch

from dit_adaln_row_amd.inputs import bf16_bits_from_f32, f32_from_u16, from_u16, to_u16
from dit_adaln_row_amd.workloads import Launch

getcontext().prec = 80
HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------------------
# exact helpers (test side)
# ---------------------------------------------------------------------------

def rn_f32(fr: Fraction) -> np.float32:
    """Round a rational to the nearest binary32, ties to even (exact)."""
    f = np.float32(float(fr))
    cands = {float(f), float(np.nextafter(f, np.float32(np.inf))),
             float(np.nextafter(f, np.float32(-np.inf)))}
    def key(c):
        return (abs(Fraction(c) - fr), int(np.float32(c).view(np.uint32)) & 1)
    return np.float32(min(cands, key=key))


def rn_bf16_exact(fr: Fraction, negative_zero=False) -> int:
    """Round a rational to the nearest bf16, ties to even (exact).  A result of
    zero takes the sign of the rational (or ``negative_zero`` for fr == 0)."""
    if fr == 0:
        return 0x8000 if negative_zero else 0x0000
    f = float(fr)
    u = int(np.float32(f).view(np.uint32)) >> 16
    cands = set()
    for d in (-2, -1, 0, 1, 2):
        v = (u + d) & 0xFFFF
        if (v & 0x7F80) == 0x7F80:
            continue
        cands.add(v)
    def key(v):
        val = Fraction(float(f32_from_u16(np.array([v], np.uint16))[0]))
        return (abs(val - fr), v & 1)
    best = min(cands, key=key)
    if (best & 0x7FFF) == 0:
        best = 0x8000 if fr < 0 else 0x0000
    return best


def dec(fr: Fraction) -> Decimal:
    return Decimal(fr.numerator) / Decimal(fr.denominator)


def exact_rstd(var: Fraction, eps32: float) -> Fraction:
    v = dec(var) + Decimal(float(np.float32(eps32)))
    return Fraction(Decimal(1) / v.sqrt())


def exact_ln(row_f32):
    vals = [Fraction(float(v)) for v in row_f32]
    n = len(vals)
    mean = sum(vals) / n
    var = sum((v - mean) ** 2 for v in vals) / n
    return mean, var


def ulp_bf16(v):
    v = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def rand_bf16(shape, mu, sigma, seed):
    g = torch.Generator().manual_seed(seed)
    return to_u16((torch.randn(shape, generator=g) * sigma + mu).to(torch.bfloat16))


def t_bf16(a):
    return from_u16(a)


def same_bits(a, b):
    """bitwise equality with NaNs compared by class."""
    a = np.asarray(a, np.uint16)
    b = np.asarray(b, np.uint16)
    an = (a & 0x7F80) == 0x7F80
    an &= (a & 0x7F) != 0
    bn = (b & 0x7F80) == 0x7F80
    bn &= (b & 0x7F) != 0
    return np.array_equal(an, bn) and np.array_equal(a[~an], b[~bn])


# ---------------------------------------------------------------------------
# rounding helpers
# ---------------------------------------------------------------------------

def test_round_f32_to_bf16_matches_torch_on_every_tie_class(orc):
    """All 2^16 upper halves x the low halves that decide RNE (exact, just below
    / at / just above the halfway point, all ones) + 2M random patterns,
    against torch's CPU float->bf16 conversion."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(7)
    pats = np.concatenate([pats, rng.integers(0, 1 << 32, 2_000_000, dtype=np.uint64).astype(np.uint32)])
    f = pats.view(np.float32)
    ours = orc.round_f32_to_bf16(f)
    ref = to_u16(torch.from_numpy(f.copy()).to(torch.bfloat16))
    assert same_bits(ours, ref)


def test_round_f64_to_bf16_single_rounding(orc):
    """Doubles straddling bf16 halfway points (where rounding through binary32
    would round twice) against exact rational rounding."""
    rng = np.random.default_rng(11)
    base = rng.standard_normal(400) * 10.0 ** rng.integers(-30, 30, 400)
    bits = bf16_bits_from_f32(base.astype(np.float32)).astype(np.uint32)
    lo = f32_from_u16(bits.astype(np.uint16)).astype(np.float64)
    hi = f32_from_u16(((bits + 1) & 0xFFFF).astype(np.uint16)).astype(np.float64)
    mid = (lo + hi) / 2.0
    tiny = np.abs(mid) * 2.0 ** -40
    cases = np.concatenate([mid, mid + tiny, mid - tiny, mid + np.abs(mid) * 2.0 ** -30,
                            base, np.array([0.0, -0.0, 1e-45, -3e-41, 1e300, -1e300])])
    cases = cases[np.isfinite(cases)]
    ours = orc.round_f64_to_bf16(cases)
    for d, o in zip(cases, ours):
        if abs(d) > 3.3e38:
            continue
        assert o == rn_bf16_exact(Fraction(float(d)), bool(np.signbit(d))), (d, hex(o))


def test_silu_bf16_is_correctly_rounded(orc):
    """SiLU(t) = t / (1 + e^-t) rounded once to bf16, against 80-digit decimal."""
    rng = np.random.default_rng(3)
    t = np.concatenate([rng.standard_normal(600).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1e-30, -1e-30, 1.0, -1.0, 20.0, -20.0, 80.0,
                                  -80.0, -87.5, -100.0, 88.0, 1e10], np.float32)])
    # add t whose binary32-rounded SiLU lands exactly on a bf16 halfway point:
    # there rounding through binary32 first would round twice
    r = np.random.default_rng(5).standard_normal(4_000_000).astype(np.float32) * 4
    s64 = r.astype(np.float64) / (1.0 + np.exp(-r.astype(np.float64)))
    s32 = s64.astype(np.float32)
    hard = (s32.view(np.uint32) & 0xFFFF) == 0x8000
    hard &= s32.astype(np.float64) != s64
    assert hard.sum() >= 10
    t = np.concatenate([t, r[hard][:40]])
    ours = orc.silu_bf16(t)
    for tv, o in zip(t, ours):
        x = Decimal(float(tv))
        s = x / (1 + (-x).exp())
        assert o == rn_bf16_exact(Fraction(s), bool(np.signbit(tv))), (tv, hex(o))


# ---------------------------------------------------------------------------
# elementwise stages vs torch's eager bf16 chain (per-op rounding)
# ---------------------------------------------------------------------------

SPECIAL = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x0001, 0x8001, 0x007F, 0x7F7F, 0xFF7F,
                    0x3F81, 0x4000, 0x3C00, 0xC2C8, 0x0080], np.uint16)


def test_modulate_matches_eager_chain(orc):
    """out = y * (1 + scale) + shift evaluated by torch on bf16 tensors (three
    kernels, each rounding to bf16), with a [B, 1, D] broadcast."""
    B, S, D = 3, 37, 64
    y = rand_bf16((B * S, D), 0, 1.5, 1)
    y[:len(SPECIAL), :len(SPECIAL)] = SPECIAL[None, :]
    sc = rand_bf16((B, D), 0, 0.3, 2)
    sh = rand_bf16((B, D), 0, 0.3, 3)
    sc[0, :len(SPECIAL)] = SPECIAL
    ref = t_bf16(y).view(B, S, D) * (1 + t_bf16(sc).view(B, 1, D)) + t_bf16(sh).view(B, 1, D)
    ours = orc.modulate(y, sc, sh, rows_per_batch=S)
    assert same_bits(ours, to_u16(ref.reshape(B * S, D)))


def test_modulate_strided_chunk_rows(orc):
    """Modulation rows taken from a [B, 6*D] embedding (adaLN chunk views):
    row stride 6*D, scale = chunk 1, shift = chunk 0."""
    B, S, D = 2, 5, 16
    emb = rand_bf16((B, 6 * D), 0, 0.2, 4)
    y = rand_bf16((B * S, D), 0, 1.0, 5)
    shift_view = emb[:, 0:D]
    scale_view = emb[:, D:2 * D]
    ref = t_bf16(y).view(B, S, D) * (1 + t_bf16(np.ascontiguousarray(scale_view)).view(B, 1, D)) \
        + t_bf16(np.ascontiguousarray(shift_view)).view(B, 1, D)
    # [B, 6*D] arrays whose row b starts where the chunk view's row b starts:
    # the same memory a strided chunk view addresses, row stride 6*D
    sc = np.concatenate([emb.ravel()[D:], np.zeros(D, np.uint16)]).reshape(B, 6 * D)
    sh = np.ascontiguousarray(emb)
    ours = orc.modulate(y, sc, sh, rows_per_batch=S)
    assert same_bits(ours, to_u16(ref.reshape(B * S, D)))


def test_gate_matches_eager_chain(orc):
    """h = residual + gate * update on bf16 tensors (two rounded kernels)."""
    B, S, D = 2, 29, 96
    upd = rand_bf16((B * S, D), 0, 1.5, 6)
    res = rand_bf16((B * S, D), 0, 1.0, 7)
    gate = rand_bf16((B, D), 0, 0.1, 8)
    upd[0, :len(SPECIAL)] = SPECIAL
    res[1, :len(SPECIAL)] = SPECIAL
    ref = t_bf16(res).view(B, S, D) + t_bf16(gate).view(B, 1, D) * t_bf16(upd).view(B, S, D)
    ours = orc.gate_residual(upd, res, gate, rows_per_batch=S)
    assert same_bits(ours, to_u16(ref.reshape(B * S, D)))


def test_bias_add_matches_aten_add_(orc):
    """xb = x.add_(bias.to(bf16)) with an fp32 bias, channels_last rows."""
    rows, C = 1000, 96
    x = rand_bf16((rows, C), 0, 1.0, 9)
    x[0, :len(SPECIAL)] = SPECIAL
    g = torch.Generator().manual_seed(10)
    bias = (torch.randn(C, generator=g) * 0.05).numpy()
    bias[:4] = [1e-9, -3.0e-3, 0.5 + 2 ** -9, 65504.0]
    ref = t_bf16(x).clone().add_(torch.from_numpy(bias).to(torch.bfloat16))
    assert same_bits(orc.bias_add(x, bias), to_u16(ref))


def test_conv_bias_epilogue_matches_eager(orc):
    """bf16(bf16(x + bf16(bias)) + h): the two roundings of conv(x) + h."""
    rows, C = 777, 384
    x = rand_bf16((rows, C), 0, 1.0, 12)
    h = rand_bf16((rows, C), 0, 1.0, 13)
    g = torch.Generator().manual_seed(14)
    bias = (torch.randn(C, generator=g) * 0.05).numpy()
    xb = t_bf16(x).clone().add_(torch.from_numpy(bias).to(torch.bfloat16))
    assert same_bits(orc.conv_bias_epilogue(x, bias), to_u16(xb))
    assert same_bits(orc.conv_bias_epilogue(x, bias, h), to_u16(xb + t_bf16(h)))


def _epilogue_inputs(dtype, bias_dtype, rows, C, seed):
    """x, h ~N(0,1) with special values planted (signed zeros, subnormals,
    infinities, a NaN, values at the type's largest finite magnitude so that
    adding the bias overflows); bias ~N(0, 0.05) in fp32 or x's type."""
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((rows, C), generator=g).to(tdt[dtype])
    h = torch.randn((rows, C), generator=g).to(tdt[dtype])
    big = torch.finfo(tdt[dtype]).max
    tiny = torch.finfo(tdt[dtype]).smallest_normal / 4  # subnormal
    special = torch.tensor([0.0, -0.0, tiny, -tiny, big, -big, float("inf"), float("-inf"),
                            float("nan")], dtype=torch.float32).to(tdt[dtype])
    x.view(-1)[:special.numel()] = special
    h.view(-1)[C:C + special.numel()] = special
    bias = (torch.randn(C, generator=g) * 0.05).to(tdt[bias_dtype])
    bias[0] = big if bias_dtype != "f32" else 3.0e38  # overflows x's type where it is narrower
    return x, h, bias


def _as_oracle(t, dtype):
    return t.numpy() if dtype == "f32" else to_u16(t)


def _same(a, b, dtype):
    if dtype == "f32":
        a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
        return np.array_equal(np.isnan(a), np.isnan(b)) and \
            np.array_equal(a[~np.isnan(a)].view(np.uint32), b[~np.isnan(b)].view(np.uint32))
    if dtype == "f16":
        an = ((a & 0x7C00) == 0x7C00) & ((a & 0x3FF) != 0)
        bn = ((b & 0x7C00) == 0x7C00) & ((b & 0x3FF) != 0)
        return np.array_equal(an, bn) and np.array_equal(a[~an], b[~bn])
    return same_bits(a, b)


@pytest.mark.parametrize("dtype,bias_dtype", [("bf16", "f32"), ("bf16", "bf16"), ("f16", "f32"),
                                              ("f16", "f16"), ("f32", "f32")])
def test_conv_bias_epilogue_dtypes_match_eager(orc, dtype, bias_dtype):
    """The Wan VAE page's epilogue for bf16 / fp16 / fp32 activations with an
    fp32 or same-type bias ("[Diffusion] Fuse the Wan VAE conv bias epilogue
    and tile the RMSNorm+SiLU kernel", Tests / docs: the aten oracle
    x.clone().add_(bias), then + h): torch's CPU eager chain, the bias cast to
    x's type first as autocast does, bit for bit -- special values included."""
    rows, C = 333, 96
    x, h, bias = _epilogue_inputs(dtype, bias_dtype, rows, C, 20)
    xb = x.clone().add_(bias.to(x.dtype))
    got = orc.conv_bias_epilogue_dt(_as_oracle(x, dtype), _as_oracle(bias, bias_dtype), None,
                                    dtype, bias_dtype)
    assert _same(got, _as_oracle(xb, dtype), dtype)
    got = orc.conv_bias_epilogue_dt(_as_oracle(x, dtype), _as_oracle(bias, bias_dtype),
                                    _as_oracle(h, dtype), dtype, bias_dtype)
    assert _same(got, _as_oracle(xb + h, dtype), dtype)
    if dtype == "bf16" and bias_dtype == "f32":  # the bf16-only form agrees
        assert same_bits(got, orc.conv_bias_epilogue(to_u16(x), bias.numpy(), to_u16(h)))


def test_conv_bias_epilogue_f32_bias_is_cast_first(orc):
    """An fp32 bias on a half-precision x is rounded to x's type before the
    add.  x = 1 and bias = 2^-11 + 2^-22 in fp16: the bias rounds to 2^-11
    (a tie, to even), and 1 + 2^-11 is again a tie that rounds to 1; the
    uncast fp32 sum 1 + 2^-11 + 2^-22 lies above that tie and would round to
    1 + 2^-10."""
    x = torch.full((1, 8), 1.0, dtype=torch.float16)
    b = torch.full((8,), 2.0 ** -11 + 2.0 ** -22, dtype=torch.float32)
    got = orc.conv_bias_epilogue_dt(to_u16(x), b.numpy(), None, "f16", "f32")
    assert np.all(got == to_u16(torch.ones((1, 8), dtype=torch.float16)))
    uncast = (x.float() + b).to(torch.float16)
    assert np.all(to_u16(uncast) == to_u16(torch.full((1, 8), 1.0 + 2.0 ** -10,
                                                      dtype=torch.float16)))


# ---------------------------------------------------------------------------
# statistics vs exact rational arithmetic
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,mu,sigma", [(4, 0, 1), (8, 3, 0.5), (16, -2, 4), (128, 0, 2),
                                        (96, 64, 0.1), (1024, 0, 1.5), (3072, 0.3, 1)])
def test_ln_stats_exact(orc, n, mu, sigma):
    x = rand_bf16((3, n), mu, sigma, 100 + n)
    mean, rstd = orc.ln_stats(x, 1e-6)
    for r in range(3):
        m, v = exact_ln(f32_from_u16(x[r]))
        assert mean[r] == rn_f32(m), (r, mean[r], float(m))
        assert rstd[r] == rn_f32(exact_rstd(v, 1e-6)), (r, rstd[r])


@pytest.mark.parametrize("n,sigma", [(8, 1), (96, 1), (384, 0.7), (4096, 1)])
def test_rms_stats_exact(orc, n, sigma):
    x = rand_bf16((3, n), 0.1, sigma, 200 + n)
    rstd = orc.rms_stats(x, 1e-6)
    for r in range(3):
        vals = [Fraction(float(v)) for v in f32_from_u16(x[r])]
        ms = sum(v * v for v in vals) / n
        assert rstd[r] == rn_f32(exact_rstd(ms, 1e-6)), r


def test_high_offset_row_guard(orc):
    """A row ~N(64, 0.1): the variance is 4e5 times smaller than E[x^2].  The
    oracle's rstd is still the correctly rounded value, while the naive fp32
    E[x^2]-E[x]^2 misses the 2e-6 tolerance by orders of magnitude (so this
    row separates a sound statistics algorithm from an unsound one)."""
    x = rand_bf16((1, 3072), 64.0, 0.1, 300)
    _, rstd = orc.ln_stats(x, 1e-6)
    m, v = exact_ln(f32_from_u16(x[0]))
    want = rn_f32(exact_rstd(v, 1e-6))
    assert rstd[0] == want
    xf = f32_from_u16(x[0]).astype(np.float32)
    naive_var = np.float32(np.mean(xf * xf, dtype=np.float32) - np.float32(np.mean(xf, dtype=np.float32)) ** 2)
    naive = 1 / math.sqrt(max(float(naive_var), 0.0) + 1e-6)
    assert abs(naive - float(want)) / float(want) > 1e-3


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def test_ln_constant_row_closed_form(orc):
    """A constant row has variance exactly 0: mean = c, rstd = fp32(1/sqrt(eps)),
    y = +0, and the modulate returns shift bit for bit."""
    cols = 256
    for c in (0x3FC0, 0xC120, 0x0000, 0x4B00):
        x = np.full((1, cols), c, np.uint16)
        sc = rand_bf16((1, cols), 0, 0.1, 400)
        sh = rand_bf16((1, cols), 0, 0.1, 401)
        r = orc.ln_modulate(x, sc, sh, 1e-6)
        assert r["mean"][0] == f32_from_u16(np.array([c], np.uint16))[0]
        assert r["rstd"][0] == rn_f32(exact_rstd(Fraction(0), 1e-6))
        assert np.all(r["y"] == 0)
        nz = (sh[0] & 0x7FFF) != 0
        assert np.array_equal(r["out"][0][nz], sh[0][nz])


def test_ln_two_valued_row_closed_form(orc):
    """Equal counts of a and b: mean = (a+b)/2 and var = (a-b)^2/4 exactly;
    y is +-rstd*(a-b)/2 rounded."""
    for a, b in ((1.0, 3.0), (-0.5, 0.25), (100.0, 96.0)):
        row = np.array([a, b] * 64, np.float32)
        x = bf16_bits_from_f32(row).reshape(1, -1)
        mean, rstd = orc.ln_stats(x, 1e-5)
        assert mean[0] == np.float32((a + b) / 2)
        want = rn_f32(exact_rstd(Fraction(a - b) ** 2 / 4, 1e-5))
        assert rstd[0] == want
        y = f32_from_u16(orc.ln_normalize(x, mean, rstd))
        half = np.float32(np.float32(a) - mean[0]) * rstd[0]
        assert np.all(y[0, 0::2] == f32_from_u16(bf16_bits_from_f32(np.array([half])))[0])


def test_zero_scale_shift_is_plain_layernorm(orc):
    rows, cols = 8, 512
    x = rand_bf16((rows, cols), 0, 1, 500)
    z = np.zeros((1, cols), np.uint16)
    r = orc.ln_modulate(x, z, z, 1e-6)
    # y * 1 + 0: equal up to the sign of zero
    assert np.array_equal(f32_from_u16(r["out"]), f32_from_u16(r["y"]))


def test_zero_gate_returns_residual(orc):
    rows, cols = 16, 128
    upd = rand_bf16((rows, cols), 0, 1.5, 501)
    res = rand_bf16((rows, cols), 0, 1, 502)
    h = orc.gate_residual(upd, res, np.zeros((1, cols), np.uint16))
    assert np.array_equal(f32_from_u16(h), f32_from_u16(res))


def test_rms_closed_forms(orc):
    cols = 4096
    w = rand_bf16((cols,), 1, 0.05, 503)
    sc = rand_bf16((1, cols), 0, 0.1, 504)
    sh = rand_bf16((1, cols), 0, 0.1, 505)
    # zero row: rstd = 1/sqrt(eps), y = 0, out = shift
    r = orc.rms_modulate(np.zeros((1, cols), np.uint16), w, sc, sh, 1e-6)
    assert r["rstd"][0] == rn_f32(exact_rstd(Fraction(0), 1e-6))
    assert np.all(f32_from_u16(r["y"]) == 0)
    assert np.array_equal(f32_from_u16(r["out"]), f32_from_u16(sh))
    # w = 1, scale = shift = 0 -> out == y; a constant row c -> y = bf16(c * rstd)
    one = np.full(cols, 0x3F80, np.uint16)
    z = np.zeros((1, cols), np.uint16)
    x = np.full((1, cols), 0x4040, np.uint16)  # 3.0
    r = orc.rms_modulate(x, one, z, z, 1e-6)
    assert r["rstd"][0] == rn_f32(exact_rstd(Fraction(9), 1e-6))
    assert np.array_equal(f32_from_u16(r["out"]), f32_from_u16(r["y"]))
    assert np.all(r["y"] == bf16_bits_from_f32(np.array([np.float32(3.0) * r["rstd"][0]]))[0])


# ---------------------------------------------------------------------------
# library cross-checks: torch float64 LayerNorm / RMSNorm
# ---------------------------------------------------------------------------

def test_ln_normalize_vs_torch_layer_norm(orc):
    rows, cols = 64, 3072
    x = rand_bf16((rows, cols), 0.2, 1.5, 600)
    mean, rstd = orc.ln_stats(x, 1e-6)
    y = f32_from_u16(orc.ln_normalize(x, mean, rstd)).astype(np.float64)
    xt = torch.from_numpy(f32_from_u16(x).astype(np.float64))
    ref = torch.nn.functional.layer_norm(xt, (cols,), eps=1e-6).numpy()
    slack = 0.5 * ulp_bf16(ref) + 4e-7 * np.abs(ref) + rstd[:, None] * np.abs(mean[:, None]) * 2.0 ** -23 + 1e-30
    assert np.all(np.abs(y - ref) <= slack)


def test_rms_normalize_vs_torch_rms_norm(orc):
    rows, cols = 64, 4096
    x = rand_bf16((rows, cols), 0, 1, 601)
    w = rand_bf16((cols,), 1, 0.05, 602)
    rstd = orc.rms_stats(x, 1e-6)
    y = f32_from_u16(orc.rms_normalize(x, rstd, w)).astype(np.float64)
    xt = torch.from_numpy(f32_from_u16(x).astype(np.float64))
    wt = torch.from_numpy(f32_from_u16(w).astype(np.float64))
    ref = torch.nn.functional.rms_norm(xt, (cols,), weight=wt, eps=1e-6).numpy()
    slack = 0.5 * ulp_bf16(ref) + 4e-7 * np.abs(ref) + 1e-30
    assert np.all(np.abs(y - ref) <= slack)


def test_wan_silu_path_vs_torch(orc):
    """channels_last rows: bias fold like add_, RMS over C, gamma, SiLU, against
    torch float64 rms_norm + silu on the bias-folded input."""
    rows, C = 2000, 96
    x = rand_bf16((rows, C), 0, 1, 603)
    g = torch.Generator().manual_seed(604)
    bias = (torch.randn(C, generator=g) * 0.05).numpy()
    gamma = f32_from_u16(rand_bf16((C,), 1, 0.05, 605))
    r = orc.rmsnorm_silu_bias(x, bias, gamma, 1e-6)
    xb_ref = t_bf16(x).clone().add_(torch.from_numpy(bias).to(torch.bfloat16))
    assert same_bits(r["xb"], to_u16(xb_ref))
    xt = xb_ref.double()
    ref = torch.nn.functional.silu(torch.nn.functional.rms_norm(
        xt, (C,), weight=torch.from_numpy(gamma.astype(np.float64)), eps=1e-6)).numpy()
    out = f32_from_u16(r["out"]).astype(np.float64)
    slack = 0.5 * ulp_bf16(ref) + 1e-6 * np.abs(ref) + 1e-30
    assert np.all(np.abs(out - ref) <= slack)
    # and the rstd is the correctly rounded exact value
    for i in (0, 1, 1999):
        vals = [Fraction(float(v)) for v in f32_from_u16(r["xb"][i])]
        assert r["rstd"][i] == rn_f32(exact_rstd(sum(v * v for v in vals) / C, 1e-6))


def test_normalised_moments(orc):
    """fp64 moments of y: mean ~ 0 and variance ~ var/(var+eps) ~ 1, within the
    bf16 rounding of the elements."""
    x = rand_bf16((32, 4096), -0.7, 2.0, 606)
    mean, rstd = orc.ln_stats(x, 1e-6)
    y = f32_from_u16(orc.ln_normalize(x, mean, rstd)).astype(np.float64)
    assert np.all(np.abs(y.mean(1)) <= 2.0 ** -9)
    assert np.all(np.abs(y.var(1) - 1.0) <= 2.0 ** -8)


# ---------------------------------------------------------------------------
# metamorphic invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("k", [-3, 5])
def test_power_of_two_scaling_invariance(orc, k):
    """f(2^k x, 4^k eps) == f(x, eps) bit for bit: every op involved scales
    exactly, and sqrt / division are correctly rounded."""
    x = rand_bf16((16, 1024), 0.5, 1.2, 700)
    xs = bf16_bits_from_f32(f32_from_u16(x) * np.float32(2.0 ** k))
    eps = 1e-6
    eps_s = float(np.float32(eps) * np.float32(4.0 ** k))
    m0, r0 = orc.ln_stats(x, eps)
    m1, r1 = orc.ln_stats(xs, eps_s)
    assert np.array_equal(m1, m0 * np.float32(2.0 ** k))
    assert np.array_equal(r1, r0 * np.float32(2.0 ** -k))
    assert np.array_equal(orc.ln_normalize(xs, m1, r1), orc.ln_normalize(x, m0, r0))
    w = rand_bf16((1024,), 1, 0.05, 701)
    q0 = orc.rms_stats(x, eps)
    q1 = orc.rms_stats(xs, eps_s)
    assert np.array_equal(q1, q0 * np.float32(2.0 ** -k))
    assert np.array_equal(orc.rms_normalize(xs, q1, w), orc.rms_normalize(x, q0, w))


def test_composites_equal_stage_chains(orc):
    """Each composite is its stages in sequence, and batch rows index the
    modulation row r // rows_per_batch."""
    B, S, D = 2, 33, 256
    x = rand_bf16((B * S, D), 0, 1.5, 800)
    res = rand_bf16((B * S, D), 0, 1, 801)
    gate = rand_bf16((B, D), 0, 0.1, 802)
    sc = rand_bf16((B, D), 0, 0.1, 803)
    sh = rand_bf16((B, D), 0, 0.1, 804)
    w = rand_bf16((D,), 1, 0.05, 805)
    r = orc.ln_modulate(x, sc, sh, 1e-6, rows_per_batch=S)
    m, s = orc.ln_stats(x, 1e-6)
    assert np.array_equal(r["mean"], m) and np.array_equal(r["rstd"], s)
    y = orc.ln_normalize(x, m, s)
    assert np.array_equal(r["y"], y)
    assert np.array_equal(r["out"], orc.modulate(y, sc, sh, rows_per_batch=S))
    for b in range(B):   # batch b only sees modulation row b
        rb = orc.ln_modulate(x[b * S:(b + 1) * S], sc[b:b + 1], sh[b:b + 1], 1e-6)
        assert np.array_equal(rb["out"], r["out"][b * S:(b + 1) * S])
    g = orc.gated_ln_modulate(x, res, gate, sc, sh, 1e-6, rows_per_batch=S)
    h = orc.gate_residual(x, res, gate, rows_per_batch=S)
    assert np.array_equal(g["h"], h)
    assert np.array_equal(g["out"], orc.ln_modulate(h, sc, sh, 1e-6, rows_per_batch=S)["out"])
    rr = orc.rms_modulate(x, w, sc, sh, 1e-6, residual=res, gate=gate, rows_per_batch=S)
    assert np.array_equal(rr["h"], h)
    q = orc.rms_stats(h, 1e-6)
    assert np.array_equal(rr["rstd"], q)
    assert np.array_equal(rr["out"], orc.modulate(orc.rms_normalize(h, q, w), sc, sh, rows_per_batch=S))


def test_qk_is_per_row_layernorm_q_then_k(orc):
    q = rand_bf16((300, 128), 0, 2, 900)
    k = rand_bf16((77, 128), 0.1, 2, 901)
    r = orc.qk_layernorm(q, k, 1e-5)
    mq, sq = orc.ln_stats(q, 1e-5)
    mk, sk = orc.ln_stats(k, 1e-5)
    assert np.array_equal(r["mean"], np.concatenate([mq, mk]))
    assert np.array_equal(r["rstd"], np.concatenate([sq, sk]))
    assert np.array_equal(r["q_out"], orc.ln_normalize(q, mq, sq))
    assert np.array_equal(r["k_out"], orc.ln_normalize(k, mk, sk))
    # row 5 of q against exact arithmetic
    m, v = exact_ln(f32_from_u16(q[5]))
    assert r["mean"][5] == rn_f32(m) and r["rstd"][5] == rn_f32(exact_rstd(v, 1e-5))


def test_rejects_bad_arguments(orc):
    x = np.zeros((4, 8), np.uint16)
    with pytest.raises(ValueError):
        orc.ln_modulate(x, np.zeros((1, 8), np.uint16), np.zeros((1, 8), np.uint16), 1e-6,
                        rows_per_batch=3)


# ---------------------------------------------------------------------------
# the byte model against the page's printed bandwidths
# ---------------------------------------------------------------------------

def test_byte_model_reproduces_page_bandwidths():
    with open(os.path.join(HERE, "golden", "page_bandwidth.json")) as f:
        g = json.load(f)
    n, c, d, hh, ww = g["shape"]
    rows = n * d * hh * ww
    for e in g["entries"]:
        if e["entry"] == "conv_bias_epilogue":
            l = Launch("e", "conv_bias_epilogue", rows, c, (), 0.0)
        else:
            l = Launch("e", "rmsnorm_silu_bias", rows, c, (), 1e-6, extra={"bias": False})
        tbps = l.algorithmic_bytes() / (e["ms"] * 1e-3) / 1e12
        assert abs(tbps - e["tbps_printed"]) <= e["printed_precision"], (e["what"], tbps)


# ---------------------------------------------------------------------------
# binary16 storage (standalone elementwise sites)
# ---------------------------------------------------------------------------

def test_round_f32_to_f16_matches_numpy_on_every_tie_class(orc):
    """All 2^16 upper halves x the low halves that decide RNE at bit 13 (exact,
    just below / at / just above the halfway point) + 2M random patterns,
    against numpy's correctly rounded float32 -> float16 conversion."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0FFF, 0x1000, 0x1001, 0x2000, 0x3000, 0x3001, 0xEFFF, 0xF000,
                     0xFFFF], np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(17)
    pats = np.concatenate([pats, rng.integers(0, 1 << 32, 2_000_000, dtype=np.uint64).astype(np.uint32)])
    f = pats.view(np.float32)
    with np.errstate(over="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    ours = orc.round_f32_to_f16(f)
    nan_o = ((ours & 0x7C00) == 0x7C00) & ((ours & 0x3FF) != 0)
    nan_r = ((ref & 0x7C00) == 0x7C00) & ((ref & 0x3FF) != 0)
    assert np.array_equal(nan_o, nan_r)
    assert np.array_equal(ours[~nan_o], ref[~nan_r])


def test_widen_f16_exact(orc):
    h = np.arange(1 << 16, dtype=np.uint16)
    ours = orc.widen_f16(h)
    ref = h.view(np.float16).astype(np.float32)
    n = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), n) and np.array_equal(ours[~n], ref[~n])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_standalone_modulate_and_gate_match_eager(orc, dtype):
    """x * (1 + scale) + shift and residual + gate * update evaluated by torch
    on CPU tensors of the storage dtype (each op rounds), (B,1,D) broadcast."""
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    B, S, D = 3, 41, 96
    g = torch.Generator().manual_seed(21)
    mk = lambda *shape, s=1.0: (torch.randn(*shape, generator=g) * s).to(tdt)
    x, sc, sh = mk(B, S, D, s=2.0), mk(B, 1, D, s=0.3), mk(B, 1, D, s=0.3)
    u, res, gate = mk(B, S, D, s=1.5), mk(B, S, D), mk(B, 1, D, s=0.1)
    x[0, 0, :6] = torch.tensor([0.0, -0.0, 65504.0, 6e-5, -1e-7, 1.0]).to(tdt)
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1, D)
    ref = x * (1 + sc) + sh
    ours = orc.modulate_dt(bits(x), bits(sc), bits(sh), dtype, rows_per_batch=S)
    assert same_bits(ours, bits(ref)) if dtype == "bf16" else np.array_equal(ours, bits(ref))
    ref = res + gate * u
    ours = orc.gate_residual_dt(bits(u), bits(res), bits(gate), dtype, rows_per_batch=S)
    assert np.array_equal(ours, bits(ref))
    if dtype == "bf16":   # the same stages as the fused paths use
        assert np.array_equal(orc.modulate_dt(bits(x), bits(sc), bits(sh), "bf16", S),
                              orc.modulate(bits(x), bits(sc), bits(sh), rows_per_batch=S))


# ---------------------------------------------------------------------------
# LN-affine folding (the lossy one-pass form; FLUX.1 page, Commit 3)
# ---------------------------------------------------------------------------

def test_folded_ln_pins(orc):
    rows, cols = 64, 3072
    x = rand_bf16((rows, cols), 0.0, 1.5, 700)
    sc = rand_bf16((1, cols), 0, 0.1, 701)
    sh = rand_bf16((1, cols), 0, 0.1, 702)
    f = orc.ln_modulate_folded(x, sc, sh, 1e-6)
    lossless = orc.ln_modulate(x, sc, sh, 1e-6)
    # the statistics are the lossless LayerNorm's
    assert np.array_equal(f["mean"].view(np.uint32), lossless["mean"].view(np.uint32))
    assert np.array_equal(f["rstd"].view(np.uint32), lossless["rstd"].view(np.uint32))

    # weight 1, bias 0: the unrounded normalised value rounded once, i.e. the
    # lossless chain's y (equal up to the sign of zero)
    z = np.zeros((1, cols), np.uint16)
    f0 = orc.ln_modulate_folded(x, z, z, 1e-6)
    assert np.array_equal(f32_from_u16(f0["out"]), f32_from_u16(lossless["y"]))

    # scale = -1: the weight bf16(1 + scale) is 0, so out == shift exactly
    m1 = np.full((1, cols), 0xBF80, np.uint16)
    fm = orc.ln_modulate_folded(x, m1, sh, 1e-6)
    assert np.array_equal(f32_from_u16(fm["out"]), np.broadcast_to(f32_from_u16(sh), (rows, cols)))

    # library: torch's LayerNorm with weight = (1 + scale) in bf16 eager and
    # bias = shift, evaluated in float64 (the page's layer_norm(x, weight=1+scale,
    # bias=shift)); one rounding of an fp32 chain on fp32 statistics lands
    # within half a bf16 ulp plus the chain's fp32 error
    w = to_u16(torch.ones(cols, dtype=torch.bfloat16) + t_bf16(sc[0]))      # eager bf16 add
    x64 = torch.from_numpy(f32_from_u16(x).astype(np.float64))
    w64 = torch.from_numpy(f32_from_u16(w).astype(np.float64))
    b64 = torch.from_numpy(f32_from_u16(sh[0]).astype(np.float64))
    ref = torch.nn.functional.layer_norm(x64, (cols,), weight=w64, bias=b64, eps=1e-6).numpy()
    tw = torch.nn.functional.layer_norm(x64, (cols,), eps=1e-6).numpy() * w64.numpy()
    out = f32_from_u16(f["out"]).astype(np.float64)
    chain = 2.0 ** -21 * (np.abs(tw) + np.abs(b64.numpy())) + \
        f["rstd"][:, None].astype(np.float64) * np.abs(f["mean"][:, None]) * np.abs(w64.numpy()) * 2.0 ** -23
    slack = 0.5 * ulp_bf16(np.abs(ref) + chain) + chain + 1e-30
    assert np.all(np.abs(out - ref) <= slack)
    assert np.mean(out == ref.astype(np.float32).astype(np.float64)) < 1.0  # it is rounded

    # against the lossless three-rounding chain: the two extra roundings (y,
    # then y * s1) and the two final ones differ by at most
    # |s1| ulp(y)/2 + ulp(p)/2 + ulp(out) -- at this scale a few hundredths
    # (the page reports a max abs difference of about 0.05 on FLUX.1 shapes)
    y = f32_from_u16(lossless["y"]).astype(np.float64)
    p = y * w64.numpy()
    bound = np.abs(w64.numpy()) * 0.5 * ulp_bf16(y) + 0.5 * ulp_bf16(p) + ulp_bf16(np.abs(p) + np.abs(b64.numpy()))
    diff = np.abs(out - f32_from_u16(lossless["out"]).astype(np.float64))
    assert np.all(diff <= bound + 1e-30)
    assert 0 < diff.max() <= 0.0625


# ---------------------------------------------------------------------------
# backward of LN + modulate (Qwen-Image final AdaLN output page): the fixed
# fp32 token-sum tree and the gradients
# ---------------------------------------------------------------------------

U24 = 2.0 ** -24


def test_tree32_shape_by_hand(orc):
    """Hand-derived results that tell the page's tree (adjacent pairs in
    groups of 32, recursively, +0 padding) from its plausible neighbours."""
    f = lambda v: float(orc.tree32_sum(np.array(v, np.float32)))
    # adjacent pairs: (1 + u) + (u + u) = 1 + 2u; a sequential sum gives 1
    assert f([1, U24, U24, U24]) == 1 + 2 * U24
    # adjacent pairs: (1 + -1) + (u + u) = 2u; pairing i with i+2 first gives u
    assert f([1, -1, U24, U24]) == 2 * U24
    # 33 values: group 0 = 1 + 15*2u exactly, group 1 = u; their sum is a tie
    # rounded to even: 1 + 32u
    assert f([1] + [U24] * 32) == 1 + 32 * U24
    # four groups whose sums are 1, u, u, u: the second level pairs them as
    # ((1 + u) + (u + u)) = 1 + 2u; adding the group sums in order gives 1
    v = np.zeros(128, np.float32)
    v[0], v[32], v[64], v[96] = 1, U24, U24, U24
    assert f(v) == 1 + 2 * U24
    # +0 padding: two -0 terms meet a padded +0, so the sum is +0
    r = orc.tree32_sum(np.array([-0.0, -0.0], np.float32))
    assert r == 0 and not np.signbit(r)
    assert orc.tree32_sum(np.array([], np.float32)) == 0
    # n equal bf16 values sum to n*c exactly
    c = np.float32(0.10009765625)
    for n in (1, 2, 3, 31, 32, 33, 100, 1000, 4096):
        assert orc.tree32_sum(np.full(n, c, np.float32)) == np.float32(n * float(c))


def test_tree32_error_bound(orc):
    rng = np.random.default_rng(5)
    for n in (7, 32, 1000, 6889):
        v = rng.standard_normal(n).astype(np.float32)
        exact = sum(Fraction(float(t)) for t in v)
        depth = 5 * max(1, math.ceil(math.log(n, 32)))
        got = Fraction(float(orc.tree32_sum(v)))
        assert abs(got - exact) <= Fraction(depth) * Fraction(U24) * sum(abs(Fraction(float(t))) for t in v)


def _torch_backward(x, sc, dout, eps, rpb):
    """Gradients of LN(x) * (1 + scale) + shift by torch autograd in float64."""
    rows, cols = x.shape
    xt = torch.from_numpy(f32_from_u16(x).astype(np.float64)).requires_grad_()
    st = torch.from_numpy(f32_from_u16(sc).astype(np.float64)).requires_grad_()
    ht = torch.zeros_like(st, requires_grad=True)
    b = torch.arange(rows) // rpb
    out = torch.nn.functional.layer_norm(xt, (cols,), eps=eps) * (1 + st[b]) + ht[b]
    out.backward(torch.from_numpy(f32_from_u16(dout).astype(np.float64)))
    xh = torch.nn.functional.layer_norm(xt.detach(), (cols,), eps=eps).numpy()
    return xt.grad.numpy(), st.grad.numpy(), ht.grad.numpy(), xh


def test_backward_vs_torch_autograd(orc):
    B, S, D = 2, 77, 1024
    x = rand_bf16((B * S, D), 0.3, 1.5, 800)
    sc = rand_bf16((B, D), 0, 0.1, 801)
    dout = rand_bf16((B * S, D), 0, 1.0, 802)
    r = orc.ln_modulate_backward(x, sc, dout, 1e-6, rows_per_batch=S)
    gx, gs, gh, xh = _torch_backward(x, sc, dout, 1e-6, S)
    # d_x: one rounding of a binary64 evaluation on fp32 statistics
    g = f32_from_u16(dout).astype(np.float64) * (1 + np.repeat(f32_from_u16(sc), S, 0))
    rstd = r["rstd"].astype(np.float64)[:, None]
    c1 = g.mean(1, keepdims=True)
    c2 = (g * xh).mean(1, keepdims=True)
    slack = 1e-6 * rstd * (np.abs(g) + np.abs(c1) + np.abs(xh * c2))
    dx = f32_from_u16(r["d_x"]).astype(np.float64)
    assert np.all(np.abs(dx - gx) <= 0.5 * ulp_bf16(np.abs(gx) + slack) + slack + 1e-30)
    assert np.mean(r["d_x"] == bf16_bits_from_f32(gx.astype(np.float32))) > 0.99
    # token sums: the fixed tree's error bound over the exact sums
    depth = 5 * 2
    tsh = np.abs(f32_from_u16(dout).astype(np.float64)).reshape(B, S, D).sum(1)
    assert np.all(np.abs(r["d_shift"] - gh) <= depth * U24 * tsh + 1e-30)
    tsc = np.abs(f32_from_u16(dout).astype(np.float64) * xh).reshape(B, S, D).sum(1)
    assert np.all(np.abs(r["d_scale"] - gs) <= (depth + 4) * U24 * tsc + 1e-30)


def test_backward_batch_invariance_and_closed_forms(orc):
    S, D = 45, 256
    xs = [rand_bf16((S, D), 0, 1, 810 + i) for i in range(3)]
    scs = [rand_bf16((1, D), 0, 0.1, 820 + i) for i in range(3)]
    ds = [rand_bf16((S, D), 0, 1, 830 + i) for i in range(3)]
    whole = orc.ln_modulate_backward(np.concatenate(xs), np.concatenate(scs), np.concatenate(ds),
                                     1e-6, rows_per_batch=S)
    for i in range(3):
        alone = orc.ln_modulate_backward(xs[i], scs[i], ds[i], 1e-6)
        assert np.array_equal(alone["d_x"], whole["d_x"][i * S:(i + 1) * S])
        assert np.array_equal(alone["d_scale"][0].view(np.uint32), whole["d_scale"][i].view(np.uint32))
        assert np.array_equal(alone["d_shift"][0].view(np.uint32), whole["d_shift"][i].view(np.uint32))
    # d_out constant c: d_shift = S*c exactly, whatever x and scale are
    c = np.full((S, D), 0x3DCD, np.uint16)                     # 0.10009765625
    r = orc.ln_modulate_backward(xs[0], scs[0], c, 1e-6)
    assert np.all(r["d_shift"] == np.float32(S * 0.10009765625))
    # scale = -1: no gradient reaches x (g = 0), the token sums do not see scale
    m1 = np.full((1, D), 0xBF80, np.uint16)
    r1 = orc.ln_modulate_backward(xs[0], m1, ds[0], 1e-6)
    r0 = orc.ln_modulate_backward(xs[0], scs[0], ds[0], 1e-6)
    assert np.all(f32_from_u16(r1["d_x"]) == 0)
    assert np.array_equal(r1["d_shift"], r0["d_shift"]) and np.array_equal(r1["d_scale"], r0["d_scale"])
    # the LN backward is orthogonal to shifts and scalings of the row: the
    # row sums of d_x and of d_x * x_hat vanish up to the bf16 rounding of d_x
    _, _, _, xh = _torch_backward(xs[0], scs[0], ds[0], 1e-6, S)
    dx = f32_from_u16(r0["d_x"]).astype(np.float64)
    half = 0.5 * ulp_bf16(dx)
    assert np.all(np.abs(dx.sum(1)) <= half.sum(1) * 1.01)
    assert np.all(np.abs((dx * xh).sum(1)) <= (half * np.abs(xh)).sum(1) * 1.01 + 1e-3 * np.abs(dx * xh).sum(1) * 2 ** -10)


# ---------------------------------------------------------------------------
# the backward's fp32 stream
# ---------------------------------------------------------------------------

def _f32_normal(shape, mu, sigma, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float64) * sigma + mu).float().numpy()


def test_backward_f32_vs_torch_autograd(orc):
    """The fp32 stream (Qwen-Image page, the FP32 column of the final stream's
    table and its BF16/FP32 accuracy gates) against torch float64 autograd of
    LN(x) * (1 + scale) + shift: d_x within its fp32 rounding plus what the
    fp32 rounding of mean and rstd moves it by; the token sums within the
    fixed tree's error bound over the exact sums."""
    B, S, D = 2, 77, 1024
    x = _f32_normal((B * S, D), 0.3, 1.5, 840)
    sc = _f32_normal((B, D), 0, 0.1, 841)
    dout = _f32_normal((B * S, D), 0, 1.0, 842)
    r = orc.ln_modulate_backward_f32(x, sc, dout, 1e-6, rows_per_batch=S)
    xt = torch.from_numpy(x.astype(np.float64)).requires_grad_()
    st = torch.from_numpy(sc.astype(np.float64)).requires_grad_()
    ht = torch.zeros_like(st, requires_grad=True)
    b = torch.arange(B * S) // S
    out = torch.nn.functional.layer_norm(xt, (D,), eps=1e-6) * (1 + st[b]) + ht[b]
    out.backward(torch.from_numpy(dout.astype(np.float64)))
    gx, gs, gh = xt.grad.numpy(), st.grad.numpy(), ht.grad.numpy()
    xh = torch.nn.functional.layer_norm(xt.detach(), (D,), eps=1e-6).numpy()
    g = dout.astype(np.float64) * (1 + np.repeat(sc.astype(np.float64), S, 0))
    rstd = r["rstd"].astype(np.float64)[:, None]
    c1 = g.mean(1, keepdims=True)
    c2 = (g * xh).mean(1, keepdims=True)
    # mean and rstd rounded to fp32 (2^-24 relative each) move x_hat and the
    # three terms by a few parts in 2^24
    slack = 8 * U24 * rstd * (np.abs(g) + np.abs(c1) + np.abs(xh * c2)) * (1 + np.abs(xh))
    assert np.all(np.abs(r["d_x"].astype(np.float64) - gx) <= U24 * np.abs(gx) + slack + 1e-30)
    depth = 5 * 2
    tsh = np.abs(dout.astype(np.float64)).reshape(B, S, D).sum(1)
    assert np.all(np.abs(r["d_shift"] - gh) <= depth * U24 * tsh + 1e-30)
    tsc = np.abs(dout.astype(np.float64) * xh).reshape(B, S, D).sum(1)
    assert np.all(np.abs(r["d_scale"] - gs) <= (depth + 4) * U24 * tsc + 1e-30)


def test_backward_f32_agrees_with_bf16_stream_on_bf16_values(orc):
    """On fp32 inputs that hold bf16 values the two streams see the same
    numbers: the statistics and both token sums are bitwise the bf16
    stream's, and d_x, rounded to fp32 there and to bf16 here from the same
    binary64 value, differs by at most one bf16 ulp after rounding the fp32
    value to bf16 (only where the fp32 value lands on a bf16 halfway point)."""
    B, S, D = 3, 40, 768
    x = rand_bf16((B * S, D), 0.2, 1.5, 850)
    sc = rand_bf16((B, D), 0, 0.1, 851)
    dout = rand_bf16((B * S, D), 0, 1.0, 852)
    rb = orc.ln_modulate_backward(x, sc, dout, 1e-6, rows_per_batch=S)
    rf = orc.ln_modulate_backward_f32(f32_from_u16(x), f32_from_u16(sc), f32_from_u16(dout), 1e-6,
                                      rows_per_batch=S)
    for k in ("mean", "rstd", "d_shift", "d_scale"):
        assert np.array_equal(rb[k].view(np.uint32), rf[k].view(np.uint32)), k
    d32 = bf16_bits_from_f32(rf["d_x"])
    d = np.abs(d32.astype(np.int32) - rb["d_x"].astype(np.int32))
    assert d.max() <= 1 and (d == 0).mean() >= 0.9999


def test_backward_f32_batch_invariance_and_closed_forms(orc):
    S, D = 45, 256
    xs = [_f32_normal((S, D), 0, 1, 860 + i) for i in range(3)]
    scs = [_f32_normal((1, D), 0, 0.1, 870 + i) for i in range(3)]
    ds = [_f32_normal((S, D), 0, 1, 880 + i) for i in range(3)]
    whole = orc.ln_modulate_backward_f32(np.concatenate(xs), np.concatenate(scs),
                                         np.concatenate(ds), 1e-6, rows_per_batch=S)
    for i in range(3):
        alone = orc.ln_modulate_backward_f32(xs[i], scs[i], ds[i], 1e-6)
        assert np.array_equal(alone["d_x"].view(np.uint32),
                              whole["d_x"][i * S:(i + 1) * S].view(np.uint32))
        for k in ("d_scale", "d_shift"):
            assert np.array_equal(alone[k][0].view(np.uint32), whole[k][i].view(np.uint32))
    # d_out constant c with few significant bits: every partial sum is exact,
    # so d_shift = S * c whatever the tree
    c = np.full((S, D), 0.375, np.float32)
    r = orc.ln_modulate_backward_f32(xs[0], scs[0], c, 1e-6)
    assert np.all(r["d_shift"] == np.float32(S * 0.375))
    r1 = orc.ln_modulate_backward_f32(xs[0], np.full((1, D), -1.0, np.float32), ds[0], 1e-6)
    assert np.all(r1["d_x"] == 0)

