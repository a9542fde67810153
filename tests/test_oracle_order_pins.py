"""Pins of the oracle's operation order inside each normalise stage (no GPU).

A normalise stage chains a few binary32 operations and rounds to bf16 once.
Which operations, in which order, decides the last bit of a few elements in a
hundred thousand, and a tolerance against a float64 library routine cannot
see that.  Here each stage's expression is evaluated in exact rational
arithmetic, rounded to binary32 or bf16 exactly where the expression rounds
(round-to-nearest-even written out from its definition below, with no
floating-point library involved), on inputs searched so that the plausible
re-associated forms give a different bf16 value.  The oracle passes only with
the stated order:

* LayerNorm normalise -- GLM-Image page ("[diffusion] GLM-Image bit-exact
  fused aten LayerNorm+modulate / qk-LN"), "What rounding-faithful means
  here": the binary32 sum of x and -mean, multiplied by rstd in binary32
  (no fused multiply-add), rounded to bf16.  Rejected: x*rstd - mean*rstd,
  fma(x, rstd, -mean*rstd), (x - mean)*rstd rounded once.
* RMSNorm normalise -- ERNIE-Image page ("[diffusion] ERNIE-Image bit-exact
  fused RMSNorm+scale/shift"), same section: the product of x, rstd and w in
  binary32, one final rounding to bf16; the products are read left to right.
  Rejected: x*(rstd*w), (x*w)*rstd (the exact product rounded once).
* LN-affine folding -- FLUX.1 page ("[diffusion] FLUX.1 fused adaLN modulate
  (bit-exact) + RoPE cache hoist, LN-affine folding behind quality=high"),
  Commit 3: LayerNorm with weight bf16(1 + scale) and bias shift applied in
  fp32 to the unrounded normalised value.  The page leaves the binary32 order
  of that affine open; the reading pinned here is the normalise's order, then
  the weight, then the bias, no fused multiply-add.  Rejected: fma(t, w,
  shift), rstd folded into the weight, the weight applied before rstd.
* Wan RMSNorm + SiLU -- Wan VAE page ("[Diffusion] Fuse the Wan VAE conv bias
  epilogue and tile the RMSNorm+SiLU kernel"), Modifications: one fp32 pass
  whose pre-activation is read as t = (xb * rstd) * gamma, SiLU rounded once.
  Rejected: xb*(rstd*gamma), (xb*gamma)*rstd.

The search for separating inputs uses numpy's float32 arithmetic and torch's
bf16 conversion (library routines) only to find candidates; every assertion
about a candidate rests on the exact evaluation.  The same library evaluation
of the stated order must also equal the oracle on every element.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import torch

from dit_adaln_row_amd.inputs import f32_from_u16

getcontext().prec = 60

F32, BF16 = 24, 8  # significand bits; both formats have binary32's exponent range


def rne(q: Fraction, p: int) -> Fraction:
    """q rounded to the nearest number with p significand bits and binary32's
    exponent range (normal numbers from 2^-126 up, subnormals spaced
    2^(-126 - p + 1) below), ties to the even significand.  No overflow occurs
    in these tests (asserted)."""
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if a < Fraction(2) ** e:
        e -= 1                      # now 2^e <= a < 2^(e+1)
    e = max(e, -126)                # below 2^-126 the spacing stays fixed
    quantum = Fraction(2) ** (e - p + 1)
    m = a / quantum
    k = m.numerator // m.denominator
    rest = m - k
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and k % 2 == 1):
        k += 1
    v = k * quantum
    assert v < Fraction(2) ** 128
    return v if q > 0 else -v


def r32(q):
    return rne(q, F32)


def bf16_bits(v: Fraction) -> int:
    """Bit pattern of a nonzero bf16-representable rational."""
    assert v != 0 and rne(v, BF16) == v
    return int(np.array(float(v), np.float32).view(np.uint32)) >> 16


def fr(v) -> Fraction:
    return Fraction(float(v))


def lib_bf16(a_f32) -> np.ndarray:
    """torch's float32 -> bf16 conversion (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a_f32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def lib_bf16_of_f64(a_f64) -> np.ndarray:
    """Candidate search only: binary64 -> binary32 -> bf16 (two roundings)."""
    return lib_bf16(np.asarray(a_f64, np.float64).astype(np.float32))


def bf16_from_normal(mu, sigma, shape, seed):
    g = torch.Generator().manual_seed(seed)
    z = torch.randn(shape, generator=g, dtype=torch.float64)
    v = torch.as_tensor(mu, dtype=torch.float64) + z * torch.as_tensor(sigma, dtype=torch.float64)
    return v.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_uniform(lo, hi, n, seed):
    g = torch.Generator().manual_seed(seed)
    return (lo + (hi - lo) * torch.rand(n, generator=g, dtype=torch.float64)).to(
        torch.float32).numpy()


def separated(name, cand, exact_page, exact_alt, oracle_bits, limit=64):
    """Among candidate positions, count those where the exact stated order
    gives the oracle's bits and the exact alternative gives other bits."""
    n = 0
    for i in cand[:limit]:
        page = exact_page(i)
        assert bf16_bits(page) == oracle_bits(i), f"{name}: the oracle departs from the stated order at {i}"
        if bf16_bits(exact_alt(i)) != oracle_bits(i):
            n += 1
    assert n >= 1, f"no input separates the stated order from {name}"
    return n


def test_ln_normalize_order_glm_page(orc):
    rows, cols = 1024, 2048
    mean = (f32_uniform(-1.0, 1.0, rows, 0x4C01) * np.float32(0.3)).astype(np.float32)
    rstd = f32_uniform(0.4, 2.5, rows, 0x4C02)
    x = bf16_from_normal(mean[:, None].astype(np.float64), 1.0 / rstd[:, None].astype(np.float64),
                         (rows, cols), 0x4C03)
    y = orc.ln_normalize(x, mean, rstd)
    xf = f32_from_u16(x)
    m, r = mean[:, None], rstd[:, None]
    page = lib_bf16(r * (xf - m))                       # binary32 ops in the stated order
    assert np.array_equal(y, page)
    flat = y.reshape(-1)

    def ex_page(i):
        a, b = divmod(int(i), cols)
        return rne(r32(fr(rstd[a]) * r32(fr(xf[a, b]) - fr(mean[a]))), BF16)

    alts = {
        "x*rstd - mean*rstd": (
            lib_bf16((xf * r) - (m * r)),
            lambda X, M, R: r32(r32(X * R) - r32(M * R))),
        "fma(x, rstd, -mean*rstd)": (
            lib_bf16_of_f64(xf.astype(np.float64) * r - (m * r).astype(np.float64)),
            lambda X, M, R: r32(X * R - r32(M * R))),
        "(x - mean)*rstd rounded once": (
            lib_bf16_of_f64((xf.astype(np.float64) - m) * r),
            lambda X, M, R: r32((X - M) * R)),
    }
    for name, (alt_np, alt_exact) in alts.items():
        cand = np.flatnonzero(alt_np.reshape(-1) != flat)

        def ex_alt(i, f=alt_exact):
            a, b = divmod(int(i), cols)
            return rne(f(fr(xf[a, b]), fr(mean[a]), fr(rstd[a])), BF16)

        separated(name, cand, ex_page, ex_alt, lambda i: int(flat[i]))
    # an exact check of a sample of ordinary elements
    for i in np.random.default_rng(5).choice(flat.size, 1500, replace=False):
        assert bf16_bits(ex_page(i)) == int(flat[i])


def test_rms_normalize_order_ernie_page(orc):
    rows, cols = 512, 4096
    x = bf16_from_normal(0.0, 1.0, (rows, cols), 0x5201)
    w = bf16_from_normal(1.0, 0.05, (cols,), 0x5202)
    rstd = f32_uniform(0.5, 2.0, rows, 0x5203)
    y = orc.rms_normalize(x, rstd, w)
    xf, wf = f32_from_u16(x), f32_from_u16(w)
    r = rstd[:, None]
    page = lib_bf16((xf * r) * wf[None, :])
    assert np.array_equal(y, page)
    flat = y.reshape(-1)

    def args(i):
        a, b = divmod(int(i), cols)
        return fr(xf[a, b]), fr(rstd[a]), fr(wf[b])

    def ex_page(i):
        X, R, W = args(i)
        return rne(r32(r32(X * R) * W), BF16)

    alts = {
        "x*(rstd*w)": (lib_bf16(xf * (r * wf[None, :])), lambda X, R, W: r32(X * r32(R * W))),
        "(x*w)*rstd": (lib_bf16((xf * wf[None, :]) * r), lambda X, R, W: r32(r32(X * W) * R)),
    }
    for name, (alt_np, alt_exact) in alts.items():
        cand = np.flatnonzero(alt_np.reshape(-1) != flat)
        separated(name, cand, ex_page, lambda i, f=alt_exact: rne(f(*args(i)), BF16),
                  lambda i: int(flat[i]))
    for i in np.random.default_rng(6).choice(flat.size, 1500, replace=False):
        assert bf16_bits(ex_page(i)) == int(flat[i])


def test_folded_affine_order_flux_page(orc):
    rows, cols = 512, 2048
    x = bf16_from_normal(0.2, 1.5, (rows, cols), 0x4601)
    scale = bf16_from_normal(0.0, 0.1, (rows, cols), 0x4602)   # one modulation row per row
    shift = bf16_from_normal(0.0, 0.1, (rows, cols), 0x4603)
    res = orc.ln_modulate_folded(x, scale, shift, 1e-6, rows_per_batch=1)
    out, mean, rstd = res["out"], res["mean"], res["rstd"]
    xf, sf, hf = f32_from_u16(x), f32_from_u16(scale), f32_from_u16(shift)
    m, r = mean[:, None], rstd[:, None]
    wt = f32_from_u16(lib_bf16(np.float32(1.0) + sf))      # the weight row keeps its bf16 rounding
    t = r * (xf - m)
    page = lib_bf16((t * wt) + hf)
    assert np.array_equal(out, page)
    flat = out.reshape(-1)

    def args(i):
        a, b = divmod(int(i), cols)
        W = rne(r32(1 + fr(sf[a, b])), BF16)
        return fr(xf[a, b]), fr(mean[a]), fr(rstd[a]), W, fr(hf[a, b])

    def ex_page(i):
        X, M, R, W, H = args(i)
        return rne(r32(r32(r32(R * r32(X - M)) * W) + H), BF16)

    alts = {
        "fma(t, w, shift)": (
            lib_bf16_of_f64(t.astype(np.float64) * wt + hf),
            lambda X, M, R, W, H: r32(r32(R * r32(X - M)) * W + H)),
        "rstd folded into the weight": (
            lib_bf16(((xf - m) * (r * wt)) + hf),
            lambda X, M, R, W, H: r32(r32(r32(X - M) * r32(R * W)) + H)),
        "weight before rstd": (
            lib_bf16((r * ((xf - m) * wt)) + hf),
            lambda X, M, R, W, H: r32(r32(R * r32(r32(X - M) * W)) + H)),
    }
    for name, (alt_np, alt_exact) in alts.items():
        cand = np.flatnonzero(alt_np.reshape(-1) != flat)
        separated(name, cand, ex_page, lambda i, f=alt_exact: rne(f(*args(i)), BF16),
                  lambda i: int(flat[i]))
    for i in np.random.default_rng(7).choice(flat.size, 1500, replace=False):
        assert bf16_bits(ex_page(i)) == int(flat[i])


def _silu_exact_bf16(t: Fraction) -> Fraction:
    """bf16 rounding of SiLU(t) = t / (1 + e^-t), evaluated to 60 digits.  The
    rounding must not move under a relative change of 2^-40 (far above the
    evaluation's error), so that it is the exact value's rounding."""
    td = Decimal(t.numerator) / Decimal(t.denominator)
    s = Fraction(td / (1 + (-td).exp()))
    v = rne(s, BF16)
    d = Fraction(1, 1 << 40)
    assert rne(s * (1 - d), BF16) == v == rne(s * (1 + d), BF16)
    return v


def test_wan_pre_activation_order(orc):
    rows, C = 4096, 384
    xb = bf16_from_normal(0.0, 1.0, (rows, C), 0x5701)
    gamma = f32_from_u16(bf16_from_normal(1.0, 0.05, (C,), 0x5702))   # bf16 values held as fp32
    rstd = f32_uniform(0.5, 2.0, rows, 0x5703)
    out = orc.silu_normalize(xb, rstd, gamma)
    flat = out.reshape(-1)
    xf, r, g = f32_from_u16(xb), rstd[:, None], gamma[None, :]
    t_page = (xf * r) * g

    def silu_np(t):
        t = t.astype(np.float64)
        return lib_bf16_of_f64(t / (1.0 + np.exp(-t)))

    page_np = silu_np(t_page)

    def args(i):
        a, b = divmod(int(i), C)
        return fr(xf[a, b]), fr(rstd[a]), fr(gamma[b])

    def ex_page(i):
        X, R, G = args(i)
        return _silu_exact_bf16(r32(r32(X * R) * G))

    alts = {
        "xb*(rstd*gamma)": (xf * (r * g), lambda X, R, G: r32(X * r32(R * G))),
        "(xb*gamma)*rstd": ((xf * g) * r, lambda X, R, G: r32(r32(X * G) * R)),
    }
    for name, (t_alt, alt_exact) in alts.items():
        cand = np.flatnonzero((silu_np(t_alt) != page_np).reshape(-1) & (t_alt != t_page).reshape(-1))
        separated(name, cand, ex_page, lambda i, f=alt_exact: _silu_exact_bf16(f(*args(i))),
                  lambda i: int(flat[i]))
    for i in np.random.default_rng(8).choice(flat.size, 600, replace=False):
        assert bf16_bits(ex_page(i)) == int(flat[i])
