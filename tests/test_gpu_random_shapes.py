"""Seeded random shapes across the entry points (a fixed list, so failures
reproduce): widths that are any multiple of 8 up to 4096 (a wavefront per
row, the balanced launch, ragged last vectors) and up to 16384 (rows in
halves, a workgroup per row), several modulation batches
with chunk-view strides, row counts that leave remainders of every size
against the 1024 SIMDs, token counts across the backward's tree levels, and
Wan pixel counts and qk head-row counts that leave ragged last groups.
Every output is compared with the oracle at the parity bar."""
import numpy as np
import pytest
import torch

from dit_adaln_row_amd import inputs as gen
from parity import check_rows_end_to_end, check_stats, dev, host, log, same_bits, ulp_diff

pytestmark = pytest.mark.gpu


def rand(shape, mu, sigma, seed):
    return gen.to_u16(gen.normal(shape, mu, sigma, seed))


def _configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        cols = int(rng.choice([8 * int(rng.integers(1, 513)), 1024 * int(rng.integers(1, 5))]))
        B = int(rng.choice([1, 1, 2, 3, 7]))
        S = int(rng.integers(1, 1400 // B + 2))
        extra = int(rng.choice([0, 0, 8, 8 * int(rng.integers(1, 64))]))  # chunk-view stride pad
        out.append((i, B, S, cols, extra))
    return out


CONFIGS = _configs(32, 20261202)
KINDS = ["ln", "gated", "rms", "gated_rms", "folded", "backward"]


def _wide_configs(n, seed):
    """Rows over 4096 columns: the half-row widths (5120-8192 in steps of
    1024) and any multiple of 8 to 16384 (a workgroup per row)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        cols = int(rng.choice([5120, 6144, 7168, 8192, 8 * int(rng.integers(513, 2049))]))
        B = int(rng.choice([1, 1, 2, 3]))
        S = int(rng.integers(1, 700 // B + 2))
        extra = int(rng.choice([0, 8, 8 * int(rng.integers(1, 64))]))
        out.append((100 + i, B, S, cols, extra))
    return out


WIDE = _wide_configs(12, 20261204)
WIDE_KINDS = ["ln", "gated", "rms", "gated_rms", "folded"]


def _pixel_configs(n, seed):
    """Wan channel counts (the two tuned widths, the other LDS-staged and
    lane-split widths, any multiple of 8) with pixel counts that leave every
    kind of ragged last group; qk head-row counts split between q and k."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        c = int(rng.choice([96, 96, 384, 384, 128, 192, 256, 512, 8 * int(rng.integers(1, 513))]))
        pixels = int(rng.integers(1, 3000))
        rq, rk = int(rng.integers(0, 2500)), int(rng.integers(0, 2500))
        out.append((i, c, pixels, bool(rng.integers(0, 2)), max(rq, 1), rk))
    return out


@pytest.mark.parametrize("i,c,pixels,bias,rq,rk", _pixel_configs(16, 20261203))
def test_random_pixels_and_heads(gpu, orc, i, c, pixels, bias, rq, rk):
    log(f"random pixels {i}: C={c} pixels={pixels} bias={bias}; qk rows {rq}+{rk}")
    x = rand((pixels, c), 0, 1, 1600 + i)
    b = gen.normal((c,), 0, 0.05, 1700 + i, "f32").numpy() if bias else None
    g = gen.normal((c,), 1, 0.05, 1800 + i, "f32_bf16vals").numpy()
    rstd = torch.empty(pixels, dtype=torch.float32, device="cuda")
    xb = torch.empty((pixels, c), dtype=torch.bfloat16, device="cuda")
    out = gpu.rmsnorm_silu_bias(dev(x), torch.from_numpy(g).cuda(),
                                torch.from_numpy(b).cuda() if bias else None, 1e-6,
                                rstd_out=rstd, xb_out=xb)
    torch.cuda.synchronize()
    ref = orc.rmsnorm_silu_bias(x, b, g, 1e-6)
    assert same_bits(host(xb), ref["xb"])
    assert np.array_equal(host(rstd).view(np.uint32), ref["rstd"].view(np.uint32))
    assert ulp_diff(host(out), ref["out"]).max() <= 1

    q = rand((rq, 128), 0, 2, 1900 + i)
    k = rand((rk, 128), 0.5, 2, 2000 + i) if rk else None
    mean = torch.empty(rq + rk, dtype=torch.float32, device="cuda")
    rs = torch.empty(rq + rk, dtype=torch.float32, device="cuda")
    qo, ko = gpu.qk_layernorm(dev(q), dev(k) if rk else None, 1e-5, mean_out=mean, rstd_out=rs)
    torch.cuda.synchronize()
    qref = orc.qk_layernorm(q, k if rk else np.zeros((0, 128), np.uint16), 1e-5)
    check_stats(host(mean), host(rs), qref["mean"], qref["rstd"], "qk")
    got = np.concatenate([host(qo)] + ([host(ko)] if rk else []))
    want = np.concatenate([qref["q_out"]] + ([qref["k_out"]] if rk else []))
    check_rows_end_to_end(got, want, "qk")


def _mod(B, cols, extra, seed):
    """B modulation rows of `cols` inside rows of cols + extra (a chunk view)."""
    full = rand((B, cols + extra), 0, 0.1, seed)
    return full, dev(full)[:, :cols], np.ascontiguousarray(full[:, :cols])


@pytest.mark.parametrize("i,B,S,cols,extra", CONFIGS)
def test_random_shape(gpu, orc, i, B, S, cols, extra):
    _check_shape(gpu, orc, i, KINDS[i % len(KINDS)], B, S, cols, extra)


@pytest.mark.parametrize("i,B,S,cols,extra", WIDE)
def test_random_wide_shape(gpu, orc, i, B, S, cols, extra):
    _check_shape(gpu, orc, i, WIDE_KINDS[i % len(WIDE_KINDS)], B, S, cols, extra)


def _check_shape(gpu, orc, i, kind, B, S, cols, extra):
    rows = B * S
    log(f"random shape {i}: {kind} B={B} S={S} cols={cols} stride pad={extra}")
    x = rand((rows, cols), 0.1 * (i % 3), 1.0 + 0.3 * (i % 4), 700 + i)
    _, scd, sc = _mod(B, cols, extra, 800 + i)
    _, shd, sh = _mod(B, cols, extra, 900 + i)
    mean, rstd = (torch.empty(rows, dtype=torch.float32, device="cuda") for _ in range(2))
    if kind in ("ln", "folded"):
        fn = gpu.ln_modulate if kind == "ln" else gpu.ln_modulate_folded
        out = host(fn(dev(x), scd, shd, 1e-6, mean_out=mean, rstd_out=rstd))
        torch.cuda.synchronize()
        ref = (orc.ln_modulate if kind == "ln" else orc.ln_modulate_folded)(
            x, sc, sh, 1e-6, rows_per_batch=S)
        check_stats(host(mean), host(rstd), ref["mean"], ref["rstd"], kind)
        check_rows_end_to_end(out, ref["out"], kind)
    elif kind == "gated":
        res = rand((rows, cols), 0, 1, 1000 + i)
        _, gd, g = _mod(B, cols, extra, 1100 + i)
        h, out = gpu.gated_ln_modulate(dev(x), dev(res), gd, scd, shd, 1e-6, mean_out=mean,
                                       rstd_out=rstd)
        torch.cuda.synchronize()
        ref = orc.gated_ln_modulate(x, res, g, sc, sh, 1e-6, rows_per_batch=S)
        assert same_bits(host(h), ref["h"])
        check_stats(host(mean), host(rstd), ref["mean"], ref["rstd"], kind)
        check_rows_end_to_end(host(out), ref["out"], kind)
    elif kind in ("rms", "gated_rms"):
        w = rand((cols,), 1, 0.05, 1200 + i)
        kw, res, g = {}, None, None
        if kind == "gated_rms":
            res = rand((rows, cols), 0, 1, 1300 + i)
            _, gd, g = _mod(B, cols, extra, 1400 + i)
            kw = dict(residual=dev(res), gate=gd)
        r = gpu.rms_modulate(dev(x), dev(w), scd, shd, 1e-6, rstd_out=rstd, **kw)
        torch.cuda.synchronize()
        ref = orc.rms_modulate(x, w, sc, sh, 1e-6, residual=res, gate=g, rows_per_batch=S)
        out = r
        if kind == "gated_rms":
            h, out = r
            assert same_bits(host(h), ref["h"])
        check_stats(None, host(rstd), None, ref["rstd"], kind)
        check_rows_end_to_end(host(out), ref["out"], kind)
    else:
        if cols > 4096:
            pytest.skip("the backward serves rows up to 4096 columns")
        dout = rand((rows, cols), 0, 1, 1500 + i)
        # outputs start as NaN: no value may survive from a reused buffer
        nan = float("nan")
        d_x = torch.full((rows, cols), nan, dtype=torch.bfloat16, device="cuda")
        d_scale = torch.full((B, cols), nan, dtype=torch.float32, device="cuda")
        d_shift = torch.full((B, cols), nan, dtype=torch.float32, device="cuda")
        d_x, d_scale, d_shift = gpu.ln_modulate_backward(dev(x), scd, dev(dout), 1e-6, d_x=d_x,
                                                         d_scale=d_scale, d_shift=d_shift,
                                                         mean_out=mean, rstd_out=rstd)
        torch.cuda.synchronize()
        ref = orc.ln_modulate_backward(x, sc, dout, 1e-6, rows_per_batch=S)
        check_stats(host(mean), host(rstd), ref["mean"], ref["rstd"], kind)
        d = ulp_diff(host(d_x), ref["d_x"])
        assert d.max() <= 1 and (d == 0).mean() >= 0.9999
        assert np.array_equal(host(d_shift), ref["d_shift"])
        assert np.array_equal(host(d_scale), ref["d_scale"])
