"""Non-finite and extreme rows through every entry point, against the oracle
bit for bit (NaN by class): a row holding +inf, one holding -inf, one
holding both, one holding a NaN, a row of huge finite values (~1e30) and an
all-zero row, mixed with ordinary rows.

By their definition the statistics of a row holding an infinity or a NaN are
NaN (inf - inf in the variance, NaN in the sums), so the whole row's output
is NaN; the RMS statistics of a row holding an infinity are rstd = 0.  The
kernels and the oracle take the same IEEE operations, so the non-finite
results agree by class and the finite ones by bits (the SiLU output within
its 1-ulp bar).
"""
import numpy as np
import pytest
import torch

from dit_adaln_row_amd import inputs as gen
from parity import dev, host, log, same_bits, ulp_diff

pytestmark = pytest.mark.gpu

PINF, NINF, QNAN = 0x7F80, 0xFF80, 0x7FC0


def rand(shape, mu, sigma, seed):
    return gen.to_u16(gen.normal(shape, mu, sigma, seed))


def special_rows(rows, cols, seed):
    x = rand((rows, cols), 0, 1, seed)
    x[0, 5 % cols] = PINF
    x[1, 7 % cols] = NINF
    x[2, 3 % cols] = PINF
    x[2, 11 % cols] = NINF
    x[3, 9 % cols] = QNAN
    x[4] = rand((1, cols), 0, 1e30, seed + 1)  # huge, finite
    x[5] = 0
    return x


def f32_same(a, b):
    """fp32 arrays bitwise equal, NaNs compared by class."""
    a = np.ascontiguousarray(a, np.float32)
    b = np.ascontiguousarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32),
                                                     b[~nb].view(np.uint32))


def f32(n):
    return torch.empty(n, dtype=torch.float32, device="cuda")


def check_nonfinite_rows_nan(out, rows=(0, 1, 2, 3)):
    """The rows holding an infinity or a NaN are NaN throughout (LN)."""
    nan = ((out & 0x7F80) == 0x7F80) & ((out & 0x7F) != 0)
    assert nan[list(rows)].all()


@pytest.mark.parametrize("cols", [1000, 3072, 5000])
def test_ln_modulate_non_finite(gpu, orc, cols):
    """cols 3072: the balanced row kernel; 1000: a wavefront per row; 5000: a
    workgroup per row."""
    x = special_rows(8, cols, 500)
    sc, sh = rand((1, cols), 0, 0.1, 501), rand((1, cols), 0, 0.1, 502)
    mean, rstd, y = f32(8), f32(8), torch.empty((8, cols), dtype=torch.bfloat16, device="cuda")
    out = gpu.ln_modulate(dev(x), dev(sc), dev(sh), 1e-6, mean_out=mean, rstd_out=rstd, y_out=y)
    torch.cuda.synchronize()
    ref = orc.ln_modulate(x, sc, sh, 1e-6)
    assert f32_same(host(mean), ref["mean"]) and f32_same(host(rstd), ref["rstd"])
    assert same_bits(host(y), ref["y"]) and same_bits(host(out), ref["out"])
    check_nonfinite_rows_nan(host(out))
    folded_mean, folded_rstd = f32(8), f32(8)
    fo = gpu.ln_modulate_folded(dev(x), dev(sc), dev(sh), 1e-6, mean_out=folded_mean,
                                rstd_out=folded_rstd)
    torch.cuda.synchronize()
    fref = orc.ln_modulate_folded(x, sc, sh, 1e-6)
    assert f32_same(host(folded_rstd), fref["rstd"])
    assert same_bits(host(fo), fref["out"])


@pytest.mark.parametrize("cols", [1000, 3072])
def test_gated_ln_modulate_non_finite(gpu, orc, cols):
    """Non-finite updates and residuals: h by the gate stage's IEEE ops, then
    the LN of h."""
    upd = special_rows(8, cols, 510)
    res = rand((8, cols), 0, 1, 511)
    res[6, 2] = PINF
    gate, sc, sh = (rand((1, cols), 0, 0.1, 512 + i) for i in range(3))
    mean, rstd = f32(8), f32(8)
    h, out = gpu.gated_ln_modulate(dev(upd), dev(res), dev(gate), dev(sc), dev(sh), 1e-6,
                                   mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    ref = orc.gated_ln_modulate(upd, res, gate, sc, sh, 1e-6)
    assert same_bits(host(h), ref["h"])
    assert f32_same(host(mean), ref["mean"]) and f32_same(host(rstd), ref["rstd"])
    assert same_bits(host(out), ref["out"])


@pytest.mark.parametrize("cols,gated", [(1000, False), (4096, False), (4096, True)])
def test_rms_modulate_non_finite(gpu, orc, cols, gated):
    """RMS: a row holding an infinity has rstd = 1/sqrt(inf) = 0, so its
    finite elements normalise to zero and the infinity to NaN."""
    x = special_rows(8, cols, 520)
    w = rand((cols,), 1, 0.05, 521)
    sc, sh = rand((1, cols), 0, 0.1, 522), rand((1, cols), 0, 0.1, 523)
    rstd = f32(8)
    kw = {}
    res = gate = None
    if gated:
        res, gate = rand((8, cols), 0, 1, 524), rand((1, cols), 0, 0.1, 525)
        kw = dict(residual=dev(res), gate=dev(gate))
    r = gpu.rms_modulate(dev(x), dev(w), dev(sc), dev(sh), 1e-6, rstd_out=rstd, **kw)
    torch.cuda.synchronize()
    ref = orc.rms_modulate(x, w, sc, sh, 1e-6, residual=res, gate=gate)
    if gated:
        h, out = r
        assert same_bits(host(h), ref["h"])
    else:
        out = r
    assert f32_same(host(rstd), ref["rstd"])
    assert same_bits(host(out), ref["out"])


def test_qk_layernorm_non_finite(gpu, orc):
    q = special_rows(40, 128, 530)
    k = special_rows(24, 128, 531)[::-1].copy()
    mean, rstd = f32(64), f32(64)
    qo, ko = gpu.qk_layernorm(dev(q), dev(k), 1e-5, mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    ref = orc.qk_layernorm(q, k, 1e-5)
    assert f32_same(host(mean), ref["mean"]) and f32_same(host(rstd), ref["rstd"])
    assert same_bits(host(qo), ref["q_out"]) and same_bits(host(ko), ref["k_out"])


@pytest.mark.parametrize("c", [96, 384, 200])
def test_rmsnorm_silu_bias_non_finite(gpu, orc, c):
    x = special_rows(64, c, 540)
    bias = gen.normal((c,), 0, 0.05, 541, "f32").numpy()
    gamma = gen.normal((c,), 1, 0.05, 542, "f32_bf16vals").numpy()
    rstd = f32(64)
    xb = torch.empty((64, c), dtype=torch.bfloat16, device="cuda")
    out = gpu.rmsnorm_silu_bias(dev(x), dev(gamma), dev(bias), 1e-6, rstd_out=rstd, xb_out=xb)
    torch.cuda.synchronize()
    ref = orc.rmsnorm_silu_bias(x, bias, gamma, 1e-6)
    assert same_bits(host(xb), ref["xb"])
    assert f32_same(host(rstd), ref["rstd"])
    o, ro = host(out), ref["out"]
    nan_g = ((o & 0x7F80) == 0x7F80) & ((o & 0x7F) != 0)
    nan_o = ((ro & 0x7F80) == 0x7F80) & ((ro & 0x7F) != 0)
    assert np.array_equal(nan_g, nan_o)
    assert ulp_diff(o[~nan_g], ro[~nan_o]).max() <= 1


@pytest.mark.parametrize("B,S,D", [(2, 8, 3072), (1, 40, 3072), (3, 5, 4096)])
def test_backward_non_finite(gpu, orc, B, S, D):
    """Non-finite x: the row's statistics are NaN, so are its d_x and every
    column's d_scale of that batch; d_shift (sums of d_out) stays finite."""
    x = special_rows(B * S, D, 550)
    sc = rand((B, D), 0, 0.1, 551)
    dout = rand((B * S, D), 0, 1, 552)
    dout[6] = 0
    mean, rstd = f32(B * S), f32(B * S)
    d_x, d_scale, d_shift = gpu.ln_modulate_backward(dev(x), dev(sc), dev(dout), 1e-6,
                                                     mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    ref = orc.ln_modulate_backward(x, sc, dout, 1e-6, rows_per_batch=S)
    assert f32_same(host(mean), ref["mean"]) and f32_same(host(rstd), ref["rstd"])
    g, r = host(d_x), ref["d_x"]
    nan_g = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)
    nan_o = ((r & 0x7F80) == 0x7F80) & ((r & 0x7F) != 0)
    assert np.array_equal(nan_g, nan_o) and nan_g[:4].all()
    assert ulp_diff(g[~nan_g], r[~nan_o]).max() <= 1
    assert f32_same(host(d_scale), ref["d_scale"]) and f32_same(host(d_shift), ref["d_shift"])
    assert np.isnan(host(d_scale)[0]).all() and np.isfinite(host(d_shift)).all()
    log(f"  backward non-finite {B}x{S}x{D}: ok")
