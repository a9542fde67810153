"""GPU parity: the HIP kernels (called through the C ABI via the binding)
against the CPU oracle, element by element, on seeded inputs.

Sizes: small and ragged cases (several tiles / workgroups plus a tail, odd
widths, batched modulation with chunk-view strides, empty launches) and every
workload at its full size, in the launch configuration the benchmark times
(no debug outputs) and with the debug outputs on for the stage checks.
"""
import numpy as np
import pytest
import torch

from dit_adaln_row_amd import inputs as gen
from dit_adaln_row_amd.workloads import WORKLOADS
from parity import (by_row_chunks, check_rows_end_to_end, check_stats, dev, host, log,
                    same_bits, ulp_diff)

pytestmark = pytest.mark.gpu
F32 = torch.float32


def rand(shape, mu, sigma, seed):
    return gen.to_u16(gen.normal(shape, mu, sigma, seed))


def empty_f32(n):
    return torch.empty(n, dtype=F32, device="cuda")


# ---------------------------------------------------------------------------
# LayerNorm + modulate (plain and gated)
# ---------------------------------------------------------------------------

def _ln_gpu(dn, x, sc, sh, eps, mod_dev=None, debug=True):
    rows, cols = x.shape
    xd = dev(x)
    scd, shd = mod_dev if mod_dev is not None else (dev(sc), dev(sh))
    kw = {}
    if debug:
        kw = dict(mean_out=empty_f32(rows), rstd_out=empty_f32(rows), y_out=torch.empty_like(xd))
    out = dn.ln_modulate(xd, scd, shd, eps, **kw)
    torch.cuda.synchronize()
    if not debug:
        return host(out), None, None, None
    return host(out), host(kw["mean_out"]), host(kw["rstd_out"]), host(kw["y_out"])


def _ln_check(orc, what, x, sc, sh, eps, rpb, out_g, mean_g, rstd_g, y_g, ref=None):
    ref = ref or orc.ln_modulate(x, sc, sh, eps, rows_per_batch=rpb)
    check_stats(mean_g, rstd_g, ref["mean"], ref["rstd"], what)
    assert same_bits(y_g, orc.ln_normalize(x, mean_g, rstd_g)), f"{what}: y stage"
    assert same_bits(out_g, orc.modulate(y_g, sc, sh, rows_per_batch=rpb)), f"{what}: modulate stage"
    check_rows_end_to_end(out_g, ref["out"], what)
    return ref


@pytest.mark.parametrize("rows,cols", [(1, 8), (3, 40), (257, 1024), (100, 3072), (37, 4096),
                                       (5, 2048), (9, 1536), (3, 16384), (1000, 512), (2, 9000),
                                       (100, 1152), (7, 2560), (33, 3584), (5, 1920), (65, 2304),
                                       (3, 2432), (17, 1088), (2, 3000)])
def test_ln_modulate_shapes(gpu, orc, rows, cols):
    log(f"ln_modulate rows={rows} cols={cols}")
    x = rand((rows, cols), 0.3, 1.5, 11 + cols)
    sc = rand((1, cols), 0, 0.1, 12)
    sh = rand((1, cols), 0, 0.1, 13)
    out, mean, rstd, y = _ln_gpu(gpu, x, sc, sh, 1e-6)
    _ln_check(orc, f"ln {rows}x{cols}", x, sc, sh, 1e-6, rows, out, mean, rstd, y)


def test_ln_modulate_batched_chunk_views(gpu, orc):
    """B = 3 modulation rows taken as chunk views of a [B, 6*D] embedding."""
    B, S, D = 3, 129, 3072
    log(f"ln_modulate batched B={B} S={S} D={D}")
    x = rand((B * S, D), 0, 1.5, 21)
    emb = rand((B, 6 * D), 0, 0.1, 22)
    embd = dev(emb)
    sc_view, sh_view = embd[:, D:2 * D], embd[:, 0:D]
    out, mean, rstd, y = _ln_gpu(gpu, x, None, None, 1e-6, mod_dev=(sc_view, sh_view))
    sc = np.concatenate([emb.ravel()[D:], np.zeros(D, np.uint16)]).reshape(B, 6 * D)
    _ln_check(orc, "ln batched", x, sc, emb, 1e-6, S, out, mean, rstd, y)


def test_ln_modulate_empty_and_inplace(gpu, orc):
    x = torch.empty((0, 1024), dtype=torch.bfloat16, device="cuda")
    s = torch.zeros((1, 1024), dtype=torch.bfloat16, device="cuda")
    assert gpu.ln_modulate(x, s, s).numel() == 0
    xs = rand((65, 1024), 0, 1, 31)
    sc, sh = rand((1, 1024), 0, 0.1, 32), rand((1, 1024), 0, 0.1, 33)
    xd = dev(xs)
    gpu.ln_modulate(xd, dev(sc), dev(sh), 1e-6, out=xd)   # in place
    torch.cuda.synchronize()
    assert same_bits(host(xd), orc.ln_modulate(xs, sc, sh, 1e-6)["out"])


def test_ln_special_rows(gpu, orc):
    """Constant rows (variance 0), an all-zero row, a high-offset row, huge and
    tiny (subnormal) magnitudes, and a NaN row."""
    cols = 3072
    x = rand((12, cols), 0, 1, 41)
    x[0] = 0x3FC0                                           # constant 1.5
    x[1] = 0                                                # zeros
    x[2] = rand((1, cols), 64.0, 0.1, 42)                   # offset row
    x[3] = rand((1, cols), 0, 1e30, 43)                     # huge
    x[4] = rand((1, cols), 0, 1e-39, 44)                    # subnormal
    x[5] = rand((1, cols), 0, 3e-38, 45)                    # tiny normal
    x[6] = np.where(np.arange(cols) % 2 == 0, 0x4040, 0xC040).astype(np.uint16)  # +-3
    x[7, 17] = 0x7FC0                                       # a NaN in a row
    sc = rand((1, cols), 0, 0.1, 46)
    sh = rand((1, cols), 0, 0.1, 47)
    out, mean, rstd, y = _ln_gpu(gpu, x, sc, sh, 1e-6)
    ref = orc.ln_modulate(x, sc, sh, 1e-6)
    fin = np.isfinite(ref["rstd"]) & np.isfinite(ref["mean"])
    _ln_check(orc, "ln special", x[fin], sc, sh, 1e-6, int(fin.sum()), out[fin], mean[fin],
              rstd[fin], y[fin])
    assert np.all(~np.isfinite(rstd[~fin]) | ~np.isfinite(mean[~fin]))
    assert same_bits(out[7], ref["out"][7])                # NaN row: NaN everywhere


@pytest.mark.parametrize("rows,cols,B", [(1, 8, 1), (257, 1024, 1), (100, 3072, 2), (37, 4096, 1),
                                         (3, 16384, 1), (2, 9000, 2), (5, 2048, 5), (9, 1536, 3)])
def test_ln_modulate_folded(gpu, orc, rows, cols, B):
    """The lossy affine-folded LN: same statistics, one fp32 chain per element."""
    log(f"ln_modulate_folded rows={rows} cols={cols} B={B}")
    x = rand((rows, cols), 0.1, 1.5, 71 + cols)
    emb = rand((B, 6 * cols), 0, 0.1, 72 + B)
    embd = dev(emb)
    sc_view, sh_view = embd[:, cols:2 * cols], embd[:, 0:cols]
    mean, rstd = empty_f32(rows), empty_f32(rows)
    xd = dev(x)
    out = gpu.ln_modulate_folded(xd, sc_view, sh_view, 1e-6, mean_out=mean, rstd_out=rstd)
    fast = gpu.ln_modulate_folded(xd, sc_view, sh_view, 1e-6)
    torch.cuda.synchronize()
    out, fast, mean, rstd = host(out), host(fast), host(mean), host(rstd)
    assert same_bits(out, fast), "statistics outputs changed the result"
    sc = np.concatenate([emb.ravel()[cols:], np.zeros(cols, np.uint16)]).reshape(B, 6 * cols)
    ref = orc.ln_modulate_folded(x, sc, emb, 1e-6, rows_per_batch=rows // B)
    check_stats(mean, rstd, ref["mean"], ref["rstd"], "folded")
    check_rows_end_to_end(out, ref["out"], "folded")


def test_gated_ln_modulate_shapes(gpu, orc):
    for rows, cols, B in [(7, 1024, 1), (300, 3072, 1), (2 * 65, 3072, 2), (33, 4096, 1)]:
        log(f"gated_ln_modulate rows={rows} cols={cols} B={B}")
        upd = rand((rows, cols), 0, 1.5, 51)
        res = rand((rows, cols), 0, 1, 52)
        gate = rand((B, cols), 0, 0.1, 53)
        sc = rand((B, cols), 0, 0.1, 54)
        sh = rand((B, cols), 0, 0.1, 55)
        kw = dict(mean_out=empty_f32(rows), rstd_out=empty_f32(rows), y_out=torch.empty(
            (rows, cols), dtype=torch.bfloat16, device="cuda"))
        h, out = gpu.gated_ln_modulate(dev(upd), dev(res), dev(gate), dev(sc), dev(sh), 1e-6, **kw)
        torch.cuda.synchronize()
        h, out = host(h), host(out)
        rpb = rows // B
        ref = orc.gated_ln_modulate(upd, res, gate, sc, sh, 1e-6, rows_per_batch=rpb)
        assert same_bits(h, ref["h"]), "gate stage"
        _ln_check(orc, "gated", h, sc, sh, 1e-6, rpb, out, host(kw["mean_out"]),
                  host(kw["rstd_out"]), host(kw["y_out"]), ref=ref)


def test_gated_inplace_residual(gpu, orc):
    rows, cols = 64, 3072
    upd, res = rand((rows, cols), 0, 1.5, 61), rand((rows, cols), 0, 1, 62)
    gate, sc, sh = (rand((1, cols), 0, 0.1, s) for s in (63, 64, 65))
    rd = dev(res)
    gpu.gated_ln_modulate(dev(upd), rd, dev(gate), dev(sc), dev(sh), 1e-6, residual_out=rd)
    torch.cuda.synchronize()
    assert same_bits(host(rd), orc.gate_residual(upd, res, gate))


# ---------------------------------------------------------------------------
# RMSNorm + modulate (plain and gated)
# ---------------------------------------------------------------------------

def _rms_run_check(gpu, orc, what, x, w, sc, sh, eps, rpb, res=None, gate=None, mod_dev=None):
    """mod_dev: device (scale, shift, gate) views to pass instead of sc, sh, gate
    (chunk views); the host arrays then describe the same memory for the oracle."""
    rows, cols = x.shape
    kw = dict(rstd_out=empty_f32(rows), y_out=torch.empty((rows, cols), dtype=torch.bfloat16,
                                                          device="cuda"))
    scd, shd, gd = mod_dev if mod_dev is not None else (dev(sc), dev(sh), dev(gate))
    if res is not None:
        h, out = gpu.rms_modulate(dev(x), dev(w), scd, shd, eps, residual=dev(res), gate=gd, **kw)
    else:
        h, out = None, gpu.rms_modulate(dev(x), dev(w), scd, shd, eps, **kw)
    torch.cuda.synchronize()
    out, rstd, y = host(out), host(kw["rstd_out"]), host(kw["y_out"])
    ref = orc.rms_modulate(x, w, sc, sh, eps, residual=res, gate=gate, rows_per_batch=rpb)
    src = x
    if res is not None:
        h = host(h)
        assert same_bits(h, ref["h"]), f"{what}: gate stage"
        src = h
    check_stats(None, rstd, None, ref["rstd"], what)
    assert same_bits(y, orc.rms_normalize(src, rstd, w)), f"{what}: y stage"
    assert same_bits(out, orc.modulate(y, sc, sh, rows_per_batch=rpb)), f"{what}: modulate stage"
    check_rows_end_to_end(out, ref["out"], what)
    assert np.all(ulp_diff(out, ref["out"]) <= 1), f"{what}: beyond 1 ulp"


@pytest.mark.parametrize("rows,cols,B,gated", [(1, 4096, 1, False), (128, 2048, 1, False),
                                               (2 * 1140, 4096, 2, False), (257, 4096, 1, True),
                                               (2 * 65, 4096, 2, True), (11, 1024, 1, True),
                                               (5, 24, 1, False), (3, 16384, 1, True),
                                               (2 * 50, 2560, 2, True), (64, 1536, 1, False),
                                               (9, 3584, 1, True), (30, 1152, 1, False)])
def test_rms_modulate_shapes(gpu, orc, rows, cols, B, gated):
    log(f"rms_modulate rows={rows} cols={cols} B={B} gated={gated}")
    x = rand((rows, cols), 0, 1, 71 + cols)
    w = rand((cols,), 1, 0.05, 72)
    sc, sh = rand((B, cols), 0, 0.1, 73), rand((B, cols), 0, 0.1, 74)
    res = rand((rows, cols), 0, 1, 75) if gated else None
    gate = rand((B, cols), 0, 0.1, 76) if gated else None
    _rms_run_check(gpu, orc, f"rms {rows}x{cols}", x, w, sc, sh, 1e-6, rows // B, res, gate)


@pytest.mark.parametrize("cols", [5120, 6144, 7168, 8192])
@pytest.mark.parametrize("kind", ["ln", "gated_ln", "rms", "gated_rms"])
@pytest.mark.parametrize("rows,B", [(74, 2), (1029, 1)])
def test_wide_rows_in_halves(gpu, orc, cols, kind, rows, B):
    """Rows of 5120-8192 columns go in halves, a wavefront each (RMS rows over
    6144 columns a workgroup per row), their modulation rows staged in LDS as
    bf16.  Two batches of 37 rows put a batch boundary inside a workgroup's
    pair of rows; the call is made with the debug outputs (stage checks) and
    without them (the timed form), and both outputs must be the same bits."""
    log(f"{kind} rows={rows} cols={cols} B={B}")
    rpb = rows // B
    x = rand((rows, cols), 0.1, 1.3, 201 + cols + rows)
    res = rand((rows, cols), 0, 1, 202) if kind.startswith("gated") else None
    gate = rand((B, cols), 0, 0.1, 203) if res is not None else None
    sc, sh = rand((B, cols), 0, 0.1, 204), rand((B, cols), 0, 0.1, 205)
    what = f"{kind} {rows}x{cols}"
    if kind.endswith("rms"):
        w = rand((cols,), 1, 0.05, 206)
        _rms_run_check(gpu, orc, what, x, w, sc, sh, 1e-6, rpb, res, gate)
        plain = gpu.rms_modulate(dev(x), dev(w), dev(sc), dev(sh), 1e-6,
                                 **({} if res is None else dict(residual=dev(res), gate=dev(gate))))
        ref = orc.rms_modulate(x, w, sc, sh, 1e-6, residual=res, gate=gate, rows_per_batch=rpb)
    elif res is None:
        out, mean, rstd, y = _ln_gpu(gpu, x, sc, sh, 1e-6)
        ref = _ln_check(orc, what, x, sc, sh, 1e-6, rpb, out, mean, rstd, y)
        plain = gpu.ln_modulate(dev(x), dev(sc), dev(sh), 1e-6)
    else:
        kw = dict(mean_out=empty_f32(rows), rstd_out=empty_f32(rows), y_out=torch.empty(
            (rows, cols), dtype=torch.bfloat16, device="cuda"))
        h, out = gpu.gated_ln_modulate(dev(x), dev(res), dev(gate), dev(sc), dev(sh), 1e-6, **kw)
        torch.cuda.synchronize()
        h, out = host(h), host(out)
        ref = orc.gated_ln_modulate(x, res, gate, sc, sh, 1e-6, rows_per_batch=rpb)
        assert same_bits(h, ref["h"]), f"{what}: gate stage"
        _ln_check(orc, what, h, sc, sh, 1e-6, rpb, out, host(kw["mean_out"]),
                  host(kw["rstd_out"]), host(kw["y_out"]), ref=ref)
        plain = gpu.gated_ln_modulate(dev(x), dev(res), dev(gate), dev(sc), dev(sh), 1e-6)
    torch.cuda.synchronize()
    if isinstance(plain, tuple):
        assert same_bits(host(plain[0]), ref["h"]), f"{what}: gate stage (timed form)"
        plain = plain[1]
    check_rows_end_to_end(host(plain), ref["out"], f"{what} (timed form)")


# ---------------------------------------------------------------------------
# qk LayerNorm
# ---------------------------------------------------------------------------

def _qk_run_check(gpu, orc, what, q, k, eps):
    rq, rk = q.shape[0], (0 if k is None else k.shape[0])
    mean, rstd = empty_f32(rq + rk), empty_f32(rq + rk)
    qo, ko = gpu.qk_layernorm(dev(q), None if k is None else dev(k), eps, mean_out=mean,
                              rstd_out=rstd)
    torch.cuda.synchronize()
    qo = host(qo)
    ko = host(ko) if k is not None else np.zeros((0, 128), np.uint16)
    kk = k if k is not None else np.zeros((0, 128), np.uint16)
    ref = orc.qk_layernorm(q, kk, eps)
    mean, rstd = host(mean), host(rstd)
    check_stats(mean, rstd, ref["mean"], ref["rstd"], what)
    both = np.concatenate([q, kk])
    got = np.concatenate([qo, ko])
    assert same_bits(got, orc.ln_normalize(both, mean, rstd)), f"{what}: normalise stage"
    check_rows_end_to_end(got, np.concatenate([ref["q_out"], ref["k_out"]]), what)


@pytest.mark.parametrize("rq,rk", [(1, 0), (4, 4), (3, 5), (17, 1), (4360 * 32, 4360 * 32),
                                   (1000, 37), (16 * 7 + 3, 16 * 5 + 1)])
def test_qk_layernorm_shapes(gpu, orc, rq, rk):
    log(f"qk_layernorm rows_q={rq} rows_k={rk}")
    q = rand((rq, 128), 0, 2, 81)
    k = rand((rk, 128), 0.1, 2, 82) if rk else None
    _qk_run_check(gpu, orc, f"qk {rq}+{rk}", q, k, 1e-5)


@pytest.mark.parametrize("d", [8, 16, 32, 40, 64, 72, 96, 112, 120])
@pytest.mark.parametrize("rq,rk", [(1, 0), (37, 11), (4096, 4093)])
def test_qk_layernorm_head_dims(gpu, orc, d, rq, rk):
    """Head dims other than 128 (multiples of 8 up to 128): 4 lanes per row up
    to 32, else 8, the vectors past the row's end masked; the statistics
    divide by d.  Statistics to the bit, the normalise stage and every output
    against the oracle."""
    log(f"qk_layernorm head_dim={d} rows_q={rq} rows_k={rk}")
    q = rand((rq, d), 0, 2, 83 + d)
    k = rand((rk, d), 0.1, 2, 84 + d) if rk else None
    mean, rstd = empty_f32(rq + rk), empty_f32(rq + rk)
    qo, ko = gpu.qk_layernorm(dev(q), None if k is None else dev(k), 1e-5, mean_out=mean,
                              rstd_out=rstd)
    torch.cuda.synchronize()
    kk = k if k is not None else np.zeros((0, d), np.uint16)
    ref = orc.qk_layernorm(q, kk, 1e-5, head_dim=d)
    mean, rstd = host(mean), host(rstd)
    what = f"qk d={d} {rq}+{rk}"
    check_stats(mean, rstd, ref["mean"], ref["rstd"], what)
    got = np.concatenate([host(qo)] + ([host(ko)] if k is not None else []))
    both = np.concatenate([q, kk])
    assert same_bits(got, orc.ln_normalize(both, mean, rstd)), f"{what}: normalise stage"
    check_rows_end_to_end(got, np.concatenate([ref["q_out"], ref["k_out"]]), what)


# ---------------------------------------------------------------------------
# channels_last RMSNorm + SiLU (+ bias) and the conv-bias epilogue
# ---------------------------------------------------------------------------

def _wan_run_check(gpu, orc, what, x, bias, gamma, eps):
    rows, c = x.shape
    rstd, xb = empty_f32(rows), torch.empty((rows, c), dtype=torch.bfloat16, device="cuda")
    out = gpu.rmsnorm_silu_bias(dev(x), dev(gamma), None if bias is None else dev(bias), eps,
                                rstd_out=rstd, xb_out=xb)
    torch.cuda.synchronize()
    out, rstd, xb = host(out), host(rstd), host(xb)
    ref = by_row_chunks(lambda lo, hi: orc.rmsnorm_silu_bias(x[lo:hi], bias, gamma, eps), None, rows)
    assert same_bits(xb, ref["xb"]), f"{what}: bias stage"
    check_stats(None, rstd, None, ref["rstd"], what)
    exact = rstd.view(np.uint32) == ref["rstd"].view(np.uint32)
    d = ulp_diff(out, ref["out"])
    log(f"  {what}: rstd exact on {exact.mean():.6f} of rows; out exact on "
        f"{(d == 0).mean():.6f} of elements, max {int(d.max())} ulp")
    # binary64 sums of squares of bf16 values are exact here and the square
    # root and divisions are the oracle's: the statistics match to the bit
    assert exact.all(), f"{what}: rstd differs from the oracle's in {int((~exact).sum())} rows"
    assert np.all(d <= 1), f"{what}: SiLU output beyond 1 ulp"
    if d.size >= 1 << 20:  # (a share is only meaningful over many elements)
        # the hardware exp2 / reciprocal are within a few 1e-7: only values
        # that close to a bf16 halfway point may round the other way
        assert (d == 0).mean() >= 0.9999, f"{what}: SiLU output exact on {(d == 0).mean():.6f}"
    return ref


@pytest.mark.parametrize("rows,c,bias", [(1, 96, True), (17, 96, True), (1000, 384, True),
                                         (333, 96, False), (64, 128, True), (77, 256, True),
                                         (50, 512, True), (13, 40, True), (9, 1000, False),
                                         (5, 4096, True), (31, 192, True), (100, 8, True),
                                         (100, 64, False), (41, 136, True), (300, 1024, True),
                                         (7, 2048, True), (3, 2056, False), (65, 520, True),
                                         (200, 24, True), (90, 72, False), (33, 200, True),
                                         (20, 264, True)])
def test_rmsnorm_silu_bias_shapes(gpu, orc, rows, c, bias):
    log(f"rmsnorm_silu_bias rows={rows} C={c} bias={bias}")
    x = rand((rows, c), 0, 1, 91 + c)
    b = gen.normal((c,), 0, 0.05, 92, "f32").numpy() if bias else None
    g = gen.normal((c,), 1, 0.05, 93, "f32_bf16vals").numpy()
    _wan_run_check(gpu, orc, f"wan {rows}x{c}", x, b, g, 1e-6)


@pytest.mark.parametrize("rows,c", [(16 * 1000 + 5, 96), (37, 96), (4 * 777 + 3, 384), (1, 384),
                                    (2 * 4160 + 1, 96)])
def test_rmsnorm_silu_bias_fold_equals_prebiased_input(gpu, rows, c):
    """Wan VAE page ("[Diffusion] Fuse the Wan VAE conv bias epilogue and tile
    the RMSNorm+SiLU kernel"), Tests / docs: the conv bias folded into the
    kernel equals the kernel run on the pre-biased tensor, bit for bit.  The
    pre-biased tensor is made the eager way, torch's add_ of the bias cast to
    bf16; ragged pixel counts leave partial pixel groups."""
    log(f"wan bias fold rows={rows} C={c}")
    x = gen.normal((rows, c), 0, 1, 3100 + c).cuda()
    b = gen.normal((c,), 0, 0.05, 3101, "f32").cuda()
    g = gen.normal((c,), 1, 0.05, 3102, "f32_bf16vals").cuda()
    r1, r2 = empty_f32(rows), empty_f32(rows)
    xb = torch.empty_like(x)
    folded = gpu.rmsnorm_silu_bias(x, g, b, 1e-6, rstd_out=r1, xb_out=xb)
    pre = x.clone().add_(b.to(torch.bfloat16))
    plain = gpu.rmsnorm_silu_bias(pre, g, None, 1e-6, rstd_out=r2)
    torch.cuda.synchronize()
    assert np.array_equal(host(xb), host(pre)), "bias stage differs from add_"
    assert np.array_equal(host(r1).view(np.uint32), host(r2).view(np.uint32)), "rstd"
    assert np.array_equal(host(folded), host(plain)), "folded bias differs from the pre-biased input"


def test_rmsnorm_silu_extreme_t(gpu, orc):
    """Large |t| (gamma up to 120): exp(-|t|) underflows / becomes subnormal."""
    rows, c = 64, 96
    x = rand((rows, c), 0, 1, 94)
    g = np.linspace(-120, 120, c).astype(np.float32)
    _wan_run_check(gpu, orc, "wan extreme", x, None, g, 1e-6)


def test_rmsnorm_silu_channels_last_5d(gpu, orc):
    n, c, d, h, w = 1, 96, 2, 12, 20
    xt = gen.normal((n, c, d, h, w), 0, 1, 95).to(memory_format=torch.channels_last_3d)
    g = gen.normal((c,), 1, 0.05, 96, "f32_bf16vals")
    b = gen.normal((c,), 0, 0.05, 97, "f32")
    out = gpu.rmsnorm_silu_bias(xt.cuda(), g.cuda(), b.cuda(), 1e-6)
    torch.cuda.synchronize()
    assert out.is_contiguous(memory_format=torch.channels_last_3d)
    rows = gen.to_u16(xt.permute(0, 2, 3, 4, 1).reshape(-1, c).contiguous())
    ref = orc.rmsnorm_silu_bias(rows, b.numpy(), g.numpy(), 1e-6)["out"]
    got = gen.to_u16(out.permute(0, 2, 3, 4, 1).reshape(-1, c).contiguous())
    assert np.all(ulp_diff(got, ref) <= 1)
    with pytest.raises(ValueError):
        gpu.rmsnorm_silu_bias(xt.contiguous().cuda(), g.cuda(), b.cuda())  # NCDHW rejected


@pytest.mark.parametrize("rows,c,res", [(1, 96, False), (1000, 96, True), (777, 384, True),
                                        (3, 8, False), (12345, 40, True), (5, 4096, True),
                                        (333, 200, False), (64, 1000, True)])
def test_conv_bias_epilogue(gpu, orc, rows, c, res):
    log(f"conv_bias_epilogue rows={rows} C={c} residual={res}")
    x = rand((rows, c), 0, 1, 101)
    h = rand((rows, c), 0, 1, 102) if res else None
    b = gen.normal((c,), 0, 0.05, 103, "f32").numpy()
    out = gpu.conv_bias_epilogue(dev(x), dev(b), None if h is None else dev(h))
    torch.cuda.synchronize()
    assert same_bits(host(out), orc.conv_bias_epilogue(x, b, h))


_TD = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _epi_case(dtype, bias_dtype, rows, c, seed):
    """x, h ~N(0,1) of the storage type with special values planted (signed
    zeros, subnormals, infinities, a NaN, the largest finite magnitude, so
    that adding the bias overflows); bias ~N(0, 0.05), fp32 or of x's type."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((rows, c), generator=g).to(_TD[dtype])
    h = torch.randn((rows, c), generator=g).to(_TD[dtype])
    fi = torch.finfo(_TD[dtype])
    sp = torch.tensor([0.0, -0.0, fi.smallest_normal / 4, -fi.smallest_normal / 4, fi.max,
                       -fi.max, float("inf"), float("-inf"), float("nan")]).to(_TD[dtype])
    n = min(sp.numel(), rows * c)
    x.view(-1)[:n] = sp[:n]
    h.view(-1)[-n:] = sp[:n]
    b = (torch.randn(c, generator=g) * 0.05).to(_TD[bias_dtype])
    return x, h, b


def _np(t, dt):
    return t.numpy() if dt == "f32" else gen.to_u16(t)


@pytest.mark.parametrize("dtype,bias_dtype", [("bf16", "f32"), ("bf16", "bf16"), ("f16", "f32"),
                                              ("f16", "f16"), ("f32", "f32")])
@pytest.mark.parametrize("rows,c,res", [(1, 8, False), (777, 96, True), (1001, 384, True),
                                        (333, 200, False), (5, 4096, True), (12345, 40, True)])
def test_conv_bias_epilogue_dtypes(gpu, orc, dtype, bias_dtype, rows, c, res):
    """Wan VAE page (Tests / docs: bf16 / fp16 / fp32 x with an fp32 or
    half-precision bias, with and without the residual): every storage type
    bitwise equal to the oracle, special values and ragged vector counts
    included."""
    log(f"conv_bias_epilogue {dtype}/{bias_dtype} rows={rows} C={c} residual={res}")
    x, h, b = _epi_case(dtype, bias_dtype, rows, c, 2100 + c + rows)
    out = gpu.conv_bias_epilogue(x.cuda(), b.cuda(), h.cuda() if res else None)
    torch.cuda.synchronize()
    ref = orc.conv_bias_epilogue_dt(_np(x, dtype), _np(b, bias_dtype),
                                    _np(h, dtype) if res else None, dtype, bias_dtype)
    got = out.cpu()
    if dtype == "f32":
        a, r = got.numpy(), ref
        assert np.array_equal(np.isnan(a), np.isnan(r))
        assert np.array_equal(a[~np.isnan(a)].view(np.uint32), r[~np.isnan(r)].view(np.uint32))
    else:
        assert same_bits(gen.to_u16(got), ref, dtype)


def test_conv_bias_epilogue_in_place_and_channels_last(gpu, orc):
    """out == x for fp16 and fp32, and a channels_last 5-D fp16 tensor."""
    for dt in ("f16", "f32"):
        x, h, b = _epi_case(dt, "f32", 300, 96, 2200)
        xd = x.cuda()
        ref = orc.conv_bias_epilogue_dt(_np(x, dt), b.numpy(), _np(h, dt), dt, "f32")
        out = gpu.conv_bias_epilogue(xd, b.cuda(), h.cuda(), out=xd)
        torch.cuda.synchronize()
        assert out.data_ptr() == xd.data_ptr()
        got = out.cpu()
        if dt == "f32":
            assert np.array_equal(np.nan_to_num(got.numpy(), nan=7.0), np.nan_to_num(ref, nan=7.0))
        else:
            assert same_bits(gen.to_u16(got), ref, dt)
    n, c, d, hh, w = 1, 96, 2, 6, 10
    xt = gen.normal((n, c, d, hh, w), 0, 1, 2201, "f16").to(memory_format=torch.channels_last_3d)
    b = gen.normal((c,), 0, 0.05, 2202, "f32")
    out = gpu.conv_bias_epilogue(xt.cuda(), b.cuda())
    torch.cuda.synchronize()
    assert out.is_contiguous(memory_format=torch.channels_last_3d)
    rows = gen.to_u16(xt.permute(0, 2, 3, 4, 1).reshape(-1, c).contiguous())
    got = gen.to_u16(out.permute(0, 2, 3, 4, 1).reshape(-1, c).contiguous())
    assert same_bits(got, orc.conv_bias_epilogue_dt(rows, b.numpy(), None, "f16", "f32"), "f16")


# ---------------------------------------------------------------------------
# every workload at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("key", list(WORKLOADS))
def test_full_workload(gpu, orc, key):
    w = WORKLOADS[key]
    log(f"full workload {key}")
    t = {k: (gen.to_u16(v) if v.dtype in (torch.bfloat16, torch.float16) else v.numpy())
         for k, v in gen.make(w).items()}
    for l in w.launches:
        log(f"  launch {l.name} rows={l.rows} cols={l.cols}")
        if l.entry == "ln_modulate":
            x, sc, sh = t["x"], t["scale"], t["shift"]
            out_fast, *_ = _ln_gpu(gpu, x, sc, sh, l.eps, debug=False)
            out, mean, rstd, y = _ln_gpu(gpu, x, sc, sh, l.eps)
            assert same_bits(out_fast, out), "debug outputs changed the result"
            ref = by_row_chunks(lambda lo, hi: orc.ln_modulate(x[lo:hi], sc, sh, l.eps), None,
                                x.shape[0])
            _ln_check(orc, f"{key}/{l.name}", x, sc, sh, l.eps, x.shape[0], out, mean, rstd, y,
                      ref=ref)
        elif l.entry == "ln_modulate_folded":
            x, sc, sh = t["x"], t["scale"], t["shift"]
            rows = x.shape[0]
            mean, rstd = empty_f32(rows), empty_f32(rows)
            out = host(gpu.ln_modulate_folded(dev(x), dev(sc), dev(sh), l.eps, mean_out=mean,
                                              rstd_out=rstd))
            torch.cuda.synchronize()
            ref = by_row_chunks(lambda lo, hi: orc.ln_modulate_folded(x[lo:hi], sc, sh, l.eps),
                                None, rows)
            check_stats(host(mean), host(rstd), ref["mean"], ref["rstd"], l.name)
            check_rows_end_to_end(out, ref["out"], l.name)
        elif l.entry == "gated_ln_modulate":
            upd, res, gate, sc, sh = (t[n] for n in ("update", "residual", "gate", "scale", "shift"))
            rows, cols = upd.shape
            _, out_fast = gpu.gated_ln_modulate(dev(upd), dev(res), dev(gate), dev(sc), dev(sh),
                                                l.eps)
            kw = dict(mean_out=empty_f32(rows), rstd_out=empty_f32(rows),
                      y_out=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda"))
            h, out = gpu.gated_ln_modulate(dev(upd), dev(res), dev(gate), dev(sc), dev(sh), l.eps,
                                           **kw)
            torch.cuda.synchronize()
            h, out = host(h), host(out)
            assert same_bits(host(out_fast), out), "debug outputs changed the result"
            ref = by_row_chunks(lambda lo, hi: orc.gated_ln_modulate(
                upd[lo:hi], res[lo:hi], gate, sc, sh, l.eps), None, rows)
            assert same_bits(h, ref["h"]), "gate stage"
            _ln_check(orc, f"{key}/{l.name}", h, sc, sh, l.eps, rows, out, host(kw["mean_out"]),
                      host(kw["rstd_out"]), host(kw["y_out"]), ref=ref)
        elif l.entry == "rms_modulate":
            gated = l.extra.get("gated", False)
            xn = "update" if gated else "x"
            _rms_run_check(gpu, orc, f"{key}/{l.name}", t[xn], t["weight"], t["scale"], t["shift"],
                           l.eps, t[xn].shape[0], t["residual"] if gated else None,
                           t["gate"] if gated else None)
        elif l.entry == "qk_layernorm":
            _qk_run_check(gpu, orc, f"{key}/{l.name}", t["q"], t["k"], l.eps)
        elif l.entry == "rmsnorm_silu_bias":
            _wan_run_check(gpu, orc, f"{key}/{l.name}", t["x"], t["bias"], t["gamma"], l.eps)
        elif l.entry == "conv_bias_epilogue":
            dt = l.extra.get("dtype", "bf16")
            td = torch.float16 if dt == "f16" else torch.bfloat16
            x, b, h = (t[n] for n in l.inputs)
            out = gpu.conv_bias_epilogue(dev(x, dtype=td), dev(b), dev(h, dtype=td))
            torch.cuda.synchronize()
            assert same_bits(host(out), orc.conv_bias_epilogue_dt(x, b, h, dt, "f32"), dt), l.name
        elif l.entry in ("modulate_scale_shift", "residual_gate_add"):
            dt = l.extra["dtype"]
            td = torch.float16 if dt == "f16" else torch.bfloat16
            a, b, c = (t[n] for n in l.inputs)
            if l.entry == "modulate_scale_shift":
                out = gpu.modulate_scale_shift(dev(a, dtype=td), dev(b, dtype=td), dev(c, dtype=td))
                ref = orc.modulate_dt(a, b, c, dt)
            else:
                out = gpu.residual_gate_add(dev(a, dtype=td), dev(b, dtype=td), dev(c, dtype=td))
                ref = orc.gate_residual_dt(a, b, c, dt)
            torch.cuda.synchronize()
            assert same_bits(host(out), ref, dt), l.name
        elif l.entry == "ln_modulate_backward":
            x, sc, dout = (t[n] for n in l.inputs)
            rpb = l.extra["rows_per_batch"]
            f32 = l.extra.get("dtype") == "f32"
            rows, cols = x.shape
            mean, rstd = empty_f32(rows), empty_f32(rows)
            # outputs start as NaN: no value may survive from a reused buffer
            nan, nb = float("nan"), rows // rpb
            d_x = torch.full((rows, cols), nan, dtype=torch.float32 if f32 else torch.bfloat16,
                             device="cuda")
            d_scale = torch.full((nb, cols), nan, dtype=torch.float32, device="cuda")
            d_shift = torch.full((nb, cols), nan, dtype=torch.float32, device="cuda")
            d_x, d_scale, d_shift = gpu.ln_modulate_backward(dev(x), dev(sc), dev(dout), l.eps,
                                                             d_x=d_x, d_scale=d_scale,
                                                             d_shift=d_shift, mean_out=mean,
                                                             rstd_out=rstd)
            torch.cuda.synchronize()
            ref = (orc.ln_modulate_backward_f32 if f32 else orc.ln_modulate_backward)(
                x, sc, dout, l.eps, rows_per_batch=rpb)
            check_stats(host(mean), host(rstd), ref["mean"], ref["rstd"], l.name)
            if f32:
                a, r = host(d_x).view(np.int32).astype(np.int64), ref["d_x"].view(np.int32).astype(np.int64)
                a = np.where(a < 0, -(a & 0x7FFFFFFF), a)
                r = np.where(r < 0, -(r & 0x7FFFFFFF), r)
                d = np.abs(a - r)
            else:
                d = ulp_diff(host(d_x), ref["d_x"])
            assert d.max() <= 1 and (d == 0).mean() >= 0.9999, l.name
            assert np.array_equal(host(d_shift), ref["d_shift"]), l.name
            assert np.array_equal(host(d_scale), ref["d_scale"]), l.name
        else:
            raise KeyError(l.entry)


# ---------------------------------------------------------------------------
# invariance and determinism
# ---------------------------------------------------------------------------

def test_row_position_batch_and_chunking_invariance(gpu, orc):
    """A row's result does not depend on where it sits, how many rows are
    launched with it (grid size), the batch split, or repeated runs."""
    cols = 3072
    x = rand((2 * 257, cols), 0, 1.5, 111)
    sc, sh = rand((1, cols), 0, 0.1, 112), rand((1, cols), 0, 0.1, 113)
    full, *_ = _ln_gpu(gpu, x, sc, sh, 1e-6, debug=False)
    again, *_ = _ln_gpu(gpu, x, sc, sh, 1e-6, debug=False)
    assert np.array_equal(full, again), "not deterministic"
    for lo, hi in [(0, 1), (5, 6), (513, 514), (31, 32 + 31), (100, 357), (0, 257), (257, 514)]:
        part, *_ = _ln_gpu(gpu, x[lo:hi], sc, sh, 1e-6, debug=False)
        assert np.array_equal(part, full[lo:hi]), (lo, hi)
    # B = 2 with equal modulation rows == B = 1
    sc2, sh2 = np.repeat(sc, 2, 0), np.repeat(sh, 2, 0)
    b2, *_ = _ln_gpu(gpu, x, sc2, sh2, 1e-6, debug=False)
    assert np.array_equal(b2, full)
    # qk: a head row alone vs inside a large launch
    q = rand((4096, 128), 0, 2, 114)
    qa, _ = gpu.qk_layernorm(dev(q), None)
    q1, _ = gpu.qk_layernorm(dev(q[1234:1235]), None)
    torch.cuda.synchronize()
    assert np.array_equal(host(qa)[1234:1235], host(q1))
    # wan: ragged pixel groups
    xw = rand((1000, 96), 0, 1, 115)
    g = gen.normal((96,), 1, 0.05, 116, "f32_bf16vals")
    b = gen.normal((96,), 0, 0.05, 117, "f32")
    wa = gpu.rmsnorm_silu_bias(dev(xw), g.cuda(), b.cuda())
    w1 = gpu.rmsnorm_silu_bias(dev(xw[999:1000]), g.cuda(), b.cuda())
    w7 = gpu.rmsnorm_silu_bias(dev(xw[3:10]), g.cuda(), b.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(host(wa)[999:1000], host(w1))
    assert np.array_equal(host(wa)[3:10], host(w7))


@pytest.mark.parametrize("cols,rows,lo", [(3072, 1024 + 300, 1024),   # halves
                                           (4096, 1024 + 16, 1024),    # quarters
                                           (2048, 2048 + 200, 2048),   # quarters
                                           # quarters first in the grid (gated forms),
                                           # 8-wavefront workgroups (plain RMS)
                                           (4096, 4096 + 120, 4096)])
@pytest.mark.parametrize("kind", ["ln", "gated_ln", "rms", "gated_rms"])
def test_split_rows_equal_whole_rows(gpu, kind, cols, rows, lo):
    """The balanced launch computes the rows past the whole rounds as half or
    quarter rows; in a launch of 700 rows (more than half a round of the 1024
    SIMDs, less than a whole one) every row runs whole, one wavefront each;
    in a launch of at most half a round every row is split again.  Every
    output and statistic is bitwise the same in all three (the segments'
    binary64 moment sums are exact)."""
    log(f"split vs whole {kind} rows={rows} cols={cols}")
    x = rand((rows, cols), 0.1, 1.5, 1300 + cols)
    res = rand((rows, cols), 0, 1, 1301 + cols)
    sc, sh, gt = (dev(rand((1, cols), 0, 0.1, 1302 + i)) for i in range(3))
    w = dev(rand((cols,), 1, 0.05, 1305))

    def run(a, b):
        n = b - a
        rstd = empty_f32(n)
        xd, rd = dev(x[a:b]), dev(res[a:b])
        if kind == "ln":
            mean = empty_f32(n)
            outs = [gpu.ln_modulate(xd, sc, sh, 1e-6, mean_out=mean, rstd_out=rstd), mean]
        elif kind == "gated_ln":
            mean = empty_f32(n)
            outs = [*gpu.gated_ln_modulate(xd, rd, gt, sc, sh, 1e-6, mean_out=mean,
                                           rstd_out=rstd), mean]
        elif kind == "rms":
            outs = [gpu.rms_modulate(xd, w, sc, sh, 1e-6, rstd_out=rstd)]
        else:
            outs = list(gpu.rms_modulate(xd, w, sc, sh, 1e-6, residual=rd, gate=gt,
                                         rstd_out=rstd))
        torch.cuda.synchronize()
        return [host(t) for t in outs + [rstd]]

    full = run(0, rows)
    for a, b in [(lo, rows), (rows - 1, rows), (lo - 3, lo + 5)]:
        w0 = b - 700  # a whole-row launch holding rows a:b
        whole = run(w0, b)
        small = run(a, b)  # at most half a round: split rows
        for f, wh, sm in zip(full, whole, small):
            got = np.asarray(f)[a:b].view(np.uint8)
            assert np.array_equal(got, np.asarray(wh)[a - w0:].view(np.uint8)), \
                f"{kind}: rows {a}:{b} differ between the split and the whole-row launch"
            assert np.array_equal(got, np.asarray(sm).view(np.uint8)), \
                f"{kind}: rows {a}:{b} differ between the large and the small launch"


def test_max_rows(gpu, orc):
    """The largest row count a call takes (2^25 - 1 rows; a launch of 4-row
    workgroups then holds 2^31 work-items), with 8-column rows: sampled rows,
    the first and the last among them, equal the oracle's."""
    rows, cols = (1 << 25) - 1, 8
    log(f"max rows: {rows} x {cols}")
    g = torch.Generator(device="cuda").manual_seed(1400)
    x = torch.randn((rows, cols), generator=g, device="cuda").to(torch.bfloat16)
    sc = dev(rand((1, cols), 0, 0.1, 1401))
    sh = dev(rand((1, cols), 0, 0.1, 1402))
    w = dev(rand((cols,), 1, 0.05, 1403))
    idx = torch.cat([torch.arange(0, 64, device="cuda"),
                     torch.randint(0, rows, (4096,), generator=g, device="cuda"),
                     torch.arange(rows - 64, rows, device="cuda")])
    xs = host(x[idx])
    out = gpu.ln_modulate(x, sc, sh, 1e-6)
    torch.cuda.synchronize()
    ref = orc.ln_modulate(xs, host(sc), host(sh), 1e-6)
    assert same_bits(host(out[idx]), ref["out"])
    del out
    out = gpu.rms_modulate(x, w, sc, sh, 1e-6)
    torch.cuda.synchronize()
    ref = orc.rms_modulate(xs, host(w), host(sc), host(sh), 1e-6)
    assert same_bits(host(out[idx]), ref["out"])


def test_max_rows_qk_and_wan(gpu, orc):
    """qk_layernorm at the largest total of head rows (2^25 - 1: 2^24 of q,
    the rest of k) and rmsnorm_silu_bias at the largest pixel count with
    C = 96 (its tuned two-group layout); sampled rows against the oracle."""
    n = (1 << 25) - 1
    g = torch.Generator(device="cuda").manual_seed(1500)

    def sample(rows):
        return torch.cat([torch.arange(0, 64, device="cuda"),
                          torch.randint(0, rows, (2048,), generator=g, device="cuda"),
                          torch.arange(rows - 64, rows, device="cuda")])

    rq = 1 << 24
    log(f"max rows qk: {rq} + {n - rq}")
    q = torch.empty((rq, 128), dtype=torch.bfloat16, device="cuda").normal_(0, 2, generator=g)
    k = torch.empty((n - rq, 128), dtype=torch.bfloat16, device="cuda").normal_(0, 2, generator=g)
    qo, ko = gpu.qk_layernorm(q, k, 1e-5)
    torch.cuda.synchronize()
    iq, ik = sample(rq), sample(n - rq)
    ref = orc.qk_layernorm(host(q[iq]), host(k[ik]), 1e-5)
    assert same_bits(host(qo[iq]), ref["q_out"]) and same_bits(host(ko[ik]), ref["k_out"])
    del q, k, qo, ko
    torch.cuda.empty_cache()

    log(f"max rows wan: {n} x 96")
    x = torch.empty((n, 96), dtype=torch.bfloat16, device="cuda").normal_(0, 1, generator=g)
    b = gen.normal((96,), 0, 0.05, 1501, "f32")
    gm = gen.normal((96,), 1, 0.05, 1502, "f32_bf16vals")
    out = gpu.rmsnorm_silu_bias(x, gm.cuda(), b.cuda(), 1e-6)
    torch.cuda.synchronize()
    ix = sample(n)
    ref = orc.rmsnorm_silu_bias(host(x[ix]), b.numpy(), gm.numpy(), 1e-6)
    assert ulp_diff(host(out[ix]), ref["out"]).max() <= 1


def test_binding_rejects_mismatched_tensors(gpu):
    """The library cannot see allocation sizes: the binding refuses, before any
    launch, outputs and companion inputs whose shape differs from the input's,
    fp32 outputs in host memory, and tensors on another device type."""
    x = torch.zeros((8, 1024), dtype=torch.bfloat16, device="cuda")
    s = torch.zeros((1, 1024), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((1024,), dtype=torch.bfloat16, device="cuda")
    small = torch.empty((4, 1024), dtype=torch.bfloat16, device="cuda")
    cases = [
        lambda: gpu.ln_modulate(x, s, s, out=small),
        lambda: gpu.ln_modulate(x, s, s, y_out=small),
        lambda: gpu.ln_modulate(x, s, s, mean_out=torch.empty(8, dtype=torch.float32)),
        lambda: gpu.ln_modulate_folded(x, s, s, out=small),
        lambda: gpu.gated_ln_modulate(x, small, s, s, s),
        lambda: gpu.gated_ln_modulate(x, x, s, s, s, residual_out=small),
        lambda: gpu.rms_modulate(x, w, s, s, out=small),
        lambda: gpu.rms_modulate(x, w.cpu(), s, s),
        lambda: gpu.rms_modulate(x, w, s, s, residual=small, gate=s),
        lambda: gpu.qk_layernorm(x.view(-1, 128), None, q_out=small.view(-1, 128)),
        lambda: gpu.modulate_scale_shift(x, s, s, out=small),
        lambda: gpu.residual_gate_add(x, small, s),
        lambda: gpu.ln_modulate_backward(x, s, small),
        lambda: gpu.ln_modulate_backward(x, s, x, d_scale=torch.empty((1, 1024))),
        lambda: gpu.copy(x, small),
    ]
    for i, call in enumerate(cases):
        with pytest.raises((ValueError, TypeError)):
            call()
    torch.cuda.synchronize()


@pytest.mark.parametrize("cols", [1024, 2048, 3072, 4096])
def test_every_launch_partition(gpu, orc, cols):
    """The balanced launch picks whole, half or quarter rows from the row count
    alone (rounds of the 1024 SIMDs, the remainder, small launches): row counts
    across every boundary of that choice give the oracle's bits."""
    n_max = 2100
    x = rand((n_max, cols), 0.1, 1.5, 1700 + cols)
    sc, sh = rand((1, cols), 0, 0.1, 1701), rand((1, cols), 0, 0.1, 1702)
    ref = orc.ln_modulate(x, sc, sh, 1e-6)["out"]
    rng = np.random.default_rng(cols)
    counts = set(range(1, 65))
    for b in (256, 512, 768, 1024, 1280, 1536, 1792, 2048):
        counts |= {b - 1, b, b + 1}
    counts |= set(int(v) for v in rng.integers(65, n_max + 1, 40))
    xd, scd, shd = dev(x), dev(sc), dev(sh)
    for n in sorted(counts):
        out = gpu.ln_modulate(xd[:n], scd, shd, 1e-6)
        torch.cuda.synchronize()
        assert same_bits(host(out), ref[:n]), f"{n} rows of {cols}"


@pytest.mark.parametrize("c", [96, 384])
def test_every_pixel_partition(gpu, orc, c):
    """rmsnorm_silu_bias takes pixels in groups (16 at C = 96, 4 at C = 384), two
    groups per wavefront and four wavefronts per workgroup: pixel counts across
    those boundaries give the oracle's bias stage and rstd bits and its SiLU
    output within 1 ulp."""
    n_max = 700
    x = rand((n_max, c), 0, 1, 1800 + c)
    b = gen.normal((c,), 0, 0.05, 1801, "f32")
    g = gen.normal((c,), 1, 0.05, 1802, "f32_bf16vals")
    ref = orc.rmsnorm_silu_bias(x, b.numpy(), g.numpy(), 1e-6)
    counts = set(range(1, 70))
    for m in (128, 256, 512):
        counts |= {m - 1, m, m + 1}
    counts.add(n_max)
    xd, bd, gd = dev(x), b.cuda(), g.cuda()
    for n in sorted(counts):
        rstd = empty_f32(n)
        xb = torch.empty((n, c), dtype=torch.bfloat16, device="cuda")
        out = gpu.rmsnorm_silu_bias(xd[:n], gd, bd, 1e-6, rstd_out=rstd, xb_out=xb)
        torch.cuda.synchronize()
        assert same_bits(host(xb), ref["xb"][:n]), f"{n} pixels: bias stage"
        assert np.array_equal(host(rstd).view(np.uint32), ref["rstd"][:n].view(np.uint32)), \
            f"{n} pixels: rstd"
        assert ulp_diff(host(out), ref["out"][:n]).max() <= 1, f"{n} pixels: out"


def test_every_qk_partition(gpu, orc):
    """qk_layernorm numbers q's head rows, then k's, 8 to a wavefront
    instruction and 32 to a workgroup, so groups straddle the q/k boundary at
    most counts: q and k counts around those boundaries against the oracle."""
    q = rand((80, 128), 0, 2, 1900)
    k = rand((80, 128), 0.5, 2, 1901)
    qd, kd = dev(q), dev(k)
    for rq in list(range(1, 41)) + [63, 64, 65, 80]:
        for rk in (0, 1, 7, 8, 9, 31, 32, 33, 80):
            qo, ko = gpu.qk_layernorm(qd[:rq], kd[:rk] if rk else None, 1e-5)
            torch.cuda.synchronize()
            ref = orc.qk_layernorm(q[:rq], k[:rk], 1e-5)
            assert same_bits(host(qo), ref["q_out"]), (rq, rk)
            if rk:
                assert same_bits(host(ko), ref["k_out"]), (rq, rk)


def test_rejections_raise(gpu):
    x = torch.zeros((4, 1024), dtype=torch.bfloat16, device="cuda")
    s = torch.zeros((1, 1024), dtype=torch.bfloat16, device="cuda")
    x1000 = torch.zeros((4, 1004), dtype=torch.bfloat16, device="cuda")
    s1000 = torch.zeros((1, 1004), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu.DitnormError) as e:
        gpu.ln_modulate(x1000, s1000, s1000)                       # cols % 8 != 0
    assert e.value.status == gpu.UNSUPPORTED
    with pytest.raises(gpu.DitnormError) as e:
        gpu.ln_modulate(x, s, s, eps=float("nan"))
    assert e.value.status == gpu.INVALID_ARGUMENT
    buf = torch.zeros(4 * 1024 + 64, dtype=torch.bfloat16, device="cuda")
    xv = buf[:4096].view(4, 1024)
    with pytest.raises(gpu.DitnormError) as e:                      # partial overlap
        gpu.ln_modulate(xv, s, s, out=buf[8:8 + 4096].view(4, 1024))
    assert e.value.status == gpu.UNSUPPORTED
    with pytest.raises(gpu.DitnormError) as e:                      # misaligned (4 bytes)
        gpu.ln_modulate(buf[2:2 + 3072].view(3, 1024), s, s,
                        out=torch.empty((3, 1024), dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == gpu.UNSUPPORTED


# ---------------------------------------------------------------------------
# the balanced launch: whole rows for whole rounds of the 1024 SIMDs, the
# remainder as half rows (two wavefronts per row, moments through LDS) or, for
# rows of 2048 or 4096 columns and a remainder of at most a quarter round, as
# quarter rows (a workgroup per row)
# ---------------------------------------------------------------------------

SPLIT_CASES = [(3072, 4096 + 512, 4096 + 512), (3072, 1024 + 1, 1025), (4096, 2048 + 257, 2305),
               (1024, 4096 + 3, 4099), (2048, 3072 + 511, 3583), (3072, 4096 + 256, 17),
               # quarters
               (4096, 1024 + 120, 1144), (2048, 2048 + 256, 2304), (4096, 1024 + 16, 13),
               (4096, 4096 + 1, 4097),
               # quarters at 4096 columns: the gated forms' remainder dispatched first
               # (at least 64 rows), batch boundaries inside its workgroups
               (4096, 4096 + 120, 17), (4096, 2048 + 256, 9), (4096, 1024 + 255, 1279),
               (4096, 1024 + 63, 1087),
               # the plain RMS form in 8-wavefront workgroups (at least four whole
               # rounds): eighths (a row per workgroup) up to an eighth of a round,
               # quarters past it, halves, every row whole with a partly live last
               # workgroup, and only whole rounds; with exactly four whole rounds
               # the eighths and quarters ride in the whole-row workgroups (two
               # quarter rows per workgroup, batch boundaries among them), with
               # five they keep workgroups of their own
               (4096, 8192 + 100, 12), (4096, 4096 + 128, 8), (4096, 4096 + 129, 13),
               (4096, 4096 + 300, 7), (4096, 4096 + 700, 11), (4096, 4096, 64),
               (4096, 4096 + 250, 41), (4096, 5120 + 100, 10)]


@pytest.mark.parametrize("cols,rows,rpb", SPLIT_CASES)
@pytest.mark.parametrize("kind", ["ln", "gated_ln", "rms", "gated_rms"])
def test_balanced_split_rows(gpu, orc, cols, rows, rpb, kind):
    """Row counts with a remainder of at most half a round take the half-row
    path (batch boundaries fall inside half-row workgroups at rpb = 17), at
    most a quarter round of 2048 or 4096 columns the quarter-row path, and in
    the plain RMS form's 8-wavefront workgroups at most an eighth of a round
    the eighth-row path."""
    log(f"balanced {kind} rows={rows} cols={cols} rpb={rpb}")
    B = rows // rpb
    x = rand((rows, cols), 0.2, 1.5, 1100 + cols + rows)
    emb = rand((B, 6 * cols), 0, 0.1, 1101 + B)
    embd = dev(emb)
    sc_d, sh_d, g_d = embd[:, cols:2 * cols], embd[:, 0:cols], embd[:, 2 * cols:3 * cols]
    sc = np.concatenate([emb.ravel()[cols:], np.zeros(cols, np.uint16)]).reshape(B, 6 * cols)
    gt = np.concatenate([emb.ravel()[2 * cols:], np.zeros(2 * cols, np.uint16)]).reshape(B, 6 * cols)
    mean, rstd = empty_f32(rows), empty_f32(rows)
    y = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    if kind in ("ln", "gated_ln"):
        if kind == "ln":
            xin = x
            out = gpu.ln_modulate(dev(x), sc_d, sh_d, 1e-6, mean_out=mean, rstd_out=rstd, y_out=y)
        else:
            res = rand((rows, cols), 0, 1, 1102)
            h, out = gpu.gated_ln_modulate(dev(x), dev(res), g_d, sc_d, sh_d, 1e-6, mean_out=mean,
                                           rstd_out=rstd, y_out=y)
            torch.cuda.synchronize()
            xin = orc.gate_residual(x, res, gt, rows_per_batch=rpb)
            assert same_bits(host(h), xin), "gate stage"
        torch.cuda.synchronize()
        ref = orc.ln_modulate(xin, sc, emb, 1e-6, rows_per_batch=rpb)
        _ln_check(orc, f"balanced {kind}", xin, sc, emb, 1e-6, rpb, host(out), host(mean),
                  host(rstd), host(y), ref=ref)
    else:
        w = rand((cols,), 1, 0.05, 1103)
        res = rand((rows, cols), 0, 1, 1104) if kind == "gated_rms" else None
        _rms_run_check(gpu, orc, f"balanced {kind}", x, w, sc, emb, 1e-6, rpb, res,
                       gt if res is not None else None, mod_dev=(sc_d, sh_d, g_d))
