"""GPU parity of ln_modulate_backward (the backward of LN + modulate with the
fixed fp32 token-sum trees) against the oracle: statistics within the
2e-6 bar and bit-identical (both sides sum exactly), d_scale / d_shift
bit-identical (the same fp32 terms through the same tree), d_x a single
rounding of the same binary64 value (bit-identical but for values within
~1e-16 of a rounding boundary), batch invariance and determinism bitwise.

Shapes span one token, ragged groups of 32, several tree levels (up to three
extra levels at 40000 tokens), many small batches, and the Qwen-Image final
stream (1, 6889, 3072)."""
import numpy as np
import pytest
import torch

import dit_adaln_row_amd as dn
from dit_adaln_row_amd import inputs as gen
from parity import check_stats, dev, host, log, ulp_diff

pytestmark = pytest.mark.gpu


def rand(shape, mu, sigma, seed):
    return gen.to_u16(gen.normal(shape, mu, sigma, seed))


def run(x, sc, dout, rpb, eps=1e-6, mod_dev=None):
    """The outputs start as NaN, so that a sum the kernels leave unwritten
    (or a value an earlier call left in a reused buffer) cannot pass."""
    rows, cols = x.shape
    nb = rows // rpb
    nan = float("nan")
    mean = torch.full((rows,), nan, dtype=torch.float32, device="cuda")
    rstd = torch.full((rows,), nan, dtype=torch.float32, device="cuda")
    d_x = torch.full((rows, cols), nan, dtype=torch.bfloat16, device="cuda")
    d_scale = torch.full((nb, cols), nan, dtype=torch.float32, device="cuda")
    d_shift = torch.full((nb, cols), nan, dtype=torch.float32, device="cuda")
    scd = dev(sc) if mod_dev is None else mod_dev
    d_x, d_scale, d_shift = dn.ln_modulate_backward(dev(x), scd, dev(dout), eps, d_x=d_x,
                                                    d_scale=d_scale, d_shift=d_shift,
                                                    mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    return dict(d_x=host(d_x), d_scale=host(d_scale), d_shift=host(d_shift), mean=host(mean),
                rstd=host(rstd))


def check(got, ref, x, sc, dout, rpb, what):
    check_stats(got["mean"], got["rstd"], ref["mean"], ref["rstd"], what)
    # d_x: the same binary64 value rounded once on both sides
    d = ulp_diff(got["d_x"], ref["d_x"])
    exact = (d == 0).mean()
    log(f"  {what}: d_x exact on {exact:.6f} of elements, max {int(d.max())} ulp")
    assert d.max() <= 1 and exact >= 0.9999, f"{what}: d_x"
    # token sums: the same fp32 terms (d_out, and d_out * x_hat from the
    # oracle's statistics bits, asserted above) through the same tree
    assert np.array_equal(got["d_shift"], ref["d_shift"]), f"{what}: d_shift"
    assert np.array_equal(got["d_scale"], ref["d_scale"]), f"{what}: d_scale"


# Token counts around the kernels' structure: a batch of at most 8 tokens (4
# over 3072 columns) in one workgroup and one launch (1, 3, 4, 5, 8), runs of
# 8 / 4 tokens folded by 4 / 8 within one 32-token group (9, 16, 32; 4-token
# runs for launches that 8-token workgroups would leave under half the chip,
# 8-token runs with many batches), one level of 128 / 256 runs (33, 1024,
# 1025, 2500, 8192), several levels (8193, 9000, 40000, 1.1M), ragged column
# counts (40, 1000, 3080) and 4096 columns.
SHAPES = [(1, 1, 8), (1, 5, 40), (1, 32, 1024), (1, 33, 1024), (2, 77, 1024), (1, 1025, 512),
          (3, 100, 3072), (2048, 3, 64), (1, 40000, 64), (4, 257, 4096), (1, 300, 1000),
          (3, 4, 3072), (2, 8, 3072), (2, 9, 3072), (5, 16, 4096), (3, 5, 4096),
          (2, 1024, 3072), (1, 9000, 3080), (1, 8192, 256), (1, 8193, 64), (2, 2500, 4096),
          (1, 1100000, 8),  # four tree launches after the fused pass
          (64, 32, 1024), (150, 9, 1024)]  # 8-token runs within one group, many batches


@pytest.mark.parametrize("B,S,D", SHAPES)
def test_backward_shapes(gpu, orc, B, S, D):
    log(f"ln_modulate_backward B={B} S={S} D={D}")
    x = rand((B * S, D), 0.2, 1.5, 900 + D + S)
    sc = rand((B, D), 0, 0.1, 901 + B)
    dout = rand((B * S, D), 0, 1.0, 902 + S)
    got = run(x, sc, dout, S)
    ref = orc.ln_modulate_backward(x, sc, dout, 1e-6, rows_per_batch=S)
    check(got, ref, x, sc, dout, S, f"bwd {B}x{S}x{D}")


# On both sides of the switch between 4- and 8-token workgroups (at most 128
# eight-token workgroups take 4-token ones), for long and short batches.
BOUNDARY = [(1, 1024, 3072), (1, 1025, 3072), (16, 64, 1024), (16, 65, 1024),
            (42, 24, 3072), (43, 24, 3072), (128, 9, 2048), (8, 129, 3072)]


@pytest.mark.parametrize("B,S,D", BOUNDARY)
def test_backward_workgroup_switch(gpu, orc, B, S, D):
    log(f"ln_modulate_backward boundary B={B} S={S} D={D}")
    x = rand((B * S, D), 0.2, 1.5, 970 + S)
    sc = rand((B, D), 0, 0.1, 971 + B)
    dout = rand((B * S, D), 0, 1.0, 972 + D)
    got = run(x, sc, dout, S)
    ref = orc.ln_modulate_backward(x, sc, dout, 1e-6, rows_per_batch=S)
    check(got, ref, x, sc, dout, S, f"bwd boundary {B}x{S}x{D}")


def test_backward_max_rows(gpu, orc):
    """The most tokens a call takes: 2^25 - 8 tokens in one batch (4194303
    eight-token workgroups of 512 work-items, 2^31 - 512 in all), 8 columns."""
    S, D = (1 << 25) - 8, 8
    log(f"ln_modulate_backward max rows: 1x{S}x{D}")
    x = rand((S, D), 0.2, 1.5, 960)
    sc = rand((1, D), 0, 0.1, 961)
    dout = rand((S, D), 0, 1.0, 962)
    got = run(x, sc, dout, S)
    ref = orc.ln_modulate_backward(x, sc, dout, 1e-6, rows_per_batch=S)
    check(got, ref, x, sc, dout, S, "bwd max rows")


def test_backward_chunk_view_scale(gpu, orc):
    """scale as a chunk view of a [B, 2*D] adaLN embedding, (scale, shift) order."""
    B, S, D = 3, 70, 3072
    x = rand((B * S, D), 0, 1.5, 910)
    emb = rand((B, 2 * D), 0, 0.1, 911)
    dout = rand((B * S, D), 0, 1, 912)
    got = run(x, None, dout, S, mod_dev=dev(emb)[:, 0:D])
    ref = orc.ln_modulate_backward(x, emb, dout, 1e-6, rows_per_batch=S)
    check(got, ref, x, emb, dout, S, "bwd chunk view")


def test_backward_batch_invariance_and_determinism(gpu, orc):
    S, D = 129, 3072
    xs = [rand((S, D), 0, 1.5, 920 + i) for i in range(3)]
    scs = [rand((1, D), 0, 0.1, 930 + i) for i in range(3)]
    ds = [rand((S, D), 0, 1, 940 + i) for i in range(3)]
    whole = run(np.concatenate(xs), np.concatenate(scs), np.concatenate(ds), S)
    again = run(np.concatenate(xs), np.concatenate(scs), np.concatenate(ds), S)
    for k in ("d_x", "d_scale", "d_shift"):
        assert np.array_equal(whole[k], again[k]), f"determinism {k}"
    for i in range(3):
        alone = run(xs[i], scs[i], ds[i], S)
        assert np.array_equal(alone["d_x"], whole["d_x"][i * S:(i + 1) * S])
        assert np.array_equal(alone["d_scale"][0].view(np.uint32), whole["d_scale"][i].view(np.uint32))
        assert np.array_equal(alone["d_shift"][0].view(np.uint32), whole["d_shift"][i].view(np.uint32))


# ---------------------------------------------------------------------------
# batch invariance as the Qwen-Image page checks it ("[WS1][Qwen-Image][CUDA]
# Final AdaLN output (final_adaln_out)", Prior art & reuse decision): bytewise,
# a singleton against every row of B = 64 / 257 / 2048, B = 2 against B = 1 at
# S = 31 / 32 / 33 / 4096 / 6032 / 6889, and one workload in five chunkings.
# ---------------------------------------------------------------------------

def _bwd_into(x, sc, dout, o, r0, r1, b0, b1):
    """Backward of rows [r0, r1) (batches [b0, b1)) written into slices of the
    output set o (device tensors)."""
    dn.ln_modulate_backward(x[r0:r1], sc[b0:b1], dout[r0:r1], 1e-6, d_x=o["d_x"][r0:r1],
                            d_scale=o["d_scale"][b0:b1], d_shift=o["d_shift"][b0:b1],
                            mean_out=o["mean"][r0:r1], rstd_out=o["rstd"][r0:r1])


def _out_set(B, S, D, fill):
    f32 = dict(dtype=torch.float32, device="cuda")
    return dict(d_x=torch.full((B * S, D), fill, dtype=torch.bfloat16, device="cuda"),
                d_scale=torch.full((B, D), fill, **f32), d_shift=torch.full((B, D), fill, **f32),
                mean=torch.full((B * S,), fill, **f32), rstd=torch.full((B * S,), fill, **f32))


def _bytes_equal(a, b, what):
    torch.cuda.synchronize()
    for k in a:
        ia = a[k].view(torch.int16 if a[k].dtype == torch.bfloat16 else torch.int32)
        ib = b[k].view(torch.int16 if b[k].dtype == torch.bfloat16 else torch.int32)
        assert torch.equal(ia, ib), f"{what}: {k} differs"


def _batched_inputs(B, S, D, seed):
    x = gen.normal((B * S, D), 0.2, 1.5, seed).cuda()
    sc = gen.normal((B, D), 0, 0.1, seed + 1).cuda()
    dout = gen.normal((B * S, D), 0, 1.0, seed + 2).cuda()
    return x, sc, dout


@pytest.mark.parametrize("B,seed", [(64, 0), (64, 127), (64, 2026), (257, 0), (2048, 0)])
def test_backward_singleton_vs_every_batch_row(gpu, B, seed):
    S, D = 3, 3072
    log(f"bwd singleton vs every row of B={B} (S={S}, seed {seed})")
    x, sc, dout = _batched_inputs(B, S, D, 5000 + seed)
    whole, alone = _out_set(B, S, D, float("nan")), _out_set(B, S, D, -3.0)
    _bwd_into(x, sc, dout, whole, 0, B * S, 0, B)
    for b in range(B):
        _bwd_into(x, sc, dout, alone, b * S, (b + 1) * S, b, b + 1)
    _bytes_equal(whole, alone, f"B={B}")


@pytest.mark.parametrize("S", [31, 32, 33, 4096, 6032, 6889])
def test_backward_two_batches_vs_one(gpu, S):
    D = 3072
    log(f"bwd B=2 vs B=1 at S={S}")
    x, sc, dout = _batched_inputs(2, S, D, 5100 + S)
    whole, alone = _out_set(2, S, D, float("nan")), _out_set(2, S, D, -3.0)
    _bwd_into(x, sc, dout, whole, 0, 2 * S, 0, 2)
    for b in range(2):
        _bwd_into(x, sc, dout, alone, b * S, (b + 1) * S, b, b + 1)
    _bytes_equal(whole, alone, f"S={S}")


def test_backward_workload_in_five_chunkings(gpu):
    B, S, D = 4096, 3, 3072
    x, sc, dout = _batched_inputs(B, S, D, 5200)
    chunkings = [[4096], [2048, 2048], [1, 4095], [1000, 1000, 2096], [257] * 15 + [241]]
    ref = None
    for parts in chunkings:
        log(f"bwd {B} samples in chunks {parts[:4]}{'...' if len(parts) > 4 else ''}")
        assert sum(parts) == B
        o = _out_set(B, S, D, float("nan"))
        b0 = 0
        for n in parts:
            _bwd_into(x, sc, dout, o, b0 * S, (b0 + n) * S, b0, b0 + n)
            b0 += n
        if ref is None:
            ref = o
        else:
            _bytes_equal(ref, o, f"chunking {parts[:4]}")


# ---------------------------------------------------------------------------
# the fp32 stream (Qwen-Image page: the FP32 column of the final stream's
# table, its BF16/FP32 accuracy gates)
# ---------------------------------------------------------------------------

def _f32_rand(shape, mu, sigma, seed):
    return gen.normal(shape, mu, sigma, seed, "f32").numpy()


def _ulp32(a, b):
    """Distance in fp32 ulps (ordered-integer difference)."""
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def check_f32(got, ref, what):
    check_stats(got["mean"], got["rstd"], ref["mean"], ref["rstd"], what)
    d = _ulp32(got["d_x"], ref["d_x"])
    log(f"  {what}: d_x exact on {(d == 0).mean():.6f} of elements, max {int(d.max())} ulp")
    assert d.max() <= 1 and (d == 0).mean() >= 0.9999, f"{what}: d_x"
    assert np.array_equal(got["d_shift"].view(np.uint32), ref["d_shift"].view(np.uint32)), what
    assert np.array_equal(got["d_scale"].view(np.uint32), ref["d_scale"].view(np.uint32)), what


def run_f32(x, sc, dout, eps=1e-6):
    rows = x.shape[0]
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    d_x, d_scale, d_shift = dn.ln_modulate_backward(dev(x), dev(sc), dev(dout), eps,
                                                    mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    return dict(d_x=host(d_x), d_scale=host(d_scale), d_shift=host(d_shift), mean=host(mean),
                rstd=host(rstd))


# one token, batches of at most 4 tokens (one launch), runs of 4 within a
# 32-token group, one and two tree levels, ragged columns, the vector-count
# forms (64, 128, 256, 512, 768 vectors of 4) and many small batches
F32_SHAPES = [(1, 1, 8), (3, 4, 3072), (2, 5, 40), (1, 32, 1024), (1, 33, 3072), (2, 77, 1000),
              (1, 1025, 512), (2048, 3, 3072), (1, 6889, 3072), (1, 9000, 2048), (5, 16, 256),
              (64, 9, 1536), (1, 300, 3064)]


@pytest.mark.parametrize("B,S,D", F32_SHAPES)
def test_backward_f32_shapes(gpu, orc, B, S, D):
    log(f"ln_modulate_backward fp32 B={B} S={S} D={D}")
    x = _f32_rand((B * S, D), 0.2, 1.5, 960 + D + S)
    sc = _f32_rand((B, D), 0, 0.1, 961 + B)
    dout = _f32_rand((B * S, D), 0, 1.0, 962 + S)
    got = run_f32(x, sc, dout)
    ref = orc.ln_modulate_backward_f32(x, sc, dout, 1e-6, rows_per_batch=S)
    check_f32(got, ref, f"bwd f32 {B}x{S}x{D}")


@pytest.mark.parametrize("S", [31, 32, 33, 6889])
def test_backward_f32_two_batches_vs_one(gpu, S):
    D = 3072
    x = _f32_rand((2 * S, D), 0.2, 1.5, 970 + S)
    sc = _f32_rand((2, D), 0, 0.1, 971)
    dout = _f32_rand((2 * S, D), 0, 1.0, 972 + S)
    whole = run_f32(x, sc, dout)
    for b in range(2):
        alone = run_f32(x[b * S:(b + 1) * S], sc[b:b + 1], dout[b * S:(b + 1) * S])
        assert np.array_equal(alone["d_x"].view(np.uint32),
                              whole["d_x"][b * S:(b + 1) * S].view(np.uint32))
        for k in ("d_scale", "d_shift"):
            assert np.array_equal(alone[k][0].view(np.uint32), whole[k][b].view(np.uint32))


def test_backward_f32_matches_bf16_stream_on_bf16_values(gpu):
    """fp32 inputs holding bf16 values: statistics and token sums bitwise the
    bf16 stream's, d_x rounded to bf16 within one ulp of it."""
    B, S, D = 3, 100, 3072
    x = rand((B * S, D), 0, 1.5, 980)
    sc = rand((B, D), 0, 0.1, 981)
    dout = rand((B * S, D), 0, 1.0, 982)
    rb = run(x, sc, dout, S)
    rf = run_f32(gen.f32_from_u16(x), gen.f32_from_u16(sc), gen.f32_from_u16(dout))
    for k in ("mean", "rstd", "d_shift", "d_scale"):
        assert np.array_equal(rb[k].view(np.uint32), rf[k].view(np.uint32)), k
    d = ulp_diff(gen.bf16_bits_from_f32(rf["d_x"]), rb["d_x"])
    assert d.max() <= 1 and (d == 0).mean() >= 0.9999


def test_backward_workspace_and_rejections(gpu):
    x = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    sc = torch.zeros((256,), dtype=torch.bfloat16, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(dn.DitnormError):
        dn.ln_modulate_backward(x, sc, x.clone(), workspace=small)
    wide = torch.zeros((4, 4104), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dn.DitnormError):
        dn.ln_modulate_backward(wide, torch.zeros(4104, dtype=torch.bfloat16, device="cuda"),
                                wide.clone())
    e = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    d_x, d_scale, d_shift = dn.ln_modulate_backward(e, sc, e)
    assert d_x.shape == (0, 256)
