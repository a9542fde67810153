"""GPU parity of ln_modulate_backward (the backward of LN + modulate with the
fixed fp32 token-sum trees) against the oracle: statistics within the
2e-6 bar (in practice bit-identical), d_scale / d_shift bit-identical when the
statistics are (the same fp32 terms through the same tree), d_x a single
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
    rows = x.shape[0]
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    scd = dev(sc) if mod_dev is None else mod_dev
    d_x, d_scale, d_shift = dn.ln_modulate_backward(dev(x), scd, dev(dout), eps,
                                                    mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    return dict(d_x=host(d_x), d_scale=host(d_scale), d_shift=host(d_shift), mean=host(mean),
                rstd=host(rstd))


def check(got, ref, x, sc, dout, rpb, what):
    differ = check_stats(got["mean"], got["rstd"], ref["mean"], ref["rstd"], what)
    # d_x: the same binary64 value rounded once on both sides
    d = ulp_diff(got["d_x"], ref["d_x"])
    exact = (d == 0).mean()
    log(f"  {what}: d_x exact on {exact:.6f} of elements, max {int(d.max())} ulp; "
        f"{int(differ.sum())} rows with last-bit stats differences")
    assert d.max() <= 1 and exact >= 0.9999, f"{what}: d_x"
    # token sums: the same fp32 terms through the same tree
    if not differ.any():
        assert np.array_equal(got["d_shift"], ref["d_shift"]), f"{what}: d_shift"
        assert np.array_equal(got["d_scale"], ref["d_scale"]), f"{what}: d_scale"
    else:
        for k in ("d_shift", "d_scale"):
            assert np.allclose(got[k], ref[k], rtol=1e-5, atol=1e-5), f"{what}: {k}"


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
