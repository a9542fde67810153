"""GPU parity of the standalone elementwise entry points (modulate_scale_shift,
residual_gate_add) in bf16 and fp16 against the oracle's eager-chain
definitions, byte for byte: ragged row counts (the kernels give each thread
several rows), batch boundaries inside a thread's rows, adaLN chunk views,
every 16-bit input pattern, in-place calls, empty launches and the full
FLUX.1-sized activation."""
import numpy as np
import pytest
import torch

import dit_adaln_row_amd as dn
from dit_adaln_row_amd import inputs as gen
from parity import dev, host, log, same_bits

pytestmark = pytest.mark.gpu

TORCH = {"bf16": torch.bfloat16, "f16": torch.float16}


def rand(shape, mu, sigma, seed, dt):
    return gen.to_u16(gen.normal(shape, mu, sigma, seed, kind=dt))


def chunk_views(emb_dev, d):
    """(scale, shift, gate) as chunk views of a [B, 6*d] embedding."""
    return emb_dev[:, d:2 * d], emb_dev[:, 0:d], emb_dev[:, 2 * d:3 * d]


def shifted(emb, start):
    """The [B, 6*d] embedding seen from element `start` of each row (what a
    chunk view starting there addresses), as a dense array for the oracle."""
    b, w = emb.shape
    flat = np.concatenate([emb.ravel()[start:], np.zeros(start, np.uint16)])
    return flat.reshape(b, w)


def _run(op, dt, x, m0, m1, b, out=None):
    """op 'mod': x, m0 = scale, m1 = shift; op 'gate': x = update, m0 = gate,
    m1 = residual."""
    if op == "mod":
        r = dn.modulate_scale_shift(x, m0, m1, out=out)
    else:
        r = dn.residual_gate_add(x, m1, m0, out=out)
    torch.cuda.synchronize()
    return host(r)


SHAPES = [(1, 8, 1), (3, 40, 1), (257, 1024, 1), (100, 3072, 2), (37, 4096, 1), (5, 16384, 1),
          (1000, 512, 4), (2, 9000, 2), (999, 1536, 3)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("op", ["mod", "gate"])
@pytest.mark.parametrize("rows,cols,B", SHAPES)
def test_elementwise_shapes(gpu, orc, dt, op, rows, cols, B):
    log(f"{op} {dt} rows={rows} cols={cols} B={B}")
    td = TORCH[dt]
    x = rand((rows, cols), 0.2, 1.5, 31 + cols + rows, dt)
    res = rand((rows, cols), 0.0, 1.0, 32 + cols, dt)
    emb = rand((B, 6 * cols), 0.0, 0.1, 33 + B, dt)
    sc, sh, gt = chunk_views(dev(emb, dtype=td), cols)
    rpb = rows // B
    if op == "mod":
        got = _run(op, dt, dev(x, dtype=td), sc, sh, B)
        ref = orc.modulate_dt(x, shifted(emb, cols), emb, dt, rpb)
    else:
        got = _run(op, dt, dev(x, dtype=td), gt, dev(res, dtype=td), B)
        ref = orc.gate_residual_dt(x, res, shifted(emb, 2 * cols), dt, rpb)
    assert same_bits(got, ref, dt), f"{int((got != ref).sum())} elements differ"


@pytest.mark.parametrize("dt,op", [("bf16", "mod"), ("f16", "mod"), ("f16", "gate")])
@pytest.mark.parametrize("u", range(1, 13))
def test_modulate_every_rows_per_thread(gpu, orc, dt, op, u):
    """The modulate (bf16 and fp16) and the fp16 gate add give each thread
    the U rows that keep every wavefront resident and the busiest SIMD least
    loaded.  At 512 columns (one wavefront per row group) a little under
    U * (4 * CUs) rows selects U: U = 1..12, each with a ragged last group
    and the batch boundaries of three batches inside a thread's rows.  (The
    bf16 gate add runs every shape at U = 2.)"""
    td = TORCH[dt]
    simds = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    cols, B = 512, 3
    rows = (simds * u - 4) // 3 * 3
    log(f"{op} {dt} U={u} rows={rows}")
    x = rand((rows, cols), 0.2, 1.5, 70 + u, dt)
    emb = rand((B, 6 * cols), 0.0, 0.1, 90 + u, dt)
    sc, sh, gt = chunk_views(dev(emb, dtype=td), cols)
    if op == "mod":
        got = _run("mod", dt, dev(x, dtype=td), sc, sh, B)
        ref = orc.modulate_dt(x, shifted(emb, cols), emb, dt, rows // B)
    else:
        res = rand((rows, cols), 0.0, 1.0, 110 + u, dt)
        got = _run("gate", dt, dev(x, dtype=td), gt, dev(res, dtype=td), B)
        ref = orc.gate_residual_dt(x, res, shifted(emb, 2 * cols), dt, rows // B)
    assert same_bits(got, ref, dt), f"{int((got != ref).sum())} elements differ"


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("op", ["mod", "gate"])
def test_elementwise_every_bit_pattern(gpu, orc, dt, op):
    """x (update) runs through all 65536 patterns; the modulation and the
    residual are random patterns too, several batches of them."""
    td = TORCH[dt]
    cols, B = 512, 4
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(-1, cols)  # 128 rows
    rows = x.shape[0]
    m0 = gen.random_bits((B, cols), 41)
    m1 = gen.random_bits((B, cols), 42)
    res = gen.random_bits((rows, cols), 43)
    log(f"{op} {dt} every bit pattern")
    if op == "mod":
        got = _run(op, dt, dev(x, dtype=td), dev(m0, dtype=td), dev(m1, dtype=td), B)
        ref = orc.modulate_dt(x, m0, m1, dt, rows // B)
    else:
        got = _run(op, dt, dev(x, dtype=td), dev(m0, dtype=td), dev(res, dtype=td), B)
        ref = orc.gate_residual_dt(x, res, m0, dt, rows // B)
    assert same_bits(got, ref, dt), f"{int((got != ref).sum())} elements differ"


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_elementwise_in_place_and_empty(gpu, orc, dt):
    td = TORCH[dt]
    rows, cols = 77, 2048
    x = rand((rows, cols), 0, 2.0, 51, dt)
    res = rand((rows, cols), 0, 1.0, 52, dt)
    sc, sh, gt = (rand((cols,), 0, 0.1, s, dt) for s in (53, 54, 55))
    xd = dev(x, dtype=td)
    r = dn.modulate_scale_shift(xd, dev(sc, dtype=td), dev(sh, dtype=td), out=xd)
    torch.cuda.synchronize()
    assert r is xd and same_bits(host(xd), orc.modulate_dt(x, sc, sh, dt), dt)
    rd = dev(res, dtype=td)
    r = dn.residual_gate_add(dev(x, dtype=td), rd, dev(gt, dtype=td), out=rd)
    torch.cuda.synchronize()
    assert r is rd and same_bits(host(rd), orc.gate_residual_dt(x, res, gt, dt), dt)
    e = torch.empty((0, cols), dtype=td, device="cuda")
    assert dn.modulate_scale_shift(e, dev(sc, dtype=td), dev(sh, dtype=td)).shape == (0, cols)
    assert dn.residual_gate_add(e, e, dev(gt, dtype=td)).shape == (0, cols)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_elementwise_full_flux_activation(gpu, orc, dt):
    """FLUX.1's [1, 4608, 3072] activation, the size the benchmark times."""
    td = TORCH[dt]
    rows, cols = 4608, 3072
    log(f"elementwise full {dt} {rows}x{cols}")
    x = rand((rows, cols), 0.0, 1.5, 61, dt)
    res = rand((rows, cols), 0.0, 1.0, 62, dt)
    sc, sh, gt = (rand((cols,), 0, 0.1, s, dt) for s in (63, 64, 65))
    got = _run("mod", dt, dev(x, dtype=td), dev(sc, dtype=td), dev(sh, dtype=td), 1)
    assert same_bits(got, orc.modulate_dt(x, sc, sh, dt), dt)
    got = _run("gate", dt, dev(x, dtype=td), dev(gt, dtype=td), dev(res, dtype=td), 1)
    assert same_bits(got, orc.gate_residual_dt(x, res, gt, dt), dt)


def test_elementwise_rejections(gpu):
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    m = torch.zeros((64,), dtype=torch.float16, device="cuda")
    with pytest.raises(TypeError):
        dn.modulate_scale_shift(x, m, m)                 # mixed storage types
    with pytest.raises(TypeError):
        dn.modulate_scale_shift(x.float(), m.float(), m.float())
    y = torch.zeros((4, 60), dtype=torch.bfloat16, device="cuda")
    s = torch.zeros((60,), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dn.DitnormError):
        dn.modulate_scale_shift(y, s, s)                 # 60 columns: not a multiple of 8
    g = torch.zeros((3, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        dn.residual_gate_add(x, x, g)                    # 4 rows over 3 batches


def test_max_vectors(gpu, orc):
    """The largest activations the one-work-item-per-vector kernels take
    (2^25 - 1 rows, the most a call takes, of 512 columns: 2^31 - 64
    vectors, 34 GB): modulate_scale_shift and conv_bias_epilogue.  Sampled
    rows, the first and last among them, against the oracle."""
    g = torch.Generator(device="cuda").manual_seed(1600)

    def sample(rows):
        return torch.cat([torch.arange(0, 64, device="cuda"),
                          torch.randint(0, rows, (2048,), generator=g, device="cuda"),
                          torch.arange(rows - 64, rows, device="cuda")])

    rows, c = (1 << 25) - 1, 512
    x = torch.empty((rows, c), dtype=torch.bfloat16, device="cuda").normal_(0, 1.5, generator=g)
    sc, sh = rand((1, c), 0, 0.1, 1601, "bf16"), rand((1, c), 0, 0.1, 1602, "bf16")
    out = dn.modulate_scale_shift(x, dev(sc), dev(sh))
    torch.cuda.synchronize()
    i = sample(rows)
    assert same_bits(host(out[i]), orc.modulate_dt(host(x[i]), sc, sh, "bf16"), "bf16")
    del x, out
    torch.cuda.empty_cache()

    x = torch.empty((rows, c), dtype=torch.bfloat16, device="cuda").normal_(0, 1, generator=g)
    bias = gen.normal((c,), 0, 0.05, 1603, "f32")
    out = dn.conv_bias_epilogue(x, bias.cuda())
    torch.cuda.synchronize()
    i = sample(rows)
    assert same_bits(host(out[i]), orc.conv_bias_epilogue(host(x[i]), bias.numpy()), "bf16")
    del x, out
    torch.cuda.empty_cache()
