"""The C ABI from a plain C program (tests/c_abi_consumer.c, built by
__graft_entry__.build()): device memory from the HIP runtime's C API, the
entry points of include/ditnorm.h with raw pointers, no Python in between.
Its outputs against the oracle at the parity bar: ln_modulate, the backward
(d_x, d_scale, d_shift over 300 tokens: chunk sums and tree levels),
gated_ln_modulate, rms_modulate, qk_layernorm (the same buffers as rows of
128) and rmsnorm_silu_bias (as pixels of 96 channels)."""
import os
import subprocess

import numpy as np
import pytest

from dit_adaln_row_amd import inputs as gen
from parity import same_bits, ulp_diff

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_bin", "c_abi_consumer")


def test_c_program_matches_oracle(gpu, orc, tmp_path):
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is not built: run __graft_entry__.build()")
    rows, cols = 300, 3072
    x = gen.to_u16(gen.normal((rows, cols), 0.2, 1.5, 2101))
    sc = gen.to_u16(gen.normal((cols,), 0, 0.1, 2102))
    sh = gen.to_u16(gen.normal((cols,), 0, 0.1, 2103))
    dout = gen.to_u16(gen.normal((rows, cols), 0, 1, 2104))
    gate = gen.to_u16(gen.normal((cols,), 0, 0.1, 2105))
    weight = gen.to_u16(gen.normal((cols,), 1.0, 0.05, 2106))
    bias = gen.normal((96,), 0, 0.05, 2107, "f32").numpy()
    gamma = gen.normal((96,), 1.0, 0.05, 2108, "f32").numpy()
    for name, arr in (("x", x), ("scale", sc), ("shift", sh), ("d_out", dout), ("gate", gate),
                      ("weight", weight)):
        np.ascontiguousarray(arr, dtype=np.uint16).tofile(tmp_path / f"{name}.bin")
    bias.astype(np.float32).tofile(tmp_path / "bias.bin")
    gamma.astype(np.float32).tofile(tmp_path / "gamma.bin")
    (tmp_path / "meta.txt").write_text(f"{rows} {cols}\n")
    r = subprocess.run([BIN, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    out = np.fromfile(tmp_path / "out.bin", np.uint16).reshape(rows, cols)
    ref = orc.ln_modulate(x, sc.reshape(1, cols), sh.reshape(1, cols), 1e-6,
                          rows_per_batch=rows)
    assert same_bits(out, ref["out"]), "ln_modulate from C"
    bref = orc.ln_modulate_backward(x, sc.reshape(1, cols), dout, 1e-6, rows_per_batch=rows)
    d_x = np.fromfile(tmp_path / "d_x.bin", np.uint16).reshape(rows, cols)
    d = ulp_diff(d_x, bref["d_x"])
    assert d.max() <= 1 and (d == 0).mean() >= 0.9999, "d_x from C"
    d_scale = np.fromfile(tmp_path / "d_scale.bin", np.float32).reshape(1, cols)
    d_shift = np.fromfile(tmp_path / "d_shift.bin", np.float32).reshape(1, cols)
    assert np.array_equal(d_shift, bref["d_shift"]), "d_shift from C"
    assert np.array_equal(d_scale, bref["d_scale"]), "d_scale from C"

    def got(name, shape):
        return np.fromfile(tmp_path / name, np.uint16).reshape(shape)

    g = orc.gated_ln_modulate(x, dout, gate.reshape(1, cols), sc.reshape(1, cols),
                              sh.reshape(1, cols), 1e-6, rows_per_batch=rows)
    assert same_bits(got("h.bin", (rows, cols)), g["h"]), "gated_ln_modulate h from C"
    assert same_bits(got("gated.bin", (rows, cols)), g["out"]), "gated_ln_modulate from C"
    r = orc.rms_modulate(x, weight, sc.reshape(1, cols), sh.reshape(1, cols), 1e-6,
                         rows_per_batch=rows)
    assert same_bits(got("rms.bin", (rows, cols)), r["out"]), "rms_modulate from C"
    q = orc.qk_layernorm(x.reshape(-1, 128), dout.reshape(-1, 128), 1e-5)
    assert same_bits(got("q_out.bin", (rows * cols // 128, 128)), q["q_out"]), "qk q from C"
    assert same_bits(got("k_out.bin", (rows * cols // 128, 128)), q["k_out"]), "qk k from C"
    w = orc.rmsnorm_silu_bias(x.reshape(-1, 96), bias, gamma, 1e-6)
    dw = ulp_diff(got("wan.bin", (rows * cols // 96, 96)), w["out"])
    assert dw.max() <= 1, "rmsnorm_silu_bias from C: beyond 1 ulp"
