"""Host-side tests of the C ABI (no GPU needed, no compute call made).

The library must load on a machine without a GPU, export every function the
header declares, and reject invalid arguments before any HIP call (every
case below returns before the library looks for a device).
"""
import ctypes
import os
import re

import pytest
import torch

import dit_adaln_row_amd as dn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ditnorm.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

A = 0x10000        # a 16-byte-aligned fake device address (never dereferenced)
B = 0x20000000
C = 0x40000000
D = 0x60000000
E = 0x80000000


def declared_functions(headers=HEADERS):
    text = "\n".join(open(h).read() for h in headers)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int64_t|int|char\s*\*|const char\s*\*)\s*\**\s*(\w+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dn.LIB_PATH):
        import dit_adaln_row_amd.build as b
        b.build(verbose=False)
    return dn.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    for must in ("ln_modulate", "ln_modulate_folded", "gated_ln_modulate", "rms_modulate", "qk_layernorm",
                 "rmsnorm_silu_bias", "conv_bias_epilogue", "modulate_scale_shift",
                 "residual_gate_add", "ln_modulate_backward",
                 "ln_modulate_backward_workspace_bytes", "ditnorm_status_string"):
        assert must in names
    for n in names:
        assert hasattr(lib, n), n
    # the measurement copy is declared apart from the method's entry points
    assert "ditnorm_copy" not in declared_functions([HEADER])
    assert "ditnorm_copy" in names


def test_status_strings(lib):
    assert lib.ditnorm_status_string(0) == b"DITNORM_OK"
    assert lib.ditnorm_status_string(1) == b"DITNORM_INVALID_ARGUMENT"
    assert lib.ditnorm_status_string(2) == b"DITNORM_UNSUPPORTED"
    assert lib.ditnorm_status_string(3) == b"DITNORM_DEVICE_ERROR"
    assert lib.ditnorm_status_string(4) == b"DITNORM_SCRATCH_EXCEEDED"
    assert lib.ditnorm_status_string(99) == b"DITNORM_UNKNOWN_STATUS"
    assert lib.ditnorm_version() >= 100


def ln(lib, x=A, sc=B, sh=C, out=D, rows=4, cols=1024, rpb=4, mbs=1024, eps=1e-6, mean=None,
       rstd=None, y=None):
    return lib.ln_modulate(x, sc, sh, out, rows, cols, rpb, mbs, eps, mean, rstd, y, None)


def test_ln_modulate_validation(lib):
    assert ln(lib, x=None) == dn.INVALID_ARGUMENT
    assert ln(lib, rows=-1) == dn.INVALID_ARGUMENT
    assert ln(lib, cols=0) == dn.INVALID_ARGUMENT
    assert ln(lib, rows=6, rpb=4) == dn.INVALID_ARGUMENT          # rows % rows_per_batch
    assert ln(lib, mbs=512) == dn.INVALID_ARGUMENT                # stride < cols
    assert ln(lib, eps=float("nan")) == dn.INVALID_ARGUMENT
    assert ln(lib, eps=-1.0) == dn.INVALID_ARGUMENT
    assert ln(lib, eps=float("inf")) == dn.INVALID_ARGUMENT
    assert ln(lib, cols=1004, mbs=1004) == dn.UNSUPPORTED          # cols % 8
    assert ln(lib, cols=16392, mbs=16392) == dn.UNSUPPORTED        # above the maximum
    assert ln(lib, x=A + 2) == dn.UNSUPPORTED                      # misaligned
    assert ln(lib, y=A + 8) == dn.UNSUPPORTED
    assert ln(lib, rows=8, rpb=4, mbs=1028) == dn.UNSUPPORTED      # batch stride breaks alignment
    assert ln(lib, out=A + 16) == dn.UNSUPPORTED                   # partial overlap with x
    assert ln(lib, y=D) == dn.UNSUPPORTED                          # two outputs overlap
    assert ln(lib, out=B) == dn.UNSUPPORTED                        # output over an input
    assert ln(lib, rows=0, x=None) == dn.OK                        # empty: no-op


def test_supported_predicates_never_touch_the_gpu(lib):
    ok = lib.ln_modulate_supported(A, B, C, D, 4, 1024, 4, 1024, 1e-6, None, None, None)
    assert ok == 1
    assert lib.ln_modulate_supported(A, B, C, A, 4, 1024, 4, 1024, 1e-6, None, None, None) == 1  # in place
    assert lib.ln_modulate_supported(A, B, C, D, 4, 1004, 4, 1004, 1e-6, None, None, None) == 0
    assert lib.gated_ln_modulate_supported(A, B, C, D, E, C + 0x10, E + 0x100000, 4, 1024, 4,
                                           1024, 1e-6, None, None, None) == 0  # residual_out over gate
    assert lib.gated_ln_modulate_supported(A, B, C, C + 0x4000, C + 0x8000, B, D, 4, 1024, 4, 1024,
                                           1e-6, None, None, None) == 1  # residual_out == residual
    assert lib.rms_modulate_supported(A, B, C, C + 0x4000, D, None, None, None, 4, 4096, 4, 4096,
                                      1e-6, None, None) == 1
    assert lib.rms_modulate_supported(A, B, C, C + 0x4000, D, E, None, None, 4, 4096, 4, 4096,
                                      1e-6, None, None) == 0   # half a gated group
    assert lib.qk_layernorm_supported(A, B, C, D, 10, 10, 128, 1e-5, None, None) == 1
    assert lib.qk_layernorm_supported(A, B, C, D, 10, 10, 64, 1e-5, None, None) == 1
    assert lib.qk_layernorm_supported(A, B, C, D, 10, 10, 72, 1e-5, None, None) == 1
    assert lib.qk_layernorm_supported(A, B, C, D, 10, 10, 8, 1e-5, None, None) == 1
    assert lib.qk_layernorm_supported(A, B, C, D, 10, 10, 60, 1e-5, None, None) == 0  # % 8
    assert lib.qk_layernorm_supported(A, B, C, D, 10, 10, 136, 1e-5, None, None) == 0  # > 128
    assert lib.qk_layernorm_supported(A, None, C, None, 10, 0, 128, 1e-5, None, None) == 1
    assert lib.qk_layernorm_supported(A, None, C, None, 10, 3, 128, 1e-5, None, None) == 0
    assert lib.rmsnorm_silu_bias_supported(A, B, C, D, 100, 96, 1e-6, None, None) == 1
    assert lib.rmsnorm_silu_bias_supported(A, None, C, D, 100, 96, 1e-6, None, None) == 1
    assert lib.rmsnorm_silu_bias_supported(A, B, C, D, 100, 100, 1e-6, None, None) == 0
    assert lib.rmsnorm_silu_bias_supported(A, B + 4, C, D, 100, 96, 1e-6, None, None) == 0
    assert lib.conv_bias_epilogue_supported(A, B, C, D, 100, 96, 0, 2) == 1
    assert lib.conv_bias_epilogue_supported(A, B, C, A, 100, 96, 0, 2) == 1   # in place
    assert lib.conv_bias_epilogue_supported(A, B, C, C, 100, 96, 0, 2) == 0   # out over h
    # storage types: fp32 or the activation's own type for the bias
    for dt, bdt, ok in ((1, 2, 1), (1, 1, 1), (2, 2, 1), (0, 0, 1), (0, 1, 0), (1, 0, 0),
                        (2, 0, 0), (2, 1, 0)):
        assert lib.conv_bias_epilogue_supported(A, B, C, D, 100, 96, dt, bdt) == ok, (dt, bdt)
    assert lib.conv_bias_epilogue(A, B, None, D, 10, 96, 3, 2, None) == dn.INVALID_ARGUMENT
    assert lib.conv_bias_epilogue(A, B, None, D, 10, 96, 0, 7, None) == dn.INVALID_ARGUMENT
    assert lib.conv_bias_epilogue(A, B, None, D, 10, 96, 2, 0, None) == dn.UNSUPPORTED
    assert lib.ln_modulate_folded_supported(A, B, C, D, 4, 3072, 4, 3072, 1e-6, None, None) == 1
    assert lib.ln_modulate_folded_supported(A, B, C, A, 4, 3072, 4, 3072, 1e-6, None, None) == 1
    assert lib.ln_modulate_folded_supported(A, B, C, D, 4, 3076, 4, 3076, 1e-6, None, None) == 0
    assert lib.ln_modulate_folded_supported(A, B, C, D, 4, 3072, 4, 3072, -1.0, None, None) == 0
    for dt in (0, 1):
        assert lib.modulate_scale_shift_supported(A, B, C, D, 8, 3072, 4, 6 * 3072, dt) == 1
        assert lib.modulate_scale_shift_supported(A, B, C, A, 8, 3072, 4, 3072, dt) == 1  # in place
        assert lib.modulate_scale_shift_supported(A, B, C, B, 8, 3072, 4, 3072, dt) == 0  # out over scale
        assert lib.modulate_scale_shift_supported(A, B, C, D, 8, 3076, 8, 3076, dt) == 0
        assert lib.modulate_scale_shift_supported(A, B, C, D, 8, 3072, 4, 3076, dt) == 0  # stride
        assert lib.residual_gate_add_supported(A, B, C, B, 8, 3072, 8, 3072, dt) == 1     # out == residual
        assert lib.residual_gate_add_supported(A, B, C, A, 8, 3072, 8, 3072, dt) == 0     # out == update
        assert lib.residual_gate_add_supported(A, B, C + 8, D, 8, 3072, 8, 3072, dt) == 0  # misaligned
    assert lib.modulate_scale_shift_supported(A, B, C, D, 8, 3072, 8, 3072, 2) == 0


def test_other_entry_validation(lib):
    assert lib.gated_ln_modulate(A, None, C, C, C, D, E, 4, 1024, 4, 1024, 1e-6, None, None,
                                 None, None) == dn.INVALID_ARGUMENT
    assert lib.rms_modulate(A, B, C, C, D, E, None, None, 4, 1024, 4, 1024, 1e-6, None, None,
                            None) == dn.INVALID_ARGUMENT
    assert lib.qk_layernorm(A, B, C, D, 4, 4, 60, 1e-5, None, None, None) == dn.UNSUPPORTED
    assert lib.qk_layernorm(A, B, C, D, 4, 4, 256, 1e-5, None, None, None) == dn.UNSUPPORTED
    assert lib.qk_layernorm(A, B, C, D, 4, 4, 0, 1e-5, None, None, None) == dn.INVALID_ARGUMENT
    # an output overlapping the other tensor's input at 64-wide rows
    assert lib.qk_layernorm(A, B, A + 64, D, 4, 4, 64, 1e-5, None, None, None) == dn.UNSUPPORTED
    assert lib.qk_layernorm(A, B, C, D, -1, 4, 128, 1e-5, None, None, None) == dn.INVALID_ARGUMENT
    assert lib.qk_layernorm(A, B, A + 128, D, 4, 4, 128, 1e-5, None, None, None) == dn.UNSUPPORTED
    assert lib.rmsnorm_silu_bias(A, B, None, D, 10, 96, 1e-6, None, None, None) == dn.INVALID_ARGUMENT
    assert lib.rmsnorm_silu_bias(A, B, C, D, 10, 4104, 1e-6, None, None, None) == dn.UNSUPPORTED
    assert lib.conv_bias_epilogue(A, None, None, D, 10, 96, 0, 2, None) == dn.INVALID_ARGUMENT
    assert lib.ln_modulate_folded(A, B, None, D, 4, 3072, 4, 3072, 1e-6, None, None,
                                  None) == dn.INVALID_ARGUMENT
    assert lib.ln_modulate_folded(A, B, C, D, 4, 3072, 3, 3072, 1e-6, None, None,
                                  None) == dn.INVALID_ARGUMENT
    assert lib.modulate_scale_shift(A, B, C, D, 8, 3072, 8, 3072, 7, None) == dn.INVALID_ARGUMENT
    assert lib.modulate_scale_shift(A, B, None, D, 8, 3072, 8, 3072, 0, None) == dn.INVALID_ARGUMENT
    assert lib.modulate_scale_shift(A, B, C, D, 8, 3072, 3, 3072, 1, None) == dn.INVALID_ARGUMENT
    assert lib.modulate_scale_shift(A, B, C, D, 8, 3072, 8, 3000, 0, None) == dn.INVALID_ARGUMENT
    assert lib.modulate_scale_shift(A, B, C, D, 0, 3072, 8, 3072, 0, None) == dn.OK   # no-op
    assert lib.residual_gate_add(A, None, C, D, 8, 3072, 8, 3072, 0, None) == dn.INVALID_ARGUMENT
    assert lib.residual_gate_add(A, B, C, D, 8, 16392, 8, 16392, 0, None) == dn.UNSUPPORTED
    # backward: workspace size, validation before any HIP call
    # the partial sums of 862 runs of 8 tokens, then of 7 values of the second level
    ws = dn.ln_modulate_backward_workspace_bytes(6889, 3072, 6889)
    assert ws >= 2 * 862 * 3072 * 4 + 2 * 7 * 3072 * 4
    assert dn.ln_modulate_backward_workspace_bytes(0, 3072, 1) == 0
    # a batch of at most 8 tokens (4 over 3072 columns) is summed in one workgroup
    assert dn.ln_modulate_backward_workspace_bytes(2048 * 3, 3072, 3) == 0
    assert dn.ln_modulate_backward_workspace_bytes(4 * 8, 3072, 8) == 0
    assert dn.ln_modulate_backward_workspace_bytes(4 * 8, 4096, 8) > 0
    assert lib.ln_modulate_backward_workspace_bytes(10, 3072, 3, 0) == -1
    assert lib.ln_modulate_backward_workspace_bytes(1 << 62, 1 << 40, 1 << 62, 0) == -1  # no overflow
    assert lib.ln_modulate_backward_workspace_bytes(4, 4104, 4, 0) == -1
    # fp32 rows: 4-token workgroups, at most 3072 columns; no other storage type
    assert lib.ln_modulate_backward_workspace_bytes(4, 4096, 4, 2) == -1
    assert lib.ln_modulate_backward_workspace_bytes(4, 3072, 4, 1) == -1
    assert dn.ln_modulate_backward_workspace_bytes(8, 3072, 8, torch.float32) > 0
    assert dn.ln_modulate_backward_workspace_bytes(2048 * 3, 3072, 3, torch.float32) == 0
    W = 0xA0000000
    bw = lambda **k: lib.ln_modulate_backward(
        k.get("x", A), k.get("sc", B), k.get("do", C), k.get("dx", D), k.get("ds", E),
        k.get("dh", E + 0x100000), k.get("rows", 64), k.get("cols", 3072), k.get("rpb", 64),
        k.get("mbs", 3072), 1e-6, k.get("ws", W), k.get("wsb", 1 << 24), None, None,
        k.get("dt", 0), None)
    assert bw(wsb=100) == dn.INVALID_ARGUMENT                  # workspace too small
    assert bw(ws=W + 16) == dn.UNSUPPORTED                     # workspace not 256-aligned
    assert bw(cols=4104, mbs=4104) == dn.UNSUPPORTED           # wider than the backward serves
    assert bw(dx=C) == dn.UNSUPPORTED                          # d_x over d_out
    assert bw(do=None) == dn.INVALID_ARGUMENT
    assert bw(rows=0) == dn.OK
    assert bw(dt=1) == dn.INVALID_ARGUMENT                     # fp16: not a backward type
    assert bw(dt=2, cols=4096, mbs=4096) == dn.UNSUPPORTED     # fp32 rows: at most 3072
    assert bw(dt=2, dx=C) == dn.UNSUPPORTED
    assert lib.ln_modulate_backward_supported(A, B, C, D, E, E + 0x100000, 64, 3072, 64, 3072,
                                              1e-6, W, 1 << 24, None, None, 0) == 1
    assert lib.ln_modulate_backward_supported(A, B, C, D, E, E + 0x100000, 64, 3072, 64, 3072,
                                              1e-6, W, 1 << 24, None, None, 2) == 1
    # the modulation row stride is bounded (byte spans stay inside int64)
    MS, T = 1 << 36, 1 << 40  # fake buffers a terabyte apart: the spans do not overlap
    assert lib.ln_modulate_supported(T, 2 * T, 3 * T, 4 * T, 16, 8, 8, MS, 1e-6, None, None,
                                     None) == 1
    assert lib.ln_modulate_supported(T, 2 * T, 3 * T, 4 * T, 16, 8, 8, MS + 8, 1e-6, None, None,
                                     None) == 0
    assert lib.ln_modulate(T, 2 * T, 3 * T, 4 * T, 16, 8, 8, 1 << 62, 1e-6, None, None, None,
                           None) == dn.UNSUPPORTED
    # size limits: rows (one wavefront per row) and 16-byte vectors per launch
    MR = 33554431
    assert lib.ln_modulate(A, B, C, D, MR + 1, 8, MR + 1, 8, 1e-6, None, None, None, None) \
        == dn.UNSUPPORTED
    assert lib.ln_modulate_supported(A, B, C, D, MR, 8, MR, 8, 1e-6, None, None, None) == 1
    assert lib.qk_layernorm(A, B, C, D, MR, 1, 128, 1e-5, None, None, None) == dn.UNSUPPORTED
    big = (1 << 63) - 1  # a sum of row counts that would overflow int64
    assert lib.qk_layernorm(A, B, C, D, big, big, 128, 1e-5, None, None, None) == dn.UNSUPPORTED
    assert lib.rmsnorm_silu_bias(A, E, E + 4096, D, MR + 1, 96, 1e-6, None, None, None) \
        == dn.UNSUPPORTED
    # 2^31 - 1 vectors of 512 per row: 4194303 rows fit, 4194304 do not (buffers 64 GB apart)
    G = 1 << 36
    for rows, ok in ((4194303, 1), (4194304, 0)):
        assert lib.conv_bias_epilogue_supported(G, E, None, 2 * G, rows, 4096, 0, 2) == ok
        # fp32 activations: 16-byte vectors of 4 values, half the rows fit
        assert lib.conv_bias_epilogue_supported(G, E, None, 2 * G, rows // 2, 4096, 2, 2) == ok
        assert lib.modulate_scale_shift_supported(G, B, C, 2 * G, rows, 4096, rows, 4096,
                                                  0) == ok
    # (fake buffers spaced so that only the size decides: d_scale / d_shift
    # of 8.4M batches span 268 MB each)
    bw3 = lambda rows: lib.ln_modulate_backward(A, B, C, D, E, E + 0x20000000, rows, 8, 3, 8,
                                                1e-6, None, 0, None, None, 0, None)
    assert bw3(3 * (MR // 4) + 3) == dn.UNSUPPORTED    # 3-token batches take 4 row slots each
    assert lib.ln_modulate_backward_supported(A, B, C, D, E, E + 0x20000000, 3 * (MR // 4), 8,
                                              3, 8, 1e-6, None, 0, None, None, 0) == 1
    # the no-allocation backward: the same checks, then the partial sums must
    # fit the library's scratch array (refused before any HIP call)
    na = lambda **k: lib.ln_modulate_backward_noalloc(
        k.get("x", A), k.get("sc", B), k.get("do", C), k.get("dx", D), k.get("ds", E),
        k.get("dh", E + 0x100000), k.get("rows", 64), k.get("cols", 3072), k.get("rpb", 64),
        k.get("mbs", 3072), 1e-6, None, None, k.get("dt", 0), None)
    assert na(do=None) == dn.INVALID_ARGUMENT
    assert na(dt=1) == dn.INVALID_ARGUMENT
    assert na(dx=C) == dn.UNSUPPORTED
    assert na(cols=4104, mbs=4104) == dn.UNSUPPORTED
    assert na(rows=0) == dn.OK
    big = 12000  # 12000 tokens of 3072 columns: 36.9 MB of partial sums
    assert dn.ln_modulate_backward_workspace_bytes(big, 3072, big) > dn.NOALLOC_SCRATCH_BYTES
    assert na(rows=big, rpb=big, dh=E + 0x1000000) == dn.SCRATCH_EXCEEDED
    assert na(rows=big, rpb=big, dh=E + 0x1000000, mbs=3000) == dn.INVALID_ARGUMENT
    assert dn.ln_modulate_backward_workspace_bytes(6889, 3072, 6889) <= dn.NOALLOC_SCRATCH_BYTES
    assert lib.ditnorm_copy(A, B, 15, None) == dn.UNSUPPORTED
    assert lib.ditnorm_copy(A, A + 16, 64, None) == dn.UNSUPPORTED


def test_missing_library_fails_loudly(tmp_path):
    import importlib
    mod = importlib.reload(dn)
    mod._lib = None
    with pytest.raises(RuntimeError):
        mod.load(str(tmp_path / "nope.so"))
    importlib.reload(dn)


def test_product_never_uses_the_oracle():
    pkg = os.path.join(ROOT, "dit_adaln_row_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle", text, flags=re.M), f
                assert "ditnorm_oracle" not in text and "libditnorm_oracle" not in text, f
    osrc = open(os.path.join(ROOT, "oracle", "ditnorm_oracle.c")).read()
    assert "#include \"" not in osrc   # the oracle includes no project header


def test_header_is_c_and_cpp_and_a_c_program_links(tmp_path):
    """include/ditnorm.h compiles as C99 and as C++11 with warnings as errors,
    and the C-ABI test's plain C program builds against the library."""
    import subprocess
    src = tmp_path / "h.c"
    src.write_text('#include "ditnorm.h"\n#include "ditnorm_measure.h"\n'
                   'int main(void) { return ditnorm_last_hip_error(); }\n')
    inc = os.path.join(ROOT, "include")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", inc, "-fsyntax-only",
                    str(src)], check=True)
    subprocess.run(["g++", "-std=c++11", "-Wall", "-Wextra", "-Werror", "-I", inc,
                    "-fsyntax-only", "-x", "c++", str(src)], check=True)
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "c_abi_consumer_build", os.path.join(ROOT, "tests", "c_abi_consumer_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert os.path.exists(mod.build(str(tmp_path / "consumer")))
