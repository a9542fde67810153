"""CPU oracle for the fused adaLN row-normalisation path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``dit_adaln_row_amd``
and its HIP library) never imports, links or calls it, and shares no code
with it: the arithmetic lives in ``ditnorm_oracle.c`` (plain C, built with
``gcc -O2 -ffp-contract=off``), this module only marshals numpy arrays.

bf16 tensors are numpy ``uint16`` arrays holding the bit patterns.

Every function here is pinned by ``tests/test_oracle_pins.py`` against
library routines, exact rational arithmetic, closed forms and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "ditnorm_oracle.c")
LIB = os.path.join(_HERE, "libditnorm_oracle.so")
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall",
          "-Wextra", "-shared", "-fPIC"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (seconds).  Returns the library path."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        sig = {
            "oracle_round_f32_to_bf16": [_f32p, _u16p, _i64],
            "oracle_round_f64_to_bf16": [_f64p, _u16p, _i64],
            "oracle_round_f32_to_f16": [_f32p, _u16p, _i64],
            "oracle_widen_f16": [_u16p, _f32p, _i64],
            "oracle_modulate_dt": [_u16p, _u16p, _u16p, _u16p, _i64, _i64, _i64, _i64, ctypes.c_int],
            "oracle_gate_residual_dt": [_u16p, _u16p, _u16p, _u16p, _i64, _i64, _i64, _i64,
                                        ctypes.c_int],
            "oracle_silu_bf16": [_f32p, _u16p, _i64],
            "oracle_ln_stats": [_u16p, _i64, _i64, ctypes.c_float, _f32p, _f32p],
            "oracle_rms_stats": [_u16p, _i64, _i64, ctypes.c_float, _f32p],
            "oracle_ln_normalize": [_u16p, _f32p, _f32p, _u16p, _i64, _i64],
            "oracle_rms_normalize": [_u16p, _f32p, _u16p, _u16p, _i64, _i64],
            "oracle_modulate": [_u16p, _u16p, _u16p, _u16p, _i64, _i64, _i64, _i64],
            "oracle_gate_residual": [_u16p, _u16p, _u16p, _u16p, _i64, _i64, _i64, _i64],
            "oracle_bias_add": [_u16p, _f32p, _u16p, _i64, _i64],
            "oracle_silu_normalize": [_u16p, _f32p, _f32p, _u16p, _i64, _i64],
            "oracle_ln_modulate": [_u16p, _u16p, _u16p, _u16p, _i64, _i64, _i64, _i64,
                                   ctypes.c_float, _f32p, _f32p, _u16p],
            "oracle_ln_modulate_folded": [_u16p, _u16p, _u16p, _u16p, _i64, _i64, _i64, _i64,
                                          ctypes.c_float, _f32p, _f32p],
            "oracle_tree32_sum": [_f32p, _i64],
            "oracle_ln_modulate_backward": [_u16p, _u16p, _u16p, _i64, _i64, _i64, _i64,
                                            ctypes.c_float, _u16p, _f32p, _f32p, _f32p, _f32p],
            "oracle_gated_ln_modulate": [_u16p, _u16p, _u16p, _u16p, _u16p, _u16p, _u16p,
                                         _i64, _i64, _i64, _i64, ctypes.c_float,
                                         _f32p, _f32p, _u16p],
            "oracle_rms_modulate": [_u16p, _u16p, _u16p, _u16p, _u16p, _u16p, _u16p, _u16p,
                                    _i64, _i64, _i64, _i64, ctypes.c_float, _f32p, _u16p],
            "oracle_qk_layernorm": [_u16p, _u16p, _u16p, _u16p, _i64, _i64, _i64,
                                    ctypes.c_float, _f32p, _f32p],
            "oracle_rmsnorm_silu_bias": [_u16p, _f32p, _f32p, _u16p, _i64, _i64,
                                         ctypes.c_float, _f32p, _u16p],
            "oracle_conv_bias_epilogue": [_u16p, _f32p, _u16p, _u16p, _i64, _i64],
            "oracle_ln_modulate_backward_f32": [_f32p, _f32p, _f32p, _i64, _i64, _i64, _i64,
                                                ctypes.c_float, _f32p, _f32p, _f32p, _f32p,
                                                _f32p],
            "oracle_conv_bias_epilogue_dt": [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, _i64, _i64, ctypes.c_int,
                                             ctypes.c_int],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            if name == "oracle_tree32_sum":
                fn.restype = ctypes.c_float
                continue
            fn.restype = None if name in ("oracle_round_f32_to_f16", "oracle_widen_f16") else \
                ctypes.c_int if name.startswith(("oracle_ln", "oracle_rms", "oracle_mod",
                                                          "oracle_gate", "oracle_bias",
                                                          "oracle_silu_norm", "oracle_gated",
                                                          "oracle_qk", "oracle_conv")) else None
        _lib = lib
    return _lib


def _p(a, typ):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(typ)


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _check(rc):
    if rc != 0:
        raise ValueError("oracle rejected its arguments (rc=%d)" % rc)


# -- conversions --------------------------------------------------------------

def round_f32_to_bf16(f):
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    _load().oracle_round_f32_to_bf16(_p(f, _f32p), _p(out, _u16p), f.size)
    return out


def round_f64_to_bf16(d):
    d = np.ascontiguousarray(d, dtype=np.float64)
    out = np.empty(d.shape, np.uint16)
    _load().oracle_round_f64_to_bf16(_p(d, _f64p), _p(out, _u16p), d.size)
    return out


def round_f32_to_f16(f):
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    _load().oracle_round_f32_to_f16(_p(f, _f32p), _p(out, _u16p), f.size)
    return out


def widen_f16(h):
    h = _u16(h)
    out = np.empty(h.shape, np.float32)
    _load().oracle_widen_f16(_p(h, _u16p), _p(out, _f32p), h.size)
    return out


DTYPES = {"bf16": 0, "f16": 1, "f32": 2}


def modulate_dt(x, scale, shift, dtype="bf16", rows_per_batch=None):
    """Standalone modulate in bf16 or fp16 storage (uint16 bit patterns)."""
    x = _u16(x)
    rows, cols = x.shape
    scale, stride = _mod_rows(scale, cols)
    shift, stride2 = _mod_rows(shift, cols)
    assert stride == stride2
    out = np.empty_like(x)
    _check(_load().oracle_modulate_dt(_p(x, _u16p), _p(scale, _u16p), _p(shift, _u16p),
                                      _p(out, _u16p), rows, cols, rows_per_batch or max(rows, 1),
                                      stride, DTYPES[dtype]))
    return out


def gate_residual_dt(update, residual, gate, dtype="bf16", rows_per_batch=None):
    """Standalone residual-gate add in bf16 or fp16 storage."""
    update, residual = _u16(update), _u16(residual)
    rows, cols = update.shape
    gate, stride = _mod_rows(gate, cols)
    out = np.empty_like(update)
    _check(_load().oracle_gate_residual_dt(_p(update, _u16p), _p(residual, _u16p), _p(gate, _u16p),
                                           _p(out, _u16p), rows, cols,
                                           rows_per_batch or max(rows, 1), stride, DTYPES[dtype]))
    return out


def silu_bf16(t):
    t = np.ascontiguousarray(t, dtype=np.float32)
    out = np.empty(t.shape, np.uint16)
    _load().oracle_silu_bf16(_p(t, _f32p), _p(out, _u16p), t.size)
    return out


# -- stages -------------------------------------------------------------------

def ln_stats(x, eps):
    x = _u16(x)
    rows, cols = x.shape
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    _check(_load().oracle_ln_stats(_p(x, _u16p), rows, cols, eps, _p(mean, _f32p), _p(rstd, _f32p)))
    return mean, rstd


def rms_stats(x, eps):
    x = _u16(x)
    rows, cols = x.shape
    rstd = np.empty(rows, np.float32)
    _check(_load().oracle_rms_stats(_p(x, _u16p), rows, cols, eps, _p(rstd, _f32p)))
    return rstd


def ln_normalize(x, mean, rstd):
    x = _u16(x)
    rows, cols = x.shape
    mean, rstd = _f32(mean), _f32(rstd)
    y = np.empty_like(x)
    _check(_load().oracle_ln_normalize(_p(x, _u16p), _p(mean, _f32p), _p(rstd, _f32p),
                                       _p(y, _u16p), rows, cols))
    return y


def rms_normalize(x, rstd, w):
    x, w = _u16(x), _u16(w)
    rows, cols = x.shape
    rstd = _f32(rstd)
    y = np.empty_like(x)
    _check(_load().oracle_rms_normalize(_p(x, _u16p), _p(rstd, _f32p), _p(w, _u16p),
                                        _p(y, _u16p), rows, cols))
    return y


def _mod_rows(mod, cols):
    """A [B, cols] (or [B, stride] with cols <= stride) modulation array."""
    mod = _u16(mod)
    if mod.ndim == 1:
        mod = mod.reshape(1, -1)
    return mod, mod.shape[1]


def modulate(y, scale, shift, rows_per_batch=None):
    y = _u16(y)
    rows, cols = y.shape
    scale, stride = _mod_rows(scale, cols)
    shift, stride2 = _mod_rows(shift, cols)
    assert stride == stride2
    rpb = rows_per_batch or max(rows, 1)
    out = np.empty_like(y)
    _check(_load().oracle_modulate(_p(y, _u16p), _p(scale, _u16p), _p(shift, _u16p),
                                   _p(out, _u16p), rows, cols, rpb, stride))
    return out


def gate_residual(update, residual, gate, rows_per_batch=None):
    update, residual = _u16(update), _u16(residual)
    rows, cols = update.shape
    gate, stride = _mod_rows(gate, cols)
    rpb = rows_per_batch or max(rows, 1)
    h = np.empty_like(update)
    _check(_load().oracle_gate_residual(_p(update, _u16p), _p(residual, _u16p), _p(gate, _u16p),
                                        _p(h, _u16p), rows, cols, rpb, stride))
    return h


def bias_add(x, bias):
    x = _u16(x)
    rows, ch = x.shape
    bias = _f32(bias)
    xb = np.empty_like(x)
    _check(_load().oracle_bias_add(_p(x, _u16p), _p(bias, _f32p), _p(xb, _u16p), rows, ch))
    return xb


def silu_normalize(xb, rstd, gamma):
    xb = _u16(xb)
    rows, ch = xb.shape
    rstd, gamma = _f32(rstd), _f32(gamma)
    out = np.empty_like(xb)
    _check(_load().oracle_silu_normalize(_p(xb, _u16p), _p(rstd, _f32p), _p(gamma, _f32p),
                                         _p(out, _u16p), rows, ch))
    return out


# -- composites (one per library entry point) ---------------------------------

def ln_modulate(x, scale, shift, eps, rows_per_batch=None, row_slice=None):
    """Returns dict(out, mean, rstd, y).  ``row_slice`` restricts to a row range
    (the modulation row index still follows the global row number)."""
    x = _u16(x)
    rows, cols = x.shape
    scale, stride = _mod_rows(scale, cols)
    shift, _ = _mod_rows(shift, cols)
    rpb = rows_per_batch or max(rows, 1)
    out = np.empty_like(x)
    y = np.empty_like(x)
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    _check(_load().oracle_ln_modulate(_p(x, _u16p), _p(scale, _u16p), _p(shift, _u16p),
                                      _p(out, _u16p), rows, cols, rpb, stride, eps,
                                      _p(mean, _f32p), _p(rstd, _f32p), _p(y, _u16p)))
    return dict(out=out, mean=mean, rstd=rstd, y=y)


def ln_modulate_folded(x, scale, shift, eps, rows_per_batch=None):
    """LN with the modulate folded into its affine (lossy one-pass form).
    Returns dict(out, mean, rstd)."""
    x = _u16(x)
    rows, cols = x.shape
    scale, stride = _mod_rows(scale, cols)
    shift, _ = _mod_rows(shift, cols)
    rpb = rows_per_batch or max(rows, 1)
    out = np.empty_like(x)
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    _check(_load().oracle_ln_modulate_folded(_p(x, _u16p), _p(scale, _u16p), _p(shift, _u16p),
                                             _p(out, _u16p), rows, cols, rpb, stride, eps,
                                             _p(mean, _f32p), _p(rstd, _f32p)))
    return dict(out=out, mean=mean, rstd=rstd)


def tree32_sum(values):
    """The fixed fp32 token-sum tree over a 1-D array of fp32 values."""
    v = np.array(values, dtype=np.float32, copy=True)
    return np.float32(_load().oracle_tree32_sum(_p(v, _f32p), v.size))


def ln_modulate_backward(x, scale, d_out, eps, rows_per_batch=None):
    """Backward of LN (no affine) + modulate.  Returns dict(d_x (bf16 bits),
    d_scale, d_shift (fp32 [B, cols]), mean, rstd)."""
    x, d_out = _u16(x), _u16(d_out)
    rows, cols = x.shape
    scale, stride = _mod_rows(scale, cols)
    rpb = rows_per_batch or max(rows, 1)
    nb = rows // rpb if rows else 0
    d_x = np.empty_like(x)
    d_scale = np.empty((nb, cols), np.float32)
    d_shift = np.empty((nb, cols), np.float32)
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    _check(_load().oracle_ln_modulate_backward(
        _p(x, _u16p), _p(scale, _u16p), _p(d_out, _u16p), rows, cols, rpb, stride, eps,
        _p(d_x, _u16p), _p(d_scale, _f32p), _p(d_shift, _f32p), _p(mean, _f32p),
        _p(rstd, _f32p)))
    return dict(d_x=d_x, d_scale=d_scale, d_shift=d_shift, mean=mean, rstd=rstd)


def ln_modulate_backward_f32(x, scale, d_out, eps, rows_per_batch=None):
    """The fp32 stream of the backward: x, scale, d_out float32; returns
    dict(d_x (float32), d_scale, d_shift, mean, rstd)."""
    x, d_out = _f32(x), _f32(d_out)
    rows, cols = x.shape
    scale = _f32(scale)
    if scale.ndim == 1:
        scale = scale.reshape(1, -1)
    stride = scale.shape[1]
    rpb = rows_per_batch or max(rows, 1)
    nb = rows // rpb if rows else 0
    d_x = np.empty_like(x)
    d_scale = np.empty((nb, cols), np.float32)
    d_shift = np.empty((nb, cols), np.float32)
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    _check(_load().oracle_ln_modulate_backward_f32(
        _p(x, _f32p), _p(scale, _f32p), _p(d_out, _f32p), rows, cols, rpb, stride, eps,
        _p(d_x, _f32p), _p(d_scale, _f32p), _p(d_shift, _f32p), _p(mean, _f32p),
        _p(rstd, _f32p)))
    return dict(d_x=d_x, d_scale=d_scale, d_shift=d_shift, mean=mean, rstd=rstd)


def gated_ln_modulate(update, residual, gate, scale, shift, eps, rows_per_batch=None):
    update, residual = _u16(update), _u16(residual)
    rows, cols = update.shape
    gate, stride = _mod_rows(gate, cols)
    scale, s2 = _mod_rows(scale, cols)
    shift, s3 = _mod_rows(shift, cols)
    assert stride == s2 == s3
    rpb = rows_per_batch or max(rows, 1)
    h = np.empty_like(update)
    out = np.empty_like(update)
    y = np.empty_like(update)
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    _check(_load().oracle_gated_ln_modulate(
        _p(update, _u16p), _p(residual, _u16p), _p(gate, _u16p), _p(scale, _u16p),
        _p(shift, _u16p), _p(h, _u16p), _p(out, _u16p), rows, cols, rpb, stride, eps,
        _p(mean, _f32p), _p(rstd, _f32p), _p(y, _u16p)))
    return dict(h=h, out=out, mean=mean, rstd=rstd, y=y)


def rms_modulate(x, weight, scale, shift, eps, residual=None, gate=None, rows_per_batch=None):
    x, weight = _u16(x), _u16(weight)
    rows, cols = x.shape
    scale, stride = _mod_rows(scale, cols)
    shift, _ = _mod_rows(shift, cols)
    rpb = rows_per_batch or max(rows, 1)
    gated = residual is not None
    if gated:
        residual = _u16(residual)
        gate, gs = _mod_rows(gate, cols)
        assert gs == stride
    h = np.empty_like(x) if gated else None
    out = np.empty_like(x)
    y = np.empty_like(x)
    rstd = np.empty(rows, np.float32)
    _check(_load().oracle_rms_modulate(
        _p(x, _u16p), _p(weight, _u16p), _p(scale, _u16p), _p(shift, _u16p), _p(out, _u16p),
        _p(residual, _u16p), _p(gate, _u16p), _p(h, _u16p), rows, cols, rpb, stride, eps,
        _p(rstd, _f32p), _p(y, _u16p)))
    return dict(out=out, h=h, rstd=rstd, y=y)


def qk_layernorm(q, k, eps, head_dim=128):
    q = _u16(q).reshape(-1, head_dim)
    k = _u16(k).reshape(-1, head_dim)
    rq, rk = q.shape[0], k.shape[0]
    qo, ko = np.empty_like(q), np.empty_like(k)
    mean = np.empty(rq + rk, np.float32)
    rstd = np.empty(rq + rk, np.float32)
    _check(_load().oracle_qk_layernorm(_p(q, _u16p), _p(k, _u16p), _p(qo, _u16p), _p(ko, _u16p),
                                       rq, rk, head_dim, eps, _p(mean, _f32p), _p(rstd, _f32p)))
    return dict(q_out=qo, k_out=ko, mean=mean, rstd=rstd)


def rmsnorm_silu_bias(x, bias, gamma, eps):
    """x: [rows, C] channels_last rows (uint16); bias: fp32 [C] or None."""
    x = _u16(x)
    rows, ch = x.shape
    bias, gamma = _f32(bias), _f32(gamma)
    out = np.empty_like(x)
    xb = np.empty_like(x)
    rstd = np.empty(rows, np.float32)
    _check(_load().oracle_rmsnorm_silu_bias(_p(x, _u16p), _p(bias, _f32p), _p(gamma, _f32p),
                                            _p(out, _u16p), rows, ch, eps, _p(rstd, _f32p),
                                            _p(xb, _u16p)))
    return dict(out=out, rstd=rstd, xb=xb)


def conv_bias_epilogue(x, bias, h=None):
    x = _u16(x)
    rows, ch = x.shape
    bias = _f32(bias)
    h = None if h is None else _u16(h)
    out = np.empty_like(x)
    _check(_load().oracle_conv_bias_epilogue(_p(x, _u16p), _p(bias, _f32p), _p(h, _u16p),
                                             _p(out, _u16p), rows, ch))
    return out


def conv_bias_epilogue_dt(x, bias, h=None, dtype="bf16", bias_dtype="f32"):
    """Conv-bias epilogue over a storage type: x, h as uint16 bit patterns
    (bf16, f16) or float32 (f32); bias float32 (bias_dtype "f32") or of x's
    type."""
    def arr(a, dt):
        return np.ascontiguousarray(a, np.float32 if dt == "f32" else np.uint16)
    x = arr(x, dtype)
    rows, ch = x.shape
    bias = arr(bias, bias_dtype)
    h = None if h is None else arr(h, dtype)
    out = np.empty_like(x)
    ptr = lambda a: None if a is None else a.ctypes.data
    _check(_load().oracle_conv_bias_epilogue_dt(ptr(x), ptr(bias), ptr(h), ptr(out), rows, ch,
                                                DTYPES[dtype], DTYPES[bias_dtype]))
    return out
