"""dit_adaln_row_amd -- fused adaLN row normalisation kernels for MI355X (gfx950).

Python binding of ``libditnorm.so`` (C ABI in ``include/ditnorm.h``).  The
binding only marshals arguments: it checks dtypes / devices / layouts,
allocates outputs with torch when the caller does not pass them, and hands
raw device pointers and the current HIP stream to the library.  Every step of
the computation runs in the library's HIP kernels; there is no other
implementation to fall back to -- if the library is missing or rejects a call,
the call raises.

Entry points (same names as the C ABI):
    ln_modulate, ln_modulate_folded, gated_ln_modulate, rms_modulate, qk_layernorm,
    rmsnorm_silu_bias, conv_bias_epilogue, modulate_scale_shift, residual_gate_add,
    ln_modulate_backward (+ ln_modulate_backward_workspace_bytes),
    ln_modulate_backward_noalloc, copy
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["load", "ln_modulate", "ln_modulate_folded", "gated_ln_modulate", "rms_modulate", "qk_layernorm",
           "rmsnorm_silu_bias", "conv_bias_epilogue", "modulate_scale_shift",
           "residual_gate_add", "ln_modulate_backward", "ln_modulate_backward_workspace_bytes",
           "ln_modulate_backward_noalloc", "copy", "DitnormError", "LIB_PATH",
           "NOALLOC_SCRATCH_BYTES"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libditnorm.so")

OK, INVALID_ARGUMENT, UNSUPPORTED, DEVICE_ERROR, SCRATCH_EXCEEDED = 0, 1, 2, 3, 4
# bytes of the library's per-device scratch array (DITNORM_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 33554432


class DitnormError(RuntimeError):
    def __init__(self, fn, status, hip_error):
        self.status = status
        self.hip_error = hip_error
        name = _lib.ditnorm_status_string(status).decode() if _lib else str(status)
        super().__init__(f"{fn}: {name} (status {status}, last hipError {hip_error})")


_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_i32 = ctypes.c_int

# storage types of the standalone elementwise entry points (DITNORM_DTYPE_*)
_DTYPE_CODES = {torch.bfloat16: 0, torch.float16: 1}
# ... of the conv-bias epilogue, and of the backward
_EPI_DTYPES = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}
_BWD_DTYPES = {torch.bfloat16: 0, torch.float32: 2}

_SIGNATURES = {
    "ln_modulate": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp],
    "ln_modulate_folded": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp],
    "gated_ln_modulate": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32,
                          _vp, _vp, _vp, _vp],
    "rms_modulate": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32,
                     _vp, _vp, _vp],
    "qk_layernorm": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _vp, _vp, _vp],
    "rmsnorm_silu_bias": [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp, _vp, _vp],
    "conv_bias_epilogue": [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _vp],
    "modulate_scale_shift": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32, _vp],
    "residual_gate_add": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32, _vp],
    "ln_modulate_backward": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _vp,
                             _i64, _vp, _vp, _i32, _vp],
    "ln_modulate_backward_noalloc": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                     _f32, _vp, _vp, _i32, _vp],
    "ditnorm_copy": [_vp, _vp, _i64, _vp],
    "ln_modulate_supported": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp],
    "ln_modulate_folded_supported": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _vp,
                                     _vp],
    "gated_ln_modulate_supported": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                    _f32, _vp, _vp, _vp],
    "rms_modulate_supported": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                               _f32, _vp, _vp],
    "qk_layernorm_supported": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _vp, _vp],
    "rmsnorm_silu_bias_supported": [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp, _vp],
    "conv_bias_epilogue_supported": [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32],
    "modulate_scale_shift_supported": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32],
    "residual_gate_add_supported": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32],
    "ln_modulate_backward_supported": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                       _f32, _vp, _i64, _vp, _vp, _i32],
    "ditnorm_last_hip_error": [],
    "ditnorm_version": [],
}


def load(path: str = LIB_PATH):
    """Load the HIP library (once).  Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m dit_adaln_row_amd.build`")
        lib = ctypes.CDLL(path)
        for name, args in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.ln_modulate_backward_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32]
        lib.ln_modulate_backward_workspace_bytes.restype = _i64
        lib.ditnorm_status_string.argtypes = [ctypes.c_int]
        lib.ditnorm_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _call(name, *args):
    lib = load()
    st = getattr(lib, name)(*args)
    if st != OK:
        raise DitnormError(name, st, lib.ditnorm_last_hip_error())


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _p(t):
    return None if t is None else t.data_ptr()


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _act(t, name, dtype=torch.bfloat16, device=None):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda or (device is not None and t.device != device):
        raise TypeError(f"{name} must be a device tensor on {device or 'the GPU'}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    return t


def _like(t, ref, name):
    """A tensor the kernels read or write with the layout of `ref`: same dtype,
    device and shape, contiguous (the library cannot check allocation sizes)."""
    _act(t, name, ref.dtype, ref.device)
    if t.shape != ref.shape:
        raise ValueError(f"{name} must have the shape of the input, {tuple(ref.shape)}")
    return t


def _mod(t, name, cols, device, dtype=torch.bfloat16):
    """Modulation rows: (cols,), (B, cols) or (B, 1, cols), last dim dense; the
    batch stride may exceed cols (a chunk view of an adaLN embedding).
    Returns (tensor, B, batch_stride)."""
    if t.dtype != dtype or t.device != device:
        raise TypeError(f"{name} must be {dtype} on {device}")
    if t.shape[-1] != cols or t.stride(-1) != 1:
        raise ValueError(f"{name}: last dim must be {cols} and dense")
    if t.dim() == 1:
        return t, 1, cols
    if t.dim() == 3:
        if t.shape[1] != 1:
            raise ValueError(f"{name}: expected (B, 1, {cols})")
        b, stride = t.shape[0], t.stride(0)
    elif t.dim() == 2:
        b, stride = t.shape[0], t.stride(0)
    else:
        raise ValueError(f"{name}: expected (cols,), (B, cols) or (B, 1, cols)")
    return t, b, (stride if b > 1 else cols)


def _f32_out(t, n, name, device):
    if t is None:
        return None
    if t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous fp32 tensor of {n} elements")
    if t.device != device:
        raise TypeError(f"{name} must be on {device}")
    return t


def _rows_cols(x):
    cols = x.shape[-1]
    return x.numel() // cols if cols else 0, cols


def _batch(rows, b):
    if b < 1 or rows % b != 0:
        raise ValueError(f"{rows} rows are not divisible by {b} modulation rows")
    return max(rows // b, 1)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def ln_modulate(x, scale, shift, eps=1e-6, out=None, *, mean_out=None, rstd_out=None,
                y_out=None):
    """out = bf16(bf16(LN(x) * bf16(1+scale)) + shift); x (..., D) bf16."""
    _act(x, "x")
    rows, cols = _rows_cols(x)
    scale, b, stride = _mod(scale, "scale", cols, x.device)
    shift, b2, stride2 = _mod(shift, "shift", cols, x.device)
    if (b, stride) != (b2, stride2):
        raise ValueError("scale and shift must have the same batch count and stride")
    out = torch.empty_like(x) if out is None else _like(out, x, "out")
    dv = x.device
    _call("ln_modulate", _p(x), _p(scale), _p(shift), _p(out), rows, cols, _batch(rows, b),
          stride, eps, _p(_f32_out(mean_out, rows, "mean_out", dv)),
          _p(_f32_out(rstd_out, rows, "rstd_out", dv)),
          _p(None if y_out is None else _like(y_out, x, "y_out")), _stream(x))
    return out


def ln_modulate_folded(x, scale, shift, eps=1e-6, out=None, *, mean_out=None, rstd_out=None):
    """The lossy one-pass form: out = bf16((rstd*(x-mean)) * bf16(1+scale) + shift),
    fp32 ops on the unrounded normalised value; x (..., D) bf16."""
    _act(x, "x")
    rows, cols = _rows_cols(x)
    scale, b, stride = _mod(scale, "scale", cols, x.device)
    shift, b2, stride2 = _mod(shift, "shift", cols, x.device)
    if (b, stride) != (b2, stride2):
        raise ValueError("scale and shift must have the same batch count and stride")
    out = torch.empty_like(x) if out is None else _like(out, x, "out")
    _call("ln_modulate_folded", _p(x), _p(scale), _p(shift), _p(out), rows, cols,
          _batch(rows, b), stride, eps, _p(_f32_out(mean_out, rows, "mean_out", x.device)),
          _p(_f32_out(rstd_out, rows, "rstd_out", x.device)), _stream(x))
    return out


def gated_ln_modulate(x, residual, gate, scale, shift, eps=1e-6, out=None, residual_out=None,
                      *, mean_out=None, rstd_out=None, y_out=None):
    """h = bf16(residual + bf16(gate * x)); out = ln_modulate(h).  Returns (h, out)."""
    _act(x, "x")
    _like(residual, x, "residual")
    rows, cols = _rows_cols(x)
    gate, b, stride = _mod(gate, "gate", cols, x.device)
    scale, b2, s2 = _mod(scale, "scale", cols, x.device)
    shift, b3, s3 = _mod(shift, "shift", cols, x.device)
    if not (b == b2 == b3 and stride == s2 == s3):
        raise ValueError("gate, scale and shift must share batch count and stride")
    h = torch.empty_like(x) if residual_out is None else _like(residual_out, x, "residual_out")
    out = torch.empty_like(x) if out is None else _like(out, x, "out")
    dv = x.device
    _call("gated_ln_modulate", _p(x), _p(residual), _p(gate), _p(scale), _p(shift), _p(h),
          _p(out), rows, cols, _batch(rows, b), stride, eps,
          _p(_f32_out(mean_out, rows, "mean_out", dv)),
          _p(_f32_out(rstd_out, rows, "rstd_out", dv)),
          _p(None if y_out is None else _like(y_out, x, "y_out")), _stream(x))
    return h, out


def rms_modulate(x, weight, scale, shift, eps=1e-6, out=None, *, residual=None, gate=None,
                 residual_out=None, rstd_out=None, y_out=None):
    """Weighted RMSNorm + modulate.  With residual and gate (the gated site) the
    norm runs on h = bf16(residual + bf16(gate * x)) and (h, out) is returned;
    otherwise out."""
    _act(x, "x")
    rows, cols = _rows_cols(x)
    _act(weight, "weight", device=x.device)
    if weight.numel() != cols:
        raise ValueError("weight must have cols elements")
    scale, b, stride = _mod(scale, "scale", cols, x.device)
    shift, b2, s2 = _mod(shift, "shift", cols, x.device)
    gated = residual is not None
    if gated != (gate is not None):
        raise ValueError("residual and gate go together")
    if gated:
        _like(residual, x, "residual")
        gate, b3, s3 = _mod(gate, "gate", cols, x.device)
        if (b3, s3) != (b, stride):
            raise ValueError("gate must share batch count and stride with scale")
        residual_out = (torch.empty_like(x) if residual_out is None
                        else _like(residual_out, x, "residual_out"))
    if (b, stride) != (b2, s2):
        raise ValueError("scale and shift must share batch count and stride")
    out = torch.empty_like(x) if out is None else _like(out, x, "out")
    _call("rms_modulate", _p(x), _p(weight), _p(scale), _p(shift), _p(out), _p(residual),
          _p(gate), _p(residual_out if gated else None), rows, cols, _batch(rows, b), stride,
          eps, _p(_f32_out(rstd_out, rows, "rstd_out", x.device)),
          _p(None if y_out is None else _like(y_out, x, "y_out")), _stream(x))
    return (residual_out, out) if gated else out


def qk_layernorm(q, k, eps=1e-5, q_out=None, k_out=None, *, mean_out=None, rstd_out=None):
    """Per-head LayerNorm of q (..., head_dim) and k (..., head_dim) in one
    launch; head_dim a multiple of 8, at most 128 (the library rejects others)."""
    _act(q, "q")
    if q.dim() == 0:
        raise ValueError("q needs a head dimension")
    head_dim = q.shape[-1]
    rows_q = q.numel() // head_dim if head_dim else 0
    if k is not None:
        _act(k, "k", device=q.device)
        if k.dim() == 0 or k.shape[-1] != head_dim:
            raise ValueError("q and k must have the same head_dim")
    rows_k = 0 if k is None else k.numel() // head_dim
    q_out = torch.empty_like(q) if q_out is None else _like(q_out, q, "q_out")
    if k is not None:
        k_out = torch.empty_like(k) if k_out is None else _like(k_out, k, "k_out")
    n = rows_q + rows_k
    _call("qk_layernorm", _p(q), _p(k), _p(q_out), _p(k_out if k is not None else None),
          rows_q, rows_k, head_dim, eps, _p(_f32_out(mean_out, n, "mean_out", q.device)),
          _p(_f32_out(rstd_out, n, "rstd_out", q.device)), _stream(q))
    return q_out, k_out


def _channels_last_rows(x):
    """[rows, C] view of a channels_last(_3d) tensor or of a dense (..., C) tensor."""
    if x.dim() in (4, 5) and not x.is_contiguous():
        fmt = torch.channels_last if x.dim() == 4 else torch.channels_last_3d
        if not x.is_contiguous(memory_format=fmt):
            raise ValueError("x must be channels_last (NCDHW/NCHW-contiguous is rejected)")
        c = x.shape[1]
        return x.permute(0, *range(2, x.dim()), 1).reshape(-1, c), c
    if x.dim() in (4, 5):
        raise ValueError("x must be channels_last (NCDHW/NCHW-contiguous is rejected)")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    return x.reshape(-1, x.shape[-1]), x.shape[-1]


def _out_like(x, out):
    if out is None:
        return torch.empty_like(x)  # keeps channels_last strides
    if (out.shape != x.shape or out.stride() != x.stride() or out.dtype != x.dtype
            or out.device != x.device):
        raise ValueError("out must match x in shape, strides, dtype and device")
    return out


def rmsnorm_silu_bias(x, gamma, bias=None, eps=1e-6, out=None, *, rstd_out=None, xb_out=None):
    """channels_last x: out = bf16(SiLU(RMSNorm_C(bf16(x + bf16(bias))) * gamma))."""
    if x.dtype != torch.bfloat16 or not x.is_cuda:
        raise TypeError("x must be a bf16 device tensor")
    rows2d, c = _channels_last_rows(x)
    rows = rows2d.shape[0]
    for t, n in ((gamma, "gamma"), (bias, "bias")):
        if t is not None and (t.dtype != torch.float32 or t.numel() != c or not t.is_contiguous()
                              or t.device != x.device):
            raise ValueError(f"{n} must be a dense fp32 [{c}] device tensor")
    out = _out_like(x, out)
    if xb_out is not None:
        xb_out = _out_like(x, xb_out)
    _call("rmsnorm_silu_bias", _p(x), _p(bias), _p(gamma), _p(out), rows, c, eps,
          _p(_f32_out(rstd_out, rows, "rstd_out", x.device)), _p(xb_out), _stream(x))
    return out


def conv_bias_epilogue(x, bias, h=None, out=None):
    """channels_last x of bf16, fp16 or fp32: out = rnd(x + rnd(bias)) [then
    rnd(out + h)], rnd the rounding to x's type (the identity for fp32); the
    bias is fp32 or of x's type."""
    if x.dtype not in _EPI_DTYPES or not x.is_cuda:
        raise TypeError("x must be a bf16, fp16 or fp32 device tensor")
    rows2d, c = _channels_last_rows(x)
    if (bias.dtype not in (torch.float32, x.dtype) or bias.numel() != c
            or not bias.is_contiguous() or bias.device != x.device):
        raise ValueError(f"bias must be a dense fp32 or {x.dtype} [{c}] tensor on {x.device}")
    if h is not None and (h.shape != x.shape or h.stride() != x.stride() or h.dtype != x.dtype
                          or h.device != x.device):
        raise ValueError("h must match x in shape, strides, dtype and device")
    out = _out_like(x, out)
    _call("conv_bias_epilogue", _p(x), _p(bias), _p(h), _p(out), rows2d.shape[0], c,
          _EPI_DTYPES[x.dtype], _EPI_DTYPES[bias.dtype], _stream(x))
    return out


def _ew_dtype(x):
    if x.dtype not in _DTYPE_CODES:
        raise TypeError(f"expected bf16 or fp16, got {x.dtype}")
    return x.dtype


def modulate_scale_shift(x, scale, shift, out=None):
    """out = rnd(rnd(x * rnd(1 + scale)) + shift), rnd the storage type of x
    (bf16 or fp16); x (..., D), scale / shift (D,), (B, D) or (B, 1, D).
    out may be x (in place)."""
    dt = _ew_dtype(x)
    _act(x, "x", dt)
    rows, cols = _rows_cols(x)
    scale, b, stride = _mod(scale, "scale", cols, x.device, dt)
    shift, b2, stride2 = _mod(shift, "shift", cols, x.device, dt)
    if (b, stride) != (b2, stride2):
        raise ValueError("scale and shift must have the same batch count and stride")
    out = torch.empty_like(x) if out is None else _like(out, x, "out")
    _call("modulate_scale_shift", _p(x), _p(scale), _p(shift), _p(out), rows, cols,
          _batch(rows, b), stride, _DTYPE_CODES[dt], _stream(x))
    return out


def residual_gate_add(update, residual, gate, out=None):
    """out = rnd(residual + rnd(gate * update)), rnd the storage type (bf16 or
    fp16); update / residual (..., D), gate (D,), (B, D) or (B, 1, D).
    out may be residual (in place)."""
    dt = _ew_dtype(update)
    _act(update, "update", dt)
    _like(residual, update, "residual")
    rows, cols = _rows_cols(update)
    gate, b, stride = _mod(gate, "gate", cols, update.device, dt)
    out = torch.empty_like(update) if out is None else _like(out, update, "out")
    _call("residual_gate_add", _p(update), _p(residual), _p(gate), _p(out), rows, cols,
          _batch(rows, b), stride, _DTYPE_CODES[dt], _stream(update))
    return out


def ln_modulate_backward_workspace_bytes(rows, cols, rows_per_batch, dtype=torch.bfloat16):
    """Bytes of device workspace ln_modulate_backward needs (host-only)."""
    n = load().ln_modulate_backward_workspace_bytes(rows, cols, rows_per_batch,
                                                    _BWD_DTYPES[dtype])
    if n < 0:
        raise ValueError("invalid sizes")
    return n


def _bwd_args(x, scale, d_out, d_x, d_scale, d_shift):
    """Checked backward operands: x, d_out (..., D) and scale (D,), (B, D) or
    (B, 1, D) of one storage type (bf16, or fp32 for the fp32 stream)."""
    if x.dtype not in _BWD_DTYPES:
        raise TypeError(f"x must be bf16 or fp32, got {x.dtype}")
    _act(x, "x", dtype=x.dtype)
    _like(d_out, x, "d_out")
    rows, cols = _rows_cols(x)
    scale, b, stride = _mod(scale, "scale", cols, x.device, dtype=x.dtype)
    rpb = _batch(rows, b)
    d_x = torch.empty_like(x) if d_x is None else _like(d_x, x, "d_x")
    f32 = dict(dtype=torch.float32, device=x.device)
    d_scale = torch.empty((b, cols), **f32) if d_scale is None else d_scale
    d_shift = torch.empty((b, cols), **f32) if d_shift is None else d_shift
    for t, nm in ((d_scale, "d_scale"), (d_shift, "d_shift")):
        if (t.dtype != torch.float32 or t.numel() != b * cols or not t.is_contiguous()
                or t.device != x.device):
            raise ValueError(f"{nm} must be a contiguous fp32 tensor of {b}x{cols} on {x.device}")
    return rows, cols, scale, stride, rpb, d_x, d_scale, d_shift


def ln_modulate_backward(x, scale, d_out, eps=1e-6, *, d_x=None, d_scale=None, d_shift=None,
                         workspace=None, mean_out=None, rstd_out=None):
    """Gradients of LN(x) * (1 + scale) + shift: returns (d_x like x,
    d_scale fp32 [B, D], d_shift fp32 [B, D]).  x, d_out (..., D) and scale
    (D,), (B, D) or (B, 1, D), all bf16 or all fp32.  The workspace (uint8
    device tensor) is allocated here when the call needs one and none is
    given."""
    rows, cols, scale, stride, rpb, d_x, d_scale, d_shift = _bwd_args(
        x, scale, d_out, d_x, d_scale, d_shift)
    dt = _BWD_DTYPES[x.dtype]
    # -1 (sizes the call rejects): no workspace, and the call reports why
    need = load().ln_modulate_backward_workspace_bytes(rows, cols, rpb, dt) if rows else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace is not None and (workspace.device != x.device or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous device tensor on {x.device}")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("ln_modulate_backward", _p(x), _p(scale), _p(d_out), _p(d_x), _p(d_scale), _p(d_shift),
          rows, cols, rpb, stride, eps, _p(workspace), ws_bytes,
          _p(_f32_out(mean_out, rows, "mean_out", x.device)),
          _p(_f32_out(rstd_out, rows, "rstd_out", x.device)), dt, _stream(x))
    return d_x, d_scale, d_shift


def ln_modulate_backward_noalloc(x, scale, d_out, eps=1e-6, *, d_x=None, d_scale=None,
                                 d_shift=None, mean_out=None, rstd_out=None):
    """ln_modulate_backward with its partial sums in the library's own
    per-device scratch array instead of a workspace: the library call
    allocates nothing (outputs not given are allocated here with torch, so a
    caller that must not allocate passes d_x, d_scale and d_shift).  Raises
    DitnormError with status SCRATCH_EXCEEDED when the partial sums do not
    fit NOALLOC_SCRATCH_BYTES.  Calls overlapping in time on one device race
    on that array."""
    rows, cols, scale, stride, rpb, d_x, d_scale, d_shift = _bwd_args(
        x, scale, d_out, d_x, d_scale, d_shift)
    _call("ln_modulate_backward_noalloc", _p(x), _p(scale), _p(d_out), _p(d_x), _p(d_scale),
          _p(d_shift), rows, cols, rpb, stride, eps,
          _p(_f32_out(mean_out, rows, "mean_out", x.device)),
          _p(_f32_out(rstd_out, rows, "rstd_out", x.device)), _BWD_DTYPES[x.dtype], _stream(x))
    return d_x, d_scale, d_shift


def copy(src, dst):
    """Plain device copy through the library's 16-byte copy kernel (measurement utility)."""
    n = src.numel() * src.element_size()
    if (not src.is_cuda or dst.device != src.device or not src.is_contiguous()
            or not dst.is_contiguous() or dst.numel() * dst.element_size() < n):
        raise ValueError("copy: contiguous device tensors on one device, dst at least src's size")
    _call("ditnorm_copy", _p(src), _p(dst), n, _stream(src))
    return dst
