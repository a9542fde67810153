"""ln_modulate_backward_noalloc against ln_modulate_backward, through the C ABI.

The no-allocation entry point runs the same kernels with the partial token
sums in the library's per-device scratch array instead of the caller's
workspace, so every output must be bitwise the workspace entry point's: d_x,
d_scale, d_shift, mean and rstd.  Two calls in a row, the second smaller, so
the second runs over the first's leftovers in the scratch array; the
workspace of the reference call is filled with NaN so that neither result can
lean on memory that starts at zero.  Then a call whose partial sums exceed the
scratch array is refused on the host (outputs untouched).
"""
import ctypes

import numpy as np
import pytest
import torch

import dit_adaln_row_amd as dn
from dit_adaln_row_amd import inputs as gen

pytestmark = pytest.mark.gpu


def _inputs(B, S, D, seed, dt=0):
    kind = "f32" if dt == 2 else "bf16"
    x = gen.normal((B * S, D), 0.2, 1.5, seed, kind).cuda()
    sc = gen.normal((B, D), 0, 0.1, seed + 1, kind).cuda()
    dout = gen.normal((B * S, D), 0, 1.0, seed + 2, kind).cuda()
    return x, sc, dout


def _outputs(B, S, D, fill, dt=0):
    f32 = dict(dtype=torch.float32, device="cuda")
    xt = torch.float32 if dt == 2 else torch.bfloat16
    return dict(d_x=torch.full((B * S, D), fill, dtype=xt, device="cuda"),
                d_scale=torch.full((B, D), fill, **f32), d_shift=torch.full((B, D), fill, **f32),
                mean=torch.full((B * S,), fill, **f32), rstd=torch.full((B * S,), fill, **f32))


def _host(o):
    torch.cuda.synchronize()
    return {k: v.view(torch.int16).cpu().numpy() if v.dtype == torch.bfloat16
            else v.cpu().numpy().view(np.uint32) for k, v in o.items()}


def _call_workspace(lib, x, sc, dout, o, B, S, D, stream, dt=0):
    need = lib.ln_modulate_backward_workspace_bytes(B * S, D, S, dt)
    assert need >= 0
    ws = torch.full((max(need, 1) // 4 + 1,), float("nan"), dtype=torch.float32, device="cuda")
    st = lib.ln_modulate_backward(x.data_ptr(), sc.data_ptr(), dout.data_ptr(),
                                  o["d_x"].data_ptr(), o["d_scale"].data_ptr(),
                                  o["d_shift"].data_ptr(), B * S, D, S, D, ctypes.c_float(1e-6),
                                  ws.data_ptr() if need else None, need,
                                  o["mean"].data_ptr(), o["rstd"].data_ptr(), dt, stream)
    assert st == dn.OK, lib.ditnorm_status_string(st)
    torch.cuda.synchronize()
    del ws
    return need


def _call_noalloc(lib, x, sc, dout, o, B, S, D, stream, dt=0):
    return lib.ln_modulate_backward_noalloc(x.data_ptr(), sc.data_ptr(), dout.data_ptr(),
                                            o["d_x"].data_ptr(), o["d_scale"].data_ptr(),
                                            o["d_shift"].data_ptr(), B * S, D, S, D,
                                            ctypes.c_float(1e-6), o["mean"].data_ptr(),
                                            o["rstd"].data_ptr(), dt, stream)


# the Qwen-Image final stream (21.4 MB of partial sums), then smaller
# launches: several batches, fewer columns, one tree level; the fp32 stream
CALLS = [(1, 6889, 3072, 7100, 0), (3, 100, 1024, 7200, 0), (2, 40, 1536, 7400, 2)]


def test_noalloc_matches_workspace_entry(gpu):
    lib = dn.load()
    stream = torch.cuda.current_stream().cuda_stream
    for B, S, D, seed, dt in CALLS:
        print(f"noalloc vs workspace: B={B} S={S} D={D} dtype={dt}", flush=True)
        x, sc, dout = _inputs(B, S, D, seed, dt)
        ref = _outputs(B, S, D, float("nan"), dt)
        need = _call_workspace(lib, x, sc, dout, ref, B, S, D, stream, dt)
        assert 0 < need <= dn.NOALLOC_SCRATCH_BYTES
        got = _outputs(B, S, D, -7.0, dt)
        st = _call_noalloc(lib, x, sc, dout, got, B, S, D, stream, dt)
        assert st == dn.OK, lib.ditnorm_status_string(st)
        r, g = _host(ref), _host(got)
        for k in r:
            assert np.array_equal(r[k], g[k]), f"B={B} S={S} D={D}: {k} differs"


def test_noalloc_refuses_beyond_scratch(gpu):
    lib = dn.load()
    B, S, D = 1, 12000, 3072  # 36.9 MB of partial sums
    assert lib.ln_modulate_backward_workspace_bytes(B * S, D, S, 0) > dn.NOALLOC_SCRATCH_BYTES
    x, sc, dout = _inputs(B, S, D, 7300)
    got = _outputs(B, S, D, -7.0)
    st = _call_noalloc(lib, x, sc, dout, got, B, S, D, torch.cuda.current_stream().cuda_stream)
    assert st == dn.SCRATCH_EXCEEDED
    assert lib.ditnorm_status_string(st) == b"DITNORM_SCRATCH_EXCEEDED"
    h = _host(got)
    assert (h["d_scale"] == np.float32(-7.0).view(np.uint32)).all()  # nothing ran
