"""HIP graph capture: the library's calls enqueue kernels only (no memset, no
allocation, no host synchronisation), so a step captured once replays with
new inputs.  One graph holds the two FLUX-like sites and the backward, another
the gated RMS site (quarter-row path), qk_layernorm and rmsnorm_silu_bias;
between replays the inputs change by ordinary eager copies, and every replay
is checked against the eager calls on the same inputs."""
import numpy as np
import pytest
import torch

from dit_adaln_row_amd import inputs as gen
from parity import dev, host

pytestmark = pytest.mark.gpu


def rand(shape, mu, sigma, seed):
    return gen.to_u16(gen.normal(shape, mu, sigma, seed))


def test_graph_capture_replays(gpu):
    rows, cols, S = 600, 3072, 600
    shapes = dict(x=(rows, cols), upd=(rows, cols), res=(rows, cols), dout=(rows, cols),
                  sc=(1, cols), sh=(1, cols), gate=(1, cols))
    static = {k: torch.empty(v, dtype=torch.bfloat16, device="cuda") for k, v in shapes.items()}

    def fill(seed):
        for i, (k, shp) in enumerate(sorted(shapes.items())):
            sigma = 0.1 if shp[0] == 1 else 1.5
            static[k].copy_(dev(rand(shp, 0, sigma, seed * 16 + i)))

    out = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    h = torch.empty_like(out)
    out2 = torch.empty_like(out)
    d_x = torch.empty_like(out)
    d_scale = torch.empty((1, cols), dtype=torch.float32, device="cuda")
    d_shift = torch.empty_like(d_scale)
    ws = torch.empty(max(gpu.ln_modulate_backward_workspace_bytes(rows, cols, S), 256),
                     dtype=torch.uint8, device="cuda")
    s = static

    def step():
        gpu.ln_modulate(s["x"], s["sc"], s["sh"], 1e-6, out=out)
        gpu.gated_ln_modulate(s["upd"], s["res"], s["gate"], s["sc"], s["sh"], 1e-6, out=out2,
                              residual_out=h)
        gpu.ln_modulate_backward(s["x"], s["sc"], s["dout"], 1e-6, d_x=d_x, d_scale=d_scale,
                                 d_shift=d_shift, workspace=ws)

    def snapshot():
        return [host(t) for t in (out, h, out2, d_x, d_scale, d_shift)]

    fill(1)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()

    for seed in (2, 3, 4):
        fill(seed)
        torch.cuda.synchronize()
        step()  # eager, same inputs
        torch.cuda.synchronize()
        eager = snapshot()
        for t in (out, h, out2, d_x, d_scale, d_shift):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref in zip(snapshot(), eager):
            assert np.array_equal(np.asarray(got).view(np.uint8), np.asarray(ref).view(np.uint8)), \
                f"replay with inputs {seed} differs from the eager calls"


def test_graph_capture_other_entries(gpu):
    """The RMS site at a row count that takes the quarter-row path (1040 rows
    of 4096), qk_layernorm and rmsnorm_silu_bias (C = 96) captured in one
    graph; three replays with new inputs, each equal to the eager calls."""
    rows, cols, heads, pixels = 1040, 4096, 3000, 5000
    shapes = dict(x=(rows, cols), res=(rows, cols), w=(cols,), sc=(1, cols), sh=(1, cols),
                  gate=(1, cols), q=(heads, 128), k=(heads // 2, 128), px=(pixels, 96))
    static = {k: torch.empty(v, dtype=torch.bfloat16, device="cuda") for k, v in shapes.items()}
    gamma = gen.normal((96,), 1, 0.05, 50, "f32_bf16vals").cuda()
    bias = gen.normal((96,), 0, 0.05, 51, "f32").cuda()

    def fill(seed):
        for i, (k, shp) in enumerate(sorted(shapes.items())):
            sigma = 0.1 if shp[0] == 1 else 1.5
            mu = 1.0 if k == "w" else 0.0
            static[k].copy_(dev(rand(shp, mu, 0.05 if k == "w" else sigma, seed * 16 + i)))

    s = static
    h = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(h)
    qo, ko = torch.empty_like(s["q"]), torch.empty_like(s["k"])
    po = torch.empty_like(s["px"])

    def step():
        gpu.rms_modulate(s["x"], s["w"], s["sc"], s["sh"], 1e-6, out=out, residual=s["res"],
                         gate=s["gate"], residual_out=h)
        gpu.qk_layernorm(s["q"], s["k"], 1e-5, q_out=qo, k_out=ko)
        gpu.rmsnorm_silu_bias(s["px"], gamma, bias, 1e-6, out=po)

    def snapshot():
        return [host(t) for t in (h, out, qo, ko, po)]

    fill(5)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()

    for seed in (6, 7, 8):
        fill(seed)
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        eager = snapshot()
        for t in (h, out, qo, ko, po):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, ref in zip(snapshot(), eager):
            assert np.array_equal(np.asarray(got).view(np.uint8), np.asarray(ref).view(np.uint8)), \
                f"replay with inputs {seed} differs from the eager calls"
