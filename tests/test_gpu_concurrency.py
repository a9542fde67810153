"""Concurrent use: entry points called from several host threads at once, each
thread on its own stream (default priority), must give the results the same
calls give one at a time -- the library keeps only per-device read-only state
(initialised under a lock on first use) and a thread-local last error."""
import threading

import numpy as np
import pytest
import torch

from dit_adaln_row_amd import inputs as gen
from parity import dev, host

pytestmark = pytest.mark.gpu


def rand(shape, mu, sigma, seed):
    return gen.to_u16(gen.normal(shape, mu, sigma, seed))


def _calls(dn, i):
    """Thread i's work: a different entry point and input per thread."""
    cols = (1024, 3072, 4096, 1000)[i % 4]
    x = dev(rand((300 + 17 * i, cols), 0, 1.5, 600 + i))
    sc = dev(rand((1, cols), 0, 0.1, 620 + i))
    sh = dev(rand((1, cols), 0, 0.1, 640 + i))
    w = dev(rand((cols,), 1, 0.05, 660 + i))
    kind = i % 3

    def run():
        if kind == 0:
            return [dn.ln_modulate(x, sc, sh, 1e-6)]
        if kind == 1:
            return [dn.rms_modulate(x, w, sc, sh, 1e-6)]
        d_x, d_scale, d_shift = dn.ln_modulate_backward(x, sc, x, 1e-6)
        return [d_x, d_scale, d_shift]
    return run


def test_concurrent_threads_and_streams(gpu):
    n = 6
    runs = [_calls(gpu, i) for i in range(n)]
    torch.cuda.synchronize()
    expected = [[host(t) for t in r()] for r in runs]
    torch.cuda.synchronize()

    results = [None] * n
    errors = []
    barrier = threading.Barrier(n)

    def worker(i):
        try:
            s = torch.cuda.Stream()
            barrier.wait(timeout=60)
            with torch.cuda.stream(s):
                outs = None
                for _ in range(20):
                    outs = runs[i]()
            s.synchronize()
            results[i] = [host(t) for t in outs]
        except Exception as e:  # reported below, in the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(n)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
    for i in range(n):
        for got, ref in zip(results[i], expected[i]):
            assert np.array_equal(np.asarray(got).view(np.uint8), np.asarray(ref).view(np.uint8)), \
                f"thread {i}: result differs from the serial call"
