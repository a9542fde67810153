"""The measurement copy (ditnorm_copy): the benchmark's bandwidth ceiling and
the counter calibration both assume it moves exactly the bytes asked for.
Its stores go through a buffer resource per workgroup, so sizes that end
inside a workgroup's 4 KB and inside a wavefront's 1 KB are checked, with a
guard region after the destination that must stay untouched."""
import pytest
import torch

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes after the destination that the copy must not touch


@pytest.mark.parametrize("nbytes", [16, 1024, 4096, 4096 + 16, 65536 - 48, 1 << 20,
                                    (1 << 20) + 4096 + 1024 + 16, 56623104])
def test_copy_moves_exactly_the_bytes(gpu, nbytes):
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.full((nbytes + GUARD,), 0xA5, dtype=torch.uint8, device="cuda")
    gpu.copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src), "copied bytes differ"
    assert bool((dst[nbytes:] == 0xA5).all()), "bytes past the copy were written"
