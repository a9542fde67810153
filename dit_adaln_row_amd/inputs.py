"""Seeded synthetic inputs, shared by the tests and the benchmark.

Only random-number generation and dtype plumbing live here (torch's seeded
generators and its float->bf16 conversion); none of the method's arithmetic.
"""
from __future__ import annotations

import numpy as np
import torch

from .workloads import WORKLOADS, Workload


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, mu, sigma, seed, kind="bf16", device="cpu") -> torch.Tensor:
    """N(mu, sigma) samples.  kind: bf16 | f16 | f32 | f32_bf16vals."""
    g = generator(seed, device)
    z = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    v = z.mul_(sigma).add_(mu)
    if kind == "bf16":
        return v.to(torch.bfloat16)
    if kind == "f16":
        return v.to(torch.float16)
    if kind == "f32":
        return v
    if kind == "f32_bf16vals":
        return v.to(torch.bfloat16).to(torch.float32)
    raise ValueError(kind)


def random_bits(shape, seed) -> np.ndarray:
    """Uniformly random 16-bit patterns (every class: zeros, subnormals,
    normals, infinities, NaNs), as numpy uint16."""
    g = generator(seed)
    v = torch.randint(0, 1 << 16, tuple(shape), generator=g, dtype=torch.int32)
    return v.numpy().astype(np.uint16)


def make(workload: Workload | str, names=None, device="cpu", seed_offset=0):
    """Dict name -> tensor for a workload (all tensors, or ``names``)."""
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    out = {}
    for t in w.tensors:
        if names is not None and t.name not in names:
            continue
        out[t.name] = normal(t.shape, t.mu, t.sigma, w.seed(t.name) + 1000003 * seed_offset,
                             t.kind, device)
    return out


def to_u16(t: torch.Tensor) -> np.ndarray:
    """bf16 or fp16 tensor -> numpy uint16 bit patterns (host copy)."""
    assert t.dtype in (torch.bfloat16, torch.float16)
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def from_u16(a: np.ndarray, device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 (or fp16) tensor."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).view(dtype).to(device)


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 with torch's conversion (input plumbing only)."""
    return to_u16(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16))


def f32_from_u16(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp32 values."""
    return (np.asarray(a, dtype=np.uint32) << 16).view(np.float32)
