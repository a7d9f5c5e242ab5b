"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

This module holds none of the decode path's arithmetic: it only draws
random tensors (with torch's generators, whose float -> bfloat16 casts round
to nearest even) and random permutations.  Both the HIP path and the CPU
oracle read the buffers it produces; neither imports the other.

Recipe (distributions of the agentic / long-context workloads):
* Q, K, V activations ~ N(0, 1), stored as bf16.
* GDN q, k ~ N(0, 1) then L2-normalised per head (in float64) and stored as
  bf16; v ~ N(0, 1) bf16; alpha ~ U(0.9, 1), beta ~ U(0, 1) as float32.
* RMSNorm weights ~ U(0.5, 1.5) float32.
* Physical pages and slot ids are drawn as seeded permutations.

Seeds are derived from a path of integers with numpy's SeedSequence so every
tensor of every layer and step has its own independent stream.
"""

import numpy as np
import torch


def seed_of(*path):
    """63-bit seed for a path of non-negative integers."""
    ss = np.random.SeedSequence([0] + [int(x) for x in path])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64((1 << 63) - 1))


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_bf16(shape, seed, device="cpu", scale=1.0):
    g = _gen(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(torch.bfloat16)


def normal_bf16_offset(shape, seed, device="cpu"):
    """N(0,1) plus a per-last-dim offset ~ U(-1, 1) (the "structured" V whose
    attention output stays O(1) at long context)."""
    g = _gen(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    off = torch.rand(shape[-1], generator=g, device=device, dtype=torch.float32) * 2 - 1
    return (x + off).to(torch.bfloat16)


def normal_f32(shape, seed, device="cpu"):
    g = _gen(seed, device)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def uniform_f32(shape, lo, hi, seed, device="cpu"):
    g = _gen(seed, device)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo


def l2_normalised_bf16(shape, seed, device="cpu"):
    """Rows (last dim) ~ N(0, I) scaled to unit L2 norm in float64, then bf16."""
    g = _gen(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float64)
    x = x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)
    return x.to(torch.bfloat16)


def permutation(n, seed):
    rng = np.random.default_rng(seed)
    return rng.permutation(n).astype(np.int32)


def integers(lo, hi, size, seed):
    """Uniform integers in [lo, hi] inclusive."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=size)


def bits(t):
    """bf16 tensor -> numpy uint16 bit patterns (CPU copy)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
