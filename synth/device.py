"""Counter-based token values computed on the device (inputs only, no attention arithmetic).

For workloads too large to generate with numpy (the mixed trace processes about half a
million tokens), every value is a pure function of
``(seed, request, tensor, position, head, dim)``: the counter is hashed with splitmix64
(Steele, Lea and Flood, "Fast splittable pseudorandom number generators", 2014) into two
53-bit uniforms, which the Box-Muller transform turns into one N(0, 1) value, rounded to
bf16 by torch's round-to-nearest-even conversion. Being stateless, the same token gets the
same value whichever batch, step or process asks for it; the values depend on the device's
float math, so a run compares values generated on one device only (the oracle receives
copies of the device-generated values).
"""

from __future__ import annotations

import math

import torch

_MASK64 = (1 << 64) - 1


def _s64(x: int) -> int:
    """A 64-bit constant as the signed value torch's int64 arithmetic wraps to."""
    x &= _MASK64
    return x - (1 << 64) if x >= (1 << 63) else x


_GOLDEN = _s64(0x9E3779B97F4A7C15)
_M1 = _s64(0xBF58476D1CE4E5B9)
_M2 = _s64(0x94D049BB133111EB)


def _lsr(z: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (z >> k) & ((1 << (64 - k)) - 1)


def splitmix64(x: torch.Tensor) -> torch.Tensor:
    z = x + _GOLDEN
    z = (z ^ _lsr(z, 30)) * _M1
    z = (z ^ _lsr(z, 27)) * _M2
    return z ^ _lsr(z, 31)


def counters(seed: int, req: torch.Tensor, tensor: int, pos: torch.Tensor, heads: int,
             dim: int) -> torch.Tensor:
    """Distinct int64 counters for ``[T][heads][dim]`` elements of tokens (req[t], pos[t])."""
    base = splitmix64(splitmix64(req.to(torch.int64) * 4 + tensor + _s64(int(seed) << 40)) ^ pos.to(torch.int64))
    lane = torch.arange(heads * dim, device=req.device, dtype=torch.int64).view(1, heads, dim)
    return base.view(-1, 1, 1) * (heads * dim) + lane


def normal_tokens(seed: int, req: torch.Tensor, tensor: str, pos: torch.Tensor, heads: int,
                  dim: int, dtype: torch.dtype = torch.bfloat16, scale: float = 1.0) -> torch.Tensor:
    """N(0, 1) * scale values ``[T][heads][dim]`` for tokens (req[t], pos[t]), as ``dtype``."""
    tid = {"q": 1, "k": 2, "v": 3}[tensor]
    c = counters(seed, req, tid, pos, heads, dim)
    a = splitmix64(c)
    b = splitmix64(c ^ _s64(0x5851F42D4C957F2D))
    u1 = (_lsr(a, 11).to(torch.float64) + 1.0) * (1.0 / (1 << 53))   # (0, 1]
    u2 = _lsr(b, 11).to(torch.float64) * (1.0 / (1 << 53))           # [0, 1)
    z = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * math.pi * u2)
    return (z * scale).to(torch.float32).to(dtype)
