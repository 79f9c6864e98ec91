"""Seeded synthetic inputs.

This module holds no attention arithmetic.  It draws i.i.d. N(0, 1) values
with numpy's PCG64 generator and, for bf16 workloads, rounds them to bf16
(round to nearest even).  The same host bits feed both the GPU upload and
any CPU check, so both sides see identical inputs.

A tensor is generated in natural sequence order, as a flat array cut into
chunks of 2**24 elements; chunk k of the tensor with seed tuple ``seed`` comes
from ``numpy.random.default_rng([*seed, k]).standard_normal(dtype=float32)``.
The result does not depend on the thread count, and any element range can be
regenerated on its own.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 24


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.
    Inputs here are finite normals, so no NaN handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_range(seed: tuple, start: int, stop: int, dtype: str = "f32") -> np.ndarray:
    """Elements [start, stop) of the flat tensor with seed tuple ``seed``.

    dtype "f32" -> float32 values; "bf16" -> uint16 bf16 bit patterns.
    """
    n = stop - start
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    if n <= 0:
        return out
    first, last = start // CHUNK, (stop - 1) // CHUNK

    def work(k: int) -> None:
        lo, hi = k * CHUNK, (k + 1) * CHUNK
        a, b = max(lo, start), min(hi, stop)
        vals = np.random.default_rng([*seed, k]).standard_normal(b - lo, dtype=np.float32)[a - lo:]
        out[a - start:b - start] = vals if dtype == "f32" else bf16_rne_bits(vals)

    ks = range(first, last + 1)
    if len(ks) == 1:
        work(first)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, ks))
    return out


def normal_tensor(shape, seed: tuple, dtype: str = "f32") -> np.ndarray:
    n = int(np.prod(shape))
    return normal_range(seed, 0, n, dtype).reshape(shape)


def to_device(shape, seed: tuple, dtype: str, device="cuda", block_chunks: int = 32):
    """Generate a tensor block by block on the host and copy each block into a
    device tensor (host memory stays bounded for multi-GiB tensors).  The bits
    equal ``normal_tensor(shape, seed, dtype)``."""
    import torch

    n = int(np.prod(shape))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = torch.empty(n, dtype=tdt, device=device)
    step = CHUNK * block_chunks
    for a in range(0, n, step):
        b = min(n, a + step)
        host = torch.from_numpy(normal_range(seed, a, b, dtype))
        if dtype == "bf16":
            host = host.view(torch.bfloat16)
        out[a:b].copy_(host)
    return out.view(*shape)
