"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no arithmetic of the method: it only draws numbers.  Both
the GPU path and the CPU oracle consume what it writes, as the same host or
device bytes.

Recipe (one tensor = one (seed, tensor id) pair):
  * ``gaussian``: N(0, std^2) drawn in fp32 by torch's generator on the target
    device, then cast once (RNE) to fp16 / bf16.  Activations and upstream
    gradients use std = 1, weights std = 0.02 (0.02 read as the standard
    deviation).
  * ``small_int``: integers uniform on {lo, ..., hi} (default -3..3), exact in
    fp16 and bf16; every fp32 partial sum of the small shapes stays an
    integer below 2^24, so sums are exact in any order.
  * Large tensors that live in pinned host memory are drawn on the GPU in
    row chunks and copied down; chunk c of tensor (seed, id) uses generator
    seed ``mix(seed, id, c)``.
"""
from __future__ import annotations

import torch

TENSOR_IDS = {"X": 1, "W": 2, "dY": 3, "W1": 4, "W2": 5}

_TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def torch_dtype(dtype: str) -> torch.dtype:
    return _TORCH_DT[dtype]


def mix(seed: int, tensor_id: int, chunk: int = 0) -> int:
    """A 63-bit generator seed per (seed, tensor, chunk) (splitmix64 finaliser)."""
    z = (seed * 0x9E3779B97F4A7C15 + tensor_id * 0xBF58476D1CE4E5B9 + chunk * 0x94D049BB133111EB + 1) & (2**64 - 1)
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & (2**64 - 1)
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & (2**64 - 1)
    z ^= z >> 31
    return z & (2**63 - 1)


def _tid(tensor) -> int:
    return TENSOR_IDS[tensor] if isinstance(tensor, str) else int(tensor)


def fill_(out: torch.Tensor, kind: str, seed: int, tensor, std: float = 1.0,
          lo: int = -3, hi: int = 3, device=None, chunk_rows: int = 0) -> torch.Tensor:
    """Fill ``out`` (2-D, fp16/bf16, CPU/pinned or CUDA) in place.

    Numbers are drawn on ``device`` (default: ``out``'s device) in chunks of
    ``chunk_rows`` rows (default: all rows at once) and copied into ``out``."""
    if out.dim() != 2:
        raise ValueError("fill_ expects a 2-D tensor")
    dev = torch.device(device) if device is not None else out.device
    rows = out.shape[0]
    step = chunk_rows if chunk_rows > 0 else max(rows, 1)
    tid = _tid(tensor)
    for c, r0 in enumerate(range(0, rows, step)):
        r1 = min(rows, r0 + step)
        g = torch.Generator(device=dev)
        g.manual_seed(mix(seed, tid, c))
        shape = (r1 - r0, out.shape[1])
        if kind == "gaussian":
            v = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
            if std != 1.0:
                v.mul_(std)
        elif kind == "small_int":
            v = torch.randint(lo, hi + 1, shape, generator=g, device=dev, dtype=torch.int32)
        else:
            raise ValueError("kind must be 'gaussian' or 'small_int'")
        out[r0:r1].copy_(v.to(out.dtype), non_blocking=False)
    return out


def new(shape, dtype: str, kind: str, seed: int, tensor, std: float = 1.0, device="cpu",
        pin: bool = False, gen_device=None, chunk_rows: int = 0) -> torch.Tensor:
    """Allocate and fill a fresh tensor (pinned host memory when ``pin``)."""
    t = torch.empty(shape, dtype=torch_dtype(dtype), device=device, pin_memory=pin)
    return fill_(t, kind, seed, tensor, std=std, device=gen_device, chunk_rows=chunk_rows)


def bits(t: torch.Tensor):
    """uint16 numpy view of a CPU fp16/bf16 tensor's bytes (no copy)."""
    import numpy as np
    if t.device.type != "cpu":
        raise ValueError("bits() needs a host tensor")
    return t.view(torch.int16).numpy().view(np.uint16)
