"""Closed forms of memory-centric tiling and the hidden-tier test, written out.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  The GPU library's planner
computes some of the same quantities in its own code; the two are compared in
tests, never shared.

Sources (page title, then section):
  [ZI-math]  ZeRO-Infinity, transformer-math page (aicassindra)
  [ZI-cn]    ZeRO-Infinity article, pwwt.cn (Chinese)
"""
from __future__ import annotations

import math

BYTES = {"f16": 2, "bf16": 2}


# --- tiling geometry ([ZI-cn] "关键技术一：Memory-centric tiling", core idea and the
#     hd=64K example; [ZI-math] "Memory-centric tiling: operators bigger than the device")

def tile_cols(M: int, N: int) -> int:
    """Output columns per tile when W[K x M] is split along M into N tiles.
    The pages split evenly; an uneven split is rejected."""
    if N < 1 or M % N:
        raise ValueError("N must divide M")
    return M // N


def tile_bytes(K: int, n: int, dtype: str = "f16") -> int:
    """Bytes of one weight tile W_i[K x n]."""
    return K * n * BYTES[dtype]


def tile_host_offset(i: int, K: int, n: int, dtype: str = "f16") -> int:
    """Byte offset of tile i in an out-major host copy W^t[M x K]: rows i*n.. of W^t."""
    return i * K * n * BYTES[dtype]


def tile_col_range(i: int, n: int):
    """Columns [i*n, (i+1)*n) of Y that tile i produces."""
    return i * n, (i + 1) * n


def working_bytes(layer_bytes: float, k: int, in_flight: bool = False) -> float:
    """Resident weight bytes with k tiles: layer_bytes/k, doubled with one
    tile in flight ([ZI-math] "Memory-centric tiling")."""
    return layer_bytes / k * (2 if in_flight else 1)


def weight_and_grad_tile_bytes(K: int, n: int, dtype: str = "f16") -> int:
    """A tile and its gradient resident together ([ZI-cn] hd=64K example)."""
    return 2 * tile_bytes(K, n, dtype)


# --- FLOPs and bytes ([ZI-math] "The FLOPs-per-byte test every tier must pass")

def flops_fwd(T: int, K: int, M: int) -> int:
    return 2 * T * K * M


def flops_bwd(T: int, K: int, M: int) -> int:
    """dX = dY W^T and dW = X^T dY: two products of the forward's size."""
    return 4 * T * K * M


def flops_checkpointed_step(P: float, T: float) -> float:
    """Forward 2P + recomputed forward 2P + backward 4P per token: 8PT."""
    return (2 * P + 2 * P + 4 * P) * T


def param_bytes_per_step(P: float, bytes_per_param: int = 2) -> float:
    """16-bit parameters climb the hierarchy twice per step: 2 * 2P bytes."""
    return 2 * bytes_per_param * P


def ait(flops: float, bytes_moved: float) -> float:
    """Arithmetic intensity: FLOPs done per byte moved."""
    return flops / bytes_moved


def ait_params(T: float) -> float:
    """8PT / 4P = 2T for checkpointed training with streamed parameters."""
    P = 1.0
    return ait(flops_checkpointed_step(P, T), param_bytes_per_step(P))


def machine_balance(R: float, BW: float) -> float:
    """R / BW: the ait a tier of bandwidth BW must reach to hide behind R FLOP/s."""
    return R / BW


def tier_hidden(ait_value: float, R: float, BW: float) -> bool:
    return ait_value >= machine_balance(R, BW)


def tokens_needed(R: float, BW: float) -> float:
    """Tokens per link that clear the bar when ait = 2T ([ZI-math] tier table)."""
    return machine_balance(R, BW) / 2.0


def efficiency(ait_value: float, R: float, BW: float) -> float:
    """min(1, ait / (R/BW)) for the binding tier ([ZI-math] "The honest cost")."""
    return min(1.0, ait_value / machine_balance(R, BW))


def adam_ait(flops_per_param: float = 12.0, bytes_per_param: float = 24.0) -> float:
    """Adam: about 12 FLOPs against 24 bytes read and written ([ZI-math] tier section)."""
    return flops_per_param / bytes_per_param


# --- fetch time and prefetch depth ([ZI-math] "Bandwidth-centric partitioning",
#     "Prefetch depth: how far ahead the pipeline must run")

def t_fetch_owner(layer_bytes: float, bw_one: float) -> float:
    return layer_bytes / bw_one


def t_fetch_striped(layer_bytes: float, dp: int, bw_one: float) -> float:
    return layer_bytes / (dp * bw_one)


def prefetch_depth(t_fetch: float, t_layer: float) -> int:
    """Smallest integer d with d >= t_fetch / t_layer (at least 1)."""
    return max(1, math.ceil(t_fetch / t_layer))


def prefetch_buffer_bytes(d: int, layer_bytes: float) -> float:
    return d * layer_bytes


# --- capacity ([ZI-math] "The ceiling that is advertised, and the one that binds")

def p_max(c_nvme_total_bytes: float, bytes_per_param: float = 16.0) -> float:
    return c_nvme_total_bytes / bytes_per_param


# --- host-link intensity of the tiled path on one GPU (our reading) ------------

def link_ait_fwd(T: int) -> float:
    """Forward: 2TKM FLOPs per K*M*2 bytes staged = T."""
    return ait(flops_fwd(T, 1, 1), 2)


def link_ait_bwd(T: int) -> float:
    """Backward: 4TKM FLOPs per K*M*2 bytes staged again = 2T."""
    return ait(flops_bwd(T, 1, 1), 2)


def link_ait_fwd_bwd(T: int) -> float:
    """Forward + backward: 6TKM FLOPs per 2*K*M*2 bytes staged = 1.5T."""
    return ait(flops_fwd(T, 1, 1) + flops_bwd(T, 1, 1), 4)


def ffn_tiled_h2d_bytes(P1: float, P2: float, bytes_per_param: int = 2) -> float:
    """FFN block with recompute when only a tile is resident: W1 staged for the
    forward, the recompute and the backward; W2 for the forward and once more
    for the recompute-plus-backward."""
    return bytes_per_param * (3 * P1 + 2 * P2)
