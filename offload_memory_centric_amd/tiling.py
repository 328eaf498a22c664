"""Convenience layer over the binding: plans, contexts and pinned buffers.

torch is used here only for plumbing: device memory (workspace, activations)
and streams.  Every step of the tiled operator runs in libzi.so.
"""
from __future__ import annotations

import ctypes
import math
import weakref
from typing import Optional

import torch

from . import zi

def inputs_dtype(dtype: str) -> torch.dtype:
    return torch.float16 if dtype == "f16" else torch.bfloat16


_ELEM = {torch.float16: 2, torch.bfloat16: 2, torch.float32: 4, torch.uint8: 1, torch.int16: 2}


def host_tensor(shape, dtype: torch.dtype) -> torch.Tensor:
    """Page-locked host tensor of exactly this size (hipHostMalloc through
    zi_host_alloc); freed when the tensor is garbage-collected."""
    nbytes = int(math.prod(shape)) * _ELEM[dtype]
    ptr = zi.zi_host_alloc(nbytes)
    buf = (ctypes.c_uint8 * nbytes).from_address(ptr)
    weakref.finalize(buf, zi.zi_host_free, ptr)
    return torch.frombuffer(buf, dtype=torch.uint8).view(dtype).view(tuple(shape))


class Plan:
    """One tiled linear operator Y[T x M] = X[T x K] W[K x M] with W^t in pinned host memory."""

    def __init__(self, T: int, K: int, M: int, N: int, d: int, dtype: str, W_host: Optional[torch.Tensor],
                 dW_host: Optional[torch.Tensor] = None, budget: int = 0, f32_out: bool = False):
        self.problem = zi.zi_problem(T=T, K=K, M=M, N=N, d=d, dtype=zi.DTYPE_CODES[dtype],
                                     flags=zi.ZI_FLAG_F32_OUT if f32_out else 0,
                                     device_budget_bytes=budget,
                                     W_host=None if W_host is None else W_host.data_ptr(),
                                     dW_host=None if dW_host is None else dW_host.data_ptr())
        if W_host is not None:
            _need(W_host, M * K, (inputs_dtype(dtype),), "W_host", device=False)
        self._keep = (W_host, dW_host)
        self.handle, self.info = zi.zi_plan_tiles(self.problem)
        self.T, self.K, self.M, self.N, self.d, self.dtype = T, K, M, N, d, dtype
        self.f32_out = f32_out

    @property
    def n(self) -> int:
        return self.info.n

    def predict(self, backward: int, flop_rate: float, h2d: float, d2h: float = 0.0):
        return zi.zi_plan_predict(self.handle, backward, flop_rate, h2d, d2h)

    def close(self):
        if self.handle:
            zi.zi_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _need(t, elems: int, dtypes, name: str, device: bool = True):
    """Host-side check that a tensor can hold what a pass will read or write."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if dtypes and t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if device and t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.numel() < elems:
        raise ValueError("%s holds %d elements, the pass needs %d" % (name, t.numel(), elems))


def _lp(plan) -> tuple:
    return (torch.float16,) if plan.dtype == "f16" else (torch.bfloat16,)


def _out(plan) -> tuple:
    return (torch.float32,) if plan.f32_out else _lp(plan)


# Compute units the copy streams may use (see zi_copy_stream_create).  The HIP
# runtime carries out some host<->device copies as copy kernels rather than on
# a DMA engine.  The device-to-host stream is confined to 8 compute units (one
# per XCD); the host-to-device stream is unconfined by default: runs of the FFN
# block with every copy forced onto copy kernels (HSA_ENABLE_SDMA=0) took the
# same time with that stream confined to 8 compute units or not, so the
# runtime's copy kernels for it do not keep to the stream's mask.
D2H_CUS = 8
H2D_CUS = 0


class Context:
    """The ring over a torch-allocated workspace and three streams.

    By default the context creates its own three streams, one after another, so
    that they sit on distinct hardware queues (see zi_stream_create): products,
    host-to-device copies (confined to ``h2d_cus`` compute units if nonzero),
    and device-to-host copies confined to ``d2h_cus`` (0: unconfined).  With ``gelu_split`` (the default) the
    workspace also holds what zi_gelu_split_bytes() asks for, so that the GeLU forward may split the
    reduction of its last, partial round of tiles.  With ``overlap`` (the default) it also
    makes a second product stream, on which forward passes whose tiles take
    few workgroup waves run every other tile's product.  The products do not run on torch's current stream: inputs
    must be complete before a call (torch.cuda.synchronize()), and outputs are
    ready once sync() returns.
    """

    def __init__(self, plan: Plan, device: str = "cuda", workspace_bytes: Optional[int] = None,
                 streams=None, d2h_cus: int = D2H_CUS, overlap: bool = True, h2d_cus: int = H2D_CUS,
                 gelu_split: bool = True):
        if workspace_bytes is None:
            # the ring, then (gelu_split) the GeLU forward's split workspace
            ring = int(plan.info.ring_bytes)
            workspace_bytes = (ring + 255) // 256 * 256 + zi.zi_gelu_split_bytes() if gelu_split else ring
        nbytes = int(workspace_bytes)
        self.handle = None
        self._own_streams = []
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        if streams is None:
            self._own_streams.append(zi.zi_stream_create())
            self._own_streams.append(zi.zi_copy_stream_create(h2d_cus) if h2d_cus else zi.zi_stream_create())
            self._own_streams.append(zi.zi_copy_stream_create(d2h_cus) if d2h_cus else zi.zi_stream_create())
            streams = tuple(self._own_streams)
        self.streams = streams
        self.handle = zi.zi_ctx_create(plan.handle, self.workspace, nbytes, *streams)
        if overlap:  # a second product stream for the forward passes (zi_ctx_set_second_stream)
            s2 = zi.zi_stream_create()
            self._own_streams.append(s2)
            zi.zi_ctx_set_second_stream(self.handle, s2)

    def fwd(self, plan: Plan, X, Y):
        _need(X, plan.T * plan.K, _lp(plan), "X")
        _need(Y, plan.T * plan.M, _out(plan), "Y")
        zi.zi_tiled_linear_fwd(self.handle, plan.handle, X, Y)

    def fwd_gelu(self, plan: Plan, X, A, H):
        """A = X W (RNE, or fp32 for an f32_out plan), H = RNE(GeLU(RNE(A)))."""
        _need(X, plan.T * plan.K, _lp(plan), "X")
        _need(A, plan.T * plan.M, _out(plan), "A")
        _need(H, plan.T * plan.M, _lp(plan), "H")
        zi.zi_tiled_linear_fwd_gelu(self.handle, plan.handle, X, A, H)

    def _bwd_args(self, plan: Plan, X, dY, dX):
        _need(X, plan.T * plan.K, _lp(plan), "X")
        _need(dY, plan.T * plan.M, _lp(plan), "dY")
        _need(dX, plan.T * plan.K, (torch.float32,), "dX")
        dW = plan._keep[1]
        if dW is None:
            raise ValueError("plan has no dW_host")
        _need(dW, plan.M * plan.K, _out(plan), "dW_host", device=False)

    def bwd(self, plan: Plan, X, dY, dX):
        self._bwd_args(plan, X, dY, dX)
        zi.zi_tiled_linear_bwd(self.handle, plan.handle, X, dY, dX)

    def bwd_recompute(self, plan: Plan, X, dY, dX, Yr):
        self._bwd_args(plan, X, dY, dX)
        _need(Yr, plan.T * plan.M, _out(plan), "Yr")
        zi.zi_tiled_linear_bwd_recompute(self.handle, plan.handle, X, dY, dX, Yr)

    def gelu_bwd(self, dtype: str, dH, A, dA, count: int):
        """dA = RNE(dH * GeLU'(A)); an fp32 dA receives the product unrounded."""
        lp = (torch.float16,) if dtype == "f16" else (torch.bfloat16,)
        _need(dH, count, (torch.float32,), "dH")
        _need(A, count, lp, "A")
        _need(dA, count, lp + (torch.float32,), "dA")
        if dA.dtype == torch.float32:
            zi.zi_gelu_bwd_f32(self.handle, zi.DTYPE_CODES[dtype], dH, A, dA, count)
        else:
            zi.zi_gelu_bwd(self.handle, zi.DTYPE_CODES[dtype], dH, A, dA, count)

    def attach_adam(self, plan: Plan, adam: Optional["Adam"]):
        """Update each tile of `plan` on the host as its gradient lands (see Adam);
        None detaches."""
        zi.zi_ctx_attach_adam(self.handle, plan.handle, None if adam is None else adam.handle)

    def attach_source(self, plan: Plan, source: Optional["FileSource"]):
        """Read `plan`'s tiles from a file source (see FileSource); None detaches."""
        zi.zi_ctx_attach_source(self.handle, plan.handle, None if source is None else source.handle)

    def sync(self):
        zi.zi_sync(self.handle)

    def set_debug(self, poison: bool = False, copy_delay_us: int = 0, dx_per_tile: bool = False):
        """Test aids (zi_ctx_set_debug): poison released slots; delay every tile copy;
        run dX products one workgroup per output block instead of persistent ones."""
        flags = (zi.ZI_DEBUG_POISON if poison else 0) | (zi.ZI_DEBUG_DX_PER_TILE if dx_per_tile else 0)
        zi.zi_ctx_set_debug(self.handle, flags, copy_delay_us)

    def set_timing(self, on: bool):
        zi.zi_ctx_set_timing(self.handle, on)

    def reset_stats(self):
        zi.zi_ctx_reset_stats(self.handle)

    def stats(self) -> dict:
        return zi.zi_ctx_stats(self.handle).as_dict()

    def timed_records(self) -> list:
        return zi.zi_ctx_timed_records(self.handle)

    def close(self):
        if self.handle:
            zi.zi_ctx_destroy(self.handle)
            self.handle = None
        while self._own_streams:
            zi.zi_stream_destroy(self._own_streams.pop())

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Adam:
    """Host Adam for one plan's weight (zi_adam_*): fp32 master, m and v of
    M x K elements each, in the layout of W^t, in host memory (torch CPU
    tensors).  master starts as the exact fp32 value of the plan's 16-bit
    W_host unless given; m and v start at zero."""

    def __init__(self, plan: Plan, lr: float = 1e-4, beta1: float = 0.9, beta2: float = 0.999,
                 eps: float = 1e-8, threads: int = 0, master: Optional[torch.Tensor] = None):
        W_host, dW_host = plan._keep
        if W_host is None or dW_host is None:
            raise ValueError("the plan needs W_host and dW_host")
        shape = (plan.M, plan.K)
        self.master = (W_host.float() if master is None else master).contiguous()
        if tuple(self.master.shape) != shape or self.master.dtype != torch.float32 or self.master.is_cuda:
            raise ValueError("master must be a host fp32 tensor of shape %s" % (shape,))
        self.m = torch.zeros(shape, dtype=torch.float32)
        self.v = torch.zeros(shape, dtype=torch.float32)
        self.hp = zi.zi_adam_hparams(lr=lr, beta1=beta1, beta2=beta2, eps=eps)
        self.plan = plan
        self.handle = zi.zi_adam_create(plan.handle, self.hp, self.master, self.m, self.v, threads)

    def wait(self):
        zi.zi_adam_wait(self.handle)

    def stats(self) -> dict:
        return zi.zi_adam_stats_get(self.handle)

    def close(self):
        if self.handle:
            zi.zi_adam_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class FileSource:
    """A plan's weight read from a file (zi_file_source_*): W^t [M x K] in the
    plan's dtype from byte `offset` on, read ahead of the passes into
    `staging` pinned tile buffers."""

    def __init__(self, plan: Plan, path: str, offset: int = 0, staging: int = 3, threads: int = 4):
        self.plan = plan
        self.handle = zi.zi_file_source_create(plan.handle, path, offset, staging, threads)

    def read(self, tile: int, dst) -> None:
        zi.zi_file_source_read(self.handle, tile, dst)

    def stats(self) -> dict:
        return zi.zi_file_source_stats_get(self.handle)

    def close(self):
        if self.handle:
            zi.zi_file_source_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Tier:
    """File sources read by one reader along the order the first step used
    them (zi_tier_*): add every source, run the steps, and call step() after
    each step's passes are enqueued."""

    def __init__(self, staging: int = 4, threads: int = 8):
        self.handle = zi.zi_tier_create(staging, threads)
        self.sources = []

    def add(self, source: FileSource) -> None:
        zi.zi_tier_add(self.handle, source.handle)
        self.sources.append(source)

    def step(self) -> None:
        zi.zi_tier_step(self.handle)

    def stats(self) -> dict:
        return zi.zi_tier_stats_get(self.handle)

    def close(self):
        if self.handle:
            zi.zi_tier_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def write_weight_file(path: str, W_host: torch.Tensor, chunk_bytes: int = 1 << 28) -> None:
    """Write a host weight's bytes to `path` (for a FileSource), in chunks."""
    flat = W_host.contiguous().view(torch.uint8).view(-1)
    with open(path, "wb") as f:
        for at in range(0, flat.numel(), chunk_bytes):
            f.write(flat[at:at + chunk_bytes].numpy())


def ffn_block_step(ctx: Context, p1: Plan, p2: Plan, X, A, H, Y, dY, dH, dA, dX, Yr, mid=None) -> None:
    """The feed-forward block with activation checkpointing, enqueued without
    host synchronisation (the ring carries prefetch across the calls):
    forward W1 (+GeLU), forward W2, recomputed forward W1 (+GeLU), backward W2
    with the recomputed W2 product, dA = dH * GeLU'(A), backward W1.  mid, if
    given, is called once the down-projection's backward is enqueued (a caller
    can mark that point on the product stream)."""
    ctx.fwd_gelu(p1, X, A, H)
    ctx.fwd(p2, H, Y)
    ctx.fwd_gelu(p1, X, A, H)
    ctx.bwd_recompute(p2, H, dY, dH, Yr)
    if mid is not None:
        mid()
    ctx.gelu_bwd(p1.dtype, dH, A, dA, A.numel())
    ctx.bwd(p1, X, dA, dX)
