"""ctypes binding of libzi.so, one Python function per entry point of include/zi.h.

Argument marshalling only: every step of the tiled operator runs inside the
library.  Pointer arguments accept an int address or a torch tensor (its
``data_ptr()``); stream arguments accept an int handle or a ``torch.cuda.Stream``.
A non-OK status raises :class:`ZiError` carrying the status and the library's
error text.  Importing this module loads the library and fails loudly if it
has not been built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzi.so")

(ZI_OK, ZI_ERR_ARG, ZI_ERR_SHAPE, ZI_ERR_BUDGET, ZI_ERR_NOT_PINNED, ZI_ERR_ALIGN, ZI_ERR_HIP, ZI_ERR_STATE,
 ZI_ERR_IO) = range(9)
STATUS_NAMES = ["ZI_OK", "ZI_ERR_ARG", "ZI_ERR_SHAPE", "ZI_ERR_BUDGET", "ZI_ERR_NOT_PINNED",
                "ZI_ERR_ALIGN", "ZI_ERR_HIP", "ZI_ERR_STATE", "ZI_ERR_IO"]
ZI_F16, ZI_BF16 = 1, 2
ZI_FLAG_F32_OUT = 0x1
ZI_NOALLOC_SCRATCH_BYTES = 64 << 20  # static tile buffer of zi_tiled_linear_fwd_noalloc
DTYPE_CODES = {"f16": ZI_F16, "bf16": ZI_BF16}


class ZiError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__("%s: %s" % (name, message))


class zi_problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("K", ctypes.c_int64), ("M", ctypes.c_int64),
                ("N", ctypes.c_int32), ("d", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("device_budget_bytes", ctypes.c_uint64),
                ("W_host", ctypes.c_void_p), ("dW_host", ctypes.c_void_p)]


class zi_plan_info(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("tile_bytes", ctypes.c_uint64),
                ("dw_tile_bytes", ctypes.c_uint64), ("d", ctypes.c_int32),
                ("dw_slots", ctypes.c_int32), ("ring_bytes", ctypes.c_uint64),
                ("flops_fwd", ctypes.c_double), ("flops_bwd", ctypes.c_double),
                ("h2d_bytes_pass", ctypes.c_double), ("d2h_bytes_bwd", ctypes.c_double),
                ("ait_fwd", ctypes.c_double), ("ait_bwd", ctypes.c_double),
                ("working_bytes_one", ctypes.c_double), ("working_bytes_two", ctypes.c_double),
                ("fwd_tile", ctypes.c_int32 * 2), ("dw_tile", ctypes.c_int32 * 2)]


class zi_prediction(ctypes.Structure):
    _fields_ = [("t_pass_s", ctypes.c_double), ("t_compute_s", ctypes.c_double),
                ("t_link_s", ctypes.c_double), ("stall_frac", ctypes.c_double),
                ("d_pages", ctypes.c_int32)]


class zi_rate_curve(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int32), ("n", ctypes.POINTER(ctypes.c_int64)),
                ("fwd", ctypes.POINTER(ctypes.c_double)), ("dx", ctypes.POINTER(ctypes.c_double)),
                ("dw", ctypes.POINTER(ctypes.c_double)), ("h2d", ctypes.POINTER(ctypes.c_double)),
                ("d2h", ctypes.POINTER(ctypes.c_double))]


class zi_choice(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("d", ctypes.c_int32), ("n", ctypes.c_int64),
                ("dw_slots", ctypes.c_int32), ("ring_bytes", ctypes.c_uint64),
                ("t_fwd_s", ctypes.c_double), ("t_bwd_s", ctypes.c_double), ("t_step_s", ctypes.c_double)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


class zi_adam_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float)]


class zi_adam_stats(ctypes.Structure):
    _fields_ = [("tiles_done", ctypes.c_int64), ("busy_s", ctypes.c_double), ("bytes", ctypes.c_double)]


class zi_source_stats(ctypes.Structure):
    _fields_ = [("tiles_read", ctypes.c_int64), ("restarts", ctypes.c_int64), ("read_s", ctypes.c_double),
                ("bytes", ctypes.c_double), ("wait_s", ctypes.c_double), ("direct", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


class zi_tier_stats(ctypes.Structure):
    _fields_ = [("trace_len", ctypes.c_int64), ("steps", ctypes.c_int64), ("tiles_read", ctypes.c_int64),
                ("restarts", ctypes.c_int64), ("demand_reads", ctypes.c_int64), ("hits", ctypes.c_int64),
                ("read_s", ctypes.c_double),
                ("bytes", ctypes.c_double), ("wait_s", ctypes.c_double)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


ZI_STATS_KERNELS = 16


class zi_kernel_stats(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 24), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("red", ctypes.c_int64), ("launches", ctypes.c_int64), ("ms", ctypes.c_double),
                ("flops", ctypes.c_double), ("solo_launches", ctypes.c_int64), ("solo_ms", ctypes.c_double)]

    def as_dict(self) -> dict:
        d = {k: getattr(self, k) for k, _ in self._fields_}
        d["name"] = bytes(self.name).split(b"\0", 1)[0].decode()
        return d


class zi_stats(ctypes.Structure):
    _fields_ = [("kind_count", ctypes.c_int32), ("kind_name", (ctypes.c_char * 24) * 8),
                ("launches", ctypes.c_int64 * 8), ("kernel_ms", ctypes.c_double * 8),
                ("flops", ctypes.c_double * 8), ("h2d_copies", ctypes.c_int64),
                ("d2h_copies", ctypes.c_int64), ("h2d_ms", ctypes.c_double),
                ("d2h_ms", ctypes.c_double), ("h2d_bytes", ctypes.c_double),
                ("d2h_bytes", ctypes.c_double), ("span_ms", ctypes.c_double),
                ("compute_busy_ms", ctypes.c_double), ("kernel_count", ctypes.c_int32),
                ("kernel", zi_kernel_stats * ZI_STATS_KERNELS)]

    def as_dict(self):
        kinds = {}
        for k in range(self.kind_count):
            name = bytes(self.kind_name[k]).split(b"\0", 1)[0].decode()
            kinds[name] = {"launches": self.launches[k], "ms": self.kernel_ms[k], "flops": self.flops[k]}
        return {"kinds": kinds, "h2d_copies": self.h2d_copies, "d2h_copies": self.d2h_copies,
                "h2d_ms": self.h2d_ms, "d2h_ms": self.d2h_ms, "h2d_bytes": self.h2d_bytes,
                "d2h_bytes": self.d2h_bytes, "span_ms": self.span_ms,
                "compute_busy_ms": self.compute_busy_ms,
                "kernels": [self.kernel[i].as_dict() for i in range(self.kernel_count)]}


class zi_timed_rec(ctypes.Structure):
    _fields_ = [("what", ctypes.c_int32), ("kind", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("red", ctypes.c_int64), ("start_ms", ctypes.c_double),
                ("end_ms", ctypes.c_double)]


if not os.path.exists(LIB_PATH):
    raise ImportError("libzi.so is not built (expected at %s); run "
                      "`python -m offload_memory_centric_amd.build`" % LIB_PATH)
# torch ships its own HIP runtime under the same soname as the system's.  Load
# torch first so that libzi binds to that copy: a process that ends up with two
# HIP runtimes finds no device in the one that initialises second.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_S = ctypes.c_int  # zi_status
_sigs = {
    "zi_plan_tiles": (_S, [ctypes.POINTER(zi_problem), ctypes.POINTER(_P), ctypes.POINTER(zi_plan_info)]),
    "zi_plan_destroy": (_S, [_P]),
    "zi_prefetch_depth": (ctypes.c_int32, [ctypes.c_double, ctypes.c_double]),
    "zi_plan_predict": (_S, [_P, ctypes.c_int32, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                             ctypes.POINTER(zi_prediction)]),
    "zi_plan_choose": (_S, [ctypes.POINTER(zi_problem), ctypes.POINTER(zi_rate_curve), ctypes.c_double,
                            ctypes.c_double, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(zi_choice),
                            ctypes.POINTER(zi_choice), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]),
    "zi_ctx_create": (_S, [_P, _P, ctypes.c_uint64, _P, _P, _P, ctypes.POINTER(_P)]),
    "zi_gelu_split_bytes": (ctypes.c_uint64, []),
    "zi_ctx_destroy": (_S, [_P]),
    "zi_tiled_linear_fwd": (_S, [_P, _P, _P, _P]),
    "zi_tiled_linear_fwd_gelu": (_S, [_P, _P, _P, _P, _P]),
    "zi_tiled_linear_bwd": (_S, [_P, _P, _P, _P, _P]),
    "zi_tiled_linear_bwd_recompute": (_S, [_P, _P, _P, _P, _P, _P]),
    "zi_gelu_bwd": (_S, [_P, ctypes.c_int32, _P, _P, _P, ctypes.c_int64]),
    "zi_gelu_bwd_f32": (_S, [_P, ctypes.c_int32, _P, _P, _P, ctypes.c_int64]),
    "zi_tiled_linear_fwd_noalloc": (_S, [_P, _P, _P, _P]),
    "zi_sync": (_S, [_P]),
    "zi_ctx_set_timing": (_S, [_P, ctypes.c_int32]),
    "zi_ctx_set_debug": (_S, [_P, ctypes.c_uint32, ctypes.c_uint32]),
    "zi_ctx_set_second_stream": (_S, [_P, _P]),
    "zi_ctx_reset_stats": (_S, [_P]),
    "zi_ctx_stats": (_S, [_P, ctypes.POINTER(zi_stats)]),
    "zi_ctx_timed_records": (_S, [_P, ctypes.POINTER(zi_timed_rec), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]),
    "zi_stream_create": (_S, [ctypes.POINTER(_P)]),
    "zi_copy_stream_create": (_S, [ctypes.c_int32, ctypes.POINTER(_P)]),
    "zi_stream_destroy": (_S, [_P]),
    "zi_adam_update": (_S, [ctypes.POINTER(zi_adam_hparams), ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                            ctypes.c_int64, _P, _P, _P, _P, _P, ctypes.c_int32]),
    "zi_adam_create": (_S, [_P, ctypes.POINTER(zi_adam_hparams), _P, _P, _P, ctypes.c_int32,
                            ctypes.POINTER(_P)]),
    "zi_adam_destroy": (_S, [_P]),
    "zi_ctx_attach_adam": (_S, [_P, _P, _P]),
    "zi_adam_wait": (_S, [_P]),
    "zi_adam_stats_get": (_S, [_P, ctypes.POINTER(zi_adam_stats)]),
    "zi_file_source_create": (_S, [_P, ctypes.c_char_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.POINTER(_P)]),
    "zi_file_source_destroy": (_S, [_P]),
    "zi_ctx_attach_source": (_S, [_P, _P, _P]),
    "zi_file_source_read": (_S, [_P, ctypes.c_int64, _P]),
    "zi_file_source_stats_get": (_S, [_P, ctypes.POINTER(zi_source_stats)]),
    "zi_tier_create": (_S, [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_P)]),
    "zi_tier_add": (_S, [_P, _P]),
    "zi_tier_step": (_S, [_P]),
    "zi_tier_destroy": (_S, [_P]),
    "zi_tier_stats_get": (_S, [_P, ctypes.POINTER(zi_tier_stats)]),
    "zi_tier_trace_get": (_S, [_P, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
    "zi_tier_simulate_reads": (_S, [ctypes.POINTER(ctypes.c_int64), ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]),
    "zi_host_alloc": (_S, [ctypes.c_uint64, ctypes.POINTER(_P)]),
    "zi_host_free": (_S, [_P]),
    "zi_last_error": (ctypes.c_char_p, []),
    "zi_version": (ctypes.c_int32, []),
}
for _name, (_res, _args) in _sigs.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_sigs)


def _ptr(x) -> int:
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "__array_interface__"):  # numpy array
        return x.__array_interface__["data"][0]
    return int(x)


def _stream(s) -> int:
    if s is None:
        return None
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    return int(s)


def _check(status: int):
    if status != ZI_OK:
        raise ZiError(status, zi_last_error())


# ---- entry points ----------------------------------------------------------------

def zi_last_error() -> str:
    return (_lib.zi_last_error() or b"").decode(errors="replace")


def zi_version() -> int:
    return _lib.zi_version()


def zi_plan_tiles(problem: zi_problem, make_plan: bool = True):
    """Returns (plan handle or None, zi_plan_info)."""
    info = zi_plan_info()
    h = _P()
    _check(_lib.zi_plan_tiles(ctypes.byref(problem), ctypes.byref(h) if make_plan else None,
                              ctypes.byref(info)))
    return (h.value if make_plan else None), info


def zi_plan_destroy(plan) -> None:
    _check(_lib.zi_plan_destroy(plan))


def zi_prefetch_depth(t_fetch_s: float, t_layer_s: float) -> int:
    return _lib.zi_prefetch_depth(t_fetch_s, t_layer_s)


def zi_plan_predict(plan, backward: int, flop_rate: float, h2d_bytes_per_s: float,
                    d2h_bytes_per_s: float = 0.0) -> zi_prediction:
    out = zi_prediction()
    _check(_lib.zi_plan_predict(plan, int(backward), flop_rate, h2d_bytes_per_s, d2h_bytes_per_s,
                                ctypes.byref(out)))
    return out


def zi_plan_choose(problem: zi_problem, n, fwd, dx=None, dw=None, h2d_bytes_per_s: float = 0.0,
                   d2h_bytes_per_s: float = 0.0, backward: int = 1, max_d: int = 2, h2d=None, d2h=None):
    """(choice, table): the chosen tiling and every candidate considered, as dicts."""
    count = len(n)

    def arr(ctype, xs):
        if xs is None:
            return None
        if len(xs) != count:
            raise ValueError("every rate list needs one entry per width")
        return (ctype * count)(*xs)

    keep = [arr(ctypes.c_int64, [int(x) for x in n]), arr(ctypes.c_double, fwd),
            arr(ctypes.c_double, dx), arr(ctypes.c_double, dw), arr(ctypes.c_double, h2d),
            arr(ctypes.c_double, d2h)]
    curve = zi_rate_curve(count, *keep)
    out = zi_choice()
    cap = max(1, count * max(1, int(max_d)))
    table = (zi_choice * cap)()
    length = ctypes.c_int32()
    _check(_lib.zi_plan_choose(ctypes.byref(problem), ctypes.byref(curve), float(h2d_bytes_per_s),
                               float(d2h_bytes_per_s), int(backward), int(max_d), ctypes.byref(out),
                               table, cap, ctypes.byref(length)))
    return out.as_dict(), [table[i].as_dict() for i in range(min(cap, length.value))]


def zi_ctx_create(plan, workspace, workspace_bytes: int, compute_stream, h2d_stream, d2h_stream):
    h = _P()
    _check(_lib.zi_ctx_create(plan, _ptr(workspace), int(workspace_bytes), _stream(compute_stream),
                              _stream(h2d_stream), _stream(d2h_stream), ctypes.byref(h)))
    return h.value


def zi_ctx_destroy(ctx) -> None:
    _check(_lib.zi_ctx_destroy(ctx))


def zi_tiled_linear_fwd(ctx, plan, X, Y) -> None:
    _check(_lib.zi_tiled_linear_fwd(ctx, plan, _ptr(X), _ptr(Y)))


def zi_tiled_linear_fwd_gelu(ctx, plan, X, A, H) -> None:
    _check(_lib.zi_tiled_linear_fwd_gelu(ctx, plan, _ptr(X), _ptr(A), _ptr(H)))


def zi_tiled_linear_bwd(ctx, plan, X, dY, dX) -> None:
    _check(_lib.zi_tiled_linear_bwd(ctx, plan, _ptr(X), _ptr(dY), _ptr(dX)))


def zi_tiled_linear_bwd_recompute(ctx, plan, X, dY, dX, Yr) -> None:
    _check(_lib.zi_tiled_linear_bwd_recompute(ctx, plan, _ptr(X), _ptr(dY), _ptr(dX), _ptr(Yr)))


def zi_tiled_linear_fwd_noalloc(plan, X, Y, stream=None) -> None:
    _check(_lib.zi_tiled_linear_fwd_noalloc(plan, _ptr(X), _ptr(Y), _stream(stream)))


def zi_gelu_bwd(ctx, dtype: int, dH, A, dA, count: int) -> None:
    _check(_lib.zi_gelu_bwd(ctx, int(dtype), _ptr(dH), _ptr(A), _ptr(dA), int(count)))


def zi_gelu_bwd_f32(ctx, dtype: int, dH, A, dA, count: int) -> None:
    _check(_lib.zi_gelu_bwd_f32(ctx, int(dtype), _ptr(dH), _ptr(A), _ptr(dA), int(count)))


def zi_gelu_split_bytes() -> int:
    return int(_lib.zi_gelu_split_bytes())


def zi_stream_create() -> int:
    h = _P()
    _check(_lib.zi_stream_create(ctypes.byref(h)))
    return h.value


def zi_copy_stream_create(n_cus: int) -> int:
    h = _P()
    _check(_lib.zi_copy_stream_create(int(n_cus), ctypes.byref(h)))
    return h.value


def zi_stream_destroy(stream) -> None:
    _check(_lib.zi_stream_destroy(_stream(stream)))


def zi_sync(ctx) -> None:
    _check(_lib.zi_sync(ctx))


def zi_ctx_set_second_stream(ctx, stream) -> None:
    _check(_lib.zi_ctx_set_second_stream(ctx, _stream(stream)))


ZI_DEBUG_POISON = 0x1
ZI_DEBUG_DX_PER_TILE = 0x2


def zi_ctx_set_debug(ctx, flags: int = 0, copy_delay_us: int = 0) -> None:
    _check(_lib.zi_ctx_set_debug(ctx, int(flags), int(copy_delay_us)))


def zi_ctx_set_timing(ctx, enable: bool) -> None:
    _check(_lib.zi_ctx_set_timing(ctx, 1 if enable else 0))


def zi_ctx_reset_stats(ctx) -> None:
    _check(_lib.zi_ctx_reset_stats(ctx))


def zi_ctx_stats(ctx) -> zi_stats:
    out = zi_stats()
    _check(_lib.zi_ctx_stats(ctx, ctypes.byref(out)))
    return out


def zi_ctx_timed_records(ctx) -> list:
    """Every launch and copy timed since the last reset: dicts with what
    ("kernel", "h2d", "d2h"), kind (index into the stats' kinds, -1 for
    copies), rows, cols, red (copies: rows = bytes), start_ms, end_ms."""
    n = ctypes.c_int32(0)
    _check(_lib.zi_ctx_timed_records(ctx, None, 0, ctypes.byref(n)))
    buf = (zi_timed_rec * max(n.value, 1))()
    _check(_lib.zi_ctx_timed_records(ctx, buf, n.value, ctypes.byref(n)))
    names = ("kernel", "h2d", "d2h")
    return [{"what": names[r.what], "kind": r.kind, "rows": r.rows, "cols": r.cols, "red": r.red,
             "start_ms": r.start_ms, "end_ms": r.end_ms} for r in buf[:n.value]]


def zi_adam_update(hp: zi_adam_hparams, dtype: int, grad_f32: int, step: int, count: int, grad, master, m, v,
                   w, threads: int = 0) -> None:
    _check(_lib.zi_adam_update(ctypes.byref(hp), int(dtype), int(grad_f32), int(step), int(count), _ptr(grad),
                               _ptr(master), _ptr(m), _ptr(v), _ptr(w), int(threads)))


def zi_adam_create(plan, hp: zi_adam_hparams, master, m, v, threads: int = 0) -> int:
    h = _P()
    _check(_lib.zi_adam_create(plan, ctypes.byref(hp), _ptr(master), _ptr(m), _ptr(v), int(threads),
                               ctypes.byref(h)))
    return h.value


def zi_adam_destroy(adam) -> None:
    _check(_lib.zi_adam_destroy(adam))


def zi_ctx_attach_adam(ctx, plan, adam) -> None:
    _check(_lib.zi_ctx_attach_adam(ctx, plan, adam))


def zi_adam_wait(adam) -> None:
    _check(_lib.zi_adam_wait(adam))


def zi_adam_stats_get(adam) -> dict:
    s = zi_adam_stats()
    _check(_lib.zi_adam_stats_get(adam, ctypes.byref(s)))
    return {"tiles_done": s.tiles_done, "busy_s": s.busy_s, "bytes": s.bytes}


def zi_file_source_create(plan, path: str, offset: int = 0, staging: int = 3, threads: int = 4) -> int:
    h = _P()
    _check(_lib.zi_file_source_create(plan, os.fsencode(path), int(offset), int(staging), int(threads),
                                      ctypes.byref(h)))
    return h.value


def zi_file_source_destroy(src) -> None:
    _check(_lib.zi_file_source_destroy(src))


def zi_ctx_attach_source(ctx, plan, src) -> None:
    _check(_lib.zi_ctx_attach_source(ctx, plan, src))


def zi_file_source_read(src, tile: int, dst) -> None:
    _check(_lib.zi_file_source_read(src, int(tile), _ptr(dst)))


def zi_file_source_stats_get(src) -> dict:
    s = zi_source_stats()
    _check(_lib.zi_file_source_stats_get(src, ctypes.byref(s)))
    return s.as_dict()


def zi_tier_create(staging: int = 4, threads: int = 8) -> int:
    h = _P()
    _check(_lib.zi_tier_create(int(staging), int(threads), ctypes.byref(h)))
    return h.value


def zi_tier_add(tier, src) -> None:
    _check(_lib.zi_tier_add(tier, src))


def zi_tier_step(tier) -> None:
    _check(_lib.zi_tier_step(tier))


def zi_tier_destroy(tier) -> None:
    _check(_lib.zi_tier_destroy(tier))


def zi_tier_stats_get(tier) -> dict:
    s = zi_tier_stats()
    _check(_lib.zi_tier_stats_get(tier, ctypes.byref(s)))
    return s.as_dict()


def zi_tier_trace_get(tier) -> list:
    n = ctypes.c_int64()
    _check(_lib.zi_tier_trace_get(tier, None, 0, ctypes.byref(n)))
    ids = (ctypes.c_int64 * max(1, n.value))()
    _check(_lib.zi_tier_trace_get(tier, ids, n.value, ctypes.byref(n)))
    return list(ids[:n.value])


def zi_tier_simulate_reads(trace, buffers: int, steps: int, window: int = 0) -> list:
    """Reads per step of the tier's policy on `trace`; window 0 means `buffers`."""
    t = (ctypes.c_int64 * max(1, len(trace)))(*[int(x) for x in trace])
    out = (ctypes.c_int64 * max(1, int(steps)))()
    _check(_lib.zi_tier_simulate_reads(t, len(trace), int(buffers), int(window or buffers), int(steps), out))
    return list(out[:int(steps)])


def zi_host_alloc(nbytes: int) -> int:
    h = _P()
    _check(_lib.zi_host_alloc(int(nbytes), ctypes.byref(h)))
    return h.value


def zi_host_free(ptr) -> None:
    _check(_lib.zi_host_free(_ptr(ptr)))
