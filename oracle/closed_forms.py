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


# --- choosing the tile width ([ZI-math] "Memory-centric tiling": resident bytes
#     fall as layer_bytes / k while finer tiles make the products smaller and
#     slower; [ZI-cn] "关键技术三：Overlap-Centric Design": copies overlap products)
#
# Our reading of the ring on one link: a pass over N tiles with d device slots
# for weight tiles.  Tile i's copy starts once the link is free and tile i - d
# has released its slot; its products start once the compute stream is free
# and the copy has landed.  In the backward, the weight slot is released after
# the products that read W (recomputed forward, then dX); dW_i is formed in a
# separate gradient slot (free once the write-back of tile i - g is done, with
# g gradient slots) or, with g = 0, in the weight slot itself, which then stays
# taken until dW_i has been written back.

def ring_bytes(K: int, n: int, d: int, dtype: str, budget: int, with_grad: bool, grad_f32: bool = False):
    """(gradient slots, device bytes) of a ring of d weight slots, or None if
    it does not fit `budget` (0 = no cap).  Slots are rounded up to 256 bytes;
    a backward gets two gradient slots if the budget leaves room, else one,
    else none (the gradient then needs to fit a weight slot)."""
    def slot(b):
        return -(-b // 256) * 256
    w = slot(tile_bytes(K, n, dtype))
    g = slot(K * n * (4 if grad_f32 else BYTES[dtype]))
    if budget and d * w > budget:
        return None
    if not with_grad:
        return 0, d * w
    slots = 2 if not budget else min(2, (budget - d * w) // g)
    if slots == 0 and g > w:
        return None
    return slots, d * w + slots * g


def ring_run(N: int, d: int, passes, grad_slots: int = 0):
    """End time of each pass when `passes` run back to back on one ring.

    Every pass stages all N tiles in order; the copies of a pass start as soon
    as the link and the slots allow, so they run ahead into the previous pass.
    Tile g of the run (counted across passes) reuses the slot of tile g - d.
    A pass is a dict: t_copy, and t_fwd for a forward; for a backward
    (backward=True) t_re (recomputed forward), t_dx, t_dw, t_back (the
    gradient's write-back) and `pairs`: the dX products of tiles 2j and 2j+1
    of the pass run as one product once both are resident (our reading of the
    grouping the library uses with gradient slots), which frees both slots;
    tile 2j then runs only its recompute and dW before tile 2j+1 arrives.
    With `re_pairs` as well, the recomputed products of the pair also run
    once tile 2j+1 is resident (tile 2j runs only its dW), as the library
    orders them where one launch over both tiles takes fewer rounds of
    workgroups than two."""
    if any(p.get("pairs") for p in passes) and not grad_slots:
        raise ValueError("pairs need gradient slots")
    release = []      # release[g]: when the g-th staged tile frees its weight slot
    grad_free = []    # grad_free[h]: when the h-th gradient frees its gradient slot
    link = comp = back = 0.0
    ends = []
    for p in passes:
        for i in range(N):
            g = len(release)
            link = max(link, release[g - d] if g >= d else 0.0) + p["t_copy"]
            start = max(comp, link)
            if not p.get("backward"):
                comp = start + p["t_fwd"]
                release.append(comp)
                continue
            h = len(grad_free)
            re2 = bool(p.get("pairs") and p.get("re_pairs"))
            if p.get("pairs") and i % 2 == 0 and i + 1 < N:
                # no dX yet (nor, with re_pairs, the recompute); the slot stays taken
                w_done = start + (0.0 if re2 else p.get("t_re", 0.0))
                release.append(None)
            elif p.get("pairs") and i % 2 == 1:
                w_done = start + (2 if re2 else 1) * p.get("t_re", 0.0) + 2 * p["t_dx"]
                release[g - 1] = w_done
                release.append(w_done)
            else:
                w_done = start + p.get("t_re", 0.0) + p["t_dx"]
                if grad_slots:
                    release.append(w_done)
            if grad_slots:
                comp = max(w_done, grad_free[h - grad_slots] if h >= grad_slots else 0.0) + p["t_dw"]
                back = max(back, comp) + p["t_back"]
            else:
                comp = w_done + p["t_dw"]
                back = max(back, comp) + p["t_back"]
                release.append(back)
            grad_free.append(back)
        ends.append(max(comp, back))
    return ends


def ring_pass_time(N: int, d: int, t_copy: float, t_fwd: float = 0.0, backward: bool = False,
                   t_re: float = 0.0, t_dx: float = 0.0, t_dw: float = 0.0, t_back: float = 0.0,
                   grad_slots: int = 0) -> float:
    """Time from the first copy to the last product (and write-back) of one pass."""
    p = {"t_copy": t_copy, "t_fwd": t_fwd, "backward": backward, "t_re": t_re, "t_dx": t_dx,
         "t_dw": t_dw, "t_back": t_back}
    return ring_run(N, d, [p], grad_slots)[0]


def steady_step_time(N: int, d: int, step, grad_slots: int = 0) -> float:
    """One step (its passes in order) among back-to-back steps: the third
    step's end minus the second's."""
    ends = ring_run(N, d, list(step) * 3, grad_slots)
    k = len(step)
    return ends[3 * k - 1] - ends[2 * k - 1]


def choose_tiling(T: int, K: int, M: int, dtype: str, budget: int, widths, r_fwd, r_dx, r_dw,
                  h2d: float, d2h: float, backward: int, max_d: int, grad_f32: bool = False,
                  c_h2d=None, c_d2h=None):
    """Every candidate (width from `widths` dividing M, multiple of 8; d in
    1..max_d; ring within the budget), priced as a step among back-to-back
    steps of one forward pass plus, for backward 1 or 2, one backward pass (2:
    the forward product recomputed per tile), with the measured rates of that
    width (copy rates c_h2d / c_d2h per width, else h2d / d2h).  Returns
    (choice, table): backward 3 is 2 with the recomputed products of a dX
    pair run together (re_pairs).  The candidate of least step time, where a candidate
    within a relative 1e-9 of the best so far counts as equal and then the
    smaller ring, the smaller d, the smaller N win; table lists every
    candidate in the order considered, each with its passes' times on their
    own as well."""
    table = []
    best = None
    for j, n in enumerate(widths):
        if M % n or n % 8:
            continue
        N = M // n
        flops = 2.0 * T * K * n
        for d in range(1, max_d + 1):
            fit = ring_bytes(K, n, d, dtype, budget, backward != 0, grad_f32)
            if fit is None:
                continue
            slots, nbytes = fit
            t_copy = tile_bytes(K, n, dtype) / (c_h2d[j] if c_h2d else h2d)
            step = [{"t_copy": t_copy, "t_fwd": flops / r_fwd[j]}]
            if backward:
                step.append({"t_copy": t_copy, "backward": True,
                             "t_re": flops / r_fwd[j] if backward >= 2 else 0.0,
                             "t_dx": flops / r_dx[j], "t_dw": flops / r_dw[j],
                             "t_back": K * n * (4 if grad_f32 else BYTES[dtype]) / (c_d2h[j] if c_d2h else d2h)})
            if backward:
                step[1]["pairs"] = slots > 0 and d >= 2 and N >= 2 and n % 64 == 0
                step[1]["re_pairs"] = backward == 3
            alone = [ring_run(N, d, [p], slots)[0] for p in step]
            c = {"N": N, "d": d, "n": n, "dw_slots": slots, "ring_bytes": nbytes,
                 "t_fwd_s": alone[0], "t_bwd_s": alone[1] if backward else 0.0,
                 "t_step_s": steady_step_time(N, d, step, slots)}
            table.append(c)
            if best is None or c["t_step_s"] < best["t_step_s"] * (1 - 1e-9):
                best = c
            elif c["t_step_s"] <= best["t_step_s"] * (1 + 1e-9):
                if (c["ring_bytes"], c["d"], c["N"]) < (best["ring_bytes"], best["d"], best["N"]):
                    best = c
    return best, table


# --- the file tier's buffers as a cache (our reading R30 of the pages' CPU
#     memory in front of NVMe; [ZI-cn] "关键技术三：Overlap-Centric Design")

def belady_reads(trace, capacity: int, steps: int):
    """Reads per step of the offline optimum (Belady): a cache of `capacity`
    items over `steps` repetitions of `trace`, evicting on a miss the item
    whose next request is farthest away (never requested again counts as
    farthest).  No policy reads fewer."""
    seq = list(trace) * steps
    L = len(trace)
    held = set()
    reads = [0] * steps
    for i, x in enumerate(seq):
        if x in held:
            continue
        reads[i // L] += 1
        if len(held) == capacity:
            def nxt(y):
                for j in range(i + 1, len(seq)):
                    if seq[j] == y:
                        return j
                return len(seq) + 1
            held.remove(max(held, key=nxt))
        held.add(x)
    return reads


def tier_policy_reads(trace, buffers: int, steps: int, window: int = 0):
    """Reads per step of the tier's policy with its read-ahead `window`
    requests ahead (0: as far as it may, `buffers`): before each request the
    reader walks the trace from its position until `window` requests are
    waiting; a tile some buffer
    holds is given that buffer without a read; otherwise the tile is read into
    a buffer no waiting request needs, an empty one first, else the one whose
    tile is next wanted latest (counted from the reader's position along the
    repeating trace).  Then the request takes the first waiting buffer."""
    L = len(trace)
    total = steps * L
    tiles = [None] * buffers          # what each buffer holds
    waiting = []                      # buffer of each request read ahead for, in order
    reads = [0] * steps
    ahead = 0                         # next position the reader looks at
    window = window or buffers
    for _ in range(total):
        while len(waiting) < window and ahead < total:
            want = trace[ahead % L]
            if want in tiles:
                waiting.append(tiles.index(want))
                ahead += 1
                continue
            free = [b for b in range(buffers) if b not in waiting]
            if not free:
                break
            empty = [b for b in free if tiles[b] is None]
            if empty:
                b = empty[0]
            else:
                def wanted_in(b):
                    for j in range(L):
                        if trace[(ahead + j) % L] == tiles[b]:
                            return j
                    return L + 1
                b = max(free, key=lambda c: (wanted_in(c), -c))
            tiles[b] = want
            reads[ahead // L] += 1
            waiting.append(b)
            ahead += 1
        waiting.pop(0)
    return reads
