"""Benchmark of the tiled linear hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input.  The
default workload is the feed-forward block of the 1T-parameter model that the
ZeRO-Infinity transformer-math page tiles in its section "Memory-centric
tiling: operators bigger than the device": up-projection W1[25600 x 102400],
GeLU, down-projection W2[102400 x 25600], both fp16 in pinned host memory and
split into 16 output-dimension tiles each, T = 32768 tokens (the batch that
the tier table's section shows clearing the slow-tier bar), prefetch depth 2.
One step = forward W1 (+GeLU), forward W2, recomputed forward W1 (+GeLU),
backward W2 with the recomputed W2 product, dA = dH * GeLU'(A), backward W1:
forward 2P + recompute 2P + backward 4P = 8PT FLOPs (the page's
FLOPs-per-byte section), every tile staged over the host link per pass and
every weight gradient written back to pinned host memory.

Prints one JSON line (rank 0, N = 1).  ``--workload linear`` times a single
tiled linear fwd+bwd instead (the mid FFN up-projection shape by default).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tiled-linear fwd+bwd TFLOP/s, % MFMA peak, exposed host-transfer stall %"
PEAK_MFMA_F16 = 2.5e15   # dense fp16/bf16 MFMA, MI355X published figure (FLOP/s)
PEAK_HBM = 8.0e12        # bytes/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", choices=["ffn", "linear"], default="ffn")
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--d", type=int, default=2)
    ap.add_argument("--dtype", choices=["f16", "bf16"], default=None)
    ap.add_argument("--K", type=int, default=None)
    ap.add_argument("--M", type=int, default=None)
    ap.add_argument("--N", type=int, default=None)
    ap.add_argument("--budget-tiles", type=float, default=0.0,
                    help="device budget of the tile buffers, in weight tiles (linear workload; "
                         "0: no cap).  With a budget of 2 tiles the gradient forms in its weight "
                         "tile's slot")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-link-peak", action="store_true")
    ap.add_argument("--link-peak-only", action="store_true",
                    help="only measure the host-link peak and print it (run as a child process)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--d2h-cus", type=int, default=None,
                    help="compute units of the device-to-host copy stream (0: unrestricted)")
    ap.add_argument("--h2d-cus", type=int, default=None,
                    help="compute units of the host-to-device copy stream (0: unrestricted)")
    ap.add_argument("--dx-per-tile", action="store_true",
                    help="run the dX products one workgroup per output block instead of one persistent "
                         "workgroup per compute unit (to compare the two forms)")
    ap.add_argument("--no-gelu-split", action="store_true",
                    help="leave out the workspace that lets the GeLU forward split the reduction of its "
                         "last, partial round of tiles between two workgroups each (to compare the two forms)")
    ap.add_argument("--max-ahead", type=int, default=0,
                    help="steps the host may enqueue ahead of the device (0: no limit)")
    ap.add_argument("--enqueue", choices=("mid", "all"), default=None,
                    help="mid: enqueue each step once the previous one has reached its middle (the "
                         "down-projection's backward done, or the linear's forward); all: every step "
                         "at once (default: mid for the FFN block, all for the tiled linear)")
    ap.add_argument("--unbounded-enqueue", dest="enqueue", action="store_const", const="all",
                    help="the same as --enqueue all")
    ap.add_argument("--ahead-poll", type=float, default=0.0,
                    help="with --max-ahead: poll the step's end event every this many ms instead of "
                         "waiting on it")
    ap.add_argument("--no-overlap", action="store_true",
                    help="no second product stream (few-wave forward tiles then run on one stream too)")
    ap.add_argument("--adam", action="store_true",
                    help="attach the host Adam to every weight: each tile is updated on the host "
                         "once its gradient has landed, overlapped with the next tiles")
    ap.add_argument("--adam-threads", type=int, default=16,
                    help="host threads that share each tile's update (one tile at a time)")
    ap.add_argument("--nvme", type=str, default=None, metavar="DIR",
                    help="read the weights from files written into DIR (the NVMe tier): each tile "
                         "goes file -> pinned staging buffer -> HBM")
    ap.add_argument("--nvme-threads", type=int, default=8,
                    help="threads that split each tile's file read")
    ap.add_argument("--nvme-staging", type=int, default=3,
                    help="pinned staging buffers per weight (with --nvme-tier: of the tier)")
    ap.add_argument("--nvme-tier", action="store_true",
                    help="read all weights with one reader that follows the order the first step "
                         "used the tiles in (the warmup step is the recorded one)")
    ap.add_argument("--choose", action="store_true",
                    help="measure the products' rates at several tile widths, let the planner "
                         "choose N and d from them, and time every width (prints its own JSON line)")
    ap.add_argument("--widths", type=str, default=None,
                    help="comma-separated tile widths for --choose (default: the 256-multiples of "
                         "the block's down-projection between 800 and 6400 columns)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain streaming kernel of known size (HBM counter calibration)")
    ap.add_argument("--summarize-trace", type=str, default=None, metavar="DIR",
                    help="summarise the rocprofv3 CSV output under DIR (kernel trace and/or counter "
                         "collection) per kernel and grid size, and exit (no GPU needed)")
    ap.add_argument("--split", action="append", default=[], metavar="LABEL=R0,R1,...",
                    help="with --summarize-trace: the dispatches of LABEL, in dispatch order, come in "
                         "repeating runs of R0, R1, ... launches of different shapes (a persistent "
                         "kernel's grid does not tell them apart); label run i 'LABEL #i'")
    return ap.parse_args()


_EPI_NAMES = {0: "lp", 1: "f32", 2: "gelu", 3: "acc", 4: "gelu_f32a"}


def kernel_label(name, grid, wg):
    """Short name of a dispatched kernel and its workgroup count: the GEMM by
    its template (type, Q and P layouts, epilogue, blocks per wave), the other
    kernels of the library by name, the rest by the start of their name."""
    import re
    groups = grid // max(wg, 1)
    m = re.search(r"gemm_kernelI(DF16_|DF16b)Lb([01])ELb([01])ELi(\d)ELb([01])ELi(\d+)ELi(\d+)E(?:Lb([01])E)?", name)
    if m:
        t = "bf16" if m.group(1) == "DF16b" else "f16"
        q = "rs" if m.group(2) == "1" else "rc"
        p = "rs" if m.group(3) == "1" else "rc"
        epi = _EPI_NAMES.get(int(m.group(4)), m.group(4))
        ragged = "" if m.group(5) == "1" else ",ragged"
        persist = ",persistent" if m.group(8) == "1" else ""
        return "gemm<%s,%s,%s,%s,%sx%s%s%s> x%d" % (t, q, p, epi, m.group(6), m.group(7), ragged, persist, groups)
    for key, label in (("gelu_bwd_kernel", "gelu_bwd"), ("gelu_table_kernel", "gelu_table"),
                       ("gelu_grad_table_kernel", "gelu_grad_table"),
                       ("copyBuffer", "__amd_rocclr_copyBuffer"), ("neg_kernel", "neg_kernel")):
        if key in name:
            return "%s x%d" % (label, groups)
    short = name[5:] if name.startswith("void ") else name
    return "%s x%d" % (short.split("(")[0][:60], groups)


def split_labels(keys, labels, splits):
    """labels[i] with ' #g' appended for the labels named in `splits`
    ({label: [r0, r1, ...]}): ordered by keys[i], the dispatches of such a label
    run through repeating runs of r0, r1, ... and g is the run's index."""
    out = list(labels)
    seen = {}
    for i in sorted(range(len(labels)), key=lambda i: keys[i]):
        runs = splits.get(labels[i])
        if not runs:
            continue
        k = seen.get(labels[i], 0)
        seen[labels[i]] = k + 1
        k %= sum(runs)
        g = 0
        while k >= runs[g]:
            k -= runs[g]
            g += 1
        out[i] = "%s #%d" % (labels[i], g)
    return out


def summarize_trace(path, splits=None):
    """Per kernel label: counter means/min/max over the dispatches (counter
    collection CSV) and durations, with the dispatches no other dispatch (or
    no other kernel of the library) overlapped (kernel trace CSV).  Prints one
    JSON object {"counters": {...}, "kernels": {...}}.  `splits` (see
    split_labels) tells apart launches of one kernel and grid by their order."""
    import csv
    import glob
    import json
    splits = splits or {}
    counters, kernels = {}, {}
    for f in sorted(glob.glob(os.path.join(path, "*counter_collection.csv"))):
        per = {}  # (label, counter) -> {dispatch: value};  label -> {dispatch: ms}
        dur = {}
        recs = list(csv.DictReader(open(f)))
        labs = [kernel_label(r["Kernel_Name"], int(r["Grid_Size"]), int(r["Workgroup_Size"])) for r in recs]
        # one row per (dispatch, counter): order the dispatches, then label their rows
        first = {}
        for i, r in enumerate(recs):
            first.setdefault(r["Dispatch_Id"], i)
        order = sorted(first, key=lambda d: int(d))
        dlab = dict(zip(order, split_labels(list(range(len(order))), [labs[first[d]] for d in order], splits)))
        for r in recs:
            lab = dlab[r["Dispatch_Id"]]
            did = r["Dispatch_Id"]
            per.setdefault((lab, r["Counter_Name"]), {})
            per[(lab, r["Counter_Name"])][did] = per[(lab, r["Counter_Name"])].get(did, 0.0) + float(r["Counter_Value"])
            dur.setdefault(lab, {})[did] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
        for (lab, cn), vals in per.items():
            v = list(vals.values())
            counters.setdefault(lab, {})[cn] = {"dispatches": len(v), "mean": sum(v) / len(v), "min": min(v),
                                                "max": max(v)}
        for lab, vals in dur.items():
            v = list(vals.values())
            counters.setdefault(lab, {})["_dur"] = {"dispatches": len(v), "mean": sum(v) / len(v), "min": min(v),
                                                    "max": max(v)}
    for f in sorted(glob.glob(os.path.join(path, "*kernel_trace.csv"))):
        recs = list(csv.DictReader(open(f)))
        labs = split_labels([int(r["Dispatch_Id"]) for r in recs],
                            [kernel_label(r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
                             for r in recs], splits)
        rows = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"].startswith("_ZN2zi"),
                       lab) for r, lab in zip(recs, labs))
        n = len(rows)

        def alone(lib_only):
            # a dispatch is alone if no other dispatch (of the library, with
            # lib_only) runs during any part of it: sorted by start, that is no
            # earlier one ending after its start and the next one starting
            # before its end
            out = [False] * n
            idx = [i for i in range(n) if rows[i][2] or not lib_only]
            mx = None
            for a_, i in enumerate(idx):
                s_, e_ = rows[i][0], rows[i][1]
                nxt = rows[idx[a_ + 1]][0] if a_ + 1 < len(idx) else None
                out[i] = (mx is None or mx <= s_) and (nxt is None or nxt >= e_)
                mx = e_ if mx is None else max(mx, e_)
            return out

        solo, solo_lib = alone(False), alone(True)
        for i, (s, e, lib, lab) in enumerate(rows):
            k = kernels.setdefault(lab, {"dispatches": 0, "ms": 0.0, "solo": 0, "solo_ms": 0.0, "solo_lib": 0,
                                         "solo_lib_ms": 0.0})
            ms = (e - s) / 1e6
            k["dispatches"] += 1
            k["ms"] += ms
            if solo[i]:
                k["solo"] += 1
                k["solo_ms"] += ms
            if solo_lib[i] and lib:
                k["solo_lib"] += 1
                k["solo_lib_ms"] += ms
        for k in kernels.values():
            k["avg_ms"] = k["ms"] / k["dispatches"]
            k["solo_avg_ms"] = k["solo_ms"] / k["solo"] if k["solo"] else None
            k["solo_lib_avg_ms"] = k["solo_lib_ms"] / k["solo_lib"] if k["solo_lib"] else None
    print(json.dumps({"counters": counters, "kernels": kernels}, indent=1, sort_keys=True))


def per_step_parts(recs, kind_names, steps):
    """Each timed step's kernel time by product kind, and its copies' rates,
    from the context's per-launch records: a step enqueues the same launches
    and copies in the same order, so the i-th share of each list is step i's
    (a copy that prefetches the next step's first tile counts with the step
    that enqueued it)."""
    ker = [r for r in recs if r["what"] == "kernel"]
    out = {"kernel_ms": {}, "kernel_span_ms": [], "h2d_GBps": [], "d2h_GBps": []}
    if steps < 1 or not ker or len(ker) % steps:
        out["error"] = "launches do not split evenly over the steps"
        return out
    per = len(ker) // steps
    for i in range(steps):
        part = ker[i * per:(i + 1) * per]
        for r in part:
            name = kind_names[r["kind"]] if 0 <= r["kind"] < len(kind_names) else str(r["kind"])
            out["kernel_ms"].setdefault(name, [0.0] * steps)[i] += r["end_ms"] - r["start_ms"]
        out["kernel_span_ms"].append(round(max(r["end_ms"] for r in part) - min(r["start_ms"] for r in part), 3))
    for what in ("h2d", "d2h"):
        cp = [r for r in recs if r["what"] == what]
        if cp and len(cp) % steps == 0:
            per = len(cp) // steps
            for i in range(steps):
                part = cp[i * per:(i + 1) * per]
                ms = sum(r["end_ms"] - r["start_ms"] for r in part)
                out[what + "_GBps"].append(round(sum(r["rows"] for r in part) / (ms * 1e-3) / 1e9, 2) if ms > 0 else None)
    out["kernel_ms"] = {k: [round(x, 3) for x in v] for k, v in out["kernel_ms"].items()}
    return out


def copy_probe(torch, nbytes=1 << 30, reps=3):
    """Plain streaming kernel: reads and writes ``nbytes`` per launch.

    Used to scale the HBM byte counters (FETCH_SIZE, WRITE_SIZE) of a profiled
    run: the counters' reading for this kernel against its known traffic.
    """
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe": "torch.neg fp32", "bytes_read_per_launch": nbytes,
                      "bytes_written_per_launch": nbytes, "launches": reps}), flush=True)


KERNEL_SOURCE = os.path.join(ROOT, "offload_memory_centric_amd", "csrc", "zi_kernels.hip")


def measured_traffic(config, kernel):
    """HBM bytes per launch of ``kernel`` from the committed counter summary.

    The summary records the workload configuration and the hash of the kernel
    source it was taken on; when either differs from this run its figures do not
    apply and the result is None.
    """
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "hbm_traffic_gemm_%s.md" % config["workload"])
    try:
        text = open(path).read()
        src = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("kernel_source_sha256") != src or d.get("config") != config:
        return None
    return d.get("hbm_bytes_per_launch", {}).get(kernel)


def link_peak(torch, tiling, nbytes=1 << 30, reps=5):
    """hipMemcpyAsync peak from pinned memory: H2D alone, D2H alone, both at once."""
    host = tiling.host_tensor((nbytes,), torch.uint8)
    host2 = tiling.host_tensor((nbytes,), torch.uint8)
    dev = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dev2 = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()

    def timed(fn):
        out = []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            out.append(time.perf_counter() - t0)
        return statistics.median(out)

    def h2d():
        with torch.cuda.stream(s1):
            dev.copy_(host, non_blocking=True)

    def d2h():
        with torch.cuda.stream(s2):
            host2.copy_(dev2, non_blocking=True)

    def both():
        h2d()
        d2h()

    h2d()
    d2h()
    t_h2d, t_d2h, t_both = timed(h2d), timed(d2h), timed(both)
    del host, host2, dev, dev2
    return {"h2d_GBps": nbytes / t_h2d / 1e9, "d2h_GBps": nbytes / t_d2h / 1e9,
            "duplex_h2d_plus_d2h_GBps": 2 * nbytes / t_both / 1e9, "bytes": nbytes, "reps": reps}


def link_peak_in_child():
    """The host-link peak, measured in a child process started before this one
    touches the GPU.  Concurrent host-to-device and device-to-host copies on two
    streams (the duplex figure) were seen to leave the HIP runtime of their
    process serialising later copies and kernels, so they get a process of
    their own."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--link-peak-only"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, timeout=300)
    if r.returncode != 0:
        log("link peak child failed:", r.stderr.decode(errors="replace")[-500:])
        return None
    return json.loads(r.stdout.decode().strip().splitlines()[-1])


class ClockSampler:
    """Samples the GPU's clocks, power, temperatures and throttle counters
    every `period` seconds on a host thread, and notes when each marked step's
    end event completes, so that every timed step gets the conditions it ran
    at.  Reads the AMD SMI library's GPU metrics when it is importable, else
    only the shader clock from the driver's pp_dpm_sclk file."""

    # gpu_metrics fields kept per sample (means per step) ...
    LEVELS = ("current_gfxclk", "current_uclk", "current_socket_power", "temperature_hotspot", "temperature_mem")
    # ... and accumulators whose increase over a step, over that of
    # accumulation_counter, is the share of the step spent in that state
    RESIDENCY = ("ppt_residency_acc", "socket_thm_residency_acc", "hbm_thm_residency_acc",
                 "vr_thm_residency_acc", "prochot_residency_acc")

    def __init__(self, period=0.02):
        import threading
        self.period = period
        self.samples = []        # (host time, {field: value})
        self.ends = {}           # step index -> host time its end event was seen complete
        self.events, self.recorded = [], 0
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        self._read = self._reader()

    @staticmethod
    def _num(v):
        return float(v) if isinstance(v, (int, float)) and v not in (0xFFFF, 0xFFFFFFFF) and v >= 0 else None

    def _reader(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            h = amdsmi.amdsmi_get_processor_handles()[0]

            def read():
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                out = {k: self._num(m.get(k)) for k in self.LEVELS + self.RESIDENCY + ("accumulation_counter",)}
                xcc = [self._num(x) for x in (m.get("current_gfxclks") or [])]
                xcc = [x for x in xcc if x]
                if xcc:
                    out["gfxclk_min_xcc"], out["gfxclk_max_xcc"] = min(xcc), max(xcc)
                return out
            read()
            self.source = "amdsmi gpu_metrics"
            return read
        except Exception as e:  # no SMI library on this host: the driver's file
            self.error = "amdsmi: %s" % (e,)
        import glob
        for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            try:
                open(path).read()
            except OSError:
                continue

            def read(path=path):
                for line in open(path):
                    if line.rstrip().endswith("*"):
                        return {"current_gfxclk": float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))}
                return {}
            self.source = path
            return read
        self.source = None
        return None

    def watch(self, events):
        """Step i ends at events[i + 1]; call mark_recorded(i + 1) after recording it."""
        self.events = events
        self.recorded = 0

    def mark_recorded(self, n):
        self.recorded = n

    def _run(self):
        while not self._stop.is_set():
            t = time.perf_counter()
            if self._read is not None:
                try:
                    self.samples.append((t, self._read()))
                except Exception as e:
                    self.error = str(e)
                    self._read = None
            for j in range(1, self.recorded + 1):
                if j not in self.ends and self.events[j].query():
                    self.ends[j] = time.perf_counter()
            self._stop.wait(self.period)

    def start(self):
        import threading
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def per_step(self, t_start, n):
        """Per step (step 0 from t_start): mean shader clock (and the slowest
        and fastest XCC's), memory clock, power and temperatures over the
        step's samples, and the share of the step each throttle state held."""
        out = []
        prev = t_start
        names = {"current_gfxclk": "sclk_MHz", "gfxclk_min_xcc": "sclk_min_xcc_MHz",
                 "gfxclk_max_xcc": "sclk_max_xcc_MHz", "current_uclk": "mclk_MHz",
                 "current_socket_power": "power_W", "temperature_hotspot": "hotspot_C",
                 "temperature_mem": "hbm_C"}
        for j in range(1, n + 1):
            end = self.ends.get(j)
            if end is None:
                out.append(None)
                continue
            sel = [x[1] for x in self.samples if prev <= x[0] <= end]
            row = {"samples": len(sel)}
            for k, nm in names.items():
                v = [x[k] for x in sel if x.get(k)]
                row[nm] = round(statistics.mean(v), 1) if v else None
            if len(sel) >= 2 and sel[0].get("accumulation_counter") and sel[-1].get("accumulation_counter"):
                dt = sel[-1]["accumulation_counter"] - sel[0]["accumulation_counter"]
                for k in self.RESIDENCY:
                    if dt > 0 and sel[0].get(k) is not None and sel[-1].get(k) is not None:
                        row[k.replace("_residency_acc", "_share")] = round((sel[-1][k] - sel[0][k]) / dt, 3)
            out.append(row)
            prev = end
        return out


def main():
    args = parse()
    if args.summarize_trace:
        splits = {}
        for sp in args.split:
            lab, _, runs = sp.rpartition("=")
            splits[lab] = [int(x) for x in runs.split(",")]
        summarize_trace(args.summarize_trace, splits)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the tiled path runs on a single device and has no "
              "multi-GPU form (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    link = None
    if not args.no_link_peak and not args.link_peak_only and not args.copy_probe:
        link = link_peak_in_child()
        log("link peak", link)

    import numpy as np
    import torch

    from offload_memory_centric_amd import inputs, tiling, zi

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(torch)
        return
    if args.link_peak_only:
        print(json.dumps(link_peak(torch, tiling)), flush=True)
        return
    if args.choose:
        print(json.dumps(choose_leg(args, torch, tiling, inputs, link)), flush=True)
        return
    dtype = args.dtype or ("f16" if args.workload == "ffn" else "bf16")
    tdt = inputs.torch_dtype(dtype)
    d = args.d
    seed = 0

    ctx_kw = {} if args.d2h_cus is None else {"d2h_cus": args.d2h_cus}
    if args.no_gelu_split:
        ctx_kw["gelu_split"] = False
    if args.h2d_cus is not None:
        ctx_kw["h2d_cus"] = args.h2d_cus
    if args.no_overlap:
        ctx_kw["overlap"] = False

    # ---------------- workload ----------------
    if args.workload == "ffn":
        T = args.T or 32768
        D, F = args.K or 25600, args.M or 102400
        N1 = N2 = args.N or 16
        log("allocating FFN block T=%d D=%d F=%d" % (T, D, F))
        X = inputs.new((T, D), dtype, "gaussian", seed, "X", device="cuda")
        dY = inputs.new((T, D), dtype, "gaussian", seed, "dY", device="cuda")
        W1t = tiling.host_tensor((F, D), tdt)
        W2t = tiling.host_tensor((D, F), tdt)
        inputs.fill_(W1t, "gaussian", seed, "W1", std=0.02, device="cuda", chunk_rows=4096)
        inputs.fill_(W2t, "gaussian", seed, "W2", std=0.02, device="cuda", chunk_rows=1024)
        dW1t = tiling.host_tensor((F, D), tdt)
        dW2t = tiling.host_tensor((D, F), tdt)
        p1 = tiling.Plan(T, D, F, N1, d, dtype, W1t, dW1t)
        p2 = tiling.Plan(T, F, D, N2, d, dtype, W2t, dW2t)
        ctx = tiling.Context(p1 if p1.info.ring_bytes >= p2.info.ring_bytes else p2, **ctx_kw)
        if args.dx_per_tile:
            ctx.set_debug(dx_per_tile=True)
        A = torch.empty((T, F), dtype=tdt, device="cuda")
        H = torch.empty_like(A)
        dA = torch.empty_like(A)
        dH = torch.empty((T, F), dtype=torch.float32, device="cuda")
        Y = torch.empty((T, D), dtype=tdt, device="cuda")
        Yr = torch.empty_like(Y)
        dX = torch.empty((T, D), dtype=torch.float32, device="cuda")
        P = D * F * 2  # parameters of the block
        flops_step = 8.0 * P * T
        h2d_bytes_step = 2.0 * (3 * D * F + 2 * D * F)

        def step(mid=None):
            tiling.ffn_block_step(ctx, p1, p2, X, A, H, Y, dY, dH, dA, dX, Yr, mid=mid)

        config = {"workload": "ffn_block_fwd_recompute_bwd", "T": T, "d_model": D, "d_ff": F,
                  "N_up": N1, "N_down": N2, "n_up": F // N1, "n_down": D // N2, "d": d,
                  "weights": "pinned host", "dtype": dtype}
        plans = (p1, p2)
    else:
        T = args.T or 4096
        K, M = args.K or 8192, args.M or 32768
        N = args.N or 8
        log("allocating linear T=%d K=%d M=%d N=%d" % (T, K, M, N))
        X = inputs.new((T, K), dtype, "gaussian", seed, "X", device="cuda")
        dY = inputs.new((T, M), dtype, "gaussian", seed, "dY", device="cuda")
        Wt = tiling.host_tensor((M, K), tdt)
        inputs.fill_(Wt, "gaussian", seed, "W", std=0.02, device="cuda", chunk_rows=4096)
        dWt = tiling.host_tensor((M, K), tdt)
        tile_bytes = K * (M // N) * 2
        budget = int(args.budget_tiles * tile_bytes)
        p = tiling.Plan(T, K, M, N, d, dtype, Wt, dWt, budget=budget)
        ctx = tiling.Context(p, **ctx_kw)
        if args.dx_per_tile:
            ctx.set_debug(dx_per_tile=True)
        Y = torch.empty((T, M), dtype=tdt, device="cuda")
        dX = torch.empty((T, K), dtype=torch.float32, device="cuda")
        flops_step = 6.0 * T * K * M
        h2d_bytes_step = 2.0 * K * M * 2

        def step(mid=None):
            ctx.fwd(p, X, Y)
            if mid is not None:
                mid()
            ctx.bwd(p, X, dY, dX)

        config = {"workload": "tiled_linear_fwd_bwd", "T": T, "K": K, "M": M, "N": N, "n": M // N,
                  "d": d, "weights": "pinned host", "dtype": dtype}
        if budget:
            config.update({"budget_tiles": args.budget_tiles, "budget_bytes": budget,
                           "gradient_slots": p.info.dw_slots, "ring_bytes": p.info.ring_bytes})
        plans = (p,)
    if args.dx_per_tile:
        config["dx_form"] = "one workgroup per output block"
    if args.no_gelu_split:
        config["gelu_split"] = False
    sources, tier = [], None
    if args.nvme:
        if args.adam:
            raise SystemExit("--nvme and --adam exclude each other (the optimizer updates host memory)")
        sources, tier = nvme_sources(args, tiling, ctx, plans)
        config["weights"] = "file -> pinned staging -> HBM"
        if tier is not None:
            pass_step = step

            def step(mid=None):
                pass_step(mid)
                tier.step()
    torch.cuda.synchronize()

    # Per-step marks: an event on the compute stream after every step.  For
    # the FFN block the host enqueues step i once step i - 1 has reached its
    # middle, so the ring's prefetch still crosses steps while about one step
    # is in flight (as in a training loop that reads its loss every step).
    # With every step enqueued at once the HIP runtime was seen, after 12-19
    # steps, to carry the tile copies out at 36-40 GB/s as copy kernels beside
    # the products (steps 15-40 % longer), and with two or more whole steps in
    # flight to stall write-backs at 13 GB/s; one step or less in flight
    # avoided both.  The tiled linear's middle is its forward, and there the
    # same gating slowed the write-backs of the step after the first to
    # 8-19 GB/s in 11 of 12 three-step runs (every step enqueued at once: none
    # of 6), so it enqueues every step at once by default.
    if args.enqueue is None:
        args.enqueue = "mid" if config["workload"] == "ffn_block_fwd_recompute_bwd" else "all"
    comp = torch.cuda.ExternalStream(ctx.streams[0])

    def marked(n, sampler=None):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        if sampler is not None:
            sampler.watch(ev)
        mids = [torch.cuda.Event() for _ in range(n)]
        ev[0].record(comp)
        for i in range(n):
            e = None
            if args.enqueue == "mid" and i >= 1:
                e = mids[i - 1]
            elif args.max_ahead and i >= args.max_ahead:
                e = ev[i - args.max_ahead + 1]
            if e is not None:
                if args.ahead_poll:
                    while not e.query():
                        time.sleep(args.ahead_poll * 1e-3)
                else:
                    e.synchronize()
            step(mid=lambda: mids[i].record(comp))
            ev[i + 1].record(comp)
            if sampler is not None:
                sampler.mark_recorded(i + 1)
        return ev

    def spans(ev):
        return [round(ev[i].elapsed_time(ev[i + 1]), 3) for i in range(len(ev) - 1)]

    # ---------------- warmup ----------------
    wev = marked(args.warmup)
    ctx.sync()
    torch.cuda.synchronize()
    warm_ms = spans(wev)

    src_before = [src.stats() for src, _ in sources]

    # ---------------- timed steps ----------------
    ctx.set_timing(True)
    ctx.reset_stats()
    sampler = ClockSampler()
    sampler.start()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tev = marked(args.steps, sampler)
    ctx.sync()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    time.sleep(2 * sampler.period)  # the sampler notes the last step's end
    sampler.stop()
    step_ms = spans(tev)
    step_clock = sampler.per_step(t0, args.steps)
    st = ctx.stats()
    step_parts = per_step_parts(ctx.timed_records(), list(st["kinds"]), args.steps)
    ctx.set_timing(False)

    ms_step = wall / args.steps * 1e3
    tflops = flops_step * args.steps / wall / 1e12
    busy_ms = st["compute_busy_ms"]
    stall = max(0.0, 1.0 - busy_ms / (wall * 1e3))
    h2d_rate = st["h2d_bytes"] / (st["h2d_ms"] * 1e-3) if st["h2d_ms"] > 0 else 0.0
    d2h_rate = st["d2h_bytes"] / (st["d2h_ms"] * 1e-3) if st["d2h_ms"] > 0 else 0.0

    kinds = {k: v for k, v in st["kinds"].items() if v["launches"]}
    # Per kernel (product and launch shape).  A launch that another kernel
    # overlapped (the two-stream forward passes) has a duration that includes
    # the time the two shared the device; a kernel's own rate comes from the
    # launches that ran alone, and its time per step is that rate applied to
    # all of its launches.
    kernel_table = []
    for k in st["kernels"]:
        fl = k["flops"] / k["launches"]
        solo = k["solo_launches"] > 0
        avg = (k["solo_ms"] / k["solo_launches"]) if solo else k["ms"] / k["launches"]
        kernel_table.append({
            "kernel": "%s %dx%dx%d" % (k["name"], k["rows"], k["cols"], k["red"]),
            "launches": k["launches"], "solo_launches": k["solo_launches"],
            "avg_ms": round(avg, 4), "avg_ms_all_launches": round(k["ms"] / k["launches"], 4),
            "ms_per_step": round(avg * k["launches"] / args.steps, 3),
            "tflops": round(fl / (avg * 1e-3) / 1e12, 1) if k["name"] != "gelu_bwd" else None,
            "flops_per_launch": fl if k["name"] != "gelu_bwd" else None})
    kernel_table.sort(key=lambda r: -r["ms_per_step"])
    dom = next(r for r in kernel_table if r["flops_per_launch"])
    achieved = dom["tflops"]
    kinds_table = {k: {"launches": v["launches"], "avg_ms": v["ms"] / v["launches"],
                       "total_ms_per_step": v["ms"] / args.steps}
                   for k, v in kinds.items()}

    # The hidden-tier rule with the measured rates: the step can go no faster
    # than its kernels (the path's FLOPs over the time some kernel ran) or its
    # host-to-device bytes over the measured link.
    pred = None
    if link and busy_ms > 0:
        R = flops_step * args.steps / (busy_ms * 1e-3)
        ait = flops_step / h2d_bytes_step
        link_roof = ait * link["h2d_GBps"] * 1e9
        attainable = min(R, link_roof)
        pred = {"kernel_flop_rate_TFLOPs": R / 1e12,
                "kernel_rate_basis": "step FLOPs / union of the kernels' intervals",
                "link_h2d_GBps": link["h2d_GBps"],
                "balance_flop_per_byte": R / (link["h2d_GBps"] * 1e9),
                "ait_step_flop_per_h2d_byte": ait,
                "link_roofline_TFLOPs": link_roof / 1e12,
                "bound": "link" if link_roof < R else "mfma",
                "attainable_TFLOPs": attainable / 1e12,
                "frac_of_attainable": tflops * 1e12 / attainable}

    result = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded Gaussian: X, dY ~ N(0,1), W ~ N(0, 0.02^2))",
        "config": config,
        "pct_mfma_peak": round(100.0 * tflops * 1e12 / PEAK_MFMA_F16, 2),
        "step_ms": step_ms,
        "warmup_step_ms": warm_ms,
        "exposed_stall_pct": round(100.0 * stall, 2),
        "h2d_GBps_achieved": round(h2d_rate / 1e9, 2),
        "d2h_GBps_achieved": round(d2h_rate / 1e9, 2),
        "link_peak": link,
        "kernels": kernel_table,
        "kinds": kinds_table,
        "model": pred,
        "roofline": {"kernel": dom["kernel"], "bound": "mfma", "achieved": achieved,
                     "peak": PEAK_MFMA_F16 / 1e12, "unit": "TFLOP/s",
                     "frac": round(achieved * 1e12 / PEAK_MFMA_F16, 4),
                     "flops_per_launch": dom["flops_per_launch"], "avg_launch_ms": dom["avg_ms"],
                     "launches_timed": dom["solo_launches"] or dom["launches"],
                     "traffic": measured_traffic(config, dom["kernel"])},
        "step_clock": {"source": sampler.source, "error": sampler.error, "per_step": step_clock},
        "step_parts": step_parts,
        "host_enqueue": ("each step once the previous one reached its middle" if args.enqueue == "mid"
                         else ("at most %d steps ahead" % args.max_ahead if args.max_ahead else "unbounded")),
    }
    if config["workload"] == "ffn_block_fwd_recompute_bwd":
        # the recomputed forward is work the step repeats; without it 7PT
        result["useful_7PT_TFLOPs"] = round(tflops * 7.0 / 8.0, 3)

    if sources:
        result["nvme"] = nvme_report(args, tiling, sources, src_before, kinds, wall, flops_step * args.steps)
        if tier is not None:
            result["nvme"]["tier"] = tier.stats()
            # the tier's buffer policy on its recorded trace, without files or
            # threads, with the read-ahead 1, 2 or every buffer ahead of the
            # requests (a reader held back by the disk runs one or two ahead)
            trace = zi.zi_tier_trace_get(tier.handle)
            tile = plans[0].info.tile_bytes
            assert all(p.info.tile_bytes == tile for p in plans), "reads are counted in tiles of one size"
            S = args.nvme_staging
            result["nvme"]["predicted_GB_read_per_step"] = {
                str(w): round(zi.zi_tier_simulate_reads(trace, S, 4, w)[-1] * tile / 1e9, 2)
                for w in sorted({1, min(2, S), S})}
            result["nvme"]["measured_GB_read_per_step"] = round(
                result["nvme"]["bytes_read_timed"] / args.steps / 1e9, 2)
    adams = []
    if args.adam:
        result["adam"] = host_adam_leg(args, torch, tiling, ctx, plans, marked, spans, ms_step)
        adams = result["adam"].pop("_objs")

    result["machine"] = machine_info(torch)

    # ---------------- CPU baseline (oracle, after the GPU timing) ----------------
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, np, torch, config, locals())
    print(json.dumps(result), flush=True)
    for pl in plans:
        ctx.attach_source(pl, None)
    ctx.close()
    for a in adams:
        a.close()
    if tier is not None:
        tier.close()
    for src, path in sources:
        src.close()
        os.remove(path)


def choose_leg(args, torch, tiling, inputs, link, steps=3):
    """Tile-width choice, measured.  For each width n (N = M/n, d = 2) one
    tiled linear fwd + bwd is run over `steps` steps with per-launch events;
    the rates of its forward, dX and dW products and of its copies make the
    planner's curve.  The step time is then taken without those events, among
    back-to-back steps (as the planner prices a step).  Both run with one
    product stream, the schedule the planner's model describes.
    zi_plan_choose then picks N and d from that curve and the host-link rates,
    and its prediction for every width stands beside the measured step time.
    Default shape: the feed-forward block's down-projection, W2[102400 x 25600]
    fp16 at T = 32768."""
    from offload_memory_centric_amd import zi
    T = args.T or 32768
    K, M = args.K or 102400, args.M or 25600
    dtype = args.dtype or "f16"
    tdt = inputs.torch_dtype(dtype)
    widths = ([int(x) for x in args.widths.split(",")] if args.widths else
              [800, 1024, 1280, 1600, 2560, 3200, 5120, 6400])
    widths = [n for n in widths if M % n == 0 and n % 8 == 0]
    if not widths or not link:
        raise SystemExit("--choose needs widths that divide M and the host-link peak")
    log("choose: T=%d K=%d M=%d %s widths %s" % (T, K, M, dtype, widths))
    X = inputs.new((T, K), dtype, "gaussian", 0, "X", device="cuda")
    dY = inputs.new((T, M), dtype, "gaussian", 0, "dY", device="cuda")
    Wt = tiling.host_tensor((M, K), tdt)
    inputs.fill_(Wt, "gaussian", 0, "W", std=0.02, device="cuda", chunk_rows=1024)
    dWt = tiling.host_tensor((M, K), tdt)
    dX = torch.empty((T, K), dtype=torch.float32, device="cuda")
    flops_step = 6.0 * T * K * M
    rows = []
    for n in widths:
        plan = tiling.Plan(T, K, M, M // n, 2, dtype, Wt, dWt)
        # the planner's ring model runs a pass's products one after another,
        # so the curve and the step times are taken with one product stream
        # (a second one would overlap forward products, and their event
        # durations would include the time they share the device)
        ctx = tiling.Context(plan, overlap=False)
        Y = torch.empty((T, M), dtype=tdt, device="cuda")
        ctx.fwd(plan, X, Y)
        ctx.bwd(plan, X, dY, dX)
        ctx.sync()
        # rates of the products and copies, from per-launch events
        ctx.set_timing(True)
        ctx.reset_stats()
        for _ in range(steps):
            ctx.fwd(plan, X, Y)
            ctx.bwd(plan, X, dY, dX)
        ctx.sync()
        st = ctx.stats()
        ctx.set_timing(False)
        # the step time among back-to-back steps, without the per-launch
        # events: marks on the compute stream after each step, and the mean
        # over the steps after the first two (which include the ring's fill)
        comp = torch.cuda.ExternalStream(ctx.streams[0])
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 3)]
        torch.cuda.synchronize()
        marks[0].record(comp)
        for k in range(steps + 2):
            ctx.fwd(plan, X, Y)
            ctx.bwd(plan, X, dY, dX)
            marks[k + 1].record(comp)
        ctx.sync()
        torch.cuda.synchronize()
        wall = marks[2].elapsed_time(marks[steps + 2]) * 1e-3 / steps
        rate = {k[len("gemm_"):]: v["flops"] / (v["ms"] * 1e-3) for k, v in st["kinds"].items() if v["launches"]}
        rows.append({"n": n, "N": M // n, "ms_per_step_measured": round(wall * 1e3, 3),
                     "TFLOPs_measured": round(flops_step / wall / 1e12, 1),
                     "fwd_TFLOPs": round(rate["fwd"] / 1e12, 1), "dx_TFLOPs": round(rate["dx"] / 1e12, 1),
                     "dw_TFLOPs": round(rate["dw"] / 1e12, 1),
                     "h2d_GBps": round(st["h2d_bytes"] / st["h2d_ms"] / 1e6, 2),
                     "d2h_GBps": round(st["d2h_bytes"] / st["d2h_ms"] / 1e6, 2)})
        log("  n=%d N=%d %.1f ms/step, fwd %.0f dx %.0f dw %.0f TFLOP/s, copies %.1f / %.1f GB/s" % (
            n, M // n, wall * 1e3, rate["fwd"] / 1e12, rate["dx"] / 1e12, rate["dw"] / 1e12,
            rows[-1]["h2d_GBps"], rows[-1]["d2h_GBps"]))
        ctx.close()
        plan.close()
        del Y
    prob = zi.zi_problem(T=T, K=K, M=M, N=1, d=1, dtype=zi.DTYPE_CODES[dtype], flags=0,
                         device_budget_bytes=0, W_host=None, dW_host=None)
    h2d, d2h = link["h2d_GBps"] * 1e9, link["d2h_GBps"] * 1e9
    choice, table = zi.zi_plan_choose(prob, [r["n"] for r in rows], [r["fwd_TFLOPs"] * 1e12 for r in rows],
                                      [r["dx_TFLOPs"] * 1e12 for r in rows],
                                      [r["dw_TFLOPs"] * 1e12 for r in rows], h2d, d2h, 1, 3,
                                      h2d=[r["h2d_GBps"] * 1e9 for r in rows],
                                      d2h=[r["d2h_GBps"] * 1e9 for r in rows])
    for r in rows:
        pred = [c for c in table if c["n"] == r["n"] and c["d"] == 2][0]
        r["ms_per_step_predicted_d2"] = round(pred["t_step_s"] * 1e3, 3)
    best = min(rows, key=lambda r: r["ms_per_step_measured"])
    mine = [r for r in rows if r["n"] == choice["n"]][0]
    return {"choose": {"workload": "tiled_linear_fwd_bwd", "T": T, "K": K, "M": M, "dtype": dtype,
                       "link": link, "widths": rows,
                       "choice": {"N": choice["N"], "d": choice["d"], "n": choice["n"],
                                  "ms_per_step_predicted": round(choice["t_step_s"] * 1e3, 3),
                                  "ms_per_step_measured_d2": mine["ms_per_step_measured"]},
                       "measured_best": {"n": best["n"], "N": best["N"],
                                         "ms_per_step": best["ms_per_step_measured"]},
                       "choice_vs_best": round(best["ms_per_step_measured"] / mine["ms_per_step_measured"], 4)}}


def nvme_sources(args, tiling, ctx, plans):
    """Write every plan's weight to a file under args.nvme and read the tiles
    from there: one source per weight, args.nvme_staging staging buffers each,
    or (--nvme-tier) all of them under one tier with that many buffers."""
    os.makedirs(args.nvme, exist_ok=True)
    out = []
    tier = tiling.Tier(staging=args.nvme_staging, threads=args.nvme_threads) if args.nvme_tier else None
    for j, pl in enumerate(plans):
        path = os.path.join(args.nvme, "zi_weight_%d.bin" % j)
        t0 = time.perf_counter()
        tiling.write_weight_file(path, pl._keep[0])
        os.sync()
        log("wrote %s (%.1f GB) in %.1f s" % (path, pl.K * pl.M * 2 / 1e9, time.perf_counter() - t0))
        src = tiling.FileSource(pl, path, staging=args.nvme_staging, threads=args.nvme_threads)
        if tier is not None:
            tier.add(src)
        ctx.attach_source(pl, src)
        out.append((src, path))
    return out, tier


def nvme_report(args, tiling, sources, before, kinds, wall, flops):
    """What the file tier delivered during the timed steps, beside the rate a
    plain sequential read of one weight file reaches with the same threads,
    and the pages' test for the tier: the step's FLOPs per byte read from the
    files against the products' rate over that read rate."""
    import numpy as np
    after = [src.stats() for src, _ in sources]
    d = {k: sum(a[k] - b[k] for a, b in zip(after, before)) for k in ("bytes", "read_s", "wait_s", "restarts")}
    src0 = sources[0][0]
    tile = src0.plan.info.tile_bytes
    raw = np.empty(tile + 4096, np.uint8)  # pageable and 4096-aligned: a direct read lands in place
    buf = raw[(-raw.ctypes.data) % 4096:][:tile]
    reps = min(src0.plan.N, 8)
    t0 = time.perf_counter()
    for t in range(reps):
        src0.read(t, buf)
    peak = reps * tile / (time.perf_counter() - t0)
    prod = {k: v for k, v in kinds.items() if k != "gelu_bwd"}
    R = sum(v["flops"] for v in prod.values()) / (sum(v["ms"] for v in prod.values()) * 1e-3)
    ait = flops / d["bytes"] if d["bytes"] else None
    return {"direct_io": bool(after[0]["direct"]), "threads_per_read": args.nvme_threads,
            "staging_per_weight": args.nvme_staging,
            "bytes_read_timed": d["bytes"], "read_busy_s": round(d["read_s"], 3),
            "pass_wait_s": round(d["wait_s"], 3), "restarts": d["restarts"],
            "read_GBps_over_timed_steps": round(d["bytes"] / wall / 1e9, 2),
            "read_GBps_sequential_peak": round(peak / 1e9, 2),
            "ait_flop_per_file_byte": ait, "balance_R_over_BW": R / peak,
            "tier_hidden": (ait >= R / peak) if ait else None}


def host_stream_GBps(torch, nelem=1 << 28, reps=3):
    """Practical host memory bandwidth: a += b over fp32 arrays of 1 GiB on
    torch's CPU threads, 12 bytes per element (a read and written in place,
    b read; no write-allocate traffic, as in the optimizer's own pattern)."""
    a = torch.ones(nelem)
    b = torch.ones(nelem)
    a.add_(b)
    best = float("inf")
    for _ in range(reps):
        t0 = time.perf_counter()
        a.add_(b)
        best = min(best, time.perf_counter() - t0)
    return 12.0 * nelem / best / 1e9


def host_adam_leg(args, torch, tiling, ctx, plans, marked, spans, ms_without):
    """The same steps again with the host Adam attached to every weight: each
    tile is updated on the host as soon as its gradient has landed, while the
    GPU goes on with the next tiles.  Reports the step time with the optimizer
    beside the step time of the path alone, and the optimizer's bandwidth
    against the host's practical bandwidth."""
    log("host Adam on %d weight(s), %d threads per tile update" % (len(plans), args.adam_threads))
    adams = []
    for pl in plans:
        a = tiling.Adam(pl, lr=1e-4, threads=args.adam_threads)
        ctx.attach_adam(pl, a)
        adams.append(a)
    # the warmup step pays the first touch of the optimizer state
    marked(max(1, args.warmup))
    ctx.sync()
    torch.cuda.synchronize()
    before = [a.stats() for a in adams]
    t0 = time.perf_counter()
    ev = marked(args.steps)
    ctx.sync()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    after = [a.stats() for a in adams]
    tiles = sum(x["tiles_done"] - y["tiles_done"] for x, y in zip(after, before))
    busy = sum(x["busy_s"] - y["busy_s"] for x, y in zip(after, before))
    nbytes = sum(x["bytes"] - y["bytes"] for x, y in zip(after, before))
    params = sum(pl.K * pl.M for pl in plans)
    ms_with = wall / args.steps * 1e3
    peak = host_stream_GBps(torch)
    achieved = nbytes / busy / 1e9 if busy > 0 else None
    return {
        "threads": args.adam_threads,
        "params": params,
        "host_state_bytes": 12 * params,
        "ms_per_step_with_optimizer": round(ms_with, 3),
        "ms_per_step_without": round(ms_without, 3),
        "exposed_ms_per_step": round(ms_with - ms_without, 3),
        "step_ms_with_optimizer": spans(ev),
        "tiles_per_step": tiles / args.steps,
        "busy_ms_per_step": round(busy / args.steps * 1e3, 3),
        "roofline": {"bound": "host memory", "achieved": round(achieved, 2) if achieved else None,
                     "peak": round(peak, 2), "unit": "GB/s",
                     "frac": round(achieved / peak, 3) if achieved else None,
                     "bytes_per_param": 28, "peak_kind": "measured a += b on the host"},
        "_objs": adams,
    }


def machine_info(torch):
    """The facts a reader needs to place the figures: device, runtime, host
    cores and memory nodes, the copy-engine switch and the clocks the driver
    reports (where rocm-smi is there to read them)."""
    import glob
    props = torch.cuda.get_device_properties(0)
    info = {"device": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hbm_bytes": props.total_memory,
            "hip_runtime": torch.version.hip, "HSA_ENABLE_SDMA": os.environ.get("HSA_ENABLE_SDMA"),
            "host_cores": len(os.sched_getaffinity(0)),
            "host_numa_nodes": len(glob.glob("/sys/devices/system/node/node[0-9]*"))}
    try:
        with open("/proc/cpuinfo") as f:
            info["host_cpu"] = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    # clocks and power limit through the AMD SMI library (no child process:
    # a program started from a process that has initialised the GPU must not
    # replace itself, and the rocm-smi script does)
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
        clk = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
        mem = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.MEM)
        info["clocks"] = {"sclk_MHz_now": clk.get("clk"), "sclk_MHz_max": clk.get("max_clk"),
                          "mclk_MHz_now": mem.get("clk")}
        try:
            pw = amdsmi.amdsmi_get_power_cap_info(h)
            info["power_cap_W"] = pw.get("power_cap") / 1e6 if pw.get("power_cap", 0) > 1e4 else pw.get("power_cap")
        except Exception:
            pass
    except Exception as e:
        info["clocks"] = {"error": str(e)[:200]}
    return info


def _bits(torch, np, t):
    if t.device.type != "cpu":
        t = t.cpu()
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def cpu_baseline(args, np, torch, config, env):
    """The oracle, as it stands, on a bounded sample of the same workload.

    The sample runs on every host core the process may use; the weight decode
    it pays (the oracle turns every 16-bit weight it reads into a double) is
    then timed on its own with the same calls, so the products' rate can be
    stated apart from it.  A second, smaller sample runs on one thread.  Both
    rates are extrapolated to the whole step (labelled as extrapolated: the
    oracle never runs the whole step here)."""
    import oracle

    oracle.set_threads(0)
    cores = oracle.get_threads()
    dtype = config["dtype"]
    t_start = time.perf_counter()
    rng = np.random.default_rng(0)
    if config["workload"] == "ffn_block_fwd_recompute_bwd":
        X, dY, W1t, W2t = (_bits(torch, np, env[k]) for k in ("X", "dY", "W1t", "W2t"))
        T, D, F = config["T"], config["d_model"], config["d_ff"]
        nt = 32
        nf = 64
        t_rows = np.sort(rng.choice(T, nt, replace=False))
        f_cols = np.sort(rng.choice(F, nf, replace=False))
        d2 = np.sort(rng.choice(D, 2, replace=False))
        dc = np.sort(rng.choice(D, 2, replace=False))
        t0 = time.perf_counter()
        oracle.ffn_sample(X, W1t, W2t, dY, dtype, t_rows, f_cols, d2, dc, chunk=4096)
        secs = time.perf_counter() - t0
        # multiply-adds the sample performs (2 FLOPs each): token rows over the whole
        # hidden dimension, hidden columns over all tokens
        flops = 2.0 * (nt * F * D * 2 + nt * F * (len(d2) + len(dc)) + nf * T * D * 2 +
                       nf * T * (len(d2) + len(dc)))
        sample = ("oracle.ffn_sample: %d token row(s) through the whole block and %d hidden "
                  "column(s) over all %d tokens (%.3g FLOPs)" % (nt, nf, T, flops))
        # the decode of both weights as the sample reads them (same calls, same chunks)
        t1 = time.perf_counter()
        for f0 in range(0, F, 4096):
            fidx = np.arange(f0, min(F, f0 + 4096), dtype=np.int64)
            oracle.gather(W1t, dtype, D, 1, fidx, F, None, D)
            oracle.gather(W2t, dtype, 1, F, fidx, F, None, D)
        decode_s = time.perf_counter() - t1
        flops_step = 8.0 * D * F * 2 * T
        # one thread: token rows of the up-projection over one tile's columns
        one_rows = rng.choice(T, 16, replace=False)
        one_cols = np.arange(F // 16)
        one_flops = 2.0 * len(one_rows) * len(one_cols) * D
        one_what = "oracle.linear_fwd_sample, 1 thread: %d token rows x %d columns of W1" % (
            len(one_rows), len(one_cols))
        one_args = (X, W1t, one_rows, one_cols)
    else:
        X, dY, Wt = (_bits(torch, np, env[k]) for k in ("X", "dY", "Wt"))
        T, K, M = config["T"], config["K"], config["M"]
        rows = np.arange(0, T, max(1, T // 32))[:32]
        # at most 16384 output columns: the oracle decodes every weight row it
        # reads into doubles (a 32 GiB weight would take 137 GB)
        cols = np.arange(min(M, 16384))
        t0 = time.perf_counter()
        oracle.linear_fwd_sample(X, Wt, rows, cols, dtype)
        secs = time.perf_counter() - t0
        flops = 2.0 * len(rows) * K * len(cols)
        sample = "oracle.linear_fwd_sample: %d rows x %d of the %d columns (%.3g FLOPs)" % (
            len(rows), len(cols), M, flops)
        t1 = time.perf_counter()
        oracle.gather(Wt, dtype, K, 1, cols, M, None, K)
        decode_s = time.perf_counter() - t1
        flops_step = 6.0 * T * K * M
        one_rows = rows[:4]
        one_cols = np.arange(min(M, 4096))
        one_flops = 2.0 * len(one_rows) * len(one_cols) * K
        one_what = "oracle.linear_fwd_sample, 1 thread: %d rows x %d columns" % (len(one_rows), len(one_cols))
        one_args = (X, Wt, one_rows, one_cols)
    oracle.set_threads(1)
    t2 = time.perf_counter()
    oracle.linear_fwd_sample(*one_args, dtype)
    one_s = time.perf_counter() - t2
    oracle.set_threads(0)
    prod_s = max(secs - decode_s, 1e-9)
    log("cpu baseline: %.1f s sample (%.1f s of it weight decode), %.1f s one thread, %.1f s total" % (
        secs, decode_s, one_s, time.perf_counter() - t_start))
    rate, rate_prod, rate_one = flops / secs, flops / prod_s, one_flops / one_s
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": sample, "seconds": round(secs, 2),
            "decode_seconds": round(decode_s, 2),
            "products_TFLOPs": rate_prod / 1e12,
            "one_thread": {"value": rate_one / 1e12, "unit": "TFLOP/s", "cores": 1, "sample": one_what,
                           "seconds": round(one_s, 2)},
            "extrapolated_full_step_s": {
                "note": "extrapolated from the sample rates, not run: step FLOPs / rate",
                "step_flops": flops_step,
                "all_cores": round(flops_step / rate, 1),
                "all_cores_products_only": round(flops_step / rate_prod, 1),
                "one_thread": round(flops_step / rate_one, 1)}}


if __name__ == "__main__":
    main()
