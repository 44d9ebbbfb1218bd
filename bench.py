#!/usr/bin/env python3
"""Benchmark of the deterministic training-linear GEMM on one MI355X.

Default workload: the bf16 transformer MLP-up linear 768 -> 3072 at M = 4096
(X[4096,768], W[768,3072] stored [in,out], bias[3072], dY[4096,3072]).  One
step = forward (bi_forward) + dX and dW (bi_linear_backward, whose dX and dW
tiles share one launch at this shape) through the C ABI on the MFMA tier; dX
and dW in launches of their own are timed beside it for reference.  Inputs are
seeded synthetic data already resident in HBM when timing starts.

Prints ONE JSON line with the whole-step throughput (TFLOP/s, from the wall
time of the timed steps), a per-kernel roofline entry for the dominant kernel
(time per launch from batches of back-to-back launches of that kernel, each
batch bracketed by HIP events recorded on the launch stream), and the CPU
oracle's throughput on a bounded sample of the same workload.

Other workloads (--workload): fp8 (e4m3 GEMM 8192x4096x4096), fp8_linear
(scaled fp8 linear forward + backward with quantisation), grouped (8
experts, 16384x2048 -> 1408, forward + dinput + dweights), sweep (forward of
W[4096,4096] at M in {1,3,17,128,1000,8192}), bias_grad (column sums of
dY[4096,3072] and dY[16384,8192], bf16), tiles (forward, dX and dW of the
default workload on each candidate tile, for the tile-choice counters), scalar
(the scalar FMA tier: bf16 768 -> 48 at M = 4096 and the f32 64x128x256
linear).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK = 2516.6   # TFLOP/s, dense bf16/f16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
FP8_PEAK = 5033.2    # TFLOP/s, dense fp8 MFMA
HBM_PEAK = 8000.0    # GB/s
# f32 FMA on the vector ALUs without packed instructions (the library is built
# without packed f32 math): 256 CU x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz
F32_VALU_PEAK = 78.6  # TFLOP/s
BF16_FLOP_PER_CLK = 256 * 4096  # dense bf16 MFMA flop per shader clock, whole chip
TARGET_FRAC = 0.60   # stated target for the default workload: forward, dX, dW each


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="linear",
                    choices=["linear", "fp8", "fp8_linear", "grouped", "sweep", "bias_grad",
                             "tiles", "copy", "scalar"])
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f16"])
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="untimed run of the step before the warm-up steps, so that the GPU "
                         "clocks have left their idle state (once per process)")
    ap.add_argument("--batch-launches", type=int, default=100,
                    help="back-to-back launches per timing batch of each op (five batches); "
                         "fewer keep profiler output small")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--traffic-record", nargs=4, metavar=("RD", "WR", "COPY_RD", "COPY_WR"),
                    help="no GPU: write the HBM traffic record of the default workload from "
                         "four rocprofv3 --pmc output folders (read and write request "
                         "counters of the default workload and of --workload copy)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """Hash of the HIP sources; a committed counter record is valid only for it."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "deterministic_invariant_gemm_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(record: str, op: str):
    """HBM bytes per launch of `op` from the committed rocprofv3 counter record
    (memory-side read and write requests counted by size), or None if the
    record is missing or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", record)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash() or op not in rec.get("kernels", {}):
        return None
    return int(rec["kernels"][op]["traffic_bytes"])


TRAFFIC_RECORD = "linear_768x3072_m4096_traffic"
# kernels of the default workload, by name: the step's forward and shared
# backward, and dX and dW in launches of their own
LINEAR_KERNELS = {"fwd": "mfma_dl_kernel<1, true, false,", "bwd": "mfma_dl_backward_kernel<1>",
                  "dX": "mfma_dl_kernel<1, true, true,", "dW": "mfma_dl_kernel<1, false, false,"}
COPY_BYTES = 512 << 20  # --workload copy


def counter_means(folder: str) -> dict:
    """{kernel name: {counter: mean per dispatch, "dispatches": n}} from the
    csv files a rocprofv3 --pmc run wrote under `folder` (each counter summed
    over its hardware instances within a dispatch)."""
    import csv
    import glob
    disp = {}
    for f in sorted(glob.glob(os.path.join(folder, "**", "*counter_collection.csv"),
                              recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                d = disp.setdefault((f, r["Dispatch_Id"]), {"kernel": r["Kernel_Name"]})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    per = {}
    for d in disp.values():
        acc = per.setdefault(d.pop("kernel"), {})
        for c, v in d.items():
            acc.setdefault(c, []).append(v)
    return {k: dict({c: sum(v) / len(v) for c, v in cs.items()},
                    dispatches=max(len(v) for v in cs.values()))
            for k, cs in per.items()}


def request_bytes(rd: dict, wr: dict):
    """HBM bytes (read, written) of one dispatch from the memory-side request
    counters: each read request moves 32, 64 or 128 bytes as its counter says;
    a write request moves 64 bytes (TCC_EA0_WRREQ_64B) or 32 bytes (the rest
    of TCC_EA0_WRREQ)."""
    read = (32 * rd.get("TCC_EA0_RDREQ_32B", 0.0) + 64 * rd.get("TCC_EA0_RDREQ_64B", 0.0)
            + 128 * rd.get("TCC_EA0_RDREQ_128B", 0.0))
    w64 = wr.get("TCC_EA0_WRREQ_64B", 0.0)
    write = 64 * w64 + 32 * (wr.get("TCC_EA0_WRREQ", w64) - w64)
    return read, write


def write_traffic_record(rd_dir: str, wr_dir: str, copy_rd_dir: str, copy_wr_dir: str):
    """Traffic record of the default workload (profiles/<TRAFFIC_RECORD>.json,
    read back by recorded_traffic, and a markdown summary beside it) from the
    four counter runs; the copy of COPY_BYTES checks the byte accounting."""
    rd, wr = counter_means(rd_dir), counter_means(wr_dir)
    crd, cwr = counter_means(copy_rd_dir), counter_means(copy_wr_dir)
    copy = [k for k in crd if "copyBuffer" in k]
    if len(copy) != 1 or copy[0] not in cwr:
        raise SystemExit("the copy runs hold no single copy kernel")
    c_read, c_write = request_bytes(crd[copy[0]], cwr[copy[0]])
    m, k, n = 4096, 768, 3072
    alg = {"fwd": (2 * (m * k + k * n + n), 2 * m * n),
           "bwd": (2 * (m * n + k * n + m * k), 2 * (m * k + k * n)),
           "dX": (2 * (m * n + k * n), 2 * m * k), "dW": (2 * (m * k + m * n), 2 * k * n)}
    kernels = {}
    for op, pat in LINEAR_KERNELS.items():
        names = [kn for kn in rd if pat in kn]
        if len(names) != 1 or names[0] not in wr:
            raise SystemExit(f"{op}: expected one kernel matching {pat!r}, found {names}")
        r, w = request_bytes(rd[names[0]], wr[names[0]])
        short = names[0].replace("(anonymous namespace)::", "").split("(")[0]
        short = short.replace("void bi::mfma::", "").replace("void bi::", "")
        kernels[op] = {"kernel": short, "read_bytes": r, "write_bytes": w, "traffic_bytes": r + w,
                       "algorithmic_read": alg[op][0], "algorithmic_write": alg[op][1],
                       "dispatches": rd[names[0]]["dispatches"]}
    rec = {"source_hash": kernel_source_hash(),
           "method": "HBM bytes per dispatch = 32, 64, 128 x TCC_EA0_RDREQ_{32B,64B,128B} "
                     "read + 64 x TCC_EA0_WRREQ_64B + 32 x (TCC_EA0_WRREQ - "
                     "TCC_EA0_WRREQ_64B) written, each counter summed over its instances",
           "copy_check": {"bytes": COPY_BYTES, "read_bytes": c_read, "write_bytes": c_write},
           "kernels": kernels}
    base = os.path.join(ROOT, "profiles", TRAFFIC_RECORD)
    with open(base + ".json", "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    cmd = ("rocprofv3 --pmc {c} --output-format csv -d {d} -o run -- "
           "python3 bench.py{w} --steps 3 --warmup 1 --settle-ms 0 --batch-launches 5 "
           "--no-cpu-baseline")
    rdc, wrc = "TCC_EA0_RDREQ_32B TCC_EA0_RDREQ_64B TCC_EA0_RDREQ_128B", \
        "TCC_EA0_WRREQ TCC_EA0_WRREQ_64B"
    lines = ["# HBM traffic: bf16 linear 768->3072 at M=4096", "",
             "Commands (repository root, one MI355X; one counter set per run):", "", "```",
             cmd.format(c=rdc, d=rd_dir, w=""), cmd.format(c=wrc, d=wr_dir, w=""),
             cmd.format(c=rdc, d=copy_rd_dir, w=" --workload copy"),
             cmd.format(c=wrc, d=copy_wr_dir, w=" --workload copy"),
             f"python3 bench.py --traffic-record {rd_dir} {wr_dir} {copy_rd_dir} {copy_wr_dir}",
             "```", "",
             "Bytes per dispatch from the memory-side request counters, each counted at its "
             "size: read = 32 x RDREQ_32B + 64 x RDREQ_64B + 128 x RDREQ_128B, write = "
             "64 x WRREQ_64B + 32 x (WRREQ - WRREQ_64B) (TCC_EA0_ counters summed over the "
             "channels).  No calibration factor: the 512 MiB device copy counts "
             f"{c_read / 2**20:.1f} MiB read and {c_write / 2**20:.1f} MiB written.", "",
             "| op | kernel | HBM read (MB) | algorithmic read (MB) | read / algorithmic | "
             "HBM write (MB) | algorithmic write (MB) |", "|---|---|---|---|---|---|---|"]
    for op, e in kernels.items():
        lines.append(f"| {op} | `{e['kernel']}` | {e['read_bytes'] / 1e6:.1f} | "
                     f"{e['algorithmic_read'] / 1e6:.1f} | "
                     f"{e['read_bytes'] / e['algorithmic_read']:.2f} | "
                     f"{e['write_bytes'] / 1e6:.1f} | {e['algorithmic_write'] / 1e6:.1f} |")
    lines += ["", "fwd and bwd (dX and dW tiles in one launch, bi_linear_backward) make the "
              "step; dX and dW are the same products in launches of their own.  Algorithmic "
              "bytes: every operand read once and the output written once (bwd reads dY once "
              "for both products).", "",
              f"Kernel sources hash at measurement: `{rec['source_hash']}` (bench.py reports "
              "this traffic only while the sources hash the same)."]
    with open(base + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def host_threads() -> int:
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        n = min(n, int(omp))
    return max(n, 1)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class HipEvents:
    """Timing events created with hipEventDisableSystemFence: recording one
    enqueues a timestamp without the system-scope cache writeback and
    invalidation a default event performs, so the events do not slow the
    kernels they bracket (default events add several microseconds per record
    on this GPU).  Elapsed times are read only after a device-wide
    synchronization."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        # the HIP runtime torch has already loaded (same soname)
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.ct = ctypes
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def new(self):
        ev = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        self.made.append(ev)
        return ev

    def record(self, ev, stream):
        rc = self.hip.hipEventRecord(ev, self.ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def ms(self, e0, e1):
        out = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(out), e0, e1)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return out.value

    def close(self):
        for ev in self.made:
            self.hip.hipEventDestroy(ev)
        self.made = []


SETTLE_MS = 400.0
SETTLE_CHUNK = 100  # steps queued between synchronisations
def timing_note():
    return ("value: wall time of the timed steps (no events), after the clock-settle phase "
            "(untimed steps) and the warm-up steps; time per launch of each op: median of "
            f"{BATCHES} batches of {BATCH_LAUNCHES} back-to-back launches of that op, each batch "
            f"bracketed by HIP events on its stream, divided by {BATCH_LAUNCHES}")
_settled = [False]


class ClockSampler:
    """Shader clock (MHz) of GPU 0 read through amdsmi every few milliseconds
    from a host thread while the step runs untimed: the current entry of the
    GFX clock table (amdsmi_get_clk_freq), else the gpu-metrics current_gfxclk
    (which some boards leave stale).  Never active during a timed region."""

    def __init__(self):
        self.samples, self.error, self._stop, self._th = [], None, False, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            self._read()
        except Exception as e:  # no SMI access on this host: report why
            self.error = f"amdsmi unavailable: {e!r}"[:200]

    def _read(self):
        smi = self._smi
        try:
            f = smi.amdsmi_get_clk_freq(self._h, smi.AmdSmiClkType.GFX)
            return float(f["frequency"][f["current"]]) / 1e6
        except Exception:
            return float(smi.amdsmi_get_gpu_metrics_info(self._h)["current_gfxclk"])

    def _loop(self):
        while not self._stop:
            try:
                self.samples.append(self._read())
            except Exception as e:
                self.error = f"amdsmi read failed: {e!r}"[:200]
                return
            time.sleep(0.004)

    def start(self):
        if self.error is None:
            import threading
            self._stop = False
            self._th = threading.Thread(target=self._loop, daemon=True)
            self._th.start()

    def stop(self):
        if self._th is not None:
            self._stop = True
            self._th.join()
            self._th = None

    def summary(self):
        if not self.samples:
            return {"mhz": None, "source": self.error or "no samples"}
        a = np.array(self.samples)
        return {"mhz": float(np.median(a)), "min": float(a.min()), "max": float(a.max()),
                "samples": int(a.size),
                "source": "amdsmi GFX clock (current entry of the clock table), sampled every "
                          "~4 ms while the step ran untimed after the timed regions"}


def settle(torch, ops):
    """Run the step, untimed, for SETTLE_MS of wall time (the first call; later
    calls, after host work such as generating the next inputs, for a quarter of
    that).  An idle MI355X takes a few hundred milliseconds of load to reach
    its working clocks; without this the first few hundred steps run up to
    15 % slower.  Work stays queued throughout (the GPU runs slower for some
    tens of milliseconds after even a few milliseconds without work)."""
    if SETTLE_MS <= 0:
        return
    budget = SETTLE_MS if not _settled[0] else SETTLE_MS / 4
    s = torch.cuda.current_stream()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < budget:
        for _ in range(SETTLE_CHUNK):
            for _, fn in ops:
                fn(s)
        torch.cuda.synchronize()
    _settled[0] = True


def measure_clock(torch, ops, ms=200.0):
    """Shader clock while the step runs untimed for `ms` of wall time, after
    every timed region: polling the SMU through amdsmi slows the GPU for some
    tens of milliseconds afterwards, so no timed region follows it."""
    s = torch.cuda.current_stream()
    clock = ClockSampler()
    t0 = time.perf_counter()
    started = False
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(SETTLE_CHUNK):
            for _, fn in ops:
                fn(s)
        if not started:
            clock.start()
            started = True
        torch.cuda.synchronize()
    clock.stop()
    return clock.summary()


BATCHES, BATCH_LAUNCHES = 5, 100
HOST_BOUND = set()


def timed_steps(torch, ops, steps, warmup):
    """ops: list of (name, fn(stream)); one step runs every op once, in order,
    through the C ABI.

    Timed region: `steps` steps with nothing else on the stream, bracketed by
    device synchronisation; the wall time gives ms per step.  Time per launch
    of each op: BATCHES batches of BATCH_LAUNCHES back-to-back launches of that
    op alone, each batch bracketed by two timing events on the stream the op
    is launched on; the median batch divided by BATCH_LAUNCHES (an event pair
    around every single launch would add its own ~2 us to each).  An op whose
    launches take the host nearly as long to enqueue as the GPU takes to run
    them is named in HOST_BOUND (its time is then the host's).
    Returns (wall ms per step, {name: ms per launch})."""
    settle(torch, ops)
    s = torch.cuda.current_stream()
    for _ in range(warmup):
        for _, fn in ops:
            fn(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for _, fn in ops:
            fn(s)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    hev = HipEvents()
    per = {}
    for name, fn in ops:
        for _ in range(3):
            fn(s)
        ev = [(hev.new(), hev.new()) for _ in range(BATCHES)]
        torch.cuda.synchronize()
        host = []
        for e0, e1 in ev:
            t = time.perf_counter()
            hev.record(e0, s)
            for _ in range(BATCH_LAUNCHES):
                fn(s)
            hev.record(e1, s)
            host.append((time.perf_counter() - t) * 1e3)
        torch.cuda.synchronize()
        gpu = sorted(hev.ms(a, b) for a, b in ev)
        per[name] = gpu[len(gpu) // 2] / BATCH_LAUNCHES
        if sorted(host)[len(host) // 2] >= 0.9 * gpu[len(gpu) // 2]:
            HOST_BOUND.add(name)
    hev.close()
    return wall, per


def cold_launches(torch, ops, reps=10, flush_bytes=1 << 30):
    """Time per launch of each op with the caches cold: before every launch a
    1 GiB buffer is overwritten on the same stream (more than the 256 MB MALL
    and the L2s hold), and only the launch itself is bracketed by events.
    Returns {name: mean ms}."""
    s = torch.cuda.current_stream()
    junk = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    hev = HipEvents()
    out = {}
    for name, fn in ops:
        ev = [(hev.new(), hev.new()) for _ in range(reps)]
        for e0, e1 in ev:
            junk.fill_(1)
            hev.record(e0, s)
            fn(s)
            hev.record(e1, s)
        torch.cuda.synchronize()
        out[name] = sum(hev.ms(a, b) for a, b in ev) / reps
    hev.close()
    del junk
    return out


def cpu_baseline_linear(d, target_s):
    """The oracle, as it is, on the first R rows of the batch (forward, dX and
    dW over those R rows); R grows until the sample takes about target_s."""
    import oracle
    thr = host_threads()
    k, n, dt = d["k"], d["n"], d["dt"]

    def run(r):
        x, dy = d["x"][:r], d["dy"][:r]
        t = time.perf_counter()
        oracle.linear_forward(dt, x, d["w"], d["b"], r, k, n, threads=thr)
        oracle.linear_dx(dt, dy, d["w"], r, k, n, threads=thr)
        oracle.linear_dw(dt, x, dy, r, k, n, threads=thr)
        return time.perf_counter() - t

    r = 16
    dt_s = run(r)
    r = int(min(d["m"], max(16, r * target_s / max(dt_s, 1e-3))))
    reps = 1
    if r == d["m"]:
        # the whole batch is cheaper than the target: time one pass, then repeat it
        reps = max(1, round(target_s / max(run(r), 1e-3)) - 1)
    t = time.perf_counter()
    for _ in range(reps):
        run(r)
    dt_s = time.perf_counter() - t
    flops = reps * 3 * 2.0 * r * k * n
    return {"value": flops / dt_s / 1e12, "unit": "TFLOP/s", "cores": thr, "kind": "oracle",
            "sample": f"forward+dX+dW on the first {r} of {d['m']} rows (K={k}, N={n}), "
                      f"{reps} pass(es), {dt_s:.1f} s, f64 accumulation, {cpu_model()}"}


def bench_linear(args, torch, dig, synth):
    dt = synth.BF16 if args.dtype == "bf16" else synth.F16
    d = synth.mlp_up_linear(dt)
    m, k, n = d["m"], d["k"], d["n"]
    dev = lambda a: torch.from_numpy(a.view(np.int16).copy()).cuda()
    x, w, b, dy = dev(d["x"]), dev(d["w"]), dev(d["b"]), dev(d["dy"])
    y = torch.empty((m, n), dtype=torch.int16, device="cuda")
    dx = torch.empty((m, k), dtype=torch.int16, device="cuda")
    dw = torch.empty((k, n), dtype=torch.int16, device="cuda")
    wsb = dig.bi_backward_dw_workspace_bytes(m, k, n, dt, 1)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    # one training step of the layer: the forward, then both gradients from one
    # call (dX and dW tiles share a launch at this shape)
    ops = [
        ("fwd", lambda s: dig.check(dig.bi_forward(y, x, w, b, m, k, n, dt, s, 1))),
        ("bwd", lambda s: dig.check(dig.bi_linear_backward(dx, dw, dy, x, w, m, k, n, dt,
                                                           ws if wsb else None, wsb, s, 1))),
    ]
    ms, per = timed_steps(torch, ops, args.steps, args.warmup)
    # the two gradients in launches of their own, for reference (not in the step)
    alone = [
        ("dX", lambda s: dig.check(dig.bi_backward_dx(dx, dy, w, m, k, n, dt, s, 1))),
        ("dW", lambda s: dig.check(dig.bi_backward_dw(dw, x, dy, m, k, n, dt,
                                                      ws if wsb else None, wsb, s, 1))),
    ]
    _, sep = timed_steps(torch, alone, args.steps, args.warmup)
    cold = cold_launches(torch, ops)
    # the same step in the other 16-bit dtype (same f32 samples rounded to it)
    odt = synth.F16 if dt == synth.BF16 else synth.BF16
    do = synth.mlp_up_linear(odt)
    xo, wo, bo, dyo = dev(do["x"]), dev(do["w"]), dev(do["b"]), dev(do["dy"])
    ops_o = [
        ("fwd", lambda s: dig.check(dig.bi_forward(y, xo, wo, bo, m, k, n, odt, s, 1))),
        ("bwd", lambda s: dig.check(dig.bi_linear_backward(dx, dw, dyo, xo, wo, m, k, n, odt,
                                                           ws if wsb else None, wsb, s, 1))),
    ]
    ms_o, per_o = timed_steps(torch, ops_o, args.steps, args.warmup)
    del xo, wo, bo, dyo
    flop = 2.0 * m * k * n
    flops = {"fwd": flop, "bwd": 2 * flop, "dX": flop, "dW": flop}
    # algorithmic bytes per launch: each operand read once, the output written once
    # (the shared backward launch reads dY once for both gradients)
    bytes_ = {"fwd": 2 * (m * k + k * n + n + m * n),
              "bwd": 2 * (m * n + k * n + m * k) + 2 * (m * k + k * n)}
    dominant = max(per, key=per.get)
    achieved = flops[dominant] / (per[dominant] * 1e-3) / 1e12
    clock = measure_clock(torch, ops)
    # the dense bf16 MFMA peak at the measured clock, for context beside the
    # fraction of the 2.4 GHz specification peak
    peak_at_clock = (BF16_FLOP_PER_CLK * clock["mhz"] * 1e6 / 1e12) if clock["mhz"] else None
    fastest = max(flops[name] / (v * 1e-3) / 1e12 for name, v in list(per.items()) + list(sep.items()))
    if peak_at_clock is not None and fastest > peak_at_clock:
        # a stale metrics table (seen under a profiler) reads far below the
        # clock the kernels must have run at: report no clock rather than it
        clock = {"mhz": None, "rejected_mhz": clock["mhz"],
                 "source": clock["source"] + "; reading rejected: the peak at that clock is "
                           "below the measured throughput"}
        peak_at_clock = None

    def op_entry(name, v):
        tf = flops[name] / (v * 1e-3) / 1e12
        e = {"us": round(v * 1e3, 2), "tflops": round(tf, 2), "frac_peak": round(tf / BF16_PEAK, 4)}
        if peak_at_clock:
            e["frac_peak_at_sclk"] = round(tf / peak_at_clock, 4)
        return e
    out = {
        "metric": "TFLOP/s and % MFMA peak, bf16 fwd/dX/dW at M=4096, 768->3072; "
                  "bit-exact determinism",
        "value": round(3 * flop / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": f"{args.dtype} training linear 768->3072 (weight [in,out]) at "
                               "M=4096: forward + dX + dW, MFMA tier",
                   "M": m, "K": k, "N": n, "bias": True,
                   "calls": "bi_forward, bi_linear_backward"},
        "timing": timing_note(),
        "roofline": {"bound": "mfma", "kernel": dominant,
                     "achieved": round(achieved, 2), "peak": BF16_PEAK, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_PEAK, 4),
                     "traffic": recorded_traffic("linear_768x3072_m4096_traffic.json", dominant),
                     "algorithmic_bytes": bytes_[dominant]},
        "ops": {name: op_entry(name, v) for name, v in per.items()},
        "separate_launches": {name: op_entry(name, v) for name, v in sep.items()},
        ("f16" if odt == synth.F16 else "bf16"): {
            "value": round(3 * flop / (ms_o * 1e-3) / 1e12, 2), "ms_per_step": round(ms_o, 5),
            "ops": {name: op_entry(name, v) for name, v in per_o.items()}},
        "cold_caches": {"note": "each launch right after 1 GiB was written on its stream (the "
                                "step's 36 MB otherwise stay in the 256 MB MALL); events around "
                                "the launch alone",
                        **{name: {"us": round(v * 1e3, 2)} for name, v in cold.items()}},
        "sclk": dict(clock, peak_bf16_at_sclk_tflops=round(peak_at_clock, 1)
                     if peak_at_clock else None),
    }
    # the stated target for this workload: each of forward, dX and dW at 60 % or
    # more of the dense bf16 peak; the gap per op, beside the result
    fracs = {name: e["frac_peak"] for name, e in out["ops"].items()}
    fracs.update({name: e["frac_peak"] for name, e in out["separate_launches"].items()})
    out["target"] = {"frac_peak": TARGET_FRAC, "met": all(f >= TARGET_FRAC for f in fracs.values()),
                     "gap": {name: round(TARGET_FRAC - f, 4) for name, f in fracs.items()},
                     "us_per_op_at_target": round(flop / (TARGET_FRAC * BF16_PEAK * 1e12) * 1e6, 2)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_linear(d, args.cpu_seconds)
    return out


def bench_fp8(args, torch, dig, synth):
    """fp8 e4m3 GEMM A[8192,4096] x B^T[4096,4096] and its first 16 rows, on the
    exact default path (codes widened to bf16, bf16 matrix instruction) and on
    the opt-in fast path (tc = 3, fp8 matrix instruction)."""
    d = synth.fp8_8192x4096x4096()
    m, k, n = d["m"], d["k"], d["n"]
    a = torch.from_numpy(d["a8"]).cuda()
    bt = torch.from_numpy(d["bt8"]).cuda()
    da = torch.tensor([float(d["da"])], dtype=torch.float32, device="cuda")
    db = torch.tensor([float(d["db"])], dtype=torch.float32, device="cuda")
    y = torch.empty((m, n), dtype=torch.int16, device="cuda")
    y16 = torch.empty((16, n), dtype=torch.int16, device="cuda")
    fast = dig.TC_FP8_FAST
    ops = [("fp8_m8192", lambda s: dig.check(dig.bi_fp8_mm(y, a, bt, da, db, m, k, n, s, 1))),
           ("fp8_m16", lambda s: dig.check(dig.bi_fp8_mm(y16, a, bt, da, db, 16, k, n, s, 1))),
           ("fp8_fast_m8192",
            lambda s: dig.check(dig.bi_fp8_mm(y, a, bt, da, db, m, k, n, s, fast))),
           ("fp8_fast_m16",
            lambda s: dig.check(dig.bi_fp8_mm(y16, a, bt, da, db, 16, k, n, s, fast)))]
    ms, per = timed_steps(torch, ops, args.steps, args.warmup)
    flop = 2.0 * m * k * n
    ach = {key: flop / (per[key] * 1e-3) / 1e12 for key in ("fp8_m8192", "fp8_fast_m8192")}
    b16 = 16 * k + n * k + 16 * n * 2
    small = {key: {"us": round(per[key] * 1e3, 2),
                   "GBps": round(b16 / (per[key] * 1e-3) / 1e9, 1),
                   "frac_hbm": round(b16 / (per[key] * 1e-3) / 1e9 / HBM_PEAK, 4)}
             for key in ("fp8_m16", "fp8_fast_m16")}
    return {
        "metric": "fp8 e4m3 GEMM TFLOP/s", "value": round(ach["fp8_m8192"], 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": "fp8 e4m3 A[8192,4096] x B^T[4096,4096], per-tensor scales, "
                               "bf16 out; plus M=16; exact path (value) and fast path",
                   "M": m, "K": k, "N": n},
        "roofline": {"bound": "mfma", "kernel": "fp8_m8192", "achieved": round(ach["fp8_m8192"], 2),
                     "peak": FP8_PEAK, "unit": "TFLOP/s",
                     "frac": round(ach["fp8_m8192"] / FP8_PEAK, 4), "traffic": None},
        "fast": {"us": round(per["fp8_fast_m8192"] * 1e3, 2),
                 "tflops": round(ach["fp8_fast_m8192"], 2),
                 "frac_peak": round(ach["fp8_fast_m8192"] / FP8_PEAK, 4)},
        "m16": small,
    }


def bench_fp8_linear(args, torch, dig, synth):
    """Scaled fp8 linear on x[8192,4096], w[4096,4096] ([out,in]), g[8192,4096]:
    forward (quantise x and w, fp8 GEMM + bias) and backward (quantise g,
    transposed copies of w, g and x, the dX and dW fp8 GEMMs), all through the
    C ABI; plus the quantiser and the transposing quantiser alone on x."""
    d = synth.fp8_linear(8192, 4096, 4096, seed=45)
    m, k, n = d["m"], d["k"], d["n"]
    dev = lambda a: torch.from_numpy(a.view(np.int16).copy()).cuda()
    x, w, g, b = dev(d["x"]), dev(d["w"]), dev(d["g"]), dev(d["b"])
    sc = {key: torch.tensor([float(d[key])], dtype=torch.float32, device="cuda")
          for key in ("sx", "sw", "sg", "sx_inv", "sw_inv", "sg_inv")}
    amax = torch.zeros(4, dtype=torch.float32, device="cuda")
    y = torch.empty((m, n), dtype=torch.int16, device="cuda")
    dx = torch.empty((m, k), dtype=torch.int16, device="cuda")
    dw = torch.empty((n, k), dtype=torch.int16, device="cuda")
    nb = dig.bi_fp8_linear_workspace_bytes(m, k, n)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    q = torch.empty(m * k, dtype=torch.uint8, device="cuda")
    a0, a1, a2 = (amax[i:i + 1] for i in range(3))
    step = [
        ("forward", lambda s: dig.check(dig.bi_fp8_linear_forward(
            y, x, w, b, sc["sx"], sc["sw"], sc["sx_inv"], sc["sw_inv"], a0, a1, m, k, n, ws, nb,
            s, 1))),
        ("backward", lambda s: dig.check(dig.bi_fp8_linear_backward(
            dx, dw, g, x, w, sc["sg"], sc["sw"], sc["sx"], sc["sg_inv"], sc["sw_inv"],
            sc["sx_inv"], a2, m, k, n, ws, nb, s, 1))),
    ]
    ms, per = timed_steps(torch, step, args.steps, args.warmup)
    alone = [
        ("quantize", lambda s: dig.check(dig.bi_fp8_quantize(q, x, sc["sx_inv"], a0, m * k,
                                                             dig.BI_FP8_E4M3, s))),
        ("transpose_quantize", lambda s: dig.check(dig.bi_fp8_transpose_quantize(
            q, x, sc["sx_inv"], a0, m, k, dig.BI_FP8_E4M3, s))),
    ]
    _, qper = timed_steps(torch, alone, args.steps, args.warmup)
    flop = 3 * 2.0 * m * k * n
    qbytes = 3 * m * k  # 2 bytes read + 1 byte written per element
    qgbps = {name: qbytes / (v * 1e-3) / 1e9 for name, v in qper.items()}
    dominant = max(qgbps, key=lambda name: qper[name])
    return {
        "metric": "scaled fp8 linear step TFLOP/s (quantisation included)",
        "value": round(flop / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": "scaled fp8 linear x[8192,4096] w[4096,4096] g[8192,4096]: "
                               "forward + backward (dX, dW), e4m3fn, bias", "M": m, "K": k,
                   "N": n},
        "ops": {name: {"us": round(v * 1e3, 2)} for name, v in per.items()},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(qgbps[dominant], 1),
                     "peak": HBM_PEAK, "unit": "GB/s",
                     "frac": round(qgbps[dominant] / HBM_PEAK, 4), "traffic": None,
                     "algorithmic_bytes": qbytes},
        "quantizers": {name: {"us": round(v * 1e3, 2), "GBps": round(qgbps[name], 1)}
                       for name, v in qper.items()},
    }


def bench_grouped(args, torch, dig, synth):
    d = synth.grouped_16384x2048x1408_e8()
    m, k, n, e = d["m"], d["k"], d["n"], d["e"]
    dev = lambda a: torch.from_numpy(a.view(np.int16).copy()).cuda()
    inp, w, dy = dev(d["input"]), dev(d["weights"]), dev(d["dy"])
    ids = torch.from_numpy(d["row_experts"].view(np.int32).copy()).cuda()
    off = torch.from_numpy(d["offsets"].view(np.int32).copy()).cuda()
    y = torch.empty((m, n), dtype=torch.int16, device="cuda")
    di = torch.empty((m, k), dtype=torch.int16, device="cuda")
    dwt = torch.empty((e, n, k), dtype=torch.float32, device="cuda")
    bt = synth.BF16
    ops = [("grouped_fwd", lambda s: dig.check(dig.bi_grouped_nt(y, inp, w, ids, off, m, k, n, e,
                                                                 bt, s, 1))),
           ("grouped_bwd", lambda s: dig.check(dig.bi_grouped_nt_backward(
               di, dwt, inp, w, dy, ids, off, m, k, n, e, bt, s, 1)))]
    ms, per = timed_steps(torch, ops, args.steps, args.warmup)
    valid = int(d["offsets"][e])
    flop = 2.0 * valid * k * n
    ach = flop / (per["grouped_fwd"] * 1e-3) / 1e12
    return {
        "metric": "grouped GEMM TFLOP/s (valid rows)", "value": round(3 * flop / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "row-routed grouped GEMM input[16384,2048] x weights[8,1408,2048]^T, "
                               "5% padding rows: forward + dinput + f32 dweights",
                   "M": m, "K": k, "N": n, "E": e, "valid_rows": valid},
        "roofline": {"bound": "mfma", "kernel": "grouped_fwd", "achieved": round(ach, 2),
                     "peak": BF16_PEAK, "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK, 4),
                     "traffic": None},
        "ops": {k_: {"us": round(v * 1e3, 2)} for k_, v in per.items()},
    }


def bench_sweep(args, torch, dig, synth):
    d = synth.square_4096_sweep()
    m, k, n = d["m"], d["k"], d["n"]
    dev = lambda a: torch.from_numpy(a.view(np.int16).copy()).cuda()
    x, w = dev(d["x"]), dev(d["w"])
    y = torch.empty((m, n), dtype=torch.int16, device="cuda")
    bt = synth.BF16
    res = {}
    for mp in (1, 3, 17, 128, 1000, 8192):
        ops = [(f"m{mp}", lambda s, mp=mp: dig.check(dig.bi_forward(y, x, w, None, mp, k, n, bt,
                                                                    s, 1)))]
        _, per = timed_steps(torch, ops, max(args.steps // 4, 10), 5)
        us = per[f"m{mp}"] * 1e3
        byt = 2 * (mp * k + k * n + mp * n)
        res[mp] = {"us": round(us, 2), "tflops": round(2.0 * mp * k * n / (us * 1e-6) / 1e12, 2),
                   "GBps": round(byt / (us * 1e-6) / 1e9, 1)}
    big = res[8192]
    return {"metric": "forward TFLOP/s, W[4096,4096] batch sweep", "value": big["tflops"],
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": big["us"] / 1e3, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "bf16 forward, W[4096,4096], M sweep", "K": k, "N": n},
            "roofline": {"bound": "mfma", "kernel": "m8192", "achieved": big["tflops"],
                         "peak": BF16_PEAK, "unit": "TFLOP/s",
                         "frac": round(big["tflops"] / BF16_PEAK, 4), "traffic": None},
            "sweep": res}


def bench_bias_grad(args, torch, dig, synth):
    """Bias gradient db = RNE(column sums of dY): the dY of the default linear
    workload [4096,3072] and a larger [16384,8192], both bf16.  HBM-bound:
    algorithmic bytes = dY read once + db written once."""
    bt = synth.BF16
    shapes = {"db_4096x3072": (4096, 3072), "db_16384x8192": (16384, 8192)}
    ops, nbytes = [], {}
    keep = []
    for name, (m, n) in shapes.items():
        dy = torch.from_numpy(synth.normal_bits((m, n), 1.0, 2, 4, bt).view(np.int16)).cuda()
        db = torch.empty(n, dtype=torch.int16, device="cuda")
        wsb = dig.bi_bias_grad_workspace_bytes(m, n, bt)
        ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device="cuda")
        keep += [dy, db, ws]
        ops.append((name, lambda s, dy=dy, db=db, ws=ws, m=m, n=n, wsb=wsb: dig.check(
            dig.bi_bias_grad(db, dy, m, n, bt, ws if wsb else None, wsb, s))))
        nbytes[name] = 2 * (m * n + n)
    ms, per = timed_steps(torch, ops, args.steps, args.warmup)
    gbps = {k_: nbytes[k_] / (v * 1e-3) / 1e9 for k_, v in per.items()}
    main_op = "db_4096x3072"
    dominant = max(per, key=per.get)
    return {"metric": "bias gradient GB/s (dY read + db write)", "value": round(gbps[main_op], 1),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "bf16 bias gradient, dY[4096,3072] (and dY[16384,8192])",
                       "M": 4096, "N": 3072},
            "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(gbps[dominant], 1),
                         "peak": HBM_PEAK, "unit": "GB/s",
                         "frac": round(gbps[dominant] / HBM_PEAK, 4), "traffic": None,
                         "algorithmic_bytes": nbytes[dominant]},
            "ops": {k_: {"us": round(v * 1e3, 2), "GBps": round(gbps[k_], 1)}
                    for k_, v in per.items()}}


def bench_scalar(args, torch, dig, synth):
    """The scalar FMA tier: the bf16 linear 768 -> 48 at M = 4096 (N < 64, so
    the forward and dW run the scalar tier; dW in 256-row chunks plus the
    ordered chunk sum) and the f32 linear X[64,128] W[128,256] (forward, dX,
    dW).  ALU-bound: f32 FMAs on the vector ALUs."""
    dev = lambda a: torch.from_numpy(a.view(np.int16 if a.dtype == np.uint16 else np.int32)
                                     .copy()).cuda()
    keep, ops, flops = [], [], {}
    for tag, d in (("n48", synth.mlp_up_linear(synth.BF16, n=48, seed=22)),
                   ("f32", synth.f32_linear_64x128x256())):
        m, k, n, dt = d["m"], d["k"], d["n"], d["dt"]
        tdt = torch.int16 if dt != synth.F32 else torch.int32
        x, w, b, dy = dev(d["x"]), dev(d["w"]), dev(d["b"]), dev(d["dy"])
        y = torch.empty((m, n), dtype=tdt, device="cuda")
        dx = torch.empty((m, k), dtype=tdt, device="cuda")
        dw = torch.empty((k, n), dtype=tdt, device="cuda")
        wsb = dig.bi_backward_dw_workspace_bytes(m, k, n, dt, 1)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        keep += [x, w, b, dy, y, dx, dw, ws]
        assert dig.bi_plan(dig.OP_FWD, dt, 1, k, n)[0] == 0  # scalar tier
        ops.append((f"{tag}_fwd", lambda s, y=y, x=x, w=w, b=b, m=m, k=k, n=n, dt=dt:
                    dig.check(dig.bi_forward(y, x, w, b, m, k, n, dt, s, 1))))
        ops.append((f"{tag}_dW", lambda s, dw=dw, x=x, dy=dy, m=m, k=k, n=n, dt=dt, ws=ws, wsb=wsb:
                    dig.check(dig.bi_backward_dw(dw, x, dy, m, k, n, dt, ws if wsb else None, wsb,
                                                 s, 1))))
        if tag == "f32":
            ops.append((f"{tag}_dX", lambda s, dx=dx, dy=dy, w=w, m=m, k=k, n=n, dt=dt:
                        dig.check(dig.bi_backward_dx(dx, dy, w, m, k, n, dt, s, 1))))
        for op in ("fwd", "dW", "dX"):
            flops[f"{tag}_{op}"] = 2.0 * m * k * n
    ms, per = timed_steps(torch, ops, args.steps, args.warmup)
    tf = {name: flops[name] / (v * 1e-3) / 1e12 for name, v in per.items()}
    main_op = "n48_fwd"
    return {"metric": "scalar FMA tier TFLOP/s (bf16 linear 768->48 at M=4096, forward)",
            "value": round(tf[main_op], 3), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": "scalar FMA tier: bf16 linear X[4096,768] W[768,48] + b "
                                   "(forward, chunked dW) and f32 linear X[64,128] W[128,256] + b "
                                   "(forward, dX, dW)"},
            "roofline": {"bound": "alu", "kernel": main_op, "achieved": round(tf[main_op], 3),
                         "peak": F32_VALU_PEAK, "unit": "TFLOP/s",
                         "frac": round(tf[main_op] / F32_VALU_PEAK, 4), "traffic": None},
            "ops": {name: {"us": round(v * 1e3, 2), "tflops": round(tf[name], 3),
                           "frac_alu_peak": round(tf[name] / F32_VALU_PEAK, 4)}
                    for name, v in per.items()}}


# Candidate MFMA tiles per op of the default workload (tile id 40 + base: direct
# loads; 100 + base: the same with copies spread between MFMAs).  Shapes:
# 41 256x256 2x2 waves, 42 256x192 2x2, 44 128x128 2x2, 45 128x96 4x1,
# 48 96x96 3x1, 49 128x192 2x2, 50 256x96 4x1, 51 256x192 4x2, 52 256x256 4x2,
# 55 128x128 2x4, 57 96x96 1x3.  The first id of each list is the default.
TILE_CANDIDATES = {
    "fwd": [111, 51, 52, 41, 42, 44, 49, 55, 115],
    "dX": [45, 44, 105, 115, 55, 50, 51, 42],
    "dW": [57, 48, 44, 45, 115, 55, 104, 108, 105],
}


def bench_tiles(args, torch, dig, synth):
    """Forward, dX and dW of the default workload on every candidate tile
    (forced with tc = 16 + id; every tile gives the same bits).  Used with
    rocprofv3 counters to compare MFMA busy time, LDS bank conflicts and HBM
    traffic between tiles."""
    d = synth.mlp_up_linear(synth.BF16)
    m, k, n, dt = d["m"], d["k"], d["n"], synth.BF16
    dev = lambda a: torch.from_numpy(a.view(np.int16).copy()).cuda()
    x, w, b, dy = dev(d["x"]), dev(d["w"]), dev(d["b"]), dev(d["dy"])
    y = torch.empty((m, n), dtype=torch.int16, device="cuda")
    dx = torch.empty((m, k), dtype=torch.int16, device="cuda")
    dw = torch.empty((k, n), dtype=torch.int16, device="cuda")
    calls = {
        "fwd": lambda s, tc: dig.check(dig.bi_forward(y, x, w, b, m, k, n, dt, s, tc)),
        "dX": lambda s, tc: dig.check(dig.bi_backward_dx(dx, dy, w, m, k, n, dt, s, tc)),
        "dW": lambda s, tc: dig.check(dig.bi_backward_dw(dw, x, dy, m, k, n, dt, None, 0, s, tc)),
    }
    flop = 2.0 * m * k * n
    res = {}
    for op, ids in TILE_CANDIDATES.items():
        ops = [(f"{op}:{t}", lambda s, f=calls[op], t=t: f(s, 16 + t)) for t in ids]
        with dig.testing_build():
            _, per = timed_steps(torch, ops, args.steps, args.warmup)
        res[op] = {str(t): {"us": round(per[f"{op}:{t}"] * 1e3, 2),
                            "tflops": round(flop / (per[f"{op}:{t}"] * 1e-3) / 1e12, 1)}
                   for t in ids}
    default_ms = sum(per_op[str(TILE_CANDIDATES[op][0])]["us"] for op, per_op in res.items()) / 1e3
    return {"metric": "forward/dX/dW time per candidate tile", "value":
            round(3 * flop / (default_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(default_ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "bf16 linear 768->3072 at M=4096, each op on each candidate "
                                   "tile", "M": m, "K": k, "N": n},
            "roofline": None, "tiles": res}


def bench_copy(args, torch, dig, synth):
    """Plain device-to-device copy of a 512 MiB buffer: the known-size kernel
    used to calibrate the FETCH_SIZE / WRITE_SIZE counters, and a measured HBM
    bandwidth reference."""
    n = 256 * 1024 * 1024
    src = torch.ones(n, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    ms, per = timed_steps(torch, [("copy", lambda s: dst.copy_(src))], args.steps, args.warmup)
    nbytes = 2 * 2 * n
    gbps = nbytes / (per["copy"] * 1e-3) / 1e9
    return {"metric": "device copy GB/s (read + write)", "value": round(gbps, 1), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
            "data": "synthetic", "config": {"workload": "copy of 512 MiB (read 512 MiB, write 512 MiB)",
                                            "bytes_read": 2 * n, "bytes_written": 2 * n},
            "roofline": {"bound": "hbm", "kernel": "copy", "achieved": round(gbps, 1),
                         "peak": HBM_PEAK, "unit": "GB/s", "frac": round(gbps / HBM_PEAK, 4),
                         "traffic": None}}


def main():
    args = parse()
    if args.traffic_record:
        write_traffic_record(*args.traffic_record)
        return
    global SETTLE_MS, BATCH_LAUNCHES
    SETTLE_MS = args.settle_ms
    BATCH_LAUNCHES = max(1, args.batch_launches)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import deterministic_invariant_gemm_amd as dig
    import synth
    dig.load()
    fn = {"linear": bench_linear, "fp8": bench_fp8, "fp8_linear": bench_fp8_linear,
          "grouped": bench_grouped,
          "sweep": bench_sweep, "bias_grad": bench_bias_grad, "tiles": bench_tiles,
          "copy": bench_copy, "scalar": bench_scalar}[args.workload]
    out = fn(args, torch, dig, synth)
    out.setdefault("timing", timing_note())
    if HOST_BOUND:
        out["host_bound_ops"] = sorted(HOST_BOUND)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
