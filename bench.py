"""Benchmark of the gfx950 dense GEMM library on one MI355X.

One step = one C = A x B on the headline workload (M = N = K = 8192, BF16
inputs drawn from N(0,1) with a fixed seed, FP32 accumulation and output),
with A, B and C resident in HBM before the timed region.

Timing protocol for the headline:
  1. one launch into a NaN-filled C, checked for unwritten outputs;
  2. settle: back-to-back launches from idle for at least 200 ms.  The board's
     power controller clamps the clock hard when a heavy load starts and
     relaxes it over the next few tens of milliseconds (a kernel trace shows
     launches 3-6 at 880-1030 us against 714 us once settled), so a window
     taken straight after idle measures that transient, not the kernel.  The
     first K of these launches are timed and reported as `cold_first_k_ms`;
  3. W untimed warm-up steps, then exactly K timed steps between HIP events
     on the stream the library launches on: `value` = 2MNK / mean step time;
  4. the steady state: the median over 5 windows of at least 50 ms each,
     reported beside `value` (with the board's clock and power sampled through
     amdsmi meanwhile, where the box allows it).

Printed on stdout as one JSON line; progress goes to stderr.  Besides the
headline it carries:
  roofline      the dominant kernel against the MI355X dense BF16 matrix peak,
                with HBM traffic from the committed rocprofv3 counter summary
                (null once the kernel sources differ from the profiled ones)
                and the kernel's resources (registers, LDS, scratch, occupancy);
  cpu_baseline  the CPU oracle timed on this host on a bounded sample of the
                same workload (whole rows of C), with the GPU rows checked
                against it;
  by_workload   the other workloads (256^3 to 8192^3; FP32, FP16, BF16, INT8;
                operand layouts, the general output step, device conversion)
                and the naive one-work-item-per-output kernel at 1024^3, each
                with its kernel's resources and, for the plain products, the
                oracle timed on a bounded sample with the GPU rows checked.

`--gpus N` with N > 1 exits with an error: the library runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOPS (2MNK/s) and % of MI355X peak at M=N=K=1024/2048/8192"
# MI355X datasheet peaks (dense): 256 CUs x 2.4 GHz x FLOP/clock/CU
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3,
               "i8": 5033.2}  # INT8: TOPS, twice the 16-bit matrix rate
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
RESOURCES_FILE = os.path.join(ROOT, "dense_gemm_16_amd", "kernel_resources.json")
SETTLE_MS = 200.0
# Small, launch-bound workloads also timed as replays of a captured HIP graph.
GRAPH_TIMED = ("c0-f16-256", "c1-f32-1024", "c2-f16-1024")
EXTRA = ["c0-f16-256", "c1-f32-1024", "c1-f32-1024-int", "c2-f16-1024", "c3-f16-2048", "c3-bf16-2048",
         "c3r-f16-2050x2047x2056", "c4f-f32-4096", "s8-bf16-1024x8192x8192",
         "s2x4-bf16-4096x2048x8192", "lk-bf16-512x512x65536", "lk-f32-512x512x16384", "i8u-1000", "f32u-2049"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    """Hash of the library sources; counter-derived traffic is only valid for this hash."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_gemm_16_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _compiler_figures():
    try:
        with open(RESOURCES_FILE) as f:
            return json.load(f).get("kernels", {})
    except (OSError, ValueError):
        return {}


class Problem:
    """Device-resident operands of one workload and a launcher for it.  The
    workspace the call asks for (migemm_workspace_size) is allocated once and
    lent to every launch (migemm_gemm_ws)."""

    def __init__(self, w, variant=-1, config=-1, alpha=1.0, beta=0.0, c_code=0, ta=False,
                 tb=False):
        import torch
        import dense_gemm_16_amd as mg
        from dense_gemm_16_amd import inputs
        self.w, self.mg = w, mg
        self.A, self.B = w.make()
        # operands given transposed are stored K x M (A) and N x K (B)
        self.dA = (self.A.t().contiguous() if ta else self.A).cuda()
        self.dB = (self.B.t().contiguous() if tb else self.B).cuda()
        self.lda, self.ldb = (w.M if ta else w.K), (w.K if tb else w.N)
        self.ops = (int(ta), int(tb))
        if w.dtype == "i8":
            c_code = 4  # INT32 C, the only output of an INT8 product
        cdt = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16, 4: torch.int32}[c_code]
        self.C = torch.empty((w.M, w.N), dtype=cdt, device="cuda")
        if beta != 0.0:
            self.C.copy_(torch.randn((w.M, w.N), generator=torch.Generator().manual_seed(w.seed + 1)))
        if self.C.dtype == torch.int32:
            self.C.zero_()
        self.epi = (float(alpha), float(beta), c_code)
        self.general = not (alpha == 1.0 and beta == 0.0 and c_code == 0)
        self.code = inputs.DTYPE_CODES[w.dtype]
        shape = (w.M, w.N, w.K, self.code, self.dA.data_ptr(), self.lda, self.dB.data_ptr(),
                 self.ldb)
        st, n = mg.migemm_workspace_size(variant, config, *self.ops, *shape)
        if st != mg.OK:
            raise RuntimeError(f"{w.name}: {mg.migemm_status_string(st)}")
        self.ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
        self.ws_args = (self.ws.data_ptr(), n) if n else (None, 0)
        self.desc = mg.describe(variant, config, *self.ops, *shape, c_code, w.N, n)
        names = [mg.migemm_variant_name(v) for v in range(mg.migemm_variant_count())]
        self.variant, self.config = names.index(self.desc["variant"]), self.desc["config"]
        self.stream = torch.cuda.current_stream()
        self.sp = self.stream.cuda_stream
        self.launches = 0  # launches of this problem so far (to find the timed ones in a trace)
        self.args = (self.variant, self.config, *self.ops, *shape, *self.epi, self.C.data_ptr(),
                     w.N, *self.ws_args, self.sp)

    def kernel_name(self):
        return (f"{self.mg.migemm_variant_name(self.variant)}["
                f"{self.mg.migemm_config_name(self.variant, self.config)}]")

    def layout(self):
        return "".join("T" if t else "N" for t in self.ops)

    def resources(self):
        """Per launch of one call: workgroups, workgroup size, the runtime's
        register / LDS / scratch / occupancy figures and the compiler's."""
        d, figs = self.desc, _compiler_figures()
        by_demangled = {v.get("demangled"): v for v in figs.values()}
        out = {"workspace_bytes": d.get("workspace_bytes", 0), "launches": []}
        for i in range(d.get("launches", 0)):
            e = {"grid": d.get(f"grid{i}"), "block": d.get(f"block{i}")}
            for key in ("kernel", "regs", "lds_bytes", "scratch_bytes", "workgroups_per_cu",
                        "waves_per_simd", "resources"):
                if f"{key}{i}" in d:
                    e[key] = d[f"{key}{i}"]
            name = e.get("kernel", "")
            comp = figs.get(name) or by_demangled.get(name)
            if comp:
                e["compiler"] = {k: v for k, v in comp.items() if k != "demangled"}
            out["launches"].append(e)
        return out

    def launch(self):
        self.launches += 1
        st = self.mg.migemm_gemm_ws(*self.args)
        if st != self.mg.OK:
            raise RuntimeError(f"{self.w.name}: {self.mg.migemm_status_string(st)} "
                               f"(hip {self.mg.migemm_last_hip_error()})")

    def _window(self, n):
        """Mean ms per launch over n back-to-back launches (HIP events on the stream)."""
        import torch
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(self.stream)
        for _ in range(n):
            self.launch()
        t1.record(self.stream)
        t1.synchronize()
        return t0.elapsed_time(t1) / n

    def time(self, steps, warmup):
        import torch
        for _ in range(warmup):
            self.launch()
        torch.cuda.synchronize()
        ms = self._window(steps)
        torch.cuda.synchronize()
        return ms

    def time_window(self, min_ms=50.0, lo=20, hi=2000):
        """Mean ms per launch over a window of at least min_ms (lo..hi launches)."""
        est = self.time(3, 2)
        n = int(min(hi, max(lo, min_ms / max(est, 1e-4))))
        return self.time(n, 0), n

    def graph_rate(self, per_graph=100, replays=5):
        """The kernels' own rate without the host's per-call launch cost: `per_graph`
        calls captured into one HIP graph on a side stream (default priority), then
        the median ms per call over `replays` replays timed with HIP events.  Also
        whether C after a replay equals C after an eager call, bit for bit (C is
        poisoned before the replay; plain overwrites only)."""
        import torch
        mg = self.mg
        self.launch()
        torch.cuda.synchronize()
        eager = self.C.clone()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=s):
            args = self.args[:-1] + (torch.cuda.current_stream().cuda_stream,)
            for _ in range(per_graph):
                st = mg.migemm_gemm_ws(*args)
                if st != mg.OK:
                    raise RuntimeError(f"{self.w.name}: {mg.migemm_status_string(st)} in capture")
        torch.cuda.synchronize()
        self.C.fill_(float("nan") if self.C.is_floating_point() else -2147483641)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(self.C, eager))
        times = []
        for _ in range(replays):
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            g.replay()
            t1.record()
            t1.synchronize()
            times.append(t0.elapsed_time(t1) / per_graph)
        del g
        return statistics.median(times), same

    def settle(self, k, min_ms=SETTLE_MS):
        """Back-to-back launches from idle until min_ms have run.  Returns the
        mean ms of the first k (the cold window), and the launches and ms in all."""
        import torch
        torch.cuda.synchronize()
        cold = self._window(k)
        n, total = k, cold * k
        while total < min_ms:
            m = int(max(10, min(2000, (min_ms - total) / max(cold, 1e-3) + 1)))
            total += self._window(m) * m
            n += m
        return cold, n, total

    def steady(self, windows=5, min_ms=50.0):
        """Median ms per launch over `windows` windows of at least min_ms each."""
        t = [self.time_window(min_ms) for _ in range(windows)]
        return statistics.median(x for x, _ in t), [round(x, 5) for x, _ in t], t[0][1]


class ClockProbe:
    """The board's graphics clock and socket power (amdsmi GPU metrics) while a
    problem runs back to back: the launches of a window of about `ms` are queued
    first, then the host samples the metrics until the window's end event has
    passed.  Reports a note instead of figures when amdsmi is not usable on the
    box or the GPU cannot be matched to an amdsmi device."""

    def __init__(self):
        self.error, self._h, self.max_clk = None, None, None
        try:
            import amdsmi
            import torch
            self._smi = amdsmi
            amdsmi.amdsmi_init()
            bus = torch.cuda.get_device_properties(0).pci_bus_id
            for h in amdsmi.amdsmi_get_processor_handles():
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                if int(bdf.split(":")[1], 16) == int(bus):
                    self._h = h
            if self._h is None:
                self.error = f"no amdsmi device on PCI bus {bus}"
            else:
                info = amdsmi.amdsmi_get_clock_info(self._h, amdsmi.AmdSmiClkType.GFX)
                self.max_clk = info.get("max_clk")
        except Exception as e:  # amdsmi missing, no permission, older torch ...
            self.error = f"{type(e).__name__}: {e}"[:200]

    def during(self, p, ms=1500.0):
        import torch
        if self._h is None:
            return {"source": "amdsmi GPU metrics", "samples": 0, "note": self.error}
        est = p.time(3, 1)
        n = int(max(20, min(5000, ms / max(est, 1e-3))))
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(p.stream)
        for _ in range(n):
            p.launch()
        t1.record(p.stream)
        samples = []
        while not t1.query():
            try:
                m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
            except Exception as e:
                self.error = f"{type(e).__name__}: {e}"[:200]
                break
            clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int)]
            pw = m.get("current_socket_power")
            if clks:
                samples.append((statistics.mean(clks), pw if isinstance(pw, (int, float)) else None,
                                m.get("temperature_hotspot")))
            time.sleep(0.002)
        t1.synchronize()
        window_ms = t0.elapsed_time(t1) / n
        # the firmware refreshes these metrics every few hundred milliseconds, and the
        # first samples can still show the idle board: the second half is the figure
        mid = samples[len(samples) // 2:]
        clk = [c for c, _, _ in mid]
        pw = [x for _, x, _ in mid if x is not None]
        tmp = [t for _, _, t in mid if isinstance(t, (int, float))]
        if not clk:
            return {"source": "amdsmi GPU metrics", "samples": 0,
                    "note": self.error or "no samples"}
        return {"source": "amdsmi GPU metrics (current_gfxclks averaged over the XCDs, "
                          "current_socket_power), sampled by the host during a window of "
                          f"{n} back-to-back launches; second half of the samples (the "
                          "firmware refreshes them every few hundred milliseconds)",
                "samples": len(mid), "window_ms_per_launch": round(window_ms, 5),
                "gfxclk_mhz_median": round(statistics.median(clk), 1),
                "gfxclk_mhz_min": round(min(clk), 1), "gfxclk_mhz_max": round(max(clk), 1),
                "gfxclk_limit_mhz": self.max_clk,
                "socket_power_w_median": round(statistics.median(pw), 1) if pw else None,
                "socket_power_w_max": max(pw) if pw else None,
                "hotspot_c_max": max(tmp) if tmp else None}


def oracle_check(p, seconds=2.0):
    """The CPU oracle on a bounded sample of p's product (whole rows of C, all of
    them when it fits the budget), timed, and p's GPU rows checked against it."""
    import numpy as np
    import oracle
    from oracle.check import compare, tolerance
    from dense_gemm_16_amd import inputs
    w = p.w
    bA, bB = inputs.to_bits(p.A), inputs.to_bits(p.B)
    thr = oracle.default_threads()
    used = oracle.threads_used(thr)
    per_row = 2.0 * w.N * w.K
    if w.M * per_row <= 2e10:
        rows = w.M
    else:
        r0 = max(used, 8)
        t = time.perf_counter()
        oracle.gemm(bA[:r0], bB, p.code, nthreads=thr)
        rate = r0 / max(time.perf_counter() - t, 1e-4)
        rows = int(min(w.M, max(used, rate * seconds)))
    t = time.perf_counter()
    ref, S = oracle.gemm(bA[:rows], bB, p.code, nthreads=thr)
    dt = time.perf_counter() - t
    got = p.C[:rows].cpu().numpy().astype(np.float64)
    chk = compare(got, ref, S, tol=None if w.exact else tolerance(p.code), exact=w.exact)
    return {"rows": rows, "seconds": round(dt, 3),
            "gflops": round(2.0 * rows * w.N * w.K / dt / 1e9, 2), "cores": used,
            "gpu_rows_vs_oracle": str(chk), "gpu_rows_ok": bool(chk.ok)}


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it still applies."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None, "no counter summary"
    e = t.get("entries", {}).get(workload)
    if not e:
        return None, "workload not profiled"
    if e.get("source_hash") != source_hash() or e.get("kernel") != kernel:
        return None, "kernel changed since the counters were taken"
    return e["hbm_bytes_per_launch"], e.get("note", "")


def cpu_baseline(p, seconds):
    """Time the CPU oracle on whole rows of C and check the GPU's rows against it."""
    import numpy as np
    import oracle
    from oracle.check import compare, tolerance
    from dense_gemm_16_amd import inputs
    w = p.w
    bA, bB = inputs.to_bits(p.A), inputs.to_bits(p.B)
    thr = oracle.default_threads()
    used = oracle.threads_used(thr)
    # Two calibration passes: a few rows, then about an eighth of the budget
    # (the first pass alone overstates the per-row time: fixed costs dominate it).
    r0 = max(used, 8)
    for frac in (None, 0.125):
        if frac is not None:
            r0 = int(min(w.M, max(r0, r0 * seconds * frac / max(t_cal, 1e-3))))
        t = time.perf_counter()
        oracle.gemm(bA[:r0], bB, p.code, nthreads=thr)
        t_cal = time.perf_counter() - t
    rows = int(min(w.M, max(r0, r0 * seconds / max(t_cal, 1e-3))))
    rows = max(used, (rows // used) * used) if rows >= used else rows
    log(f"cpu_baseline: calibration {r0} rows in {t_cal:.2f}s -> sample {rows} rows")
    t = time.perf_counter()
    ref, S = oracle.gemm(bA[:rows], bB, p.code, nthreads=thr)
    dt = time.perf_counter() - t
    flop = 2.0 * rows * w.N * w.K
    got = p.C[:rows].cpu().numpy()
    chk = compare(got, ref, S, tol=None if w.exact else tolerance(p.code), exact=w.exact)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": flop / dt / 1e12, "unit": "TOPS" if w.dtype == "i8" else "TFLOPS",
            "cores": used, "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of C ({rows}x{w.N} outputs, K={w.K}), "
                      f"fp64 ascending-k sums over the same {w.dtype} inputs; {dt:.1f} s",
            "seconds": round(dt, 3), "cpu_model": cpu_model,
            "gpu_rows_vs_oracle": str(chk), "gpu_rows_ok": bool(chk.ok)}


def conversion_lines(w):
    """migemm_convert FP32 -> BF16 on the workload's A (HBM GB/s: 4 bytes read and
    2 written per element), and FP32 operands converted then multiplied in BF16."""
    import torch
    import dense_gemm_16_amd as mg
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed)
    a32 = torch.randn((w.M, w.K), generator=g, device="cuda")
    b32 = torch.randn((w.K, w.N), generator=g, device="cuda")
    a16 = torch.empty((w.M, w.K), dtype=torch.bfloat16, device="cuda")
    b16 = torch.empty((w.K, w.N), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream

    def conv_a():
        st = mg.migemm_convert(0, 2, w.M, w.K, a32.data_ptr(), w.K, a16.data_ptr(), w.K, s)
        if st != mg.OK:
            raise RuntimeError(mg.migemm_status_string(st))

    def full():
        conv_a()
        st = mg.migemm_convert(0, 2, w.K, w.N, b32.data_ptr(), w.N, b16.data_ptr(), w.N, s)
        st = st or mg.migemm_gemm(w.M, w.N, w.K, 2, a16.data_ptr(), w.K, b16.data_ptr(), w.N,
                                  c.data_ptr(), w.N, s)
        if st != mg.OK:
            raise RuntimeError(mg.migemm_status_string(st))

    def timed(f, reps):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            f()
        t1.record()
        t1.synchronize()
        return t0.elapsed_time(t1) / reps

    out = {}
    ms = timed(conv_a, 200)
    nbytes = w.M * w.K * (4 + 2)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out["convert-f32-to-bf16-" + f"{w.M}x{w.K}"] = {
        "gbs": round(gbs, 1), "ms": round(ms, 5), "bound": "hbm",
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "bytes_per_launch": nbytes, "kernel": "migemm_convert f32->bf16"}
    log(f"extra convert f32->bf16 {w.M}x{w.K}: {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM peak)")
    ms = timed(full, 40)
    tf = w.flop / (ms * 1e-3) / 1e12
    out[w.name + "/from-f32"] = {
        "tflops": round(tf, 2), "ms": round(ms, 5),
        "frac_of_peak": round(tf / PEAK_TFLOPS[w.dtype], 4),
        "kernel": "migemm_convert x2 + migemm_gemm (BF16)",
        "note": "FP32 A and B converted to BF16 on the device, then the BF16 product"}
    log(f"extra {w.name} from FP32 data (convert A, B + BF16 product): {tf:.1f} TFLOPS")
    return out


def device_info():
    import torch
    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", ""),
            "cus": pr.multi_processor_count,
            "hbm_gib": round(pr.total_memory / 2 ** 30, 1)}


def profile_pass(p, reps):
    """Untimed launches for rocprofv3 counter runs: a plain 1 GiB copy (the counter
    calibration kernel: 1 GiB read, 1 GiB written) then the GEMM `reps` times."""
    import torch
    n = 1 << 28  # 2^28 floats = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        p.launch()
    torch.cuda.synchronize()
    log(f"profile pass: 3 x copy of {n * 4} bytes, {reps} x {p.kernel_name()}")


def _counter_rows(d):
    """(kernel name, counter value) per dispatch from a rocprofv3 --pmc CSV directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"bench.py: expected one *counter_collection.csv under {d}, found {files}")
    rows = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            k = int(r["Dispatch_Id"])
            name, v = r["Kernel_Name"], float(r["Counter_Value"])
            rows[k] = (name, rows.get(k, (name, 0.0))[1] + v)
    return [rows[k] for k in sorted(rows)]


def digest_counters(w, fetch_dir, write_dir, reps):
    """HBM bytes per call of the selected configuration from two profile-mode counter
    runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled so that the 1 GiB
    device copy of the same run reads as 1 GiB; the last `reps` calls' dispatches (one
    per launch of the call) are summed per call and the median call is kept, with the
    per-launch figures beside it.  The entry is written to the traffic summary under
    this workload."""
    import statistics
    import dense_gemm_16_amd as mg
    from dense_gemm_16_amd import inputs
    code = inputs.DTYPE_CODES[w.dtype]
    c_code = 4 if w.dtype == "i8" else 0
    d = mg.describe(-1, -1, 0, 0, w.M, w.N, w.K, code, None, w.K, None, w.N, c_code, w.N,
                    1 << 40)
    kernel = f"{d['variant']}[{d['config_name']}]"
    launches = int(d["launches"])
    gib_kib = float(1 << 20)
    e = {"kernel": kernel, "source_hash": source_hash(), "launches_per_call": launches}
    for label, d in (("fetch", fetch_dir), ("write", write_dir)):
        rows = _counter_rows(d)
        copies = [x for n, x in rows if "copyBuffer" in n]
        gemm = rows[-reps * launches:]
        if len(copies) < 2 or any("copyBuffer" in n for n, _ in gemm):
            raise SystemExit(f"bench.py: {d} does not hold a profile pass (copies then GEMMs)")
        cal = statistics.median(copies[-2:])
        calls = [sum(x for _, x in gemm[i:i + launches]) for i in range(0, len(gemm), launches)]
        raw = statistics.median(calls)
        scale = gib_kib / cal * 1024
        e[f"{label}_kib_raw"] = raw
        e[f"copy_{label}_kib_raw"] = cal
        e[f"{label}_factor"] = round(gib_kib / cal, 5)
        e[f"{label}_bytes_per_launch"] = int(round(raw * scale))
        if launches > 1:
            e[f"{label}_bytes_by_launch"] = [
                [gemm[j][0][:80], int(round(statistics.median(
                    gemm[i + j][1] for i in range(0, len(gemm), launches)) * scale))]
                for j in range(launches)]
        e[f"{label}_kernel_in_csv"] = gemm[-1][0][:160]
    e["hbm_bytes_per_launch"] = e["fetch_bytes_per_launch"] + e["write_bytes_per_launch"]
    e["note"] = (f"HBM read {e['fetch_bytes_per_launch'] / 1e9:.3f} GB + write "
                 f"{e['write_bytes_per_launch'] / 1e9:.3f} GB per launch; compulsory "
                 f"{w.compulsory_bytes() / 1e9:.3f} GB")
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        t = {}
    t["note_general"] = (
        "HBM bytes per launch of the dominant kernel from rocprofv3 FETCH_SIZE and WRITE_SIZE "
        "(KiB per dispatch), each scaled by the factor that makes the same counter read 1 GiB "
        "for a plain 1 GiB device copy (__amd_rocclr_copyBuffer) in the same run; median over "
        "the GEMM launches of the profile pass.  Valid only while the library sources hash to "
        "source_hash.  Written by bench.py --digest-counters.")
    t.setdefault("entries", {})[w.name] = e
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
        f.write("\n")
    log(f"digest: {kernel}: {e['note']}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c4-bf16-8192")
    ap.add_argument("--variant", type=int, default=-1)
    ap.add_argument("--config", type=int, default=-1)
    ap.add_argument("--dist", default="",
                    help="override the workload's input distribution (e.g. zeros: the same "
                         "kernel on inputs whose products switch no bits, to separate clock "
                         "and power effects from cycle counts)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="also time every configuration of every variant on every workload")
    ap.add_argument("--sweep-only", default="",
                    help="comma-separated workloads the sweep covers (default: all)")
    ap.add_argument("--profile-pass", type=int, default=0, metavar="REPS",
                    help="only run the copy calibration and REPS launches (for rocprofv3)")
    ap.add_argument("--digest-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn the CSV output of two profile-pass runs (rocprofv3 --pmc "
                         "FETCH_SIZE, then WRITE_SIZE) into the traffic summary entry")
    ap.add_argument("--digest-reps", type=int, default=3,
                    help="GEMM launches per profile pass (the REPS given to --profile-pass)")
    a = ap.parse_args()
    if a.digest_counters:
        from dense_gemm_16_amd import inputs
        digest_counters(inputs.WORKLOADS[a.workload], *a.digest_counters, a.digest_reps)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {a.gpus} (WORLD_SIZE={world}) "
              "is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_gemm_16_amd as mg
    from dense_gemm_16_amd import inputs
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    mg.lib()  # fail loudly if the library is missing

    w = inputs.WORKLOADS[a.workload]
    if a.dist and a.dist != w.dist:
        import dataclasses
        w = dataclasses.replace(w, dist=a.dist)
    log(f"bench: generating {w.name} inputs ({w.dist})")
    p = Problem(w, a.variant, a.config)
    if a.profile_pass:
        profile_pass(p, a.profile_pass)
        return

    # correctness launch into a NaN-filled C (integer C: a sentinel)
    p.C.fill_(-2147483647 if p.C.dtype == torch.int32 else float("nan"))
    p.launch()
    torch.cuda.synchronize()
    unwritten = int((p.C == -2147483647).sum() if p.C.dtype == torch.int32
                    else torch.isnan(p.C).sum())
    if unwritten:
        raise SystemExit(f"bench.py: {unwritten} outputs of {w.name} left unwritten")
    cold, settle_n, settle_ms = p.settle(a.steps)
    log(f"bench: settled over {settle_n} launches ({settle_ms:.0f} ms); the first {a.steps} "
        f"from idle took {cold:.4f} ms each")
    log(f"bench: {w.name} on {p.kernel_name()}, warmup {a.warmup}, steps {a.steps}")
    first_timed = p.launches + a.warmup + 1
    ms = p.time(a.steps, a.warmup)
    log(f"bench: the timed steps are launches {first_timed}..{p.launches} of this kernel "
        "in this process")
    tflops = w.flop / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    log(f"bench: {ms:.4f} ms/step, {tflops:.1f} TFLOPS ({100 * tflops / peak:.1f}% of {peak})")
    st_med, st_windows, st_n = p.steady()
    clock = ClockProbe().during(p)
    st_tf = w.flop / (st_med * 1e-3) / 1e12
    log(f"bench: steady state {st_med:.4f} ms ({st_tf:.1f} TFLOPS), median of "
        f"{len(st_windows)} windows of {st_n} launches; clock {clock.get('gfxclk_mhz_median')} MHz, "
        f"power {clock.get('socket_power_w_median')} W")
    timing = {"protocol": f"NaN-filled correctness launch; {settle_n} back-to-back launches "
                          f"({settle_ms:.0f} ms) so the power controller settles; {a.warmup} "
                          f"warm-up and {a.steps} timed steps (value); 5 windows of at least "
                          "50 ms (steady_state)",
              "timed_launches": [first_timed, first_timed + a.steps - 1],
              "cold_first_k_ms": round(cold, 5),
              "cold_first_k_tflops": round(w.flop / (cold * 1e-3) / 1e12, 2),
              "settle_launches": settle_n, "settle_ms": round(settle_ms, 1),
              "steady_state": {"median_ms": round(st_med, 5), "windows_ms": st_windows,
                               "launches_per_window": st_n, "tflops": round(st_tf, 2),
                               "frac_of_peak": round(st_tf / peak, 4)},
              "clock": clock}

    traffic, tnote = traffic_for(p.kernel_name(), w.name)
    roof = {"bound": "mfma", "kernel": p.kernel_name(), "achieved": round(tflops, 2),
            "peak": peak, "unit": "TOP/s" if w.dtype == "i8" else "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": traffic, "traffic_note": tnote,
            "algorithmic_flop_per_launch": w.flop,
            "compulsory_bytes_per_launch": w.compulsory_bytes(),
            "resources": p.resources()}
    if traffic:
        roof["traffic_gbs"] = round(traffic / (ms * 1e-3) / 1e9, 1)
        roof["traffic_frac_of_hbm_peak"] = round(traffic / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)

    sweep = {}
    if a.sweep:
        names = [w.name] + EXTRA
        if a.sweep_only:
            names = [n for n in names if n in a.sweep_only.split(",")]
        for name in names:
            wx = inputs.WORKLOADS[name]
            px = p if name == w.name else Problem(wx)
            res = {}
            for v in range(mg.migemm_variant_count()):
                if not mg.migemm_variant_supports(v, px.code):
                    continue
                if v == mg.NAIVE and wx.flop > 5e10:
                    continue
                for c in range(mg.migemm_config_count(v)):
                    q = Problem.__new__(Problem)
                    q.__dict__.update(px.__dict__)
                    q.variant, q.config = v, c
                    q.args = (v, c) + px.args[2:]
                    t, n = q.time_window()
                    res[q.kernel_name()] = round(wx.flop / (t * 1e-3) / 1e12, 2)
            best = max(res, key=res.get)
            log(f"sweep {name}: best {best} {res[best]} TFLOPS; selected "
                f"{px.kernel_name()} {res.get(px.kernel_name())}")
            sweep[name] = res
            if px is not p:
                del px

    extra = {}
    if not a.no_extra:
        def line(px, unit="tflops"):
            """Settled, then the median of 3 windows of at least 50 ms."""
            px.settle(5, 50.0)
            t, windows, n = px.steady(3)
            tf = px.w.flop / (t * 1e-3) / 1e12
            return {unit: round(tf, 2), "ms": round(t, 5), "launches": n,
                    "windows_ms": windows,
                    "frac_of_peak": round(tf / PEAK_TFLOPS[px.w.dtype], 4),
                    "kernel": px.kernel_name(), "resources": px.resources()}, tf

        for name in EXTRA:
            wx = inputs.WORKLOADS[name]
            px = Problem(wx)
            extra[name], tf = line(px, "tops" if wx.dtype == "i8" else "tflops")
            px.launch()
            torch.cuda.synchronize()
            extra[name]["oracle"] = oracle_check(px)
            log(f"extra {name}: {tf:.1f} {'TOPS' if wx.dtype == 'i8' else 'TFLOPS'} on "
                f"{px.kernel_name()}; oracle "
                f"{extra[name]['oracle']['gflops']} GFLOPS on {extra[name]['oracle']['rows']} "
                f"rows, {extra[name]['oracle']['gpu_rows_vs_oracle']}")
            if name in GRAPH_TIMED:
                # launch-bound sizes: the same calls replayed from a HIP graph
                gms, same = px.graph_rate()
                gtf = wx.flop / (gms * 1e-3) / 1e12
                extra[name]["graph"] = {"tflops": round(gtf, 2), "ms": round(gms, 5),
                                        "launches_per_graph": 100, "matches_eager": same}
                log(f"extra {name} from a HIP graph: {gtf:.1f} TFLOPS ({gms * 1e3:.2f} us per call); "
                    f"replay {'matches' if same else 'DIFFERS FROM'} the eager call")
                if not same:
                    raise SystemExit(f"bench.py: {name} replayed from a graph differs from the eager call")
            if not extra[name]["oracle"]["gpu_rows_ok"]:
                raise SystemExit(f"bench.py: {name} does not match the oracle")
            if name == "c1-f32-1024":
                # the baselines, each in its fastest configuration at this size
                # (configuration sweep: naive 64x4, LDS 32x32, VALU 64x64x16 4x4)
                for v, c, label in ((mg.NAIVE, 0, "naive"), (mg.LDS_TILED, 0, "lds_tiled"),
                                    (mg.REGTILE_VALU, 2, "regtile_valu")):
                    pn = Problem(wx, v, c)
                    extra[f"{name}/{label}"], tf = line(pn)
                    log(f"extra {name}/{label}: {tf:.2f} TFLOPS on {pn.kernel_name()}")
                    del pn
            del px
        # operands given transposed on the headline shape
        if w.name == "c4-bf16-8192":
            for ta, tb in ((False, True), (True, False), (True, True)):
                px = Problem(w, ta=ta, tb=tb)
                e, tf = line(px)
                e["layout"] = (f"A {'K x M (given transposed)' if ta else 'M x K'}, "
                               f"B {'N x K (given transposed)' if tb else 'K x N'}")
                extra[f"{w.name}/{px.layout()}"] = e
                log(f"extra {w.name} layout {px.layout()}: {tf:.1f} TFLOPS")
                del px
        # INT8 -> INT32 at the headline size
        if w.name == "c4-bf16-8192":
            wi = inputs.WORKLOADS["i8-8192"]
            px = Problem(wi)
            e, tf = line(px, "tops")
            e["peak_tops"] = PEAK_TFLOPS["i8"]
            px.launch()
            torch.cuda.synchronize()
            e["oracle"] = oracle_check(px)
            extra[wi.name] = e
            log(f"extra {wi.name}: {tf:.1f} TOPS ({100 * tf / PEAK_TFLOPS['i8']:.1f}% of "
                f"{PEAK_TFLOPS['i8']}) on {px.kernel_name()}; oracle {e['oracle']['gpu_rows_vs_oracle']}")
            if not e["oracle"]["gpu_rows_ok"]:
                raise SystemExit(f"bench.py: {wi.name} does not match the oracle")
            del px
            for ta, tb in ((False, True), (True, False), (True, True)):
                px = Problem(wi, ta=ta, tb=tb)
                extra[f"{wi.name}/{px.layout()}"], tf = line(px, "tops")
                log(f"extra {wi.name} layout {px.layout()}: {tf:.1f} TOPS")
                del px
        # FP32 data on the 16-bit path: device conversion, alone and followed by the product
        if w.name == "c4-bf16-8192":
            extra.update(conversion_lines(w))
        # the general output step on the headline shape: scaled update, BF16 C
        if w.name == "c4-bf16-8192":
            px = Problem(w, alpha=0.5, beta=-1.0, c_code=2)
            e, tf = line(px)
            e["kernel"] += " general output step"
            e["update"] = "C = 0.5 A B - 1.0 C, C stored as BF16"
            extra[w.name + "/alpha-beta-bf16-out"] = e
            log(f"extra {w.name} general (alpha 0.5, beta -1, BF16 C): {tf:.1f} TFLOPS")
            del px

    cpu = None
    if not a.no_cpu_baseline:
        # re-run once so C holds this workload's product for the row check
        p.launch()
        torch.cuda.synchronize()
        cpu = cpu_baseline(p, a.cpu_seconds)
        log(f"cpu_baseline: {cpu['value'] * 1e3:.2f} GFLOPS on {cpu['cores']} threads; "
            f"GPU rows {cpu['gpu_rows_vs_oracle']}")

    # INT8 products count integer operations and accumulate and output in INT32
    integer = w.dtype == "i8"
    out = {"metric": METRIC, "value": round(tflops, 2), "unit": "TOPS" if integer else "TFLOPS",
           "n_gpus": 1,
           "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
           "data": "synthetic",
           "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "inputs": w.dtype,
                      "accumulate": "i32" if integer else "f32",
                      "output": "i32" if integer else "f32", "distribution": w.dist,
                      "seed": w.seed, "layout": "row-major, dense leading dimensions",
                      "parallelism": "single GPU"},
           "frac_of_peak": round(tflops / peak, 4), "peak_tflops": peak,
           "roofline": roof, "cpu_baseline": cpu, "timing": timing, "by_workload": extra,
           "device": device_info(), "source_hash": source_hash()}
    if sweep:
        out["sweep"] = sweep
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
