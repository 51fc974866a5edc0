"""Benchmark of the packed varlen attention head on one MI355X.

One step = one pass of the whole hot path over the S = 20,423 packed request
(video 10x30x54 + six 20x30 references + 623 audio tokens; 24 heads, d = 128,
rotary on 96 dims): build the rotary table, fused RMSNorm + rotary of q and k,
then the per-segment attention (whose tile plan is cached after the first
call).  Inputs are synthetic and already resident in HBM when timing starts.

Prints one JSON line.  `value` is attention TFLOP/s over the whole step,
F = 4 * D * heads * sum(L^2) divided by the step time; `roofline` reports the
attention kernel alone (HIP events on its launch stream) against the bf16
dense MFMA peak; `cpu_baseline` times the fp64 oracle on a bounded sample of
the same workload.  The GPU clock is sampled during the timed work
(`sclk_mhz`) and the attention rate is also given against the peak scaled to
that clock; the steps run untimed for `--settle` seconds before the warmup
steps so the clock has left its idle level.

--config runs another bf16 workload of the same family through the same step
(its own rotary table mode, grouped K/V heads, causal mask); F then counts the
visible (query, key) pairs, sum(L (L + 1) / 2) when causal.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--no-cpu-baseline] [--config NAME]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 MFMA
PEAK_HBM_GBPS = 8000.0
METRIC = "varlen attn TFLOP/s and % bf16 MFMA peak at S=20,423, 24 heads, d=128"
HEADLINE = "h3_s20423_bf16"
ATTN_SRC = os.path.join(ROOT, "packed_varlen_attention_head_amd", "csrc", "attn_fwd_bf16.hip")
NORM_SRC = os.path.join(ROOT, "packed_varlen_attention_head_amd", "csrc", "qk_norm_rope.hip")
TABLE_SRC = os.path.join(ROOT, "packed_varlen_attention_head_amd", "csrc", "rope_table.hip")
ATTN_KERNEL = "attn_fwd_bf16_kernel<128>"
NORM_KERNEL = "qk_norm_rope_kernel<h3a::(anonymous namespace)::Bf16Tag, 128, 0, 0>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_h3_s20423_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=HEADLINE, help="bf16 workload name (synth.configs.BF16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fp8", action="store_true",
                    help="step = table + q/k norm/rotary to E4M3 + transposed E4M3 V + attention with both products "
                         "in FP8")
    ap.add_argument("--fp8-qk", action="store_true",
                    help="step = table + q/k norm/rotary writing E4M3 codes + FP8-score attention")
    ap.add_argument("--i8-qk", action="store_true",
                    help="step = table + q/k norm/rotary + INT8 codes of q (one scale per token) and k (one per 64 "
                         "keys of a segment) + INT8-score attention")
    ap.add_argument("--i8-fp8pv", action="store_true",
                    help="step = table + q/k norm/rotary writing INT8 q + INT8 codes of k + transposed E4M3 V + "
                         "attention with INT8 QK^T and FP8 PV")
    ap.add_argument("--i8-smooth", action="store_true",
                    help="with --i8-qk or --i8-fp8pv: subtract each segment's mean key before the key codes "
                         "(two mean passes added to the step)")
    ap.add_argument("--fused-q", action="store_true",
                    help="step = table + K-only norm/rotary + attention that normalises and rotates Q itself")
    ap.add_argument("--split", choices=("auto", "never", "always"), default="auto",
                    help="key-range splitting of attention plans (h3a_set_split_policy)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup steps, so the GPU clock has left its idle state")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (for scaling HBM counters)")
    ap.add_argument("--rocprof-summary", metavar="RESULTS_DB",
                    help="print a per-kernel duration table from a rocprofv3 --kernel-trace results.db")
    ap.add_argument("--summary-last", type=int, default=10, metavar="N",
                    help="with --rocprof-summary: also average each kernel's last N dispatches (the timed ones)")
    ap.add_argument("--rocprof-traffic", nargs=4, metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB", "COPY_WRITE_DB"),
                    help="HBM bytes per launch of each h3a kernel from FETCH_SIZE/WRITE_SIZE runs, scaled by "
                         "the same counters on the --calibrate-copy run; prints JSON")
    ap.add_argument("--rocprof-counters", nargs="+", metavar="RESULTS_DB",
                    help="per-dispatch averages of every counter in rocprofv3 --pmc results databases, per kernel, "
                         "and the attention kernel's MFMA utilisation; prints markdown")
    return ap.parse_args()


def _rocpd_rows(db, query):
    import sqlite3

    con = sqlite3.connect(db)
    try:
        return list(con.execute(query))
    finally:
        con.close()


def _short_kernel(name):
    """attn_fwd_*_kernel<D> (bidirectional) or <D, causal>, and the other kernels' short names."""
    import re

    m = re.search(r"(attn_fwd_(?:bf16|f32)_kernel)<([^>]*)>", name)
    if m:
        a = [x.strip() for x in m.group(2).split(",")]
        tags = [a[0]]
        if len(a) > 1 and a[1] == "true":
            tags.append("causal")
        if len(a) > 3 and a[2] == "true":
            tags.append(f"qnorm r{32 * int(a[3])}")
        if len(a) > 4 and a[4] in ("true", "1"):
            tags.append("fp8qk")
        if len(a) > 4 and a[4] == "2":
            tags.append("fp8")
        if len(a) > 4 and a[4] == "3":
            tags.append("i8qk")
        if len(a) > 4 and a[4] == "4":
            tags.append("i8qk fp8pv")
        return f"{m.group(1)}<{', '.join(tags)}>"
    m = re.search(r"(qk_norm_rope_kernel<[^>]*>|rope_table_kernel|"
                  r"__amd_rocclr_\w+|elementwise_kernel|vectorized_elementwise_kernel|reduce_kernel)", name)
    return m.group(1) if m else name[:60]


def rocprof_summary(db, last):
    """Per-kernel table (calls, total, average, and the average of the last
    `last` dispatches) from a rocprofv3 --kernel-trace results database."""
    import collections

    rows = _rocpd_rows(db, "select name, total_calls, total_duration, average, percentage from top_kernels")
    durations = collections.defaultdict(list)
    for name, start, end in _rocpd_rows(db, "select name, start, end from kernels order by start"):
        durations[name].append((end - start) / 1e3)
    print(f"| kernel | calls | total (us) | average (us) | average of the last {last} (us) | share |")
    print("|---|---|---|---|---|---|")
    for name, calls, total, avg, pct in rows:
        tail = durations.get(name, [])[-last:]
        tail_avg = f"{sum(tail) / len(tail):.1f}" if tail else ""
        print(f"| {_short_kernel(name)} | {calls} | {total:.1f} | {avg:.1f} | {tail_avg} | {pct:.2f}% |")
    return 0


def rocprof_traffic(fetch_db, write_db, copy_fetch_db, copy_write_db):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel, converted to bytes with the
    factor the same counter reads for a 1 GiB copy (bytes moved / counter bytes)."""
    import collections

    def per_kernel(db, counter):
        acc = collections.defaultdict(list)
        for name, value in _rocpd_rows(db, f"select kernel_name, value from counters_collection "
                                           f"where counter_name = '{counter}'"):
            acc[_short_kernel(name)].append(value * 1024.0)
        return {k: sum(v) / len(v) for k, v in acc.items()}

    copy_bytes = float(1 << 30)
    cf = per_kernel(copy_fetch_db, "FETCH_SIZE")
    cw = per_kernel(copy_write_db, "WRITE_SIZE")
    cname = max(cf, key=cf.get)
    f_scale = copy_bytes / cf[cname]
    w_scale = copy_bytes / cw[max(cw, key=cw.get)]
    fetch, write = per_kernel(fetch_db, "FETCH_SIZE"), per_kernel(write_db, "WRITE_SIZE")
    out = {"kernel_source_sha256_16": source_hash(ATTN_SRC),
           "source_sha256_16": {os.path.basename(p): source_hash(p) for p in (ATTN_SRC, NORM_SRC, TABLE_SRC)},
           "copy_kernel": cname, "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    for k in sorted(set(fetch) | set(write)):
        if not (k.startswith("attn") or k.startswith("qk_norm") or k.startswith("rope")):
            continue
        rb, wb = fetch.get(k, 0.0) * f_scale, write.get(k, 0.0) * w_scale
        out["kernels"][k] = {"hbm_read_bytes": rb, "hbm_write_bytes": wb, "hbm_bytes_per_launch": rb + wb}
    print(json.dumps(out, indent=1))
    return 0


def rocprof_counters(dbs):
    """Counter values per dispatch (mean over dispatches) for each kernel, from
    one or more --pmc runs, and for the attention kernel: MFMA flops executed
    (512 per bf16 MOP) against the algorithmic F of the headline workload, and
    MFMA-busy cycles over the SIMD-cycles of the dispatch."""
    import collections

    from synth import configs

    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for db in dbs:
        for name, counter, value in _rocpd_rows(db, "select kernel_name, counter_name, value "
                                                    "from counters_collection"):
            acc[_short_kernel(name)][counter].append(value)
    mean = {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in acc.items()}
    # average dispatch durations (us) where a run also traced the kernels
    durations = {}
    for db in dbs:
        try:
            for name, avg in _rocpd_rows(db, "select name, average from top_kernels"):
                durations[_short_kernel(name)] = avg
        except Exception:  # noqa: BLE001 - a counters-only run has no kernel table
            pass
    counters = sorted({c for d in mean.values() for c in d})
    kernels = sorted(k for k in mean if k.startswith(("attn", "qk_norm", "rope")))
    print("| kernel | " + " | ".join(counters) + " |")
    print("|---|" + "---|" * len(counters))
    for k in kernels:
        print(f"| {k} | " + " | ".join(f"{mean[k][c]:.4g}" if c in mean[k] else "" for c in counters) + " |")
    F = configs.BF16[HEADLINE].attention_flops()
    for k in kernels:
        m = mean[k]
        if not k.startswith("attn_fwd_bf16_kernel<128>"):
            continue
        print()
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in m:
            flop = 512.0 * m["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
            print(f"- {k}: bf16 MFMA flops executed {flop:.4g} per dispatch = {flop / F:.4f} x the "
                  f"algorithmic F = {F:.4g} of {HEADLINE}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m and "GRBM_GUI_ACTIVE" in m:
            # GRBM_GUI_ACTIVE adds up the busy cycles of the 8 XCDs
            simd_cycles = m["GRBM_GUI_ACTIVE"] / 8 * 256 * 4
            print(f"- {k}: MFMA busy {m['SQ_VALU_MFMA_BUSY_CYCLES']:.4g} cycles / (GRBM_GUI_ACTIVE "
                  f"{m['GRBM_GUI_ACTIVE']:.4g} / 8 XCDs x 256 CUs x 4 SIMDs) = "
                  f"{100.0 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:.1f}%")
        dur = durations.get(k)
        if dur and "GRBM_GUI_ACTIVE" in m:
            print(f"- {k}: GRBM_GUI_ACTIVE / 8 over the traced average duration {dur / 1e3:.3f} ms = "
                  f"{m['GRBM_GUI_ACTIVE'] / 8 / dur:.0f} MHz (the clock during the counted dispatches)")
    return 0


def calibrate_copy():
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch, five
    launches.  Its FETCH_SIZE / WRITE_SIZE readings convert the counters of the
    other kernels into bytes."""
    import torch

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n, "launches": 5}))
    return 0


NOMINAL_SCLK_MHZ = 2400.0  # the clock the published MFMA peaks assume


class SclkSampler:
    """Samples the GPU's current shader clock (the starred level of the
    driver's pp_dpm_sclk file) and board power (hwmon power1_input of the same
    device) from a host thread while timed work runs; stop() returns the
    median clock in MHz, or None when the file is absent or ambiguous (several
    GPUs and no PCI address to match), and leaves the median power in
    `power_w` (None without a power sensor).  The clock file shows the DPM
    level the driver requested; under load the hardware's own current and
    power limiters can run the shader clock below it."""

    def __init__(self, period_s=0.005):
        self.period = period_s
        self.samples = []
        self.path = None
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        if len(paths) == 1:
            self.path = paths[0]
        elif paths:
            try:
                import torch

                bus = str(getattr(torch.cuda.get_device_properties(0), "pci_bus_id", "")).lower()
                match = [p for p in paths if bus and os.path.basename(os.path.realpath(os.path.dirname(p))).lower()
                         .endswith(bus)]
                self.path = match[0] if len(match) == 1 else None
            except Exception:  # noqa: BLE001 - clock reporting is best effort
                self.path = None
        self.power_path = None
        self.power_samples = []
        self.power_w = None
        if self.path:
            pw = sorted(glob.glob(os.path.join(os.path.dirname(self.path), "hwmon", "hwmon*", "power1_input")))
            self.power_path = pw[0] if pw else None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        with open(self.path) as f:
            for line in f:
                if "*" in line:
                    mhz = line.split(":", 1)[1].strip().split("Mhz")[0].split("MHz")[0]
                    return float(mhz)
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
                if v:
                    self.samples.append(v)
                if self.power_path:
                    with open(self.power_path) as f:
                        self.power_samples.append(int(f.read()) / 1e6)  # microwatts
            except (OSError, ValueError, IndexError):
                return
            self._stop.wait(self.period)

    def start(self):
        if self.path:
            self._thread.start()

    def stop(self):
        if not self.path:
            return None
        self._stop.set()
        self._thread.join()
        self.power_w = float(np.median(self.power_samples)) if self.power_samples else None
        return float(np.median(self.samples)) if self.samples else None


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel, src):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, if it was taken on the current source `src` of that kernel; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16", {}).get(os.path.basename(src)) != source_hash(src):
        return None
    k = t.get("kernels", {}).get(kernel)
    return k.get("hbm_bytes_per_launch") if k else None


def cpu_model():
    """The host CPU's model name (Linux), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(w, T, target_s):
    """fp64 oracle on a bounded sample of query rows (all heads, rows spread
    evenly over the packed sequence), scaled to TFLOP/s with the same F (a
    row costs 4 D heads times the keys it sees)."""
    import oracle
    from synth import rng

    # The oracle's products run in numpy's BLAS: give it every core this
    # process may run on, and report that count beside the machine's.
    allowed = sorted(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else list(range(os.cpu_count() or 1))
    limiter = None
    np.ones((2, 2)) @ np.ones((2, 2))  # load the BLAS so threadpoolctl sees it
    try:
        from threadpoolctl import threadpool_info, threadpool_limits

        limiter = threadpool_limits(limits=len(allowed), user_api="blas")
        cores = max([int(p.get("num_threads", 1)) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        cores = len(allowed)
    cu = oracle.cu_seqlens(w.segments)
    qf = rng.as_f64(T.q, w.dtype)
    kf = rng.as_f64(T.k, w.dtype)
    vf = rng.as_f64(T.v, w.dtype)
    lens = np.diff(cu)
    seg = oracle.segment_of_rows(cu, np.arange(w.tokens))
    grouped = w.causal or w.kv != w.heads

    def flops(rows):
        keys = (rows - cu[seg[rows]] + 1) if w.causal else lens[seg[rows]]
        return float(np.sum(4.0 * w.head_dim * w.heads * keys))

    n = 32
    spent, done_flops, done_rows = 0.0, 0.0, 0
    while True:
        rows = np.linspace(0, w.tokens - 1, n).astype(np.int64)
        t0 = time.perf_counter()
        if grouped:
            oracle.varlen_attention_gqa_rows(qf, kf, vf, cu, w.scale, rows, causal=w.causal)
        else:
            oracle.varlen_attention_rows(qf, kf, vf, cu, w.scale, rows)
        dt = time.perf_counter() - t0
        spent, done_flops, done_rows = dt, flops(rows), n
        if dt >= target_s * 0.5 or n >= w.tokens:
            break
        n = min(w.tokens, int(n * max(2.0, min(16.0, target_s / max(dt, 1e-3)))))
    if limiter is not None:
        limiter.unregister()
    return {
        "value": done_flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "cpu_count": os.cpu_count(),
        "affinity_cores": len(allowed),
        "cpu": cpu_model(),
        "kind": "oracle",
        "sample": f"fp64 numpy oracle attention on {done_rows} query rows spread evenly over the "
                  f"S={w.tokens} packed sequence, all {w.heads} heads, each against its segment's keys "
                  f"({'causal, ' if w.causal else ''}{done_flops:.3e} flop in {spent:.1f} s); same F convention",
    }


def main():
    args = parse()
    if args.calibrate_copy:
        return calibrate_copy()
    if args.rocprof_summary:
        return rocprof_summary(args.rocprof_summary, args.summary_last)
    if args.rocprof_traffic:
        return rocprof_traffic(*args.rocprof_traffic)
    if args.rocprof_counters:
        return rocprof_counters(args.rocprof_counters)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the path is not sharded across GPUs in this build.", file=sys.stderr)
        return 2

    import torch

    import packed_varlen_attention_head_amd as h3a
    from synth import configs

    if args.config not in configs.BF16:
        print(f"unknown workload {args.config!r}; bf16 workloads: {', '.join(sorted(configs.BF16))}",
              file=sys.stderr)
        return 2
    w = configs.BF16[args.config]
    T = configs.make_tensors(w)
    h3a.set_split_policy({"auto": h3a.H3A_SPLIT_AUTO, "never": h3a.H3A_SPLIT_NEVER,
                          "always": h3a.H3A_SPLIT_ALWAYS}[args.split])
    dev = "cuda:0"
    torch.cuda.set_device(0)
    bf = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    q, k, v = bf(T.q), bf(T.k), bf(T.v)
    gq = torch.from_numpy(T.gamma_q).to(dev)
    gk = torch.from_numpy(T.gamma_k).to(dev)
    tab = torch.empty((2, w.tokens, w.rot_dim // 2), dtype=torch.float32, device=dev)
    qn, kn = torch.empty_like(q), torch.empty_like(k)
    stream = torch.cuda.current_stream()

    o = torch.empty_like(q)

    def table():
        if w.rope_mode == 0:
            return h3a.build_rope_table(w.segments, w.rot_dims, w.base, tab, stream=stream)
        return h3a.build_rope_table_ex(w.segments, w.rope_mode, w.rot_dims, w.base, tab, start=w.lin_start,
                                       stop=w.lin_stop, stream=stream)

    fused, fp8, fp8pv, i8pv = args.fused_q, args.fp8_qk or args.fp8, args.fp8, args.i8_fp8pv
    i8 = args.i8_qk or i8pv
    if fused and (w.causal or w.rot_dim % 32 != 0 or fp8):
        print(f"--fused-q needs a bidirectional workload with rot_dim a multiple of 32, without --fp8-qk "
              f"({w.name})", file=sys.stderr)
        return 2
    if args.i8_smooth and not i8:
        print("--i8-smooth needs --i8-qk or --i8-fp8pv", file=sys.stderr)
        return 2
    if i8 and (fused or fp8):
        print("--i8-qk and --i8-fp8pv exclude --fused-q, --fp8 and --fp8-qk", file=sys.stderr)
        return 2
    if i8:  # int8 codes: q with an fp32 scale per token, k with one per 64 keys of a segment
        nb = h3a.i8_key_blocks(np.concatenate([[0], np.cumsum(w.lengths)]))
        q8 = (torch.empty(q.shape, dtype=torch.int8, device=dev),
              torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=dev))
        k8 = (torch.empty(k.shape, dtype=torch.int8, device=dev),
              torch.empty((k.shape[1], max(nb, 1)), dtype=torch.float32, device=dev))
        if args.i8_smooth:  # segment means of k and their chunk-sum workspace
            nseg = len(w.lengths)
            kmu = torch.empty((nseg, k.shape[1], k.shape[2]), dtype=torch.float32, device=dev)
            kws = torch.empty((max(h3a.i8_key_mean_chunks(np.concatenate([[0], np.cumsum(w.lengths)])), 1),
                               k.shape[1], k.shape[2]), dtype=torch.float32, device=dev)
    if fp8:  # E4M3 codes and one E8M0 scale per 32 head dims
        q8 = (torch.empty(q.shape, dtype=torch.uint8, device=dev),
              torch.empty((q.shape[1], q.shape[0], q.shape[2] // 32), dtype=torch.uint8, device=dev))
        k8 = (torch.empty(k.shape, dtype=torch.uint8, device=dev),
              torch.empty((k.shape[1], k.shape[0], k.shape[2] // 32), dtype=torch.uint8, device=dev))
    if fp8pv or i8pv:  # transposed codes and one scale per 32 keys of each head dim
        cols = h3a.vt_e4m3_columns(np.concatenate([[0], np.cumsum(w.lengths)]))
        vt8 = (torch.empty((w.kv, w.head_dim, cols), dtype=torch.uint8, device=dev),
               torch.empty((w.kv, cols // 64, 2, 32, w.head_dim // 32), dtype=torch.uint8, device=dev))

    def norm():
        if fused:
            return h3a.rmsnorm_rope(k, gk, w.eps, tab, w.rot_dim, x_out=kn, stream=stream)
        if fp8:  # one pass: norm + rotary writing E4M3 codes
            return h3a.qk_rmsnorm_rope_e4m3(q, k, gq, gk, w.eps, tab, w.rot_dim, q8=q8[0], k8=k8[0], q_scale=q8[1],
                                            k_scale=k8[1], stream=stream)
        if i8:  # one pass: norm + rotary writing INT8 q codes with per-token scales, bf16 k
            return h3a.qk_rmsnorm_rope_i8q(q, k, gq, gk, w.eps, tab, w.rot_dim, q8=q8[0], q_scale=q8[1], k_out=kn,
                                           stream=stream)
        return h3a.qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim, q_out=qn, k_out=kn, stream=stream)

    def vt_prep(cu):  # V as transposed E4M3 tiles (changes every step, like q and k)
        h3a.prepare_vt_e4m3(v, cu, out=vt8[0], scale_out=vt8[1], stream=stream)

    def k_quant(cu):  # INT8 codes of the normalised, rotated k, one scale per 64 keys of a segment
        if args.i8_smooth:  # of the centred keys
            h3a.segment_key_means(kn, cu, out=kmu, workspace=kws, stream=stream)
            h3a.quantize_i8_keys(kn, cu, out=k8[0], scale_out=k8[1], mu=kmu, stream=stream)
        else:
            h3a.quantize_i8_keys(kn, cu, out=k8[0], scale_out=k8[1], stream=stream)

    def vprep(cu):
        if fp8pv or i8pv:
            vt_prep(cu)
        if i8:
            k_quant(cu)

    def attention(cu):
        if i8pv:
            return h3a.varlen_attn_fwd_i8qk_fp8pv(q8, k8, vt8, cu, w.scale, causal=w.causal, out=o, stream=stream)
        if i8:
            return h3a.varlen_attn_fwd_i8qk(q8, k8, v, cu, w.scale, causal=w.causal, out=o, stream=stream)
        if fp8pv:
            return h3a.varlen_attn_fwd_fp8(q8, k8, vt8, cu, w.scale, causal=w.causal, out=o, stream=stream)
        if fp8:
            return h3a.varlen_attn_fwd_fp8qk(q8, k8, v, cu, w.scale, causal=w.causal, out=o, stream=stream)
        if fused:  # raw q, normalised and rotated in the attention's prologue
            return h3a.varlen_attn_fwd_qnorm(q, kn, v, cu, w.scale, gq, w.eps, tab, w.rot_dim, out=o, stream=stream)
        if w.causal or w.kv != w.heads:
            return h3a.varlen_attn_fwd_ex(qn, kn, v, cu, w.scale, causal=w.causal, out=o, stream=stream)
        return h3a.varlen_attn_fwd(qn, kn, v, cu, w.scale, out=o, stream=stream)

    def step():
        cu = table()
        norm()
        vprep(cu)
        attention(cu)
        return cu

    # The GPU idles at a low clock and takes a few hundred ms of load to reach
    # its working clock: run the step untimed for `settle` seconds first.
    cu = step()
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        cu = step()
    torch.cuda.synchronize()
    clock = SclkSampler()
    clock.start()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    checksum = float(o.double().sum().item())
    if not np.isfinite(checksum):
        raise SystemExit("non-finite attention output")

    # Per-kernel average launch duration: HIP events on the launch stream
    # around n back-to-back launches of that call alone, divided by n.  (An
    # event pair per launch would add the runtime's per-event cost to short
    # kernels.)  Ten untimed launches are queued right before the first event,
    # with no host synchronisation between them: the clock drops within
    # milliseconds whenever the GPU idles and takes tens of milliseconds of
    # load to recover.
    def timed(fn, n, warm=10):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(warm):
            fn()
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / 1e3 / n

    # The attention kernel is long enough for an event pair per launch: its
    # median is reported beside the mean.
    def timed_each(fn, n, warm=10):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        for _ in range(warm):
            fn()
        ev[0].record(stream)
        for i in range(n):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        each = [ev[i].elapsed_time(ev[i + 1]) / 1e3 for i in range(n)]
        return ev[0].elapsed_time(ev[n]) / 1e3 / n, float(np.median(each))

    n_ev = max(args.steps, 10)
    attn_s, attn_med_s = timed_each(lambda: attention(cu), n_ev)
    sclk = clock.stop()
    norm_s = timed(norm, n_ev)
    table_s = timed(table, n_ev)
    vt_s = timed(lambda: vt_prep(cu), n_ev) if (fp8pv or i8pv) else 0.0
    kq_s = timed(lambda: k_quant(cu), n_ev) if i8 else 0.0

    F = w.attention_flops()
    attn_tflops = F / attn_s / 1e12
    # FP8 QK^T (half of F) at the FP8 dense peak and bf16 PV at the bf16 one:
    # F / (F/2 / 5000 + F/2 / 2500) = 3333 TFLOP/s for the kernel as a whole.
    # (INT8 QK^T at the INT8 dense peak, the same figure, with bf16 PV: 3333 too)
    peak = (PEAK_FP8_TFLOPS if (fp8pv or i8pv) else 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS) if (fp8 or i8)
            else PEAK_BF16_TFLOPS)
    S, H, Hkv, D = w.tokens, w.heads, w.kv, w.head_dim
    # q and k (H + Hkv heads; k only when fused) read and written, the table and gains read
    normed_heads = Hkv if fused else H + Hkv
    norm_bytes = 2 * (S * normed_heads * D * 2) + 2 * S * (w.rot_dim // 2) * 4 + (1 if fused else 2) * D * 4
    if fp8:  # the norm + rotary pass writes one byte per element (and a scale per 32) instead of two
        norm_bytes -= S * (H + Hkv) * D - S * (H + Hkv) * (D // 32)
    if i8:  # q written as one byte per element and an fp32 scale per row
        norm_bytes -= S * H * D - S * H * 4
    copy_src = torch.empty(norm_bytes // 2, dtype=torch.uint8, device=dev)
    copy_dst = torch.empty_like(copy_src)
    copy_gbps = 2 * copy_src.numel() / timed(lambda: copy_dst.copy_(copy_src), n_ev) / 1e9
    del copy_src, copy_dst
    # Q read and O written (H heads), K and V read (Hkv heads), once each
    attn_alg_bytes = 2 * S * H * D * 2 + 2 * S * Hkv * D * 2
    result = {
        "metric": METRIC if w.name == HEADLINE else f"varlen attn TFLOP/s and % bf16 MFMA peak on {w.name}",
        "value": F / step_s / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8 e4m3 QK^T and PV" if fp8pv else "fp8 e4m3 QK^T, bf16 PV" if fp8
                  else "int8 QK^T, fp8 e4m3 PV" if i8pv else "int8 QK^T, bf16 PV" if i8 else "bf16"),
        "data": f"synthetic: Q,K,V ~ N(0,1) bf16, gains ~ {w.gamma_mean:g}+N(0,{w.gamma_std:g}) fp32, "
                f"SplitMix64 seed {w.seed}",
        "config": {
            "workload": w.name,
            "S": S, "heads": H, "kv_heads": Hkv, "causal": w.causal, "head_dim": D,
            "rot_dims": list(w.rot_dims), "rope_mode": w.rope_mode,
            "segments": [list(s) for s in w.segments],
            "parallelism": "single GPU",
            "split": args.split,
            "step": ("rope table + k norm/rotary + attention with q norm/rotary fused in its prologue" if fused
                     else "rope table + q/k norm/rotary to E4M3 codes + transposed E4M3 V + attention with both "
                          "products in FP8" if fp8pv
                     else "rope table + q/k norm/rotary to E4M3 codes + attention with FP8 QK^T" if fp8
                     else "rope table + q/k norm/rotary writing INT8 q + INT8 codes of k" +
                          (" (centred on segment means)" if args.i8_smooth else "") + " + transposed E4M3 V + "
                          "attention with INT8 QK^T and FP8 PV" if i8pv
                     else "rope table + q/k norm/rotary writing INT8 q + INT8 codes of k" +
                          (" (centred on segment means)" if args.i8_smooth else "") + " + attention with INT8 QK^T" if i8
                     else "rope table + q/k norm/rotary + attention"),
        },
        "pct_bf16_peak_step": 100.0 * F / step_s / 1e12 / PEAK_BF16_TFLOPS,
        "attn_ms": attn_s * 1e3,
        "attn_ms_median": attn_med_s * 1e3,
        "attn_tflops": attn_tflops,
        # GPU clock sampled during the timed steps and attention launches, and
        # the attention rate against the peak scaled to that clock
        "sclk_mhz": sclk,
        # board power over the same samples (hwmon power1_input; MI355X's board limit is 1,400 W)
        "power_w": clock.power_w,
        "pct_peak_at_sclk": (100.0 * attn_tflops / (peak * sclk / NOMINAL_SCLK_MHZ)) if sclk else None,
        "norm_rope_ms": norm_s * 1e3,
        "norm_rope_GBps": norm_bytes / norm_s / 1e9,
        "rope_table_ms": table_s * 1e3,
        "v_e4m3_ms": vt_s * 1e3,
        "i8_k_quant_ms": kq_s * 1e3,
        "checksum_o": checksum,
        "roofline": {
            "bound": "mfma",
            "achieved": attn_tflops,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": attn_tflops / peak,
            "traffic": (measured_traffic(ATTN_KERNEL, ATTN_SRC) if (w.name == HEADLINE and not (fp8 or fused or i8))
                        else None),
            "kernel": f"attn_fwd_bf16_kernel<{D}{', fp8' if fp8pv else ', fp8qk' if fp8 else ', i8qk fp8pv' if i8pv else ', i8qk' if i8 else ''}"
                      f"{', qnorm' if fused else ''}>",
            "algorithmic_flop_per_launch": F,
            "algorithmic_bytes_per_launch": attn_alg_bytes,
        },
        "norm_rope_roofline": {
            "bound": "hbm",
            "achieved": norm_bytes / norm_s / 1e9,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": norm_bytes / norm_s / 1e9 / PEAK_HBM_GBPS,
            "traffic": measured_traffic(NORM_KERNEL, NORM_SRC) if (w.name == HEADLINE and not (fp8 or fused or i8)) else None,
            "kernel": "qk_norm_rope_kernel<bf16, 128>",
            "algorithmic_bytes_per_launch": norm_bytes,
            # a plain device-to-device copy moving the same bytes (half read,
            # half written), timed the same way: what HBM gives a pure stream
            "copy_reference_GBps": copy_gbps,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, T, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
