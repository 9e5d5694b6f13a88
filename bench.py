"""Benchmark of ragged paged GQA attention on one MI355X.

One step = one rpa_forward call (plan, the tiles of both classes, split-KV
merge) over one batch of seeded synthetic inputs already
resident in HBM; with --append, an rpa_kv_append of the step's new K/V rows
first.

The headline workload is the largest named one that fits one GPU, the long
context batch (16 sequences x 128 query tokens, kv_len U[65536, 131072],
32 q / 2 kv heads, head_dim 256, page 64, bf16); --workload picks another.
After the headline, the other named workloads are measured the same way
(--no-sweep skips them) and reported under "configs" of the same line.

Prints ONE JSON line on stdout (diagnostics go to stderr):
  value         query tokens/s of the headline workload over the K timed steps
  roofline      the dominant kernel's algorithmic flops (or bytes) per launch
                over its mean launch time, measured with HIP events recorded
                around each kernel on the launch stream during the timed steps
  timing        per-call HIP-event samples of the headline: warm (inputs and
                plan already in cache from the previous call) and cold (a
                1 GiB buffer written between samples, outside the events,
                evicting L2 and the 256 MB Infinity Cache): median, p10, p90
  configs       the same measurements for every other named workload, with a
                call-level and a kernel-level roofline fraction
  practical_ceilings
                what the chip sustains in the same session outside this
                library (a read-only stream, a dense bf16 matmul), and the
                headline kernel's rate as a fraction of the matching one
  cpu_baseline  the f64 CPU oracle timed on a bounded sample of the headline
                workload on the host cores (a reported baseline, not a target)

Host-only modes (no GPU): --ingest-counters turns rocprofv3 FETCH_SIZE /
WRITE_SIZE runs into the traffic file; --summarize-trace turns a rocprofv3
kernel-stats CSV into a Markdown table.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "ragged paged attn: query tokens/s, KV HBM GB/s + TFLOP/s, % of roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
HEADLINE = 5                   # the largest named workload
FLUSH_BYTES = 1 << 30          # written between cold samples (> 256 MB MALL + 8 x 4 MB L2)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: every line of the .h / .hip files
    with // comments and surrounding blanks removed, so that a comment edit
    does not void the counter-measured traffic."""
    import re

    d = os.path.join(ROOT, "ragged_paged_gqa_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".h", ".hip")):
            h.update(name.encode())
            with open(os.path.join(d, name), encoding="utf-8") as f:
                for line in f:
                    code = re.sub(r"//.*", "", line).strip()
                    if code:
                        h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def algorithmic_work(w):
    """Flops and bytes the method must compute and move (masked work and
    block over-fetch excluded), from the realized metadata, split by the
    kernel class that handles each sequence (<= 16 packed rows: decode)."""
    c = w.cfg
    G = c.num_q_heads // c.num_kv_heads
    b_kv = 1 if c.kv_dtype in ("fp8_e4m3fn", "fp8_e5m2", "int8") else 2  # bf16 and f16: 2
    b_q = 4 if c.q_dtype == "f32" else 2  # q and out elements
    sw = c.sliding_window or 0
    res = {"decode": [0.0, 0.0, 0], "prefill": [0.0, 0.0, 0]}  # flops, bytes, tokens
    for s in range(w.n_seqs):
        q0, q1 = int(w.cu_q_lens[s]), int(w.cu_q_lens[s + 1])
        ql, kvl = q1 - q0, int(w.kv_lens[s])
        if ql <= 0:
            continue
        i = np.arange(ql, dtype=np.int64)
        p = kvl - ql + i
        hi = np.minimum(p + 1, kvl) if c.is_causal else np.full(ql, kvl)
        lo = np.maximum(0, p - sw + 1) if sw > 0 else np.zeros(ql, np.int64)
        n_vis = np.maximum(hi - lo, 0)
        flops = float(c.num_q_heads * 4 * c.head_dim * n_vis.sum())
        r_s = max(0, int(hi.max()) - int(lo.min()))
        byts = float(c.num_kv_heads * 2 * c.head_dim * b_kv * r_s + ql * c.num_q_heads * (2 * b_q * c.head_dim + 4))
        cls = "decode" if ql * G <= 16 else "prefill"
        res[cls][0] += flops
        res[cls][1] += byts
        res[cls][2] += ql
    return res


def host_cpu():
    """CPU model and whether SMT is on, from /proc and /sys (Linux)."""
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    smt = None
    try:
        with open("/sys/devices/system/cpu/smt/active") as f:
            smt = f.read().strip() == "1"
    except OSError:
        pass
    return model, smt


def cpu_baseline(w, target_s: float = 15.0):
    """The oracle on the first n query tokens (all q heads), n sized for ~target_s."""
    import oracle

    oracle.build(force=False)
    threads = oracle.default_threads()
    T = w.valid_tokens()
    Hq = w.cfg.num_q_heads

    def run(n):
        toks = np.repeat(np.arange(n), Hq)
        heads = np.tile(np.arange(Hq), n)
        t0 = time.perf_counter()
        oracle.rows(w, toks, heads, nthreads=threads)
        return time.perf_counter() - t0

    # grow the sample until one run takes about target_s (10-30 s of CPU work)
    n = min(T, 2)
    dt = run(n)
    while dt < 0.6 * target_s and n < T:
        n = min(T, max(n + 1, int(n * min(8.0, target_s / max(dt, 1e-3)))))
        dt = run(n)
    model, smt = host_cpu()
    return {"value": n / dt, "unit": "query tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "smt": smt,
            "sample": f"first {n} of {T} query tokens, all {Hq} q heads, f64 oracle, {dt:.1f} s"}


def load_traffic(kernel: str, workload: int):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(f"{kernel}:cfg{workload}")
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def _counter_per_kernel(path: str, counter: str) -> dict:
    """Mean value (KiB per dispatch) of one rocprofv3 counter, per kernel name."""
    import csv
    import collections

    agg = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


KERNEL_CLASSES = ("tiles_pp_kernel", "tiles_kernel", "plan_kernel", "combine_kernel")


def kernel_class(name: str):
    for k in KERNEL_CLASSES:
        if f"rpa::{k}<" in name or f"rpa::{k}(" in name:
            return k
    return None


def ingest_counters(pmc_dir: str, workload: int) -> dict:
    """Turns two rocprofv3 --pmc runs of this benchmark (FETCH_SIZE, then
    WRITE_SIZE) plus the same two runs of `--copy-calibration` into HBM bytes
    per launch of each attention kernel, scaled by what each counter reads
    per true byte of the plain 1 GiB copy; stores them in the traffic file."""
    scale = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        copies = [v for k, v in _counter_per_kernel(
            os.path.join(pmc_dir, f"copy_{c}", "run_counter_collection.csv"), c).items() if "copyBuffer" in k]
        if not copies:
            raise SystemExit(f"no copy kernel in the {c} calibration run")
        scale[c] = copies[0] * 1024.0 / float(1 << 30)  # counter bytes per true byte
    per = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        for k, v in _counter_per_kernel(
                os.path.join(pmc_dir, f"w{workload}_{c}", "run_counter_collection.csv"), c).items():
            name = kernel_class(k)
            if name:
                per.setdefault(name, {})[c] = v * 1024.0 / scale[c]
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        t = {}
    h = kernel_source_hash()
    for name, d in per.items():
        if "FETCH_SIZE" in d and "WRITE_SIZE" in d:
            t[f"{name}:cfg{workload}"] = {
                "bytes_per_launch": round(d["FETCH_SIZE"] + d["WRITE_SIZE"]),
                "read_bytes": round(d["FETCH_SIZE"]), "write_bytes": round(d["WRITE_SIZE"]),
                "fetch_counter_per_byte": round(scale["FETCH_SIZE"], 4),
                "write_counter_per_byte": round(scale["WRITE_SIZE"], 4),
                "source_hash": h}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1, sort_keys=True)
        f.write("\n")
    return {k: v for k, v in t.items() if k.endswith(f":cfg{workload}")}


def summarize_trace(stats_csv: str) -> str:
    """A rocprofv3 kernel-stats CSV (--kernel-trace --stats) as a Markdown
    table: calls, average, min and max duration (us) and share, per kernel."""
    import csv

    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            name = r["Name"]
            if name.startswith(("__amd_rocclr", "Cijk_")) or "at::" in name or "elementwise" in name:
                continue  # torch's upload, fill and matmul kernels (the practical-ceiling probe)
            rows.append((name, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    out = ["| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, pct in sorted(rows, key=lambda x: -x[5]):
        out.append(f"| `{name}` | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.1f} % |")
    return "\n".join(out)


def practical_ceilings(torch) -> dict:
    """What the chip sustains in this session outside this library, as context
    for the roofline fractions (taken against the nominal peaks): a read-only
    stream (torch's row sums of a 65536-row view of 4 GiB of f32: of the torch
    reductions tried, the one that reads fastest) and a dense bf16 matrix
    product (torch.matmul, 8192 x 8192 x 8192, contiguous operands). Best of 5
    after a warm-up, HIP events."""
    def best_ms(fn, n=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts)
    n = 1 << 30  # f32 elements: 4 GiB
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    t_read = best_ms(lambda: x.view(65536, -1).sum(dim=1))
    del x
    m = 8192
    a = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    b = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    t_mm = best_ms(lambda: torch.matmul(a, b))
    del a, b
    torch.cuda.empty_cache()
    read_gbs = 4.0 * n / (t_read * 1e-3) / 1e9
    mm_tflops = 2.0 * m * m * m / (t_mm * 1e-3) / 1e12
    return {"read_stream_gbs": round(read_gbs, 1), "bf16_matmul_tflops": round(mm_tflops, 1),
            "how": "best of 5 (HIP events): torch row sums over 4 GiB f32 (read-only), "
                   "torch.matmul 8192^3 bf16"}


def stats(samples_ms) -> dict:
    a = np.asarray(samples_ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "mean": round(float(a.mean()), 4), "n": int(a.size)}


def roofline_of(flops: float, byts: float, seconds: float, prefer_mfma: bool) -> dict:
    """Achieved rate against the roofline that bounds this work: MFMA (bf16
    dense peak) when its arithmetic intensity is above the ridge point (or the
    caller says it is matrix-bound), else HBM."""
    ai = flops / max(byts, 1.0)
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if prefer_mfma or ai >= ridge:
        achieved = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    achieved = byts / seconds / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4)}


class Runner:
    """One workload resident on the GPU, with its timing helpers."""

    def __init__(self, number, args, headline=False):
        import torch

        import ragged_paged_gqa_amd as rpa
        import workloads as wl
        from gpu_util import Device, upload_q_bits

        self.torch, self.rpa = torch, rpa
        self.number = number
        kw = dict(kv_dtype=args.kv_dtype, q_dtype=args.q_dtype) if headline else {}
        log(f"[bench] generating workload {number}: {wl.WORKLOADS[number]}")
        t0 = time.perf_counter()
        w = wl.named(number, **kw)
        if headline and args.sinks:
            w = wl.with_sinks(w, number)
        log(f"[bench] generated in {time.perf_counter() - t0:.1f} s; uploading")
        self.w = w
        self.dev = Device(w)
        self.work = algorithmic_work(w)
        c = self.dev.cfg
        odt = torch.float32 if c.q_dtype == rpa.DTYPE_F32 else torch.bfloat16  # f16 bits fit a bf16 buffer
        self.out = torch.empty((c.num_q_tokens, c.num_q_heads, c.head_dim), dtype=odt, device="cuda")
        self.lse = torch.empty((c.num_q_tokens, c.num_q_heads), dtype=torch.float32, device="cuda")
        self.stream = torch.cuda.current_stream()
        self.append_new = None
        if headline and args.append:
            k_np, v_np = wl.new_kv(w, 1000 + number)
            self.append_new = (upload_q_bits(k_np, w.cfg.q_dtype), upload_q_bits(v_np, w.cfg.q_dtype))

    def call(self):
        d = self.dev
        self.rpa.forward(d.q, d.kv, d.kv_lens, d.page_indices, d.cu_q_lens, d.num_seqs, d.cfg,
                         workspace=d.workspace, out=self.out, lse=self.lse, sinks=d.sinks)

    def append(self):
        d = self.dev
        self.rpa.kv_append(self.append_new[0], self.append_new[1], d.kv, d.kv_lens, d.page_indices, d.cu_q_lens,
                           d.num_seqs, d.cfg, stream=self.stream)

    def timed_steps(self, steps, warmup, min_warm_s=0.0):
        """W untimed steps (and, with min_warm_s, as many more as fill that
        many seconds), then exactly K steps between synchronizations;
        per-kernel HIP events of the K calls (rpa_profile_*); with --append
        the append of each step is timed on its own with events."""
        torch = self.torch
        t0 = time.perf_counter()
        n = 0
        while n < warmup or time.perf_counter() - t0 < min_warm_s:
            if self.append_new is not None:
                self.append()
            self.call()
            n += 1
            if min_warm_s > 0.0 and n % 8 == 0:
                torch.cuda.synchronize()  # host time follows the GPU's
        torch.cuda.synchronize()
        self.warmup_calls = n
        ap_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        self.rpa.profile_begin(steps)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            if self.append_new is not None:
                ap_ev[i][0].record(self.stream)
                self.append()
                ap_ev[i][1].record(self.stream)
            self.call()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        kms, ncalls = self.rpa.profile_end()
        kmean = {k: v / max(ncalls, 1) for k, v in kms.items()}
        ams = (sum(a.elapsed_time(b) for a, b in ap_ev) / steps) if self.append_new is not None else None
        return (t1 - t0) * 1e3 / steps, kmean, ams

    def samples(self, n, flush_buf=None):
        """n single-call samples, each bracketed by HIP events on the call's
        stream; with flush_buf, the buffer is rewritten before each sample,
        outside the events."""
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            if flush_buf is not None:
                flush_buf.fill_(i & 0xFF)
            ev[i][0].record(self.stream)
            self.call()
            ev[i][1].record(self.stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    def summary(self, steps, warmup, n_samples, flush_buf, min_warm_s=0.0):
        """Everything measured for this workload (the headline's steps
        included), as one JSON-ready dict."""
        ms_step, kmean, ams = self.timed_steps(steps, warmup, min_warm_s)
        warm = stats(self.samples(n_samples))
        cold = stats(self.samples(n_samples, flush_buf))
        work = self.work
        F = work["decode"][0] + work["prefill"][0]
        B = work["decode"][1] + work["prefill"][1]
        T = self.w.valid_tokens()
        # one launch holds both classes: its work is theirs together, bound
        # by whichever peak it needs longer on
        t_ms, kf, kb = kmean["tiles"], F, B
        kroof = roofline_of(kf, kb, t_ms * 1e-3, prefer_mfma=False)
        kname = "tiles_pp_kernel" if self._uses_pp() else "tiles_kernel"
        kroof["kernel"] = kname
        kroof["kernel_ms"] = round(t_ms, 4)
        kroof["algorithmic_flops"] = kf
        kroof["algorithmic_bytes"] = kb
        kroof["kernel_name"] = kname
        kroof["traffic"] = load_traffic(kname, self.number)
        t_call = warm["median"] * 1e-3
        call_frac = max(F / (BF16_PEAK_TFLOPS * 1e12), B / (HBM_PEAK_GBS * 1e9)) / t_call
        res = {
            "workload": self._name(), "query_tokens": T, "ms_per_step": round(ms_step, 4),
            "warmup_calls": self.warmup_calls,
            "ms_per_call_warm": warm, "ms_per_call_cold": cold,
            "tokens_per_s": round(T / t_call, 1),
            "tflops": round(F / t_call / 1e12, 2), "kv_hbm_gbs": round(B / t_call / 1e9, 1),
            "roofline_frac_call": round(call_frac, 4),
            "mfma_frac_call": round(F / t_call / (BF16_PEAK_TFLOPS * 1e12), 4),
            "hbm_frac_call": round(B / t_call / (HBM_PEAK_GBS * 1e9), 4),
            "roofline_kernel": kroof,
            "kernel_ms": {k: round(v, 4) for k, v in kmean.items()},
            "algorithmic": {"flops": F, "bytes": B, "prefill_flops": work["prefill"][0],
                            "prefill_bytes": work["prefill"][1], "decode_flops": work["decode"][0],
                            "decode_bytes": work["decode"][1]},
        }
        if ams is not None:
            c = self.w.cfg
            import workloads as wl
            b_kv = 1 if wl.is_fp8(c.kv_dtype) else 2
            b_in = 4 if c.q_dtype == wl.Q_F32 else 2
            ab = float(T * 2 * c.num_kv_heads * c.head_dim * (b_in + b_kv))
            res["kv_append"] = {"kernel": "kv_append_kernel", "kernel_ms": round(ams, 5), "algorithmic_bytes": ab,
                                "achieved": round(ab / (ams * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": round(ab / (ams * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[bench] workload {self.number}: {ms_step:.4f} ms/step; warm median {warm['median']:.4f} ms "
            f"(p10 {warm['p10']:.4f}, p90 {warm['p90']:.4f}); cold median {cold['median']:.4f} ms; kernels (ms): "
            + ", ".join(f"{k} {v:.4f}" for k, v in kmean.items()))
        return res

    def _uses_pp(self):
        c = self.dev.cfg
        return c.head_dim == 256 and c.q_dtype in (self.rpa.DTYPE_BF16, self.rpa.DTYPE_F16) \
            and c.kv_dtype == c.q_dtype

    def _name(self):
        import workloads as wl
        return wl.WORKLOADS[self.number]

    def free(self):
        del self.dev, self.out, self.lse
        self.torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--samples", type=int, default=50, help="single-call samples, warm and cold each")
    ap.add_argument("--warm-seconds", type=float, default=0.0,
                    help="keep warming up past --warmup calls until this many seconds have passed "
                         "(the other named workloads of the sweep always take at least 0.2 s)")
    ap.add_argument("--workload", type=int, default=HEADLINE, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-sweep", action="store_true", help="measure the headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kv-dtype", choices=["bf16", "f16", "fp8_e4m3fn", "fp8_e5m2", "int8"], default=None,
                    help="store the headline workload's K/V cache in this type instead of its own")
    ap.add_argument("--q-dtype", choices=["bf16", "f16", "f32"], default=None,
                    help="q/out type of the headline workload (f16: a bf16 cache becomes f16 too)")
    ap.add_argument("--sinks", action="store_true",
                    help="attach seeded attention-sink logits (one per q head) and call rpa_forward_sinks")
    ap.add_argument("--append", action="store_true",
                    help="each step first writes the step's new K/V rows into the cache (rpa_kv_append), "
                         "then attends; the append kernel is timed on its own as well")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--ingest-counters", metavar="DIR", default=None,
                    help="host only: turn rocprofv3 FETCH_SIZE/WRITE_SIZE runs under DIR "
                         "(copy_<C>/ and w<workload>_<C>/) into the traffic file")
    ap.add_argument("--summarize-trace", metavar="CSV", default=None,
                    help="host only: print a rocprofv3 kernel-stats CSV as a Markdown table")
    args = ap.parse_args()

    if args.ingest_counters:
        print(json.dumps(ingest_counters(args.ingest_counters, args.workload), sort_keys=True))
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence or kv head with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(3)]
        for e0, e1 in ev:
            e0.record()
            b.copy_(a)
            e1.record()
        torch.cuda.synchronize()
        # the copy reads and writes n bytes: its rate is the HBM rate a plain
        # stream reaches, beside the 8 TB/s peak
        ms = [e0.elapsed_time(e1) for e0, e1 in ev]
        print(json.dumps({"copy_bytes": n, "copies": 3, "copy_ms": [round(m, 4) for m in ms],
                          "copy_gbs_best": round(2 * n / (min(ms) * 1e-3) / 1e9, 1)}))
        return

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import workloads as wl

    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    head = Runner(args.workload, args, headline=True)
    hs = head.summary(args.steps, args.warmup, args.samples, flush_buf, min_warm_s=args.warm_seconds)
    w = head.w
    T = w.valid_tokens()
    ms = hs["ms_per_step"]
    roof = dict(hs["roofline_kernel"])
    dtype = w.cfg.q_dtype if w.cfg.kv_dtype == w.cfg.q_dtype \
        else f"{w.cfg.q_dtype} q / {w.cfg.kv_dtype.replace('_', ' ')} kv"
    result = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        **({"warmup_calls": hs["warmup_calls"]} if hs["warmup_calls"] != args.warmup else {}),
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, shuffled page table)",
        "config": {"workload": wl.WORKLOADS[args.workload], "num_seqs": w.n_seqs, "query_tokens": T,
                   "num_q_heads": w.cfg.num_q_heads, "num_kv_heads": w.cfg.num_kv_heads,
                   "head_dim": w.cfg.head_dim, "page_size": w.cfg.page_size,
                   **({"attention_sinks": True} if args.sinks else {}),
                   **({"kv_append": True} if args.append else {}),
                   **({"kv_dtype": w.cfg.kv_dtype} if args.kv_dtype or args.q_dtype else {}),
                   **({"q_dtype": w.cfg.q_dtype} if args.q_dtype else {})},
        "tflops": round(hs["algorithmic"]["flops"] / (ms * 1e-3) / 1e12, 2),
        "kv_hbm_gbs": round(hs["algorithmic"]["bytes"] / (ms * 1e-3) / 1e9, 1),
        "roofline_frac_step": round(max(hs["algorithmic"]["flops"] / (BF16_PEAK_TFLOPS * 1e12),
                                        hs["algorithmic"]["bytes"] / (HBM_PEAK_GBS * 1e9)) / (ms * 1e-3), 4),
        "kernel_ms": hs["kernel_ms"],
        "roofline": roof,
        "timing": {"warm": hs["ms_per_call_warm"], "cold": hs["ms_per_call_cold"],
                   "note": "per-call HIP events; cold = a 1 GiB buffer written before each sample, "
                           "outside the events"},
    }
    if "kv_append" in hs:
        result["kv_append"] = hs["kv_append"]
    cpu_w = None if args.no_cpu_baseline else w
    head.free()
    del head

    # the other named workloads, the same measurements each
    configs = {f"w{args.workload}": hs}
    plain = not (args.kv_dtype or args.q_dtype or args.sinks or args.append)
    if not args.no_sweep and plain:
        for number in (1, 2, 3, 4, 5):
            if number == args.workload:
                continue
            r = Runner(number, args)
            # at least 0.2 s of warm-up calls: a short workload's first
            # ~20 ms of back-to-back calls run up to a third slower than
            # the calls after them
            configs[f"w{number}"] = r.summary(args.steps, args.warmup, args.samples, flush_buf,
                                              min_warm_s=max(0.2, args.warm_seconds))
            r.free()
            del r
    if len(configs) > 1:
        result["configs"] = configs
    log("[bench] practical ceilings (read stream, bf16 matmul)")
    ceil = practical_ceilings(torch)
    if roof.get("unit") == "TFLOP/s":
        ceil["roofline_frac_of_practical"] = round(roof["achieved"] / ceil["bf16_matmul_tflops"], 4)
    else:
        ceil["roofline_frac_of_practical"] = round(roof["achieved"] / ceil["read_stream_gbs"], 4)
    result["practical_ceilings"] = ceil
    if cpu_w is not None:
        log("[bench] timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(cpu_w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
