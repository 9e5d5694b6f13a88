"""Benchmark of ragged paged GQA attention on one MI355X.

One step = one rpa_forward call (plan, prefill-class tiles, decode-class
tiles, split-KV merge inside them) over one batch of seeded synthetic inputs
already resident in HBM; with --append, an rpa_kv_append of the step's new
K/V rows first.
The default workload is the decode batch (256 sequences x 1 query token,
kv_len U[512, 8192], 32 q / 8 kv heads, head_dim 128, page 16, bf16).

Prints ONE JSON line on stdout (diagnostics go to stderr):
  value      query tokens/s of the whole call
  roofline   the dominant kernel's algorithmic bytes (or flops) per launch
             over its mean launch time, measured with HIP events recorded
             around each kernel on the launch stream during the timed steps
  cpu_baseline  the f64 CPU oracle timed on a bounded sample of the same
             workload on the host cores (a reported baseline, not a target)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    d = os.path.join(ROOT, "ragged_paged_gqa_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".h", ".hip")):
            h.update(name.encode())
            with open(os.path.join(d, name), "rb") as f:
                h.update(f.read())
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

    n = min(T, 2)
    dt = run(n)
    while dt < target_s / 8 and n < T:
        n = min(T, max(n + 1, int(n * min(8.0, target_s / max(dt, 1e-3)))))
        dt = run(n)
    return {"value": n / dt, "unit": "query tokens/s", "cores": threads, "kind": "oracle",
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
            for name in ("decode_kernel", "prefill_kernel", "plan_kernel", "combine_kernel"):
                if f"rpa::{name}" in k:
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kv-dtype", choices=["bf16", "f16", "fp8_e4m3fn", "fp8_e5m2", "int8"], default=None,
                    help="store the workload's K/V cache in this type instead of its own")
    ap.add_argument("--q-dtype", choices=["bf16", "f16", "f32"], default=None,
                    help="q/out type (f16: a bf16 cache becomes f16 too)")
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
    args = ap.parse_args()

    if args.ingest_counters:
        print(json.dumps(ingest_counters(args.ingest_counters, args.workload), sort_keys=True))
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

    import ragged_paged_gqa_amd as rpa
    import workloads as wl

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import Device, upload_q_bits

    log(f"[bench] generating workload {args.workload}: {wl.WORKLOADS[args.workload]}")
    t0 = time.perf_counter()
    w = wl.named(args.workload, kv_dtype=args.kv_dtype, q_dtype=args.q_dtype)
    if args.sinks:
        w = wl.with_sinks(w, args.workload)
    log(f"[bench] generated in {time.perf_counter() - t0:.1f} s; uploading")
    dev = Device(w)
    work = algorithmic_work(w)
    T = w.valid_tokens()
    F = work["decode"][0] + work["prefill"][0]
    B = work["decode"][1] + work["prefill"][1]

    if args.append:
        k_np, v_np = wl.new_kv(w, 1000 + args.workload)
        k_new = upload_q_bits(k_np, w.cfg.q_dtype)
        v_new = upload_q_bits(v_np, w.cfg.q_dtype)
        stream = torch.cuda.current_stream()
        ap_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps)]

    def append(i=None):
        if i is not None:
            ap_ev[i][0].record(stream)
        rpa.kv_append(k_new, v_new, dev.kv, dev.kv_lens, dev.page_indices, dev.cu_q_lens, dev.num_seqs,
                      dev.cfg, stream=stream)
        if i is not None:
            ap_ev[i][1].record(stream)

    for _ in range(args.warmup):
        if args.append:
            append()
        dev.run()
    torch.cuda.synchronize()
    rpa.profile_begin(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if args.append:
            append(i)
        rpa.forward(dev.q, dev.kv, dev.kv_lens, dev.page_indices, dev.cu_q_lens, dev.num_seqs, dev.cfg,
                    workspace=dev.workspace, out=dev_out(dev), lse=dev_lse(dev), sinks=dev.sinks)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kms, ncalls = rpa.profile_end()
    ms = (t1 - t0) * 1e3 / args.steps
    kmean = {k: v / max(ncalls, 1) for k, v in kms.items()}
    log(f"[bench] {ms:.4f} ms/step; kernels (ms): " + ", ".join(f"{k} {v:.4f}" for k, v in kmean.items()))

    dom = "decode" if kmean["decode"] >= kmean["prefill"] else "prefill"
    f_dom, b_dom = work[dom][0], work[dom][1]
    t_dom = kmean[dom] * 1e-3
    ai = f_dom / max(b_dom, 1.0)
    if dom == "decode" or ai < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        achieved = b_dom / t_dom / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = f_dom / t_dom / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    roof["kernel"] = f"{dom}_kernel"
    roof["kernel_ms"] = round(kmean[dom], 4)
    roof["algorithmic_bytes"] = b_dom
    roof["algorithmic_flops"] = f_dom
    roof["traffic"] = load_traffic(f"{dom}_kernel", args.workload)

    step_s = ms * 1e-3
    result = {
        "metric": METRIC,
        "value": round(T / step_s, 1),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.cfg.q_dtype if w.cfg.kv_dtype == w.cfg.q_dtype
        else f"{w.cfg.q_dtype} q / {w.cfg.kv_dtype.replace('_', ' ')} kv",
        "data": "synthetic (seeded N(0,1) Q/K/V, shuffled page table)",
        "config": {"workload": wl.WORKLOADS[args.workload], "num_seqs": w.n_seqs, "query_tokens": T,
                   "num_q_heads": w.cfg.num_q_heads, "num_kv_heads": w.cfg.num_kv_heads,
                   "head_dim": w.cfg.head_dim, "page_size": w.cfg.page_size,
                   **({"attention_sinks": True} if args.sinks else {}),
                   **({"kv_dtype": w.cfg.kv_dtype} if args.kv_dtype or args.q_dtype else {}),
                   **({"q_dtype": w.cfg.q_dtype} if args.q_dtype else {})},
        "kv_hbm_gbs": round(B / step_s / 1e9, 1),
        "tflops": round(F / step_s / 1e12, 2),
        "roofline_frac_step": round(max(F / (BF16_PEAK_TFLOPS * 1e12), B / (HBM_PEAK_GBS * 1e9)) / step_s, 4),
        "kernel_ms": {k: round(v, 4) for k, v in kmean.items()},
        "roofline": roof,
    }
    if args.append:
        # bytes the append must move: each new K and V element read once in
        # the q type and written once in the cache type
        c = w.cfg
        b_kv = 1 if wl.is_fp8(c.kv_dtype) else 2
        b_in = 4 if c.q_dtype == wl.Q_F32 else 2
        ab = float(T * 2 * c.num_kv_heads * c.head_dim * (b_in + b_kv))
        ams = sum(a.elapsed_time(b) for a, b in ap_ev) / args.steps
        result["config"]["kv_append"] = True
        result["kv_append"] = {"kernel": "kv_append_kernel", "kernel_ms": round(ams, 5), "algorithmic_bytes": ab,
                               "achieved": round(ab / (ams * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": round(ab / (ams * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[bench] kv_append {ams * 1e3:.2f} us, {ab / 1e6:.2f} MB")
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


_outs = {}


def dev_out(dev):
    import torch

    import ragged_paged_gqa_amd as rpa
    key = id(dev)
    if key not in _outs:
        c = dev.cfg
        # out in the q type's width (f16 bits fit a bf16 buffer)
        odt = torch.float32 if c.q_dtype == rpa.DTYPE_F32 else torch.bfloat16
        _outs[key] = (torch.empty((c.num_q_tokens, c.num_q_heads, c.head_dim), dtype=odt, device="cuda"),
                      torch.empty((c.num_q_tokens, c.num_q_heads), dtype=torch.float32, device="cuda"))
    return _outs[key][0]


def dev_lse(dev):
    dev_out(dev)
    return _outs[id(dev)][1]


if __name__ == "__main__":
    main()
