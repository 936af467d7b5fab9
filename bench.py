"""Benchmark of the attention hot path on one MI355X.

One step = one exact attention forward on the LLM-prefill workload (B=4,
Hq=Hkv=32, Nq=Nk=2048, d=128, bf16, causal) followed by one split-KV decode
(split + combine) on the decode workload (64 sequences, Hq=32, Hkv=8, d=128,
bf16, L ~ U[512, 32768], 512-key chunks). Inputs are resident in HBM before the
timed region starts. HIP events on the launch stream bracket every kernel of
every timed step.

Prints ONE JSON line:
  value       prefill TFLOP/s = 4*B*H*N*N*d/2 / mean forward kernel time
  decode      KV GB/s = sum_b 2*Hkv*L_b*d*2 bytes / mean (split + combine) time
  bwd           the backward (dQ, dK, dV) on the prefill workload, TFLOP/s at 2.5x
                the forward's flops, timed in a loop of its own
  fwd_local     sliding-window attention (512 keys back) on the prefill shapes
  fwd_qkvpacked the prefill attention read from one packed [B, N, 3, H, d] tensor
  fwd_varlen    a packed causal prefill batch (8192 tokens in sequences of seeded
                lengths U[256, 4096]), TFLOP/s, timed in a loop of its own
  decode_auto   the same decode through attn_decode (the library's chunk length)
  decode_paged  the same decode over a paged cache (64-row pages, shuffled pool,
                block tables), timed in a loop of its own after the steps
  decode_fused  the same decode (512-key chunks) with the combine fused into the
                split kernel (attn_decode_fused), one launch per decode
  decode_fused_paged  the same over the paged cache (attn_decode_fused_paged)
  fwd_tiny      the tiny fp16 workload (B=1 H=2 N=128 d=64), causal and not,
                microseconds per call (launch-bound; no roofline claim)
  roofline    the forward kernel against the bf16 dense MFMA peak
  cpu_baseline  the fp64 CPU oracle on every row of the prefill workload, in the
                same TFLOP/s unit, plus the tiny workload in full, seeded row
                subsets of the GQA-prefill and long-context workloads (with the
                full-workload time extrapolated from the subset's share of the
                work) and the whole decode workload in KV GB/s
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s (bf16, d=128, causal) + split-KV decode KV GB/s"
PEAK_BF16_TFLOPS = 2516.6  # 256 CUs x 4096 dense bf16 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# The sources each recorded kernel is built from (a recorded traffic figure is
# used only while they are unchanged).
_CSRC = os.path.join(ROOT, "exact_attention_46_amd", "csrc")
KERNEL_SOURCES = {
    "attn_fwd_kernel": ["common.hpp", "attn_fwd.hip"],
    "attn_decode_split_kernel": ["common.hpp", "attn_decode.hip"],
    "attn_bwd_dq_kernel": ["common.hpp", "attn_bwd.hip"],
    "attn_bwd_dkdv_kernel": ["common.hpp", "attn_bwd.hip"],
    "attn_bwd_delta_kernel": ["common.hpp", "attn_bwd.hip"],
    "attn_bwd_dq_ds_kernel": ["common.hpp", "attn_bwd.hip"],
    "attn_decode_combine_kernel": ["common.hpp", "attn_decode.hip"],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first (the clocks settle within a few hundred)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (used for profiler runs)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the backward measurement")
    ap.add_argument("--no-local", action="store_true",
                    help="skip the sliding-window measurement")
    ap.add_argument("--no-qkv", action="store_true",
                    help="skip the packed-qkv measurement")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the packed variable-length prefill measurement")
    ap.add_argument("--no-auto", action="store_true",
                    help="skip the one-call decode (library chunk) measurement")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the paged-cache decode measurements")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the fused-combine decode measurements")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the forward on the GQA-prefill and long-context workloads")
    ap.add_argument("--only", choices=["all", "prefill", "decode"] + ONLY_EXTRA, default="all",
                    help="restrict the timed step (for per-kernel profiles); the extra choices "
                         "run only that measurement, --steps times after --warmup untimed runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a plain streaming kernel of known size "
                         "(the calibration of HBM byte counters)")
    ap.add_argument("--record-traffic", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "RUN"),
                    help="no GPU: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "'bench.py --copy-calibration' (RUN = step) or 'bench.py --only RUN "
                         "--copy-calibration' into entries of " + TRAFFIC_FILE)
    return ap.parse_args()


# Single measurements for counter runs (bench.py --only NAME): the forward on
# another workload, the backward, the fused decode and its paged form.
ONLY_EXTRA = ["fwd_gqa_prefill", "fwd_long_context", "bwd", "bwd_ds", "decode_fused",
              "decode_fused_paged", "fwd_local", "fwd_qkvpacked", "fwd_varlen", "decode_auto"]

COPY_CAL_BYTES = 256 << 20  # bytes read (and written) by one calibration launch
COPY_CAL_MATCH = "neg"      # the calibration kernel's name contains this


def copy_calibration(torch, dev):
    """Three launches of a plain elementwise kernel that reads COPY_CAL_BYTES and
    writes as many (y = -x over bf16)."""
    x = torch.ones(COPY_CAL_BYTES // 2, dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()


def _counter_means(folder, counter):
    """Mean value per dispatch of `counter`, by kernel name, over every
    *counter_collection.csv under `folder`."""
    import csv
    import glob
    vals = {}
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % folder)
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


# Kernels whose HBM traffic a profiled run records: run -> [(entry, kernel-name match)].
# Every run holds the calibration kernel too.
TRAFFIC_RUNS = {
    "step": [("attn_fwd_kernel/llm_prefill", "attn_fwd_kernel"),
             ("attn_decode_split_kernel/decode", "attn_decode_split_kernel<0, 128, false, false, false>"),
             ("attn_decode_split_kernel/decode_paged",
              "attn_decode_split_kernel<0, 128, true, false, false>")],
    "fwd_gqa_prefill": [("attn_fwd_kernel/gqa_prefill", "attn_fwd_kernel")],
    "fwd_long_context": [("attn_fwd_kernel/long_context", "attn_fwd_kernel")],
    "fwd_local": [("attn_fwd_kernel/local", "attn_fwd_kernel<0, 128, false, false, true,")],
    "bwd": [("attn_bwd_dq_kernel/llm_prefill", "attn_bwd_dq_kernel<"),
            ("attn_bwd_dkdv_kernel/llm_prefill", "attn_bwd_dkdv_kernel<0, 128, true, false>")],
    "bwd_ds": [("attn_bwd_delta_kernel/llm_prefill", "attn_bwd_delta_kernel"),
               ("attn_bwd_dkdv_kernel/llm_prefill_ds", "attn_bwd_dkdv_kernel<0, 128, true, true>"),
               ("attn_bwd_dq_ds_kernel/llm_prefill", "attn_bwd_dq_ds_kernel")],
    "decode_fused": [("attn_decode_split_kernel/decode_fused",
                      "attn_decode_split_kernel<0, 128, false, false, true>")],
    "decode_fused_paged": [("attn_decode_split_kernel/decode_fused_paged",
                            "attn_decode_split_kernel<0, 128, true, false, true>")],
    "fwd_qkvpacked": [("attn_fwd_kernel/qkvpacked", "attn_fwd_kernel")],
    "fwd_varlen": [("attn_fwd_kernel/varlen", "attn_fwd_kernel")],
    "decode_auto": [("attn_decode_split_kernel/decode_auto",
                     "attn_decode_split_kernel<0, 128, false, false, false>"),
                    ("attn_decode_combine_kernel/decode_auto", "attn_decode_combine_kernel")],
}


def record_traffic(fetch_dir, write_dir, run):
    """HBM bytes per launch of a run's kernels: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each divided by what the same counter reads per byte of the
    calibration kernel; merged into the traffic file."""
    if run not in TRAFFIC_RUNS:
        raise SystemExit("unknown run %r (one of %s)" % (run, ", ".join(TRAFFIC_RUNS)))
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")

    def pick(table, key):
        hits = [v for k, v in table.items() if key in k]
        if len(hits) != 1:
            raise SystemExit("expected one kernel matching %r, found %d" % (key, len(hits)))
        return hits[0]

    f_cal = pick(fetch, COPY_CAL_MATCH) * 1024.0 / COPY_CAL_BYTES
    w_cal = pick(write, COPY_CAL_MATCH) * 1024.0 / COPY_CAL_BYTES
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec.setdefault("_calibration", {})[run] = {
        "kernel": "torch.neg over %d bytes of bf16" % COPY_CAL_BYTES,
        "fetch_counter_bytes_per_byte": round(f_cal, 4),
        "write_counter_bytes_per_byte": round(w_cal, 4)}
    for name, match in TRAFFIC_RUNS[run]:
        fb = pick(fetch, match) * 1024.0 / f_cal
        wb = pick(write, match) * 1024.0 / w_cal
        rec[name] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                     "bytes_per_launch": round(fb + wb), "source_hash": source_hash(name)}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({k: rec[k] for k, _ in TRAFFIC_RUNS[run]}, indent=1))


def source_hash(entry):
    """Hash of the sources of the kernel a traffic entry ("kernel/workload") names."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[entry.split("/")[0]]:
        with open(os.path.join(_CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """Measured HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by
    a copy-kernel calibration), if recorded for the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel)
    if not ent or ent.get("source_hash") != source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


def _rows_flops(rows, N, d):
    """Metric flops of causal rows (row i attends i + 1 keys)."""
    import numpy as np
    return float(np.sum(4.0 * (rows[:, 2] + 1) * d))


def cpu_baseline(w, q, k, v, target_s):
    """The fp64 oracle as it stands on the host's cores: every row of the prefill
    workload (its whole fp64 forward), and a seeded row sample of it on one thread."""
    import numpy as np

    import oracle
    from exact_attention_46_amd import workloads as wl

    qb, kb, vb = wl.bits(q), wl.bits(k), wl.bits(v)
    cores = oracle.max_threads()  # the oracle keeps the last thread count it was given
    t0 = time.perf_counter()
    oracle.attn_fwd(qb, kb, vb, 0, w.scale, True, nthreads=cores)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.B * w.Hq * w.N * w.N * w.d / 2.0  # the metric's causal convention
    # one thread, on seeded random rows worth about a tenth of target_s
    rng = np.random.default_rng(12345)
    n1 = int(max(64, w.B * w.Hq * w.N * min(1.0, 0.1 * target_s / max(dt * cores, 1e-3))))
    rows1 = np.stack([rng.integers(0, w.B, n1), rng.integers(0, w.Hq, n1),
                      rng.integers(0, w.N, n1)], axis=1).astype(np.int64)
    t0 = time.perf_counter()
    oracle.attn_fwd_rows(qb, kb, vb, 0, w.scale, True, rows1, nthreads=1)
    dt1 = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": "all %d rows of the llm_prefill workload, each once (its whole exact "
                      "fp64 causal forward), %.2f s" % (w.B * w.Hq * w.N, dt),
            "seconds": dt,
            "one_thread": {"value": _rows_flops(rows1, w.N, w.d) / dt1 / 1e12,
                           "unit": "TFLOP/s",
                           "sample": "%d seeded random rows of the same workload on one "
                                     "thread, %.2f s" % (n1, dt1)},
            "host": {"nproc": os.cpu_count(), "cpu_model": _cpu_model()}}


def cpu_baseline_tiny(cores):
    """The oracle on the whole tiny fp16 workload, both masks."""
    import oracle
    from exact_attention_46_amd import workloads as wl

    w = wl.WORKLOADS["tiny"]
    q, k, v = (wl.bits(t) for t in wl.workload_prefill_inputs(w))
    out = {}
    for causal in (False, True):
        reps = 20
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.attn_fwd(q, k, v, 1, w.scale, causal, nthreads=cores)
        dt = (time.perf_counter() - t0) / reps
        out["causal" if causal else "non_causal"] = {"us": round(dt * 1e6, 1)}
    out["sample"] = "the whole tiny workload (B=1 H=2 N=128 d=64 fp16), mean of 20 calls"
    return out


def cpu_baseline_subset(name, cores, n_rows, seed):
    """The oracle on a seeded subset of rows of a large prefill workload; the
    full workload's time is extrapolated by the subset's share of its flops."""
    import numpy as np

    import oracle
    from exact_attention_46_amd import workloads as wl

    w = wl.WORKLOADS[name]
    q, k, v = (wl.bits(t) for t in wl.workload_prefill_inputs(w))
    rng = np.random.default_rng(seed)
    rows = np.stack([rng.integers(0, w.B, n_rows), rng.integers(0, w.Hq, n_rows),
                     rng.integers(0, w.N, n_rows)], axis=1).astype(np.int64)
    t0 = time.perf_counter()
    oracle.attn_fwd_rows(q, k, v, 0, w.scale, True, rows, nthreads=cores)
    dt = time.perf_counter() - t0
    fl = _rows_flops(rows, w.N, w.d)
    full = 4.0 * w.B * w.Hq * w.N * w.N * w.d / 2.0
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
            "sample": "%d seeded random query rows (%.3f %% of the workload's flops), %.2f s"
                      % (n_rows, 100.0 * fl / full, dt),
            "seconds": dt,
            "est_full_seconds": round(dt * full / fl, 1),
            "extrapolation": "full time = subset time x (workload flops / subset flops)"}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_decode(wd, sl, dq, kc, vc, cores, n_seq=None):
    """Times the fp64 decode oracle on the decode workload (all sequences unless
    n_seq picks a seeded sample; every key of each); KV GB/s like the metric."""
    import numpy as np

    import oracle
    from exact_attention_46_amd import workloads as wl

    rng = np.random.default_rng(777)
    n_seq = dq.shape[0] if n_seq is None else n_seq
    idx = np.sort(rng.choice(dq.shape[0], size=n_seq, replace=False))
    lens = sl.numpy()[idx].astype(np.int64)
    L = int(lens.max())
    import torch

    ti = torch.as_tensor(idx, dtype=torch.long, device=dq.device)
    q = dq.index_select(0, ti).cpu()
    k = kc.index_select(0, ti)[:, :, :L].cpu()
    v = vc.index_select(0, ti)[:, :, :L].cpu()
    t0 = time.perf_counter()
    oracle.decode(wl.bits(q), wl.bits(k), wl.bits(v), lens.astype(np.int32), 0, wd.scale,
                  nthreads=cores)
    dt = time.perf_counter() - t0
    kv = float(np.sum(2 * wd.Hkv * lens * wd.d * 2))
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": "%d of the decode workload's %d sequences (%d keys in all, every "
                      "query head), %.1f s" % (n_seq, dq.shape[0], int(lens.sum()), dt),
            "seconds": dt}


PAGE_SIZE = 64


def bench_decode_auto(args, torch, np, ea, wd, sl, dq, sld, kc, vc, stream):
    """attn_decode on the decode workload: the library picks the chunk length (2048
    keys here) instead of the workload's 512. Timed in a loop of its own."""
    print("bench: one-call decode", file=sys.stderr, flush=True)
    B, Hq, d = dq.shape
    n = ea.attn_decode_workspace(B, Hq, kc.shape[1], kc.shape[2], d)
    ws = torch.empty((n,), dtype=torch.float32, device=dq.device) if n else None
    o = torch.empty((B, Hq, d), dtype=dq.dtype, device=dq.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dq.device)

    def run():
        ea.attn_decode(dq, kc, vc, sld, o, lse, ws, wd.scale, stream)

    for _ in range(max(1, args.warmup)):
        run()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in events:
        e[0].record(stream)
        run()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    lens = sl.numpy().astype(np.int64)
    kv_bytes = float(np.sum(2 * wd.Hkv * lens * wd.d * 2))
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    slots = n // (B * Hq * (d + 1)) if n else 1  # chunk slots per (b, h)
    return {"value": round(gbs, 1), "unit": "GB/s", "ms": round(ms, 4),
            "chunk_slots": slots, "chunk": -(-kc.shape[2] // slots), "workspace_floats": n,
            "roofline": {"kernel": "attn_decode_split_kernel + combine (library chunk)",
                         "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": _sum_traffic(["attn_decode_split_kernel/decode_auto",
                                                  "attn_decode_combine_kernel/decode_auto"])}}


def _sum_traffic(names):
    vals = [load_traffic(n) for n in names]
    return sum(vals) if all(v is not None for v in vals) else None


VARLEN_TOKENS, VARLEN_MIN, VARLEN_MAX = 8192, 256, 4096


def bench_bwd(args, torch, np, ea, wp, qg, kg, vg, og, lseg, stream, stored_ds=False):
    """Backward on the llm_prefill workload (dO drawn like the inputs). TFLOP/s with
    the usual convention: 2.5x the forward's flops (five products of the forward's
    size). attn_bwd performs seven (S and dP are recomputed by both the dK/dV and
    the dQ kernels); stored_ds: attn_bwd_ds, which performs five and moves dS
    through a workspace in HBM (a D kernel, dK/dV storing dS^T, dQ = dS K).
    Timed in a loop of its own after the steps."""
    print("bench: backward%s" % (" (stored dS)" if stored_ds else ""), file=sys.stderr, flush=True)
    g = torch.Generator(device="cpu").manual_seed(wp.seed + 100)
    do = torch.randn(qg.shape, generator=g).to(qg.dtype).to(qg.device)
    dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    delta = torch.empty_like(lseg)
    ds = ea.ds_workspace(qg, kg) if stored_ds else None

    def run():
        if stored_ds:
            ea.attn_bwd_ds(qg, kg, vg, og, do, lseg, delta, ds, dq, dk, dv, True, wp.scale, stream)
        else:
            ea.attn_bwd(qg, kg, vg, og, do, lseg, delta, dq, dk, dv, True, wp.scale, stream)

    for _ in range(max(1, args.warmup)):
        run()
    torch.cuda.synchronize()
    n = max(5, args.steps // 5)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    for e in events:
        e[0].record(stream)
        run()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    flops = 2.5 * 4.0 * wp.B * wp.Hq * wp.N * wp.N * wp.d / 2.0
    tf = flops / (ms * 1e-3) / 1e12
    out = {"value": round(tf, 2), "unit": "TFLOP/s", "ms": round(ms, 4),
           "flop_convention": "2.5 x forward (causal halved)",
           "roofline": {"kernel": ("attn_bwd_ds (delta + dkdv storing dS + dq from dS kernels)"
                                   if stored_ds else "attn_bwd (dq + dkdv kernels)"),
                        "bound": "mfma",
                        "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                        "traffic": _bwd_traffic(stored_ds)}}
    if stored_ds:
        out["workspace_bytes"] = int(ds.numel())
    return out


def _bwd_traffic(stored_ds=False):
    names = (["attn_bwd_delta_kernel/llm_prefill", "attn_bwd_dkdv_kernel/llm_prefill_ds",
              "attn_bwd_dq_ds_kernel/llm_prefill"] if stored_ds else
             ["attn_bwd_dq_kernel/llm_prefill", "attn_bwd_dkdv_kernel/llm_prefill"])
    vals = [load_traffic(n) for n in names]
    return sum(vals) if all(v is not None for v in vals) else None


LOCAL_WINDOW = 512


def bench_local(args, torch, np, ea, wp, qg, kg, vg, stream):
    """Sliding-window attention on the llm_prefill shapes: each row sees its own
    key and the LOCAL_WINDOW keys before it. TFLOP/s counts 4*d flops per allowed
    (row, key) pair. Timed in a loop of its own after the steps."""
    print("bench: sliding-window attention", file=sys.stderr, flush=True)
    o = torch.empty_like(qg)
    lse = torch.empty(qg.shape[:3], dtype=torch.float32, device=qg.device)

    def run():
        ea.attn_fwd_local(qg, kg, vg, o, lse, LOCAL_WINDOW, 0, wp.scale, stream)

    for _ in range(max(1, args.warmup)):
        run()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in events:
        e[0].record(stream)
        run()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    pairs = float(sum(min(i, LOCAL_WINDOW) + 1 for i in range(wp.N)))
    flops = 4.0 * wp.B * wp.Hq * wp.d * pairs
    tf = flops / (ms * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "ms": round(ms, 4),
            "window": [LOCAL_WINDOW, 0],
            "roofline": {"kernel": "attn_fwd_kernel<bf16,128,local>", "bound": "mfma",
                         "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": load_traffic("attn_fwd_kernel/local")}}


def bench_fwd_workload(args, torch, np, ea, wl, name, dev, stream):
    """The causal forward on another prefill workload (inputs built like the
    step's), timed in a loop of its own after the steps."""
    print("bench: forward on %s" % name, file=sys.stderr, flush=True)
    w = wl.WORKLOADS[name]
    q, k, v = (t.to(dev) for t in wl.workload_prefill_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    def run():
        ea.attn_fwd(q, k, v, o, lse, True, w.scale, stream)

    steps = max(1, min(args.steps, 20))
    for _ in range(max(1, min(args.warmup, 50))):
        run()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in events:
        e[0].record(stream)
        run()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    flops = 4.0 * w.B * w.Hq * w.N * w.N * w.d / 2
    tf = flops / (ms * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "ms": round(ms, 4),
            "shape": {"B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d, "causal": True},
            "roofline": {"kernel": "attn_fwd_kernel<bf16,128,causal>", "bound": "mfma",
                         "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": load_traffic("attn_fwd_kernel/" + name),
                         "algorithmic_bytes": (2 * w.B * w.Hq * w.N + 2 * w.B * w.Hkv * w.N) * w.d
                         * 2 + w.B * w.Hq * w.N * 4}}


def bench_qkvpacked(args, torch, np, ea, wp, stream):
    """The llm_prefill attention read from one packed [B, N, 3, H, d] tensor (no
    permute) with o written [B, N, H, d]. Timed in a loop of its own."""
    print("bench: packed qkv input", file=sys.stderr, flush=True)
    g = torch.Generator(device="cpu").manual_seed(wp.seed + 200)
    qkv = torch.randn((wp.B, wp.N, 3, wp.Hq, wp.d), generator=g).to(torch.bfloat16).cuda()
    o = torch.empty((wp.B, wp.N, wp.Hq, wp.d), dtype=qkv.dtype, device=qkv.device)
    lse = torch.empty((wp.B, wp.Hq, wp.N), dtype=torch.float32, device=qkv.device)

    def run():
        ea.attn_fwd_qkvpacked(qkv, o, lse, True, wp.scale, stream)

    for _ in range(max(1, args.warmup)):
        run()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in events:
        e[0].record(stream)
        run()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    tf = 4.0 * wp.B * wp.Hq * wp.N * wp.N * wp.d / 2.0 / (ms * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "ms": round(ms, 4),
            "roofline": {"kernel": "attn_fwd_kernel<bf16,128,causal,token-major>", "bound": "mfma",
                         "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": load_traffic("attn_fwd_kernel/qkvpacked")}}


def bench_varlen(args, torch, np, ea, wl, dev, stream):
    """A packed causal prefill batch with the llm_prefill token budget (8192 tokens,
    Hq = Hkv = 32, d = 128, bf16) split into sequences of seeded lengths
    U[256, 4096]; TFLOP/s with the metric's convention, 4*H*N_b^2*d/2 per
    sequence. Timed in a loop of its own after the steps."""
    print("bench: packed variable-length prefill", file=sys.stderr, flush=True)
    lens = wl.varlen_lengths(VARLEN_TOKENS, VARLEN_MIN, VARLEN_MAX, seed=1)
    q, k, v, cq, ck = wl.varlen_inputs(lens, lens, 32, 32, 128, "bf16", seed=1)
    q, k, v, cq, ck = (t.to(dev) for t in (q, k, v, cq, ck))
    o = torch.empty_like(q)
    lse = torch.empty((32, q.shape[0]), dtype=torch.float32, device=dev)
    scale = 1.0 / 128 ** 0.5

    def run():
        ea.attn_fwd_varlen(q, k, v, o, lse, cq, ck, max(lens), True, scale, stream)

    for _ in range(max(1, args.warmup)):
        run()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in events:
        e[0].record(stream)
        run()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    flops = float(sum(4.0 * 32 * n * n * 128 / 2.0 for n in lens))
    tf = flops / (ms * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "ms": round(ms, 4),
            "seq_lens": lens,
            "roofline": {"kernel": "attn_fwd_kernel<bf16,128,causal,varlen>", "bound": "mfma",
                         "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": load_traffic("attn_fwd_kernel/varlen")}}


def bench_paged(args, torch, np, ea, wl, wd, sl, dq, sld, kc, vc, stream):
    """The decode workload laid out in PAGE_SIZE-row pages of a shuffled pool
    (block table per sequence): split-KV decode over the paged cache, timed like
    the contiguous one but outside the step."""
    print("bench: paged decode (page %d)" % PAGE_SIZE, file=sys.stderr, flush=True)
    kp, vp, table = wl.paged_from_padded(kc, vc, sl, PAGE_SIZE, seed=wd.seed)
    td = table.to(kc.device)
    bufs = ea.decode_buffers(dq, table.shape[1] * PAGE_SIZE, wd.chunk)

    def run(ev=None):
        if ev is not None:
            ev[0].record(stream)
        ea.attn_decode_split_paged(dq, kp, vp, td, sld, bufs[0], bufs[1], wd.chunk, wd.scale,
                                   stream)
        if ev is not None:
            ev[1].record(stream)
        ea.attn_decode_combine(bufs[0], bufs[1], sld, bufs[2], bufs[3], wd.chunk, stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(max(1, args.warmup)):
        run()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        run(events[i])
    torch.cuda.synchronize()
    split_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    comb_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    lens = sl.numpy().astype(np.int64)
    kv_bytes = float(np.sum(2 * wd.Hkv * lens * wd.d * 2))
    gbs = kv_bytes / ((split_ms + comb_ms) * 1e-3) / 1e9
    del kp, vp
    return {"value": round(gbs, 1), "unit": "GB/s", "page_size": PAGE_SIZE,
            "split_ms": round(split_ms, 4), "combine_ms": round(comb_ms, 4),
            "roofline": {"kernel": "attn_decode_split_kernel<bf16,128,paged>", "bound": "hbm",
                         "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": load_traffic("attn_decode_split_kernel/decode_paged")}}


def bench_decode_fused(args, torch, np, ea, wl, wd, sl, dq, sld, kc, vc, stream, paged):
    """The decode workload at its 512-key chunks with the combine fused into the
    split kernel (one launch, no separate combine), contiguous or paged (64-row
    pages of a shuffled pool). Timed in a loop of its own."""
    print("bench: fused decode%s" % (" (paged)" if paged else ""), file=sys.stderr, flush=True)
    B, Hq, d = dq.shape
    o = torch.empty((B, Hq, d), dtype=dq.dtype, device=dq.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dq.device)
    if paged:
        kp, vp, table = wl.paged_from_padded(kc, vc, sl, PAGE_SIZE, seed=wd.seed)
        td = table.to(kc.device)
        ws = ea.fused_workspace(B, Hq, kc.shape[1], table.shape[1] * PAGE_SIZE, d, wd.chunk,
                                dq.device)

        def run():
            ea.attn_decode_fused_paged(dq, kp, vp, td, sld, o, lse, ws, wd.chunk, wd.scale,
                                       stream)
    else:
        ws = ea.fused_workspace(B, Hq, kc.shape[1], kc.shape[2], d, wd.chunk, dq.device)

        def run():
            ea.attn_decode_fused(dq, kc, vc, sld, o, lse, ws, wd.chunk, wd.scale, stream)

    for _ in range(max(1, args.warmup)):
        run()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in events:
        e[0].record(stream)
        run()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    lens = sl.numpy().astype(np.int64)
    kv_bytes = float(np.sum(2 * wd.Hkv * lens * wd.d * 2))
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    kern = "attn_decode_split_kernel<bf16,128,%sfused>" % ("paged," if paged else "")
    return {"value": round(gbs, 1), "unit": "GB/s", "ms": round(ms, 4), "chunk": wd.chunk,
            "roofline": {"kernel": kern, "bound": "hbm", "achieved": round(gbs, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": load_traffic("attn_decode_split_kernel/decode_fused"
                                                 + ("_paged" if paged else ""))}}


def bench_tiny(args, torch, np, ea, wl, dev, stream):
    """The tiny fp16 workload, causal and not: microseconds per forward (events
    around a loop of back-to-back calls; launch-bound, no roofline claim)."""
    print("bench: tiny workload", file=sys.stderr, flush=True)
    w = wl.WORKLOADS["tiny"]
    q, k, v = (t.to(dev) for t in wl.workload_prefill_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    out = {"unit": "us", "shape": {"B": w.B, "H": w.Hq, "N": w.N, "d": w.d, "dtype": "fp16"}}
    for causal in (False, True):
        for _ in range(50):
            ea.attn_fwd(q, k, v, o, lse, causal, w.scale, stream)
        torch.cuda.synchronize()
        reps = 200
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            ea.attn_fwd(q, k, v, o, lse, causal, w.scale, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        out["causal_us" if causal else "non_causal_us"] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
    return out


def run_only(args, torch, np, ea, wl, wp, wd, dev):
    """One measurement alone (bench.py --only NAME), for counter runs: the
    kernels of that measurement only, so that each profiled dispatch belongs
    to one workload."""
    stream = torch.cuda.current_stream()
    name = args.only
    if name in ("fwd_gqa_prefill", "fwd_long_context"):
        return {name: bench_fwd_workload(args, torch, np, ea, wl, name[4:], dev, stream)}
    if name == "fwd_qkvpacked":
        return {name: bench_qkvpacked(args, torch, np, ea, wp, stream)}
    if name == "fwd_varlen":
        return {name: bench_varlen(args, torch, np, ea, wl, dev, stream)}
    if name in ("bwd", "bwd_ds", "fwd_local"):
        q, k, v = (t.to(dev) for t in wl.workload_prefill_inputs(wp))
        if name == "fwd_local":
            return {name: bench_local(args, torch, np, ea, wp, q, k, v, stream)}
        o, lse = ea.fwd(q, k, v, causal=True, scale=wp.scale)
        return {name: bench_bwd(args, torch, np, ea, wp, q, k, v, o, lse, stream,
                                stored_ds=(name == "bwd_ds"))}
    sl, dq, kc, vc = wl.workload_decode_inputs(wd, device=dev)
    dq, sld = dq.to(dev), sl.to(dev)
    if name == "decode_auto":
        return {name: bench_decode_auto(args, torch, np, ea, wd, sl, dq, sld, kc, vc, stream)}
    return {name: bench_decode_fused(args, torch, np, ea, wl, wd, sl, dq, sld, kc, vc, stream,
                                     paged=(name == "decode_fused_paged"))}


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_attention_46_amd as ea
    from exact_attention_46_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ea.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wp = wl.WORKLOADS["llm_prefill"]
    wd = wl.WORKLOADS["decode"]
    if args.only in ONLY_EXTRA:
        res = run_only(args, torch, np, ea, wl, wp, wd, dev)
        if args.copy_calibration:
            copy_calibration(torch, dev)
        print(json.dumps(res), flush=True)
        return
    do_pre = args.only in ("all", "prefill")
    do_dec = args.only in ("all", "decode")

    print("bench: generating inputs", file=sys.stderr, flush=True)
    q, k, v = wl.workload_prefill_inputs(wp)
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    og = torch.empty_like(qg)
    lseg = torch.empty((wp.B, wp.Hq, wp.N), dtype=torch.float32, device=dev)

    sl, dq, kc, vc = (None,) * 4
    if do_dec:
        sl, dq, kc, vc = wl.workload_decode_inputs(wd, device=dev)
        dq, sld = dq.to(dev), sl.to(dev)
        bufs = ea.decode_buffers(dq, wd.l_max, wd.chunk)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if do_pre:
            ea.attn_fwd(qg, kg, vg, og, lseg, True, wp.scale, stream)
        if ev is not None:
            ev[1].record(stream)
        if do_dec:
            ea.attn_decode_split(dq, kc, vc, sld, bufs[0], bufs[1], wd.chunk, wd.scale, stream)
            if ev is not None:
                ev[2].record(stream)
            ea.attn_decode_combine(bufs[0], bufs[1], sld, bufs[2], bufs[3], wd.chunk, stream)
        elif ev is not None:
            ev[2].record(stream)
        if ev is not None:
            ev[3].record(stream)

    print("bench: warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print("bench: timed %d steps in %.3f s" % (args.steps, wall), file=sys.stderr, flush=True)

    if args.copy_calibration:
        copy_calibration(torch, dev)

    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    split_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    comb_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in events]))

    flops = 4.0 * wp.B * wp.Hq * wp.N * wp.N * wp.d / 2.0
    tflops = flops / (fwd_ms * 1e-3) / 1e12 if do_pre else None
    out = {
        "metric": METRIC,
        "value": round(tflops, 2) if tflops else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded randn inputs, no dataset)",
        "config": {"workload": "llm_prefill: B=4 Hq=Hkv=32 Nq=Nk=2048 d=128 bf16 causal, "
                               "then decode: 64 seqs Hq=32 Hkv=8 d=128 bf16 "
                               "L~U[512,32768] chunk=512",
                   "fwd_ms": round(fwd_ms, 4)},
    }
    if do_pre:
        traffic = load_traffic("attn_fwd_kernel/llm_prefill")
        out["roofline"] = {"kernel": "attn_fwd_kernel<bf16,128,causal>", "bound": "mfma",
                           "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                           "traffic": traffic,
                           "algorithmic_bytes": 4 * wp.B * wp.Hq * wp.N * wp.d * 2
                           + wp.B * wp.Hq * wp.N * 4}
    if do_dec:
        lens = sl.numpy().astype(np.int64)
        kv_bytes = float(np.sum(2 * wd.Hkv * lens * wd.d * 2))
        dec_ms = split_ms + comb_ms
        gbs = kv_bytes / (dec_ms * 1e-3) / 1e9
        # every byte the two kernels must move: K/V, q, the partials (O fp32 + LSE of each
        # valid chunk and query head, written then read), O and LSE
        chunks = float(np.sum(-(-lens // wd.chunk)))
        part = chunks * wd.Hq * (wd.d + 1) * 4
        total_bytes = kv_bytes + dq.numel() * 2 + 2 * part + wd.B * wd.Hq * (wd.d * 2 + 4)
        out["decode"] = {"value": round(gbs, 1), "unit": "GB/s", "split_ms": round(split_ms, 4),
                         "combine_ms": round(comb_ms, 4),
                         "split_only_GBs": round(kv_bytes / (split_ms * 1e-3) / 1e9, 1),
                         "kv_bytes": int(kv_bytes),
                         "total_bytes": int(total_bytes),
                         "total_GBs": round(total_bytes / (dec_ms * 1e-3) / 1e9, 1),
                         "roofline": {"kernel": "attn_decode_split_kernel<bf16,128>",
                                      "bound": "hbm", "achieved": round(gbs, 1),
                                      "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": round(gbs / PEAK_HBM_GBS, 4),
                                      "traffic": load_traffic("attn_decode_split_kernel/decode")}}
    if do_pre and not args.no_bwd:
        out["bwd"] = bench_bwd(args, torch, np, ea, wp, qg, kg, vg, og, lseg, stream)
        out["bwd_ds"] = bench_bwd(args, torch, np, ea, wp, qg, kg, vg, og, lseg, stream,
                                  stored_ds=True)
    if do_pre and not args.no_local:
        out["fwd_local"] = bench_local(args, torch, np, ea, wp, qg, kg, vg, stream)
    if do_pre and not args.no_qkv:
        out["fwd_qkvpacked"] = bench_qkvpacked(args, torch, np, ea, wp, stream)
    if do_pre and not args.no_varlen:
        out["fwd_varlen"] = bench_varlen(args, torch, np, ea, wl, dev, stream)
    if do_pre and not args.no_configs:
        out["fwd_gqa_prefill"] = bench_fwd_workload(args, torch, np, ea, wl, "gqa_prefill", dev,
                                                    stream)
        out["fwd_long_context"] = bench_fwd_workload(args, torch, np, ea, wl, "long_context",
                                                     dev, stream)
    if do_dec and not args.no_auto:
        out["decode_auto"] = bench_decode_auto(args, torch, np, ea, wd, sl, dq, sld, kc, vc,
                                               stream)
    if do_dec and not args.no_paged:
        out["decode_paged"] = bench_paged(args, torch, np, ea, wl, wd, sl, dq, sld, kc, vc,
                                          stream)
    if do_dec and not args.no_fused:
        out["decode_fused"] = bench_decode_fused(args, torch, np, ea, wl, wd, sl, dq, sld, kc, vc,
                                                 stream, paged=False)
        if not args.no_paged:
            out["decode_fused_paged"] = bench_decode_fused(args, torch, np, ea, wl, wd, sl, dq,
                                                           sld, kc, vc, stream, paged=True)
    if do_pre and not args.no_configs:
        out["fwd_tiny"] = bench_tiny(args, torch, np, ea, wl, dev, stream)
    if not args.no_cpu_baseline and do_pre:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        cb = cpu_baseline(wp, q, k, v, args.cpu_seconds)
        cores = cb["cores"]
        cb["tiny"] = cpu_baseline_tiny(cores)
        if not args.no_configs:
            cb["gqa_prefill"] = cpu_baseline_subset("gqa_prefill", cores, 2048, 21)
            cb["long_context"] = cpu_baseline_subset("long_context", cores, 512, 22)
        if do_dec:
            cb["decode"] = cpu_baseline_decode(wd, sl, dq, kc, vc, cores)
        out["cpu_baseline"] = cb
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
