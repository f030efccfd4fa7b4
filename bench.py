#!/usr/bin/env python3
"""Benchmark one full absorbed-MLA decode step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
  mla_absorb_q (q_nope . W_UK, concat q_rope)  ->  mla_decode (split plan,
  split-KV attention against the latent cache, log-sum-exp combine)  ->
  mla_absorb_o (out . W_UV).
Default workload: DeepSeek-V2/V3-shaped decode, bf16, batch 64, 128 heads,
4096 cached tokens per sequence (latent cache [64, 4096, 576]).  That
configuration gives no projection weights; the absorb inputs (q_nope, q_rope,
W_UK, W_UV) are synthesized with the recipe of the end-to-end configuration.

Timing: W untimed warm-up steps, then exactly K timed steps.  Before each
timed step a 512 MiB buffer is read (outside the timed events) so the latent
cache cannot be served from the 4 MB L2s or the 256 MB Infinity Cache; the
eviction reads rather than writes so that no dirty lines are left whose
write-back the timed step would pay for.
HIP events on the library's stream bracket every step and, through the
library's profiling hook, the split-KV attention kernel alone.  The whole
timed loop is bracketed by torch.cuda.synchronize() on both sides.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA decode TFLOP/s + HBM GB/s (% of roofline), b=64 h=128 T=4096 bf16"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
D_C, D_R, D_QK, D_K, D_V = 512, 64, 576, 128, 128
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
# sources of the split-KV attention kernels: a traffic figure in TRAFFIC_FILE
# is only valid while the common files and its kernel's own file are unchanged
_CSRC = os.path.join(ROOT, "head_latent_attention_decode_amd", "csrc")
KERNEL_SRCS = [os.path.join(_CSRC, f) for f in ("bf16_common.h", "mla355_internal.h", "plan_build.h")]
FAMILY_SRCS = {"decode_wide_kernel": "decode_wide.hip", "decode_wide_causal_kernel": "decode_wide.hip",
               "decode_bf16_kernel": "decode_bf16.hip", "decode_pair_kernel": "decode_bf16.hip",
               "decode_colsplit_kernel": "decode_colsplit.hip", "decode_f32_kernel": "decode_f32.hip"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def work_counts(b, h, lens, elt=2, q_len=1):
    """Algorithmic FLOPs and bytes of each step stage.  With q_len causal query
    tokens per row, new token i of a row of L cached rows scores the first
    L - q_len + 1 + i of them; the cache is still read once per row."""
    sum_l = int(sum(lens))
    visible = sum(min(max(int(L) - q_len + 1 + i, 0), int(L)) for L in lens for i in range(q_len))
    nq = b * q_len  # query tokens
    dec_flop = 2 * (D_QK + D_C) * h * visible
    dec_bytes = sum_l * D_QK * elt + nq * h * (D_QK * elt + D_C * elt + 4)
    aq_flop = 2 * nq * h * D_K * D_C
    aq_bytes = nq * h * (D_K + D_R + D_QK) * elt + h * D_K * D_C * elt
    ao_flop = 2 * nq * h * D_C * D_V
    ao_bytes = nq * h * (D_C + D_V) * elt + h * D_C * D_V * elt
    return {"decode": (dec_flop, dec_bytes), "absorb_q": (aq_flop, aq_bytes),
            "absorb_o": (ao_flop, ao_bytes)}


class Hip:
    """Just enough of the HIP runtime (events) through ctypes."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, ctypes.c_void_p(stream.cuda_stream)) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)


def kernel_source_hash(kernel=None):
    """Hash of the code lines of the common kernel sources, plus the file of
    `kernel` (a name such as "decode_wide_kernel<4, 2, false>") if given."""
    h = hashlib.sha256()
    files = list(KERNEL_SRCS)
    if kernel is not None:
        files.append(os.path.join(_CSRC, FAMILY_SRCS[kernel.split("<")[0].strip()]))
    for path in files:
        with open(path) as f:
            for line in f:
                # code only: comments and blank lines do not change the kernel
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def load_traffic(workload, kernel, path=None):
    """HBM bytes per launch of `kernel` on `workload` from committed rocprofv3
    --pmc runs (TRAFFIC_FILE maps workload names to entries), valid only while
    the kernel's sources are unchanged since the counters were taken."""
    try:
        with open(path or TRAFFIC_FILE) as f:
            t = json.load(f).get(workload)
    except (OSError, ValueError, AttributeError):
        return None
    if not isinstance(t, dict) or t.get("kernel") != kernel:
        return None
    if t.get("kernel_source_sha") != kernel_source_hash(kernel):
        return None
    return t.get("hbm_bytes_per_launch")


def copy_bandwidth(torch, dev, hip, stream, nbytes=1 << 30):
    """Device-to-device copy of 1 GiB (context for the HBM figures): bytes
    read plus bytes written over the best of three copies, GB/s."""
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    best = None
    for _ in range(3):
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, stream)
        dst.copy_(src)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        t = hip.elapsed_ms(e0, e1)
        best = t if best is None else min(best, t)
    del src, dst
    return round(2 * nbytes / (best * 1e-3) / 1e9, 1)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(w, q_nope, q_rope, w_uk, w_uv, target_s=12.0, max_rows=None, q_len=1):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same
    workload: whole batch rows, all heads (and query tokens), absorb -> latent
    decode -> absorb."""
    import numpy as np
    import oracle
    orc = oracle.default()
    lens = w.seqlens.cpu().tolist()
    wk = w_uk.cpu()
    wv = w_uv.cpu()
    qn_all = q_nope.view(w.b, q_len, w.h, -1)
    qr_all = q_rope.view(w.b, q_len, w.h, -1)

    def run(rows):
        L = max(int(lens[r]) for r in rows)
        n = len(rows)
        qn = qn_all[rows].reshape(n * q_len, w.h, -1).cpu()
        qr = qr_all[rows].reshape(n * q_len, w.h, -1).cpu()
        c = w.cache[rows, :L].cpu()
        sl = np.array([lens[r] for r in rows], np.int32)
        cf = oracle._f64(c)  # widen outside the timed region
        t0 = time.perf_counter()
        qp = orc.absorb_q(qn, wk, qr)
        if q_len == 1:
            out, _ = orc.decode_latent(qp, cf, sl, w.scale)
        else:
            out, _ = orc.decode_latent_causal(qp.reshape(n, q_len, w.h, -1), cf, sl, w.scale)
        orc.absorb_o(out.reshape(n * q_len, w.h, -1), wv)
        dt = time.perf_counter() - t0
        cnt = work_counts(n, w.h, [lens[r] for r in rows], q_len=q_len)
        return dt, sum(f for f, _ in cnt.values())

    dt1, f1 = run([0])
    n = int(min(w.b if max_rows is None else max_rows, max(1, round(target_s / max(dt1, 1e-3)))))
    rows = list(range(n))
    dt, fl = run(rows)
    toks = "" if q_len == 1 else " x %d query tokens" % q_len
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": orc.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d of %d batch rows%s, all %d heads, %d cached tokens each: fp64 absorb_q -> "
                      "latent-form decode -> absorb_o, %.1f s" % (n, w.b, toks, w.h, lens[0], dt)}


PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o trace -- "
             "python3 bench.py --steps 10 --warmup 3 --no-cpu-baseline --no-context{cfg}",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR -o fetch -- "
             "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-context{cfg}",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR -o write -- "
             "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-context{cfg}",
    "cfetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR -o cfetch -- "
              "python3 bench.py --calibrate-copy 256",
    "cwrite": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR -o cwrite -- "
              "python3 bench.py --calibrate-copy 256",
}


def summarize_profiles(dirs, cid=2, out_dir=None):
    """Turn the five rocprofv3 runs of PROFILE_CMDS for configuration `cid`
    (output directories in that order) into the committed summaries:
    profiles/<kernel>_<workload>.md and the workload's entry of the traffic
    figures bench.py reports (profiles/decode_traffic.json).  Pure file
    processing, no GPU.  out_dir replaces profiles/ (tests)."""
    import csv
    import glob
    import workloads
    cfg = workloads.CONFIGS[cid]
    workload = cfg.name
    lens = workloads.lengths(cid)
    cfg_arg = "" if cid == 2 else " --config %d" % cid

    def rows(d, suffix):
        files = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
        if not files:
            raise SystemExit("no *%s under %s" % (suffix, d))
        with open(files[0], newline="") as f:
            return list(csv.DictReader(f))

    def counter_means(d):
        acc = {}
        for r in rows(d, "counter_collection.csv"):
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])  # sum over XCD/SE instances
        per = {}
        for (name, _), v in acc.items():
            per.setdefault(name, []).append(v)
        return {n: sum(v) / len(v) for n, v in per.items()}

    stats = rows(dirs[0], "kernel_stats.csv")
    fetch, write = counter_means(dirs[1]), counter_means(dirs[2])
    cfetch, cwrite = counter_means(dirs[3]), counter_means(dirs[4])
    copy_kib = 256 * 1024.0
    cf = max((v for n, v in cfetch.items() if "copy" in n.lower()), default=None)
    cw = max((v for n, v in cwrite.items() if "copy" in n.lower()), default=None)
    if cf is None or cw is None:
        raise SystemExit("no copy kernel in the calibration runs")
    fs, ws_ = copy_kib / cf, copy_kib / cw
    dec = [n for n in fetch if "decode_" in n and "_kernel" in n]
    if len(dec) != 1:
        raise SystemExit("expected one attention kernel in the counter runs, got %s" % dec)
    dname = dec[0]
    import re
    short = re.search(r"decode_\w+(<[^>]*>)?", dname).group(0)
    family = short.split("<")[0]
    hbm = int(round((fetch[dname] * fs + write[dname] * ws_) * 1024))
    w = work_counts(cfg.b, cfg.h, lens, elt=cfg.dtype.itemsize)["decode"][1]
    traffic = {
        "kernel": short, "kernel_source_sha": kernel_source_hash(short), "workload": workload,
        "hbm_bytes_per_launch": hbm, "fetch_kib_per_launch": round(fetch[dname], 1),
        "write_kib_per_launch": round(write[dname], 1), "fetch_scale": round(fs, 4),
        "write_scale": round(ws_, 4),
        "calibration": "plain 256 MiB device copy (bench.py --calibrate-copy 256): FETCH_SIZE "
                       "%.1f KiB, WRITE_SIZE %.1f KiB per copy" % (cf, cw)}
    toks = ("%d cached tokens" % lens[0] if len(set(lens)) == 1 else
            "%d to %d cached tokens, %d in all" % (min(lens), max(lens), sum(lens)))
    lines = ["# %s on %s (%s, b=%d, h=%d, %s)" % (short, workload, str(cfg.dtype).split(".")[-1], cfg.b,
                                                  cfg.h, toks), "",
             "MI355X (gfx950), ROCm 7.2, one GPU.  Commands, run from the repository root with",
             "`export TMPDIR=/tmp` (DIR: any output directory), then this summary:", "", "```"]
    lines += [PROFILE_CMDS[k].replace("{cfg}", cfg_arg) for k in ("trace", "fetch", "write", "cfetch", "cwrite")]
    lines += ["python3 bench.py --summarize-profiles TRACE_DIR FETCH_DIR WRITE_DIR CFETCH_DIR CWRITE_DIR%s" % cfg_arg,
              "```", "", "## Kernel trace (`*_kernel_stats.csv`), durations in microseconds", "",
              "Calls include warm-up steps; `reduce_kernel` is the cache-evicting read of a",
              "512 MiB buffer between steps and `__amd_rocclr_fillBufferAligned` the zeroing",
              "that reduction does first (both outside the timed region).", "",
              "| kernel | calls | avg | min | max | % |", "|---|---|---|---|---|---|"]
    for r in stats:
        nm = r["Name"]
        nm = nm if len(nm) <= 90 else nm[:87] + "..."
        lines.append("| %s | %s | %.1f | %.1f | %.1f | %.2f |" % (
            nm.replace("|", "/"), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    lines += ["", "## HBM traffic per dispatch (`FETCH_SIZE`, `WRITE_SIZE`, KiB; mean over dispatches)", "",
              "Calibration: a plain 256 MiB device-to-device copy reads FETCH_SIZE %.1f KiB and" % cf,
              "WRITE_SIZE %.1f KiB, so FETCH_SIZE is scaled by %.4f and WRITE_SIZE by %.4f to give bytes." % (cw, fs, ws_),
              "", "| kernel | FETCH_SIZE | WRITE_SIZE | HBM MB (scaled) |", "|---|---|---|---|"]
    for n in fetch:
        if "mla355" not in n:
            continue
        nm = n if len(n) <= 90 else n[:87] + "..."
        lines.append("| %s | %.1f | %.1f | %.1f |" % (nm, fetch[n], write.get(n, 0.0),
                                                      (fetch[n] * fs + write.get(n, 0.0) * ws_) * 1024 / 1e6))
    lines += ["", "Algorithmic bytes of one attention launch: %.1f MB (latent cache, queries," % (w / 1e6),
              "outputs and lse).  Measured %.1f MB; the difference is mostly the split-KV" % (hbm / 1e6),
              "partials (written here, read back by the combine kernel)."]
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    traffic_file = os.path.join(out_dir, os.path.basename(TRAFFIC_FILE))
    os.makedirs(out_dir, exist_ok=True)
    md = os.path.join(out_dir, "%s_%s.md" % (family, workload))
    with open(md, "w") as f:
        f.write("\n".join(lines) + "\n")
    try:
        with open(traffic_file) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    if not isinstance(table, dict) or "kernel" in table:
        table = {}
    table[workload] = traffic
    with open(traffic_file, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(md)
    print(traffic_file)


def bench_append(args, torch, mla, workloads, dev):
    """Time mla_cache_append alone: b rows of hidden width d_model projected to
    [x W_DKV ; RoPE(x W_KR)] and written at row t_max - 1 of the config's cache."""
    import numpy as np
    cfg = workloads.CONFIGS[args.config]
    w = workloads.make(args.config, device="cuda", poison=False)
    d_model = args.append
    g = torch.Generator().manual_seed(4243)
    x = torch.randn(w.b, d_model, generator=g).to(torch.bfloat16).to(dev)
    wd = (torch.randn(d_model, D_C, generator=g) / d_model ** 0.5).to(torch.bfloat16).to(dev)
    wr = (torch.randn(d_model, D_R, generator=g) / d_model ** 0.5).to(torch.bfloat16).to(dev)
    ang = np.arange(w.t_max)[:, None] * 10000.0 ** (-np.arange(D_R // 2)[None, :] / (D_R // 2))
    cos_t = torch.from_numpy(np.cos(ang).astype(np.float32)).to(dev)
    sin_t = torch.from_numpy(np.sin(ang).astype(np.float32)).to(dev)
    pos = torch.full((w.b,), w.t_max - 1, dtype=torch.int32, device=dev)
    ws = torch.empty(mla.mla_cache_append_workspace_bytes(w.b, d_model), dtype=torch.uint8, device=dev)
    flush = None if args.no_flush else torch.ones(128 << 20, dtype=torch.float32, device=dev)
    hip = Hip()
    stream = torch.cuda.current_stream()
    K, W = args.steps, args.warmup
    ev = [[hip.event() for _ in range(2)] for _ in range(K)]

    def step():
        mla.mla_cache_append(x, wd, wr, cos_t, sin_t, w.cache, pos, workspace=ws)

    for _ in range(W):
        if flush is not None:
            flush.sum()
        step()
    torch.cuda.synchronize()
    for i in range(K):
        if flush is not None:
            flush.sum()
        hip.record(ev[i][0], stream)
        step()
        hip.record(ev[i][1], stream)
    torch.cuda.synchronize()
    ms = sum(hip.elapsed_ms(e[0], e[1]) for e in ev) / K
    flop = 2 * w.b * d_model * D_QK
    byts = d_model * D_QK * 2 + w.b * d_model * 2 + w.b * (D_QK * 2 + 4)  # weights, x, rows
    gbs = byts / (ms * 1e-3) / 1e9
    res = {"metric": "MLA cache append GB/s (% of roofline)", "value": round(gbs, 1), "unit": "GB/s",
           "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": cfg.name + "_append_d%d" % d_model, "batch": w.b, "d_model": d_model,
                      "step": "mla_cache_append (projection, RoPE, row write)",
                      "cache_evicted_between_steps": flush is not None},
           "roofline": {"kernel": "append_proj_kernel + append_finish_kernel", "bound": "hbm",
                        "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                        "launch_us": round(ms * 1e3, 2), "alg_bytes_per_launch": byts},
           "mfma": {"achieved": round(flop / (ms * 1e-3) / 1e12, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "alg_flop_per_launch": flop}}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload configuration (1..5)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true", help="do not evict caches between steps")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context measurements (back-to-back steps, engine clock, device "
                         "copy), so that a profiled run holds only evicted-cache launches")
    ap.add_argument("--n-chunks", type=int, default=0)
    ap.add_argument("--hpg", type=int, default=0, help="heads per workgroup (0 = auto)")
    ap.add_argument("--variant", type=int, default=0)
    ap.add_argument("--fp8", action="store_true",
                    help="quantise the cache to per-token e4m3 (outside the timed region) and "
                         "decode it with mla_decode_fp8")
    ap.add_argument("--paged", type=int, default=0, metavar="BLOCK",
                    help="read the cache through a paged pool of BLOCK-token blocks (shuffled "
                         "block table) with mla_decode_paged")
    ap.add_argument("--q-len", type=int, default=1, metavar="N",
                    help="N causal query tokens per batch row (the last N cached rows), decoded "
                         "with mla_decode_mtp")
    ap.add_argument("--append", type=int, default=0, metavar="D_MODEL",
                    help="time mla_cache_append alone (hidden width D_MODEL, one new row per batch "
                         "row of the configuration) instead of the decode step")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (three times) and exit: "
                         "the reference for scaling HBM traffic counters")
    ap.add_argument("--print-source-hash", action="store_true",
                    help="print the hash of the attention kernel's sources and exit")
    ap.add_argument("--summarize-profiles", nargs=5, metavar="DIR",
                    help="write the profile summaries under profiles/ from the output directories "
                         "of the five rocprofv3 runs (trace, fetch, write, copy fetch, copy write) "
                         "and exit (no GPU needed)")
    args = ap.parse_args()
    if args.print_source_hash:
        print(kernel_source_hash("decode_wide_kernel"))
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.config)
        return

    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(asked for --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import head_latent_attention_decode_amd as mla
    import workloads

    torch.cuda.init()
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}), flush=True)
        return
    if args.append:
        bench_append(args, torch, mla, workloads, dev)
        return
    cfg = workloads.CONFIGS[args.config]
    t_setup = time.perf_counter()
    w = workloads.make(args.config, device="cuda", poison=False)
    if cfg.raw_query:
        q_nope, q_rope, w_uk, w_uv = w.q_nope, w.q_rope, w.w_uk, w.w_uv
    else:
        q_nope, q_rope, w_uk, w_uv = workloads.make_step_weights(w.b, w.h, dtype=w.dtype,
                                                                 device="cuda")
    lens = w.seqlens.cpu().tolist()
    sched = {}
    if args.n_chunks:
        sched["n_chunks"] = args.n_chunks
    if args.hpg:
        sched["heads_per_group"] = args.hpg
    if args.variant:
        sched["variant"] = args.variant
    bufs = mla.alloc_step(w.b, w.h, w.t_max, w.dtype, config=sched or None)
    pool = block_table = None
    codes = scales = None
    if args.fp8 and args.paged:
        print("--fp8 and --paged cannot be combined", file=sys.stderr)
        sys.exit(2)
    q_len = args.q_len
    mtp = None
    if q_len > 1:
        if args.fp8 or args.paged or args.hpg or args.variant:
            print("--q-len takes neither --fp8, --paged, --hpg nor --variant", file=sys.stderr)
            sys.exit(2)
        # q-side tensors for b * q_len query tokens (same heads and weights)
        q_nope, q_rope, w_uk, w_uv = workloads.make_step_weights(w.b * q_len, w.h, dtype=w.dtype,
                                                                 device="cuda")
        mtp = {"q_prime": torch.empty((w.b * q_len, w.h, D_QK), dtype=w.dtype, device=dev),
               "out": torch.empty((w.b, q_len, w.h, D_C), dtype=w.dtype, device=dev),
               "lse": torch.empty((w.b, q_len, w.h), dtype=torch.float32, device=dev),
               "y": torch.empty((w.b * q_len, w.h, D_V), dtype=w.dtype, device=dev),
               "ws": torch.empty(mla.mla_decode_mtp_workspace_bytes(w.b, q_len, w.h, w.t_max,
                                                                   sched or None),
                                 dtype=torch.uint8, device=dev)}
    if args.fp8:
        codes, scales = mla.mla_quantize_cache_fp8(w.cache)
        need = mla.mla_decode_fp8_workspace_bytes(w.b, w.h, w.t_max, sched or None)
        bufs.workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if args.paged:
        # every row's cache rows scattered over a seeded random permutation of blocks
        bs = args.paged
        mb = -(-w.t_max // bs)
        g = torch.Generator().manual_seed(4242)
        perm = torch.randperm(w.b * mb, generator=g).reshape(w.b, mb)
        pool = torch.zeros((w.b * mb, bs, D_QK), dtype=w.dtype, device=dev)
        padded = torch.zeros((w.b, mb * bs, D_QK), dtype=w.dtype, device=dev)
        padded[:, : w.t_max] = w.cache
        pool[perm.reshape(-1).to(dev)] = padded.reshape(w.b * mb, bs, D_QK)
        del padded
        block_table = perm.to(torch.int32).to(dev)
        need = mla.mla_decode_paged_workspace_bytes(w.b, w.h, pool.shape[0], bs, mb, sched or None)
        bufs.workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    # Cache eviction between steps: READ a 512 MiB buffer (more than the 4 MB
    # L2s plus the 256 MB Infinity Cache).  Reading leaves only clean lines
    # behind; overwriting the buffer instead would leave ~256 MB of dirty lines
    # whose write-back the next step would pay for.
    flush = None if args.no_flush else torch.ones(128 << 20, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log("setup %.1f s: %s b=%d h=%d t_max=%d sum(L)=%d dtype=%s" %
        (time.perf_counter() - t_setup, cfg.name, w.b, w.h, w.t_max, sum(lens), w.dtype))

    hip = Hip()
    stream = torch.cuda.current_stream()
    K, W = args.steps, args.warmup
    ev = [[hip.event() for _ in range(4)] for _ in range(K)]

    def step(i=None, clock=False):
        c = dict(sched)
        if i is not None:
            c["profile_events"] = (ev[i][1].value, ev[i][2].value)
        if clock:
            c["record_clock"] = True
        if mtp is not None:
            mla.mla_absorb_q(q_nope, w_uk, q_rope, mtp["q_prime"])
            mla.mla_decode_mtp(mtp["q_prime"].view(w.b, q_len, w.h, D_QK), w.cache, w.seqlens,
                               w.scale, mtp["out"], mtp["lse"], mtp["ws"], config=c or None)
            mla.mla_absorb_o(mtp["out"].view(w.b * q_len, w.h, D_C), w_uv, mtp["y"])
        elif codes is not None:
            mla.mla_absorb_q(q_nope, w_uk, q_rope, bufs.q_prime)
            mla.mla_decode_fp8(bufs.q_prime, codes, scales, w.seqlens, w.scale, bufs.out, bufs.lse,
                               bufs.workspace, config=c or None)
            mla.mla_absorb_o(bufs.out, w_uv, bufs.y)
        elif pool is None:
            mla.mla_step(q_nope, q_rope, w_uk, w_uv, w.cache, w.seqlens, w.scale, bufs,
                         config=c or None)
        else:
            mla.mla_absorb_q(q_nope, w_uk, q_rope, bufs.q_prime)
            mla.mla_decode_paged(bufs.q_prime, pool, block_table, w.seqlens, w.scale, bufs.out,
                                 bufs.lse, bufs.workspace, config=c or None)
            mla.mla_absorb_o(bufs.out, w_uv, bufs.y)

    for _ in range(W):
        if flush is not None:
            flush.sum()
        step()
    torch.cuda.synchronize()
    # The K timed steps run as a caller would run them: events only at the
    # step boundaries.  Events recorded between the kernels of a step cost
    # 5-10 us per step on this platform, so the attention kernel is timed in a
    # second pass of K steps (same eviction) with events around it.
    t0 = time.perf_counter()
    for i in range(K):
        if flush is not None:
            flush.sum()
        hip.record(ev[i][0], stream)
        step()
        hip.record(ev[i][3], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [hip.elapsed_ms(e[0], e[3]) for e in ev]
    # the kernel pass: at least 50 launches for the median and minimum
    KK = max(K, 50)
    ev += [[hip.event() for _ in range(4)] for _ in range(KK - K)]
    for i in range(KK):
        if flush is not None:
            flush.sum()
        hip.record(ev[i][0], stream)
        step(i)
        hip.record(ev[i][3], stream)
    torch.cuda.synchronize()
    kern_ms = [hip.elapsed_ms(e[1], e[2]) for e in ev[:KK]]
    step_instr_ms = sum(hip.elapsed_ms(e[0], e[3]) for e in ev[:KK]) / KK

    # back-to-back steps (no eviction): context only; the engine clock is
    # sampled from the host (amdsmi) while a longer run of them executes
    b2b_ms = clock = copy_gbs = None
    if not args.no_context:
        torch.cuda.synchronize()
        b0, b1 = hip.event(), hip.event()
        hip.record(b0, stream)
        for _ in range(K):
            step()
        hip.record(b1, stream)
        torch.cuda.synchronize()
        b2b_ms = hip.elapsed_ms(b0, b1) / K
        # engine clock during the attention kernel, from its first
        # workgroup's stamps (shader clock against the 100 MHz real-time
        # counter), over 20 launches after cache eviction
        ws_t = mtp["ws"] if mtp is not None else bufs.workspace
        mhz = []
        for _ in range(20):
            if flush is not None:
                flush.sum()
            ws_t[-mla.CLOCK_BYTES:].zero_()
            step(clock=True)
            torch.cuda.synchronize()
            v = mla.read_clock_mhz(ws_t)
            if v is not None:
                mhz.append(v)
        clock = None if not mhz else {
            "median": round(statistics.median(mhz), 1), "min": round(min(mhz), 1), "max": round(max(mhz), 1),
            "launches": len(mhz),
            "source": "s_memtime / s_memrealtime of the attention kernel's workgroup 0, launches after "
                      "cache eviction"}
        copy_gbs = copy_bandwidth(torch, dev, hip, stream)

    cnt = work_counts(w.b, w.h, lens, elt=w.dtype.itemsize, q_len=q_len)
    if args.fp8:
        # the cache streams 576 code bytes + a 4-byte scale per token
        f, _ = cnt["decode"]
        cnt["decode"] = (f, int(sum(lens)) * (D_QK + 4) + w.b * w.h * (D_QK * 2 + D_C * 2 + 4))
    step_flop = sum(f for f, _ in cnt.values())
    step_bytes = sum(bb for _, bb in cnt.values())
    dec_flop, dec_bytes = cnt["decode"]
    ms = sum(step_ms) / K
    kms = sum(kern_ms) / len(kern_ms)
    value = step_flop / (ms * 1e-3) / 1e12
    k_gbs = dec_bytes / (kms * 1e-3) / 1e9
    k_tfl = dec_flop / (kms * 1e-3) / 1e12
    kname = (mla.mla_decode_paged_kernel_name(w.h, sched or None) if args.paged
             else mla.mla_decode_fp8_kernel_name(w.h, sched or None) if args.fp8
             else mla.mla_decode_mtp_kernel_name(q_len, w.h) if mtp is not None
             else mla.mla_decode_kernel_name(w.dtype, w.h, sched or None))
    traffic = None if (args.paged or args.fp8 or mtp is not None) else load_traffic(cfg.name, kname)
    # the roof the attention kernel meets first: HBM bytes or MFMA FLOPs
    mfma_bound = dec_flop / (MFMA_BF16_PEAK_TFLOPS * 1e12) > dec_bytes / (HBM_PEAK_GBS * 1e9)
    log("step: mean %.2f us (min %.2f, max %.2f); split-KV kernel mean %.2f us (min %.2f); "
        "back-to-back step %.2f us; wall %.3f s for %d steps" %
        (ms * 1e3, min(step_ms) * 1e3, max(step_ms) * 1e3, kms * 1e3, min(kern_ms) * 1e3,
         (b2b_ms or 0.0) * 1e3, wall, K))
    log("split-KV kernel: %.1f GB/s (%.1f%% of HBM), %.1f TFLOP/s (%.1f%% of bf16 MFMA)" %
        (k_gbs, 100 * k_gbs / HBM_PEAK_GBS, k_tfl, 100 * k_tfl / MFMA_BF16_PEAK_TFLOPS))

    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": w.b, "heads": w.h, "cached_tokens": w.t_max,
                   "sum_cached_tokens": int(sum(lens)), "d_latent": D_C, "d_rope": D_R,
                   "step": ("absorb_q + decode (plan, split-KV, combine) + absorb_o" if q_len == 1 else
                            "absorb_q + causal multi-token decode (plan, split-KV, combine) + absorb_o"),
                   "cache_evicted_between_steps": flush is not None,
                   "schedule": sched or "auto",
                   "cache_layout": ("paged, %d-token blocks, shuffled block table" % args.paged
                                    if args.paged else "contiguous"),
                   "cache_dtype": "e4m3 codes + fp32 per-token scale" if args.fp8 else str(w.dtype),
                   "query_tokens_per_row": q_len},
        "hbm_gbps_step": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "step_flop": step_flop,
        "step_bytes": step_bytes,
        "ms_per_step_back_to_back": None if b2b_ms is None else round(b2b_ms, 5),
        "ms_per_step_kernel_events": round(step_instr_ms, 5),
        "step_us": {"mean": round(ms * 1e3, 2), "median": round(statistics.median(step_ms) * 1e3, 2),
                    "min": round(min(step_ms) * 1e3, 2), "runs": K},
        "kernel_us": {"mean": round(kms * 1e3, 2), "median": round(statistics.median(kern_ms) * 1e3, 2),
                      "min": round(min(kern_ms) * 1e3, 2), "runs": len(kern_ms)},
        "engine_clock_mhz": clock,
        "copy_1gib_gbps": copy_gbs,
        "roofline": {"kernel": kname,
                     "bound": "hbm", "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "launch_us": round(kms * 1e3, 2),
                     "alg_bytes_per_launch": dec_bytes},
        "mfma": {"achieved": round(k_tfl, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(k_tfl / MFMA_BF16_PEAK_TFLOPS, 4), "alg_flop_per_launch": dec_flop},
    }
    if mfma_bound:
        # compute-bound shape: the roofline object reports the MFMA roof, the
        # byte rate moves to the secondary object
        r = res["roofline"]
        res["hbm"] = {k: r[k] for k in ("achieved", "peak", "unit", "frac", "alg_bytes_per_launch")}
        r.update({"bound": "mfma", "achieved": round(k_tfl, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                  "unit": "TFLOP/s", "frac": round(k_tfl / MFMA_BF16_PEAK_TFLOPS, 4),
                  "alg_flop_per_launch": dec_flop})
        del r["alg_bytes_per_launch"]
        del res["mfma"]
    if not args.no_cpu_baseline:
        t_c = time.perf_counter()
        res["cpu_baseline"] = cpu_baseline(w, q_nope, q_rope, w_uk, w_uv, q_len=q_len)
        log("cpu baseline %.1f s" % (time.perf_counter() - t_c))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
