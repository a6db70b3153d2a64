"""Benchmark of the FLARE forward hot path on one MI355X.

One step = one full pass of the operator over one batch of synthetic inputs
that are already resident in HBM: split-N encode -> combine -> decode (FLARE),
or the five-launch FLARE++ sequence, through the C ABI's caller-workspace
entry point. Default workload: the PDE-mesh shape B=4, H=8, N=65536, M=128,
D=32 in bf16 (the throughput metric is quoted on N=65536, M=128).

Before the warmup steps the step runs back to back for --ramp-seconds (untimed)
so that the GPU reaches its steady clocks; the timed region is always exactly
--steps full steps, back to back (hot: whatever the last-level caches still
hold of the previous step). Prints one JSON line with
  * throughput (tokens*heads/s) of the timed region;
  * the roofline position of the dominant kernel: its average duration over a
    second pass of the same steps, from HIP events that the library binds to
    each kernel's dispatch on the launch stream (hipExtLaunchKernel), i.e. the
    kernel's own execution time as a rocprofv3 kernel trace reports it;
  * a cold-cache pass (--cold-mib): each step timed on its own after a write
    that evicts the L2s and the Infinity Cache, with its own kernel durations;
  * the fp64 CPU oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
_BF16_SRC = ["rank_latent_attention_flare_amd/csrc/kernels_bf16.hip", "rank_latent_attention_flare_amd/csrc/gfx950_ops.h"]
_COMMON_SRC = ["rank_latent_attention_flare_amd/csrc/kernels_common.hip"]


def kernel_sources(kind: str, dtype: str = "bf16") -> list:
    """The sources that define a kernel kind for a storage type (the fp32
    encode and decode live with the combine)."""
    if kind == "combine" or dtype != "bf16":
        return _COMMON_SRC
    return _BF16_SRC


def source_hash(kind: str, dtype: str = "bf16") -> str:
    """Hash of the code (comments and blank space removed) of the sources that
    define a kernel: recorded with its hardware counters, so that counters taken
    on an older version of the kernel are not reported against the current one."""
    h = hashlib.sha256()
    for rel in kernel_sources(kind, dtype):
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def cpu_model() -> str:
    """The host CPU's model name (first processor entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def trace_summary(path: str, steps: int, cold: bool) -> str:
    """Markdown summary of a rocprofv3 kernel trace (kernel_trace.csv) of one
    default bench.py run: per kernel, the average duration over all launches
    and over each pass of the run, told apart by launch order. The passes, in
    order: the clock ramp and warmup, the timed region (back to back; each
    kernel's duration there includes the wait for the previous kernel's tail),
    the kernel pass (the durations bench.py reports: isolated kernels) and, if
    run, the cold pass. Each of the last three holds `steps` steps."""
    import csv
    import statistics
    rows = sorted(csv.DictReader(open(path, newline="")), key=lambda r: int(r["Start_Timestamp"]))
    by = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    passes = ["timed", "kernel pass"] + (["cold"] if cold else [])
    out = ["| kernel | launches | avg us (all) | " + " | ".join(f"avg us ({p})" for p in passes) + " |",
           "|---|---|---|" + "---|" * len(passes)]
    # kernels that run every step (copies, fills and the flush run far fewer
    # times); the least frequent of them runs once per step
    step_kernels = {k: d for k, d in by.items() if len(d) >= steps * len(passes)}
    once = min(len(d) for d in step_kernels.values())
    for name, d in sorted(step_kernels.items(), key=lambda kv: -sum(kv[1])):
        n = len(d)
        k = steps * round(n / once)
        cols = []
        for i in range(len(passes)):
            lo = n - (len(passes) - i) * k
            cols.append(f"{statistics.mean(d[lo:lo + k]):.2f}")
        short = name.replace("void ", "").replace("flare::(anonymous namespace)::", "").split("(")[0]
        out.append(f"| {short} | {n} | {statistics.mean(d):.2f} | " + " | ".join(cols) + " |")
    return "\n".join(out)


SQ_SETS = (
    "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_SALU SQ_INSTS_LDS SQ_WAVE_CYCLES "
    "SQ_BUSY_CYCLES",
    "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY SQ_VALU_MFMA_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_ANY "
    "SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_SCA SQ_ACTIVE_INST_MISC",
    "SQ_INSTS_VALU_FMA_F32 SQ_INSTS_VALU_CVT SQ_INSTS_VALU_MUL_F32 SQ_INSTS_VALU_ADD_F32 SQ_INSTS_VALU_INT32 "
    "SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT SQ_INSTS_BRANCH",
    "GRBM_GUI_ACTIVE GRBM_COUNT SQ_CYCLES SQ_BUSY_CU_CYCLES",
)


def sq_summary(paths: list, workload) -> str:
    """Markdown table of the SQ and GRBM counter passes (rocprofv3 --pmc with
    each of SQ_SETS, one run each, in that order) of this script on one
    workload: per kernel that works on score tiles (encodes, decodes and the
    backward's token and latent kernels), averages over all its dispatches of
      shader clock = GRBM_GUI_ACTIVE / 8 XCDs / duration,
      MFMA busy    = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8),
    instruction counts per 32x32 tile of scores (B*H*N*M/1024 per launch),
    and SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES."""
    import csv
    import statistics

    vals, names, dur = {}, {}, {}
    for path in paths:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                key = (path, r["Dispatch_Id"])
                names[key] = r["Kernel_Name"]
                c = vals.setdefault(key, {})
                c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                    dur[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    blocks = workload.B * workload.H * workload.N * workload.M / 1024.0
    per = {}  # kernel -> counter -> list of per-dispatch values
    for key, c in vals.items():
        short = names[key].replace("void ", "").replace("flare::(anonymous namespace)::", "").split("(")[0]
        if not any(t in short for t in ("encode_partial", "decode_", "bw_")) or "combine" in short:
            continue
        k = per.setdefault(short, {})
        for cn, v in c.items():
            k.setdefault(cn, []).append(v)
        if key in dur:
            k.setdefault("_us", []).append(dur[key])
    out = ["| kernel | avg us (counter runs) | shader clock GHz | MFMA busy | MFMA / block | VALU / block "
           "| of which exp, fma, cvt | LDS / block | LDS bank-conflict cycles / block "
           "| SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES |",
           "|---|---|---|---|---|---|---|---|---|---|"]

    def m(k, cn):
        return statistics.mean(k[cn]) if cn in k and k[cn] else float("nan")

    for short, k in sorted(per.items(), key=lambda kv: -m(kv[1], "GRBM_GUI_ACTIVE")):
        us = m(k, "_us")
        gui = m(k, "GRBM_GUI_ACTIVE")
        clock = gui / 8 / (us * 1e3) if us == us else float("nan")
        busy = m(k, "SQ_VALU_MFMA_BUSY_CYCLES") / (1024 * gui / 8)
        out.append(
            f"| {short} | {us:.1f} | {clock:.2f} | {100 * busy:.0f}% | {m(k, 'SQ_INSTS_MFMA') / blocks:.2f} "
            f"| {m(k, 'SQ_INSTS_VALU') / blocks:.1f} | {m(k, 'SQ_INSTS_VALU_TRANS_F32') / blocks:.1f}, "
            f"{m(k, 'SQ_INSTS_VALU_FMA_F32') / blocks:.1f}, {m(k, 'SQ_INSTS_VALU_CVT') / blocks:.1f} "
            f"| {m(k, 'SQ_INSTS_LDS') / blocks:.2f} | {m(k, 'SQ_LDS_BANK_CONFLICT') / blocks:.2f} "
            f"| {m(k, 'SQ_WAIT_INST_ANY') / m(k, 'SQ_WAVE_CYCLES'):.2f} |")
    return "\n".join(out)


def kernel_kind(name: str) -> str | None:
    """The library's kernel kind of a kernel symbol (None for other kernels)."""
    for kind, tag in (("encode_partial", "encode_partial"), ("decode", "decode_"), ("combine", "combine_kernel"),
                      ("copy", "copy_kernel")):
        if tag in name:
            return kind
    return None


def pmc_summary(fetch_csv: str, write_csv: str, workload, layout: str, variant: str, copy_mib: int,
                kernel_trace_csv: str | None, bench_args: str = "", trace_args: str = "") -> list:
    """HBM traffic per launch of the forward kernels from two rocprofv3 --pmc
    runs of bench.py (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch, with the
    arguments bench_args), each scaled so that the same counter over the
    library's plain copy kernel (copy_mib MiB each way, launched once before
    the timed steps) reads copy_mib MiB. The optional kernel trace (of a run
    with the arguments trace_args) gives each kernel's average duration.
    Returns one record per kernel kind (averages over all its dispatches),
    with the hash of its source."""
    import csv

    def per_dispatch(path: str, counter: str) -> dict:
        vals, names = {}, {}
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                d = r["Dispatch_Id"]
                vals[d] = vals.get(d, 0.0) + float(r["Counter_Value"])
                names[d] = r["Kernel_Name"]
        return {d: (names[d], v) for d, v in vals.items()}

    fetch, write = per_dispatch(fetch_csv, "FETCH_SIZE"), per_dispatch(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mib << 20

    def scale(table):
        c = [v for n, v in table.values() if kernel_kind(n) == "copy"]
        if not c:
            raise SystemExit("no copy-kernel dispatch in the counter run (run bench.py with --calib-copy-mib > 0)")
        return copy_bytes / (c[0] * 1024.0)

    fs, ws = scale(fetch), scale(write)
    dur = {}
    if kernel_trace_csv:
        with open(kernel_trace_csv, newline="") as f:
            for r in csv.DictReader(f):
                k = kernel_kind(r["Kernel_Name"])
                if k:
                    dur.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    e = 2 if workload.dtype == "bf16" else 4
    alg = {"encode_partial": 2 * workload.B * workload.H * workload.N * workload.D * e,
           "decode": 2 * workload.B * workload.H * workload.N * workload.D * e}
    out = []
    for kind in ("encode_partial", "combine", "decode"):
        fv = [(n, v) for n, v in fetch.values() if kernel_kind(n) == kind]
        wv = [v for n, v in write.values() if kernel_kind(n) == kind]
        if not fv or not wv:
            continue
        rd = sum(v for _, v in fv) / len(fv) * 1024.0 * fs
        wr = sum(wv) / len(wv) * 1024.0 * ws
        lay = ("" if layout == "bhnd" else "_bnhd") + ("" if variant == "flare" else "_" + variant)
        rec = {"kernel": kind,
               "kernel_symbol": fv[0][0].replace("void ", "").replace("flare::(anonymous namespace)::", "").split("(")[0],
               "workload": workload.name + lay, "source": kernel_sources(kind, workload.dtype),
               "source_hash": source_hash(kind, workload.dtype),
               "avg_duration_us": round(sum(dur[kind]) / len(dur[kind]), 2) if kind in dur else None,
               "launches": len(fv), "hbm_read_bytes_per_launch": int(rd), "hbm_write_bytes_per_launch": int(wr),
               "hbm_bytes_per_launch": int(rd + wr), "alg_bytes_per_launch": alg.get(kind),
               "calibration": {"copy_bytes": copy_bytes, "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)},
               "commands": [f"rocprofv3 --pmc {c} -d <out> -o {o} --output-format csv -- python3 bench.py {bench_args}"
                            for c, o in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write"))]
               + ([f"rocprofv3 --kernel-trace --stats -d <out> -o kt --output-format csv -- python3 bench.py "
                   f"{trace_args or bench_args}"] if kernel_trace_csv else [])}
        out.append(rec)
    return out


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", type=int, default=2, help="workload number 1-7 (default 2)")
    p.add_argument("--variant", choices=["flare", "skill", "backward"], default="flare",
                   help="flare: the workload's forward (default); skill: the FLARE skill page's layer, "
                        "flare_encode then flare_attend with separate token queries (FLARE forward workloads only); "
                        "backward: the gradients of Q, K, V (flare_backward, or flare_pp_backward on the "
                        "FLARE++ workload)")
    p.add_argument("--layout", choices=["bhnd", "bnhd"], default="bhnd",
                   help="layout of K, V and Y: [B,H,N,D] (default) or token-major [B,N,H,D]")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true", help="time one replay of a HIP graph holding the K steps")
    p.add_argument("--no-events", action="store_true",
                   help="skip the second pass that times every kernel with HIP events")
    p.add_argument("--cold-mib", type=int, default=1024,
                   help="cold-cache pass: write this many MiB between individually timed steps, which evicts the "
                        "L2s and the 256 MB Infinity Cache, and report it beside the back-to-back (hot) figures; "
                        "0 skips the pass")
    p.add_argument("--cold-flush", choices=["read", "write"], default="read",
                   help="how the cold pass evicts the caches: read the flush buffer (default) or write it")
    p.add_argument("--calib-copy-mib", type=int, default=512,
                   help="size of the plain copy kernel run once before the timed steps (counter calibration)")
    p.add_argument("--no-calibrate", action="store_true",
                   help="skip the in-run peak calibration (a timed copy and the MFMA and exp probes)")
    p.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                   help="print the per-pass kernel summary of a rocprofv3 kernel trace of a default run of this "
                        "script with the same --steps and --cold-mib, and exit")
    p.add_argument("--pmc-summary", nargs="+", metavar="CSV",
                   help="FETCH_CSV WRITE_CSV [KERNEL_TRACE_CSV]: write profiles/<kernel>_<workload>_pmc.json (the "
                        "traffic the roofline reports) from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE runs of "
                        "this script with the same --workload, --layout, --variant, --steps, --warmup and "
                        "--ramp-seconds (the kernel trace: of a run with the same --workload, --layout and --variant "
                        "and the default steps), and exit")
    p.add_argument("--sq-summary", nargs=4, metavar="CSV",
                   help="print the SQ/GRBM counter table from four rocprofv3 --pmc runs of this script with the "
                        "counter sets of SQ_SETS, in order, on the same --workload, and exit")
    p.add_argument("--ramp-seconds", type=float, default=1.0,
                   help="run the step back to back for this long before the warmup steps, so that the GPU "
                        "reaches its steady clocks (a cold MI355X needs ~0.1-0.2 s); 0 disables")
    return p.parse_args()


def main():
    args = parse()
    if args.pmc_summary:
        from flare_inputs import WORKLOADS
        if len(args.pmc_summary) not in (2, 3):
            raise SystemExit("--pmc-summary takes FETCH_CSV WRITE_CSV [KERNEL_TRACE_CSV]")
        w = WORKLOADS[args.workload]
        bench_args = f"--workload {args.workload} --no-cpu-baseline" + \
            ("" if args.layout == "bhnd" else f" --layout {args.layout}") + \
            ("" if args.variant == "flare" else f" --variant {args.variant}") + \
            ("" if args.steps == 200 else f" --steps {args.steps}") + \
            ("" if args.warmup == 20 else f" --warmup {args.warmup}") + \
            ("" if args.ramp_seconds == 1.0 else f" --ramp-seconds {args.ramp_seconds:g}")
        trace_args = f"--workload {args.workload} --no-cpu-baseline" + \
            ("" if args.layout == "bhnd" else f" --layout {args.layout}") + \
            ("" if args.variant == "flare" else f" --variant {args.variant}")
        recs = pmc_summary(args.pmc_summary[0], args.pmc_summary[1], w, args.layout, args.variant,
                           args.calib_copy_mib, args.pmc_summary[2] if len(args.pmc_summary) == 3 else None,
                           bench_args, trace_args)
        for rec in recs:
            path = os.path.join(ROOT, "profiles", f"{rec['kernel']}_{rec['workload']}_pmc.json")
            with open(path, "w") as f:
                json.dump(rec, f, indent=1)
                f.write("\n")
            print(path, rec["hbm_bytes_per_launch"], rec["alg_bytes_per_launch"])
        return
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.steps, args.cold_mib > 0))
        return
    if args.sq_summary:
        from flare_inputs import WORKLOADS
        print(sq_summary(args.sq_summary, WORKLOADS[args.workload]))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); multi-GPU runs are not part of this "
              "build: the kernels shard by (batch, head) or by tokens, see the design notes.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from flare_inputs import WORKLOADS, recipe, workload_inputs
    from rank_latent_attention_flare_amd import flare as F

    if not os.path.exists(F.LIB_PATH):
        from rank_latent_attention_flare_amd.build import build
        build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    w = WORKLOADS[args.workload]
    op = F.FLARE_OP_PP_FORWARD if w.op == "pp_forward" else F.FLARE_OP_FORWARD
    fn = F.flare_pp_forward if op == F.FLARE_OP_PP_FORWARD else F.flare_forward
    if args.layout == "bnhd":
        fn_ex = F.flare_pp_forward_ex if op == F.FLARE_OP_PP_FORWARD else F.flare_forward_ex

        def fn(Q, K, V, out=None, workspace=None, stream=None):
            return fn_ex(Q, K, V, F.FLARE_LAYOUT_BNHD, out=out, workspace=workspace, stream=stream)

    Qh, Kh, Vh = workload_inputs(w)

    def dev(a):
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
        return t.view(torch.bfloat16) if a.dtype == np.uint16 else t

    Q, K, V = dev(Qh), dev(Kh), dev(Vh)
    ws = F.workspace_for(op, Q, K)
    if args.variant == "skill" and op != F.FLARE_OP_FORWARD:
        print(f"--variant {args.variant} needs a FLARE forward workload", file=sys.stderr)
        sys.exit(2)
    if args.variant == "backward":
        # the backward of the workload's operator: flare_backward, or
        # flare_pp_backward on the FLARE++ workload (their _ex forms in the
        # token-major layout)
        pp = op == F.FLARE_OP_PP_FORWARD
        bw_op = F.FLARE_OP_PP_BACKWARD if pp else F.FLARE_OP_BACKWARD
        bw_fn = F.flare_pp_backward if pp else F.flare_backward
        bw_ex = F.flare_pp_backward_ex if pp else F.flare_backward_ex
        ws = torch.empty(F.flare_workspace_size(bw_op, w.B, w.H, w.N, w.M, w.D, Q.dtype),
                         dtype=torch.uint8, device=Q.device)
        dYt = V.flip(2).contiguous()  # upstream gradient: the values in reverse token order
        if args.layout == "bnhd":
            dYt = dYt.transpose(1, 2).contiguous()
        grads = None

        def fn(Q, K, V, out=None, workspace=None, stream=None):
            nonlocal grads
            if grads is None:
                grads = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))
            if args.layout == "bnhd":
                bw_ex(Q, K, V, dYt, F.FLARE_LAYOUT_BNHD, stream=stream, workspace=workspace, out=grads)
            else:
                bw_fn(Q, K, V, dYt, stream=stream, workspace=workspace, out=grads)
            return grads[1]
    if args.variant == "skill":
        ws = F.workspace_for(F.FLARE_OP_ENCODE, Q, K)
        qtok = V.flip(2).contiguous()  # separate token queries: the values in reverse token order
        Zlat = torch.empty((w.B, w.H, w.M, w.D), dtype=Q.dtype, device=Q.device)
    if args.layout == "bnhd":  # token-major copies, made before any timing
        K, V = K.transpose(1, 2).contiguous(), V.transpose(1, 2).contiguous()
        if args.variant == "skill":
            qtok = qtok.transpose(1, 2).contiguous()
    Y = torch.empty_like(K)
    lay_code = F.FLARE_LAYOUT_BNHD if args.layout == "bnhd" else F.FLARE_LAYOUT_BHND
    if args.variant == "skill":
        def fn(Q, K, V, out=None, workspace=None, stream=None):
            F.flare_encode_ex(Q, K, V, lay_code, out=Zlat, workspace=workspace, stream=stream)
            return F.flare_attend(qtok, Zlat, lay_code, out=out, stream=stream)
    stream = torch.cuda.current_stream()

    # plain copy of known size (scales hardware memory counters to bytes)
    if args.calib_copy_mib > 0:
        nb = args.calib_copy_mib << 20
        a = torch.empty(nb, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        F.flare_copy_kernel(a, b)
        torch.cuda.synchronize()
        del a, b

    # Clock ramp: the step back to back for a fixed wall time (untimed), then
    # the W warmup steps, then the timed region.
    ramp_steps = 0
    if args.ramp_seconds > 0:
        t_end = time.perf_counter() + args.ramp_seconds
        while time.perf_counter() < t_end:
            for _ in range(20):
                fn(Q, K, V, out=Y, workspace=ws)
            ramp_steps += 20
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        fn(Q, K, V, out=Y, workspace=ws)
    torch.cuda.synchronize()

    # Timed region: exactly K steps, no instrumentation between the launches.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.graph:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            g.capture_begin()
            for _ in range(args.steps):
                fn(Q, K, V, out=Y, workspace=ws, stream=cap)
            g.capture_end()
        stream.wait_stream(cap)
        g.replay()
    torch.cuda.synchronize()
    start.record(stream)
    if args.graph:
        g.replay()
    else:
        for _ in range(args.steps):
            fn(Q, K, V, out=Y, workspace=ws)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    # Per-kernel durations: the same K steps again, each kernel launched with
    # a HIP event pair bound to its dispatch (its own start and end).
    # The pass is itself timed like the timed region: dispatch-bound events add
    # no packets to the stream, so its step time should match (reported).
    kt = {}
    ev_ms_step = None
    if not args.no_events:
        F.flare_timing_enable(True)
        start.record(stream)
        for _ in range(args.steps):
            fn(Q, K, V, out=Y, workspace=ws)
        end.record(stream)
        torch.cuda.synchronize()
        ev_ms_step = start.elapsed_time(end) / args.steps
        kt = F.flare_timing_read()
        F.flare_timing_enable(False)
    # Cold-cache pass: every step timed on its own, after a pass over
    # --cold-mib MiB that leaves none of the step's inputs in the L2s or the
    # Infinity Cache; kernel durations again from dispatch-bound events. The
    # default flush reads (a sum): a written flush leaves the caches full of
    # dirty lines whose write-back then runs during the timed step.
    cold = None
    if args.cold_mib > 0:
        flush = torch.ones(args.cold_mib << 20, dtype=torch.uint8, device="cuda")
        flush_sink = torch.empty((), dtype=torch.int32, device="cuda")
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps)]
        F.flare_timing_enable(True)
        for a_ev, b_ev in pairs:
            if args.cold_flush == "write":
                flush.fill_(1)
            else:
                flush_sink.copy_(flush.sum(dtype=torch.int32))
            a_ev.record(stream)
            fn(Q, K, V, out=Y, workspace=ws)
            b_ev.record(stream)
        torch.cuda.synchronize()
        kt_cold = F.flare_timing_read()
        F.flare_timing_enable(False)
        del flush
        step_ms = sorted(a_ev.elapsed_time(b_ev) for a_ev, b_ev in pairs)
        med = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (step_ms[len(step_ms) // 2 - 1]
                                                                          + step_ms[len(step_ms) // 2])
        cold = {"flush_mib": args.cold_mib, "flush": args.cold_flush, "steps": args.steps, "ms_per_step_median": round(med, 5),
                "ms_per_step_min": round(step_ms[0], 5),
                "value_median": round(w.B * w.H * w.N / (med * 1e-3), 1),
                "kernels": {k: {"avg_us": round(1e3 * ms / cnt, 3), "launches_per_step": cnt / args.steps}
                            for k, (ms, cnt) in kt_cold.items() if cnt}}
    # In-run peak calibration, after the timed passes (so that the probes'
    # heat and power do not reach them), at the clocks the warm GPU runs at:
    # a streaming read and the plain copy kernel (1:1 read/write HBM traffic),
    # the bf16 MFMA probe and the v_exp_f32 probe, each launched once untimed
    # and once timed with events.
    calib = None
    if not args.no_calibrate:
        def timed_once(launch):
            launch()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            r = launch()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e-3, r
        nb = max(args.calib_copy_mib, 64) << 20
        ca = torch.empty(nb, dtype=torch.uint8, device="cuda")
        cb = torch.empty_like(ca)
        t_copy, _ = timed_once(lambda: F.flare_copy_kernel(ca, cb))
        probe_out = torch.empty(F.flare_probe_lanes(), dtype=torch.float32, device="cuda")
        t_read, _ = timed_once(lambda: F.flare_read_kernel(ca, probe_out))
        del ca, cb
        t_mfma, mfma_work = timed_once(lambda: F.flare_probe_peak(F.FLARE_PROBE_MFMA_BF16, 2000, probe_out))
        t_exp, exp_work = timed_once(lambda: F.flare_probe_peak(F.FLARE_PROBE_EXP, 4000, probe_out))
        calib = {"read_gbs": round(nb / t_read / 1e9, 1), "copy_gbs": round(2 * nb / t_copy / 1e9, 1),
                 "copy_mib": nb >> 20,
                 "mfma_bf16_tflops": round(mfma_work / t_mfma / 1e12, 1),
                 "exp_per_s": float(f"{exp_work / t_exp:.4g}"),
                 "note": "rates this GPU sustained during the run: a streaming read, a plain copy (bytes read "
                         "+ written), independent v_mfma_f32_32x32x16_bf16 chains and independent v_exp_f32 "
                         "chains, four waves per SIMD"}

    outs = grads if args.variant == "backward" else (Y,)
    if not all(torch.isfinite(t.float()).all() for t in outs):
        print("non-finite output", file=sys.stderr)
        sys.exit(1)

    ms_step = total_ms / args.steps
    tok_heads = w.B * w.H * w.N
    value = tok_heads / (ms_step * 1e-3)
    e = 2 if w.dtype == "bf16" else 4
    kv_bytes = w.B * w.H * w.N * w.D * e
    passes = 2 if op == F.FLARE_OP_PP_FORWARD else 1
    flops_step = (12 if passes == 2 else 8) * w.B * w.H * w.N * w.M * w.D
    kern = {}
    for kind, (ms, cnt) in kt.items():
        if cnt:
            kern[kind] = {"avg_us": 1e3 * ms / cnt, "launches_per_step": cnt / args.steps,
                          "share_of_step": ms / total_ms}
    # Algorithmic work per launch. Each encode launch is a full pass: it reads
    # K and V once. The decode reads K and writes Y once per step, over its
    # launches per step (two when its latent range is split in halves). Both
    # contract 4*M*N*D flops per (b, h) per pass.
    dec_launches = kern["decode"]["launches_per_step"] if "decode" in kern else 1.0
    pass_flops = 4 * w.B * w.H * w.N * w.M * w.D
    alg_bytes = {"encode_partial": 2 * kv_bytes, "decode": int(round(2 * kv_bytes / dec_launches))}
    alg_flops = {"encode_partial": pass_flops, "decode": int(round(pass_flops / dec_launches))}
    if args.variant == "backward":
        # contraction work of the backward kernels per (b, h): logits and the products and
        # accumulations of each kernel (stats 6, dZ 4, dK/dV 10, dQ 8) x M*N*D flops; on the
        # bf16 matrix core for bf16 heads (over latent ranges where Q, Z and dZ of the head do
        # not fit in LDS), fp32 VALU for fp32 storage
        # FLARE++: the second stage's 28, plus the first stage's: on the matrix core its
        # encode-only dK/dV (8: logits, dl from dZ V^T, and the dK and dV products) and dQ
        # (6: logits, dZ V^T, dl K) kernels, with no statistics kernel; the fp32 kernels
        # compute the full formula with dY = 0 (statistics 6, dK/dV 10, dQ 8)
        on_mfma = w.dtype == "bf16"
        pp_first = 14 if on_mfma else 24
        bw_flops = ((28 + pp_first) if op == F.FLARE_OP_PP_FORWARD else 28) * w.B * w.H * w.N * w.M * w.D
        bw_ms = kt.get("backward", (0.0, 0))[0] / args.steps if kt else ms_step
        achieved_tf = bw_flops / (bw_ms * 1e-3) / 1e12
        peak = BF16_MFMA_PEAK_TFLOPS if on_mfma else 157.3
        roofline = {"bound": "mfma" if on_mfma else "alu", "kernel": "backward", "achieved": round(achieved_tf, 2),
                    "peak": peak, "unit": "TFLOP/s", "frac": round(achieved_tf / peak, 4), "traffic": None,
                    "alg_flops_per_step": bw_flops}
    else:
        if "encode_partial" in kern and "decode" in kern:
            dominant = max(("encode_partial", "decode"),
                           key=lambda k: kern[k]["avg_us"] * kern[k]["launches_per_step"])
            dur_s = kern[dominant]["avg_us"] * 1e-6
        else:  # no per-kernel events: attribute the step to one kernel (lower bound)
            dominant = "decode"
            dur_s = ms_step * 1e-3
        # The bound: whichever takes longer at the published peaks, the
        # kernel's HBM bytes or its matrix-core work (bf16 only; the fp32 path
        # runs on the VALU with M*N*D far below the HBM balance). A decode or
        # encode pass does 2M/e flops per byte, so bf16 turns matrix-core bound
        # above M = 312.
        on_mfma = w.dtype == "bf16" and (alg_flops[dominant] / (BF16_MFMA_PEAK_TFLOPS * 1e12)
                                         > alg_bytes[dominant] / (HBM_PEAK_GBS * 1e9))

        def position(seconds):
            if on_mfma:
                a = alg_flops[dominant] / seconds / 1e12
                return a, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s"
            a = alg_bytes[dominant] / seconds / 1e9
            return a, HBM_PEAK_GBS, "GB/s"
        achieved, peak, unit = position(dur_s)
        traffic = None
        lay = ("" if args.layout == "bhnd" else "_bnhd") + ("" if args.variant == "flare" else "_" + args.variant)
        pmc_path = os.path.join(ROOT, "profiles", f"{dominant}_{w.name}{lay}_pmc.json")
        if os.path.exists(pmc_path):
            with open(pmc_path) as f:
                pmc = json.load(f)
            if pmc.get("source_hash") == source_hash(dominant, w.dtype):
                traffic = pmc.get("hbm_bytes_per_launch")
        if cold and dominant in cold["kernels"]:
            cold_a, _, _ = position(cold["kernels"][dominant]["avg_us"] * 1e-6)
            cold["roofline"] = {"kernel": dominant, "bound": "mfma" if on_mfma else "hbm",
                                "achieved": round(cold_a, 1), "unit": unit, "frac": round(cold_a / peak, 4),
                                "hbm_frac_step": round((4 if passes == 1 else 6) * kv_bytes
                                                       / (cold["ms_per_step_median"] * 1e-3) / 1e9
                                                       / HBM_PEAK_GBS, 4)}
        roofline = {"bound": "mfma" if on_mfma else "hbm", "kernel": dominant, "achieved": round(achieved, 1),
                    "peak": peak, "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic,
                    "alg_bytes_per_launch": alg_bytes[dominant], "alg_flops_per_launch": alg_flops[dominant],
                    "mfma_tflops_step": round(flops_step / (ms_step * 1e-3) / 1e12, 2),
                    "mfma_frac_step": round(flops_step / (ms_step * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                    "hbm_frac_step": round((4 if passes == 1 else 6) * kv_bytes / (ms_step * 1e-3) / 1e9
                                           / HBM_PEAK_GBS, 4)}
        if calib:
            # the same position against what this GPU sustained in the run:
            # the MFMA probe, or for a bandwidth-bound kernel the streaming
            # read (encode: reads only) or the copy (decode: reads K, writes Y)
            ref = calib["mfma_bf16_tflops"] if on_mfma else (calib["read_gbs"] if dominant == "encode_partial"
                                                             else calib["copy_gbs"])
            roofline["frac_of_calibrated"] = round(achieved / ref, 4)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
        bw_n = min(w.N, 16384)
        t0 = time.perf_counter()
        done = 0
        # whole heads in order, cycling over the workload's heads again when all
        # are done before the budget is spent (a small workload is repeated)
        while True:
            b, h = heads[done % len(heads)]
            q = Qh[h]
            if args.variant == "backward" and op == F.FLARE_OP_PP_FORWARD:
                oracle.pp_backward_head(oracle.widen(q), oracle.widen(Kh[b, h, :bw_n]),
                                        oracle.widen(Vh[b, h, :bw_n]), oracle.widen(Vh[b, h, :bw_n][::-1]))
            elif op == F.FLARE_OP_PP_FORWARD:
                oracle.pp_forward_head(oracle.widen(q), oracle.widen(Kh[b, h]), oracle.widen(Vh[b, h]))
            elif args.variant == "backward":
                # the first bw_n tokens of the head (the fp64 backward keeps N x M matrices)
                oracle.backward_head(oracle.widen(q), oracle.widen(Kh[b, h, :bw_n]), oracle.widen(Vh[b, h, :bw_n]),
                                     oracle.widen(Vh[b, h, :bw_n][::-1]))
            elif args.variant == "skill":
                z = oracle.encode_head(oracle.widen(q), oracle.widen(Kh[b, h]), oracle.widen(Vh[b, h]))
                oracle.attend_head(oracle.widen(Vh[b, h][::-1]), z)
            else:
                qq, kk = oracle.widen(q), oracle.widen(Kh[b, h])
                z = oracle.encode_head(qq, kk, oracle.widen(Vh[b, h]))
                oracle.decode_head(qq, kk, z)
            done += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        el = time.perf_counter() - t0
        ntok = bw_n if args.variant == "backward" else w.N
        cores = 1 if args.variant == "backward" else oracle.threads()  # the fp64 backward is one loop nest
        sample = (f"{done} heads ({done / len(heads):.2f} passes over the {len(heads)} heads) of {w.name}, "
                  f"N={ntok} of {w.N}, fp64 {w.op if args.variant == 'flare' else args.variant}, {el:.1f} s")
        cpu = {"value": round(done * ntok / el, 1), "unit": "tokens*heads/s", "cores": cores,
               "cpu_model": cpu_model(), "kind": "oracle", "sample": sample}

    line = {
        "metric": "FLARE fwd tokens*heads/s (N=65536, M=128) + roofline fraction",
        "value": round(value, 1), "unit": "tokens*heads/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ramp": {"seconds": args.ramp_seconds, "steps": ramp_steps},
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_kernel_pass": None if ev_ms_step is None else round(ev_ms_step, 5),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (" + recipe() + ")",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "M": w.M, "D": w.D, "op": w.op,
                   "layout": args.layout, "variant": args.variant,
                   "plan": F.flare_describe_plan(op, w.B, w.H, w.N, w.M, w.D, Q.dtype)},
        "kernels": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in kern.items()},
        "roofline": roofline,
        "calibration": calib,
        "cold": cold,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
