"""Benchmark of the FLARE forward hot path on one MI355X.

One step = one full pass of the operator over one batch of synthetic inputs
that are already resident in HBM: split-N encode -> combine -> decode (FLARE),
or the five-launch FLARE++ sequence, through the C ABI's caller-workspace
entry point. Default workload: the PDE-mesh shape B=4, H=8, N=65536, M=128,
D=32 in bf16 (the throughput metric is quoted on N=65536, M=128).

Before the warmup steps the step runs back to back for --ramp-seconds (untimed)
so that the GPU reaches its steady clocks; the timed region is always exactly
--steps full steps. Prints one JSON line with throughput (tokens*heads/s), the roofline position
of the dominant kernel (its average duration measured with HIP events on the
launch stream during the timed steps), and the fp64 CPU oracle's throughput
on a bounded sample of the same workload as a baseline.
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
KERNEL_SOURCES = {
    "encode_partial": ["rank_latent_attention_flare_amd/csrc/kernels_bf16.hip",
                       "rank_latent_attention_flare_amd/csrc/gfx950_ops.h"],
    "decode": ["rank_latent_attention_flare_amd/csrc/kernels_bf16.hip",
               "rank_latent_attention_flare_amd/csrc/gfx950_ops.h"],
    "combine": ["rank_latent_attention_flare_amd/csrc/kernels_common.hip"],
}


def source_hash(kind: str) -> str:
    """Hash of the code (comments and blank space removed) of the sources that
    define a kernel: recorded with its hardware counters, so that counters taken
    on an older version of the kernel are not reported against the current one."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", type=int, default=2, help="workload number 1-6 (default 2)")
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
    p.add_argument("--calib-copy-mib", type=int, default=512,
                   help="size of the plain copy kernel run once before the timed steps (counter calibration)")
    p.add_argument("--ramp-seconds", type=float, default=1.0,
                   help="run the step back to back for this long before the warmup steps, so that the GPU "
                        "reaches its steady clocks (a cold MI355X needs ~0.1-0.2 s); 0 disables")
    return p.parse_args()


def main():
    args = parse()
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
        # flare_pp_backward on the FLARE++ workload
        if args.layout != "bhnd":
            print("--variant backward takes the [B,H,N,D] layout", file=sys.stderr)
            sys.exit(2)
        pp = op == F.FLARE_OP_PP_FORWARD
        bw_op = F.FLARE_OP_PP_BACKWARD if pp else F.FLARE_OP_BACKWARD
        bw_fn = F.flare_pp_backward if pp else F.flare_backward
        ws = torch.empty(F.flare_workspace_size(bw_op, w.B, w.H, w.N, w.M, w.D, Q.dtype),
                         dtype=torch.uint8, device=Q.device)
        dYt = V.flip(2).contiguous()  # upstream gradient: the values in reverse token order
        grads = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))

        def fn(Q, K, V, out=None, workspace=None, stream=None):
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
    # Per-kernel durations: the same K steps again with a HIP event pair
    # recorded on the launch stream around every kernel.
    kt = {}
    if not args.no_events:
        F.flare_timing_enable(True)
        for _ in range(args.steps):
            fn(Q, K, V, out=Y, workspace=ws)
        torch.cuda.synchronize()
        kt = F.flare_timing_read()
        F.flare_timing_enable(False)
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
    # algorithmic bytes per launch: encode reads K and V; decode reads K and writes Y
    alg_bytes = {"encode_partial": 2 * kv_bytes, "decode": 2 * kv_bytes}
    if args.variant == "backward":
        # contraction work of the backward kernels per (b, h): logits and the products and
        # accumulations of each kernel (stats 6, dZ 4, dK/dV 10, dQ 8) x M*N*D flops; on the
        # bf16 matrix core for bf16 heads whose Q, Z and dZ fit in LDS (D = 32, or D = 64 with
        # M <= 256), else fp32 VALU
        # FLARE++: the second stage's 28, plus the first stage's statistics, dK/dV and dQ
        # kernels (6 + 10 + 8), which run with dY = 0 and the given dZ
        bw_flops = (52 if op == F.FLARE_OP_PP_FORWARD else 28) * w.B * w.H * w.N * w.M * w.D
        bw_ms = kt.get("backward", (0.0, 0))[0] / args.steps if kt else ms_step
        achieved_tf = bw_flops / (bw_ms * 1e-3) / 1e12
        on_mfma = w.dtype == "bf16" and (w.D == 32 or (w.D == 64 and w.M <= 256))
        peak = BF16_MFMA_PEAK_TFLOPS if on_mfma else 157.3
        roofline = {"bound": "mfma" if on_mfma else "alu", "kernel": "backward", "achieved": round(achieved_tf, 2),
                    "peak": peak, "unit": "TFLOP/s", "frac": round(achieved_tf / peak, 4), "traffic": None,
                    "alg_flops_per_step": bw_flops}
    else:
        if "encode_partial" in kern and "decode" in kern:
            dominant = max(("encode_partial", "decode"),
                           key=lambda k: kern[k]["avg_us"] * kern[k]["launches_per_step"])
            achieved = alg_bytes[dominant] / (kern[dominant]["avg_us"] * 1e-6) / 1e9
        else:  # no per-kernel events: attribute the step to one kernel (lower bound)
            dominant = "decode"
            achieved = alg_bytes[dominant] / (ms_step * 1e-3) / 1e9
        traffic = None
        lay = ("" if args.layout == "bhnd" else "_bnhd") + ("" if args.variant == "flare" else "_" + args.variant)
        pmc_path = os.path.join(ROOT, "profiles", f"{dominant}_{w.name}{lay}_pmc.json")
        if os.path.exists(pmc_path):
            with open(pmc_path) as f:
                pmc = json.load(f)
            if pmc.get("source_hash") == source_hash(dominant):
                traffic = pmc.get("hbm_bytes_per_launch")
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "alg_bytes_per_launch": alg_bytes[dominant],
                    "mfma_tflops_step": round(flops_step / (ms_step * 1e-3) / 1e12, 2),
                    "mfma_frac_step": round(flops_step / (ms_step * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                    "hbm_frac_step": round((4 if passes == 1 else 6) * kv_bytes / (ms_step * 1e-3) / 1e9
                                           / HBM_PEAK_GBS, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
        bw_n = min(w.N, 16384)
        t0 = time.perf_counter()
        done = 0
        for (b, h) in heads:
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
        cpu = {"value": round(done * ntok / el, 1), "unit": "tokens*heads/s", "cores": cores,
               "kind": "oracle", "sample": f"{done} of {len(heads)} heads of {w.name}, N={ntok} of {w.N}, "
                                            f"fp64 {w.op if args.variant == 'flare' else args.variant}, "
                                            f"{el:.1f} s"}

    line = {
        "metric": "FLARE fwd tokens*heads/s (N=65536, M=128) + roofline fraction",
        "value": round(value, 1), "unit": "tokens*heads/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ramp": {"seconds": args.ramp_seconds, "steps": ramp_steps},
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (" + recipe() + ")",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "M": w.M, "D": w.D, "op": w.op,
                   "layout": args.layout, "variant": args.variant,
                   "plan": F.flare_describe_plan(op, w.B, w.H, w.N, w.M, w.D, Q.dtype)},
        "kernels": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in kern.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
