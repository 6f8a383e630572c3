"""Benchmark of the dropless MoE expert MLP hot path on one MI355X.

One step = the whole path over one batch: route -> counts/offsets -> permute
-> FC1+SwiGLU -> FC2 -> combine, then gather dO -> FC2 dgrad+dSwiGLU (+dS)
-> FC2 wgrad -> FC1 dgrad -> FC1 wgrad -> unpermute-sum. Inputs are seeded
synthetic tensors already resident in HBM when timing starts.

value = algorithmic GEMM FLOPs of the step (real routed rows only,
18 * T*k * d * n) / step time, in TFLOP/s. The dominant kernel (FC1 +
SwiGLU) is also timed with HIP events on the stream it runs on, inside the
timed steps, for the roofline object. The CPU oracle is timed on a bounded
sample of the same workload for the cpu_baseline object.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
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

METRIC = "grouped-MLP TFLOP/s fwd & bwd (% of MFMA peak); permute/quant GB/s (% HBM)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_MXFP8_TFLOPS = 5000.0    # MI355X dense MXFP8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
# HBM traffic of the FC1 kernel measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
# (calibrated on a plain device copy); valid only for the kernel sources it names
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fc1_swiglu_balanced_traffic.txt")
KERNEL_SOURCES = ["gemm.hip", "gemm_common.hpp", "common.hpp", "mx_common.hpp", "launch.hpp"]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "ragged_grouped_gemm_device_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """Bytes per FC1 launch from the committed counter summary, or None when the
    kernel sources changed since it was taken (or it does not exist)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != kernel_source_hash() or kv.get("workload") != workload:
        return None
    return float(kv["traffic_bytes_per_launch"])


def _t16(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baseline(wl, inp, target_s=15.0, act="swiglu"):
    """Time the oracle on the first R tokens (routed like the full batch)."""
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as O

    def run(R):
        x = O.from_bf16(inp["x"][:R])
        w1 = O.from_bf16(inp["w1"])       # [E, d, n] already for the non-gated sReLU
        w2 = O.from_bf16(inp["w2"])
        t0 = time.perf_counter()
        f = O.forward(x, inp["logits"][:R], w1, w2, wl.k, act=act)
        O.mlp_backward(f["x_perm"], w1, w2, f["H"], f["Y"], O.from_bf16(inp["dout"][:R]),
                       f["topk_w"], f["counts"], f["offsets"], f["row_of"], f["src_of"], wl.k,
                       act=act)
        return time.perf_counter() - t0

    # the run time is a fixed part (per-expert loops, the fp64 weight-gradient buffers) plus a
    # part linear in the tokens: two probes fix both, so the sample lands near target_s
    r1, r2 = 128, min(wl.T, 1024)
    t1, t2 = run(r1), run(r2)
    slope = max((t2 - t1) / max(r2 - r1, 1), 1e-7)
    R2 = int(min(wl.T, max(r1, (target_s - max(t1 - slope * r1, 0.0)) / slope)))
    R2 = max(128, R2 // 128 * 128)
    dt2 = run(R2)
    flops = (12.0 if act == "srelu" else 18.0) * R2 * wl.k * wl.d * wl.n
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": flops / dt2 / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "sample": f"first {R2} of {wl.T} tokens of the {wl.name} workload (top-{wl.k}), whole "
                  f"forward+backward in numpy fp64, {dt2:.1f} s wall",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="balanced")
    ap.add_argument("--act", choices=["swiglu", "geglu", "srelu"], default="swiglu",
                    help="gate activation of the GLU epilogues")
    ap.add_argument("--gather", action="store_true",
                    help="GEMMs read x and dO rows through src_of (no permuted copies)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph-replays", type=int, default=20,
                    help="after the eager steps, capture one step in a hipGraph and time this many "
                         "replays (0: skip)")
    ap.add_argument("--detail", action="store_true", help="also time every stage alone (stderr)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy first (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the path has no "
              "collectives (experts would shard across GPUs with an all-to-all dispatch and combine)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from ragged_grouped_gemm_device_amd import moe as M
    from ragged_grouped_gemm_device_amd import workloads as W

    M.load()
    wl = W.WORKLOADS[args.workload]
    mx_mode = args.workload == "mxfp8"
    act = {"swiglu": M.MOE_ACT_SWIGLU, "geglu": M.MOE_ACT_GEGLU, "srelu": M.MOE_ACT_SRELU}[args.act]
    glu = {"swiglu": "SwiGLU", "geglu": "GeGLU", "srelu": "sReLU"}[args.act]
    gated = args.act != "srelu"
    if mx_mode and not gated:
        print("the MXFP8 workload runs the gated (GLU) forms only", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    t_gen = time.perf_counter()
    inp = W.make_inputs(wl)
    if not gated:   # non-gated FC1: W1_e [d, n], the first n columns of the generated weights
        inp = dict(inp)
        inp["w1"] = np.ascontiguousarray(inp["w1"][:, :, :wl.n])
    print(f"[bench] inputs for {wl.name} generated in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)
    torch.cuda.set_device(0)
    x, w1, w2, dout = (_t16(inp[key], torch) for key in ("x", "w1", "w2", "dout"))
    logits = torch.from_numpy(inp["logits"]).cuda()
    buf = M.Buffers(wl.T, wl.k, wl.E, wl.d, wl.n, mx=mx_mode, gated=gated)
    stream = torch.cuda.current_stream()
    mx = None
    if mx_mode:
        # W2 (for FC2) and W1 (for the FC1 dgrad) quantized once (weights), outside the timed step
        buf.quantize_weights(w1, w2)
        mx = buf.mx_fwd()   # FC1 on x_q / w1t_q, FC2 on a_q / w2t_q

    # (start, end) events of the launches timed inside every timed step: FC1 (the roofline
    # kernel) and the memory-bound permute / combine kernels (the bandwidth object)
    ev = {}

    def timed(record, name, fn):
        if not record:
            fn()
            return
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        ev.setdefault(name, []).append((e0, e1))

    QRC = M.MOE_QUANT_ROWWISE | M.MOE_QUANT_COLWISE

    def step(record=False):
        M.moe_route_counts(logits, wl.k, buf.topk_idx, buf.topk_w, buf.counts, buf.offsets,
                           buf.row_of, buf.src_of, buf.M_cap, buf.err, buf.route_ws)
        if mx_mode:
            # X_perm only as MXFP8: row-wise (FC1) and column-wise (FC1 wgrad), fused with the permute
            timed(record, "permute+quant x", lambda: M.moe_permute_quant_mxfp8(
                x, buf.src_of, wl.k, wl.E, QRC, buf.x_q, buf.x_s, buf.xt_q, buf.xt_s))
            buf.xt_from_forward = True
        elif not args.gather:
            timed(record, "permute x", lambda: M.moe_permute(x, buf.row_of, buf.src_of, buf.offsets,
                                                             wl.k, wl.E, buf.x_perm))
        if args.gather:
            timed(record, "fc1", lambda: M.moe_grouped_mlp_fwd(
                x, w1, w2, buf.offsets, buf.h, buf.a, buf.y, M.MOE_STAGE_FC1 | M.MOE_GATHER_ROWS,
                mx=mx, act=act, src_of=buf.src_of, k=wl.k))
        else:
            # with MXFP8 the bf16 A is not written: FC2 reads its MXFP8 copy
            timed(record, "fc1", lambda: M.moe_grouped_mlp_fwd(
                buf.x_perm, w1, w2, buf.offsets, buf.h, None if mx_mode else buf.a, buf.y,
                M.MOE_STAGE_FC1, mx=mx, act=act))
        M.moe_grouped_mlp_fwd(buf.x_perm, w1, w2, buf.offsets, buf.h, None if mx_mode else buf.a, buf.y,
                              M.MOE_STAGE_FC2, mx=mx, act=act)
        timed(record, "combine", lambda: M.moe_combine(buf.y, buf.row_of, buf.topk_w, wl.k, buf.out))
        # backward: the same calls as moe.backward, written out so that the memory-bound
        # launches can be timed one by one
        if mx_mode:
            timed(record, "permute+quant dO", lambda: M.moe_permute_quant_mxfp8(
                dout, buf.src_of, wl.k, wl.E, QRC, buf.dy_q, buf.dy_s, buf.dyt_q, buf.dyt_s))
            # the FC2 dgrad writes only the MXFP8 copies of dH and A' (all the later MXFP8 GEMMs read)
        # dgrad2, wgrad2 and dgrad1 first; the unpermute-sum reads dX_perm while the last-level
        # cache still holds it, before the FC1 wgrad's fp32 dW1 stores go through that cache
        early = M.MOE_STAGES_BWD & ~M.MOE_STAGE_WGRAD1
        if mx_mode:
            bwd = lambda st: M.moe_grouped_mlp_bwd(
                buf.x_perm, w1, w2, buf.h, buf.dy_u, buf.topk_w, buf.src_of, buf.row_of, buf.offsets,
                None, None, buf.ds, buf.dx_perm, buf.dw1, buf.dw2, buf.bwd_ws, st, act=act, mx=buf.mx_bwd(True))
        elif args.gather:
            bwd = lambda st: M.moe_grouped_mlp_bwd(
                x, w1, w2, buf.h, dout, buf.topk_w, buf.src_of, buf.row_of, buf.offsets, buf.dh, buf.a_w,
                buf.ds, buf.dx_perm, buf.dw1, buf.dw2, buf.bwd_ws, st | M.MOE_GATHER_ROWS, act=act)
        else:
            timed(record, "permute dO", lambda: M.moe_permute(dout, buf.row_of, buf.src_of, buf.offsets,
                                                              wl.k, wl.E, buf.dy_u))
            bwd = lambda st: M.moe_grouped_mlp_bwd(
                buf.x_perm, w1, w2, buf.h, buf.dy_u, buf.topk_w, buf.src_of, buf.row_of, buf.offsets,
                buf.dh, buf.a_w, buf.ds, buf.dx_perm, buf.dw1, buf.dw2, buf.bwd_ws, st, act=act)
        bwd(early)
        timed(record, "unpermute-sum dX", lambda: M.moe_combine(buf.dx_perm, buf.row_of, None, wl.k, buf.dx))
        bwd(M.MOE_STAGE_WGRAD1)
        M.moe_route_bwd(logits, buf.topk_idx, buf.ds, buf.dlogits)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    wall0 = time.perf_counter()
    for i in range(args.steps):
        step(record=True)
        if i % 10 == 9:
            print(f"[bench] step {i + 1}/{args.steps}", file=sys.stderr, flush=True)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / args.steps
    avg_ms = {name: sum(a.elapsed_time(b) for a, b in pairs) / len(pairs) for name, pairs in ev.items()}
    fc1_ms = avg_ms["fc1"]
    assert int(buf.err.item()) == 0
    bandwidth = _bandwidth(wl, buf, avg_ms, mx_mode)
    for name, r in bandwidth["kernels"].items():
        print(f"[bench] {name:18s} {r['us']:8.1f} us  {r['GBps']:8.1f} GB/s ({100 * r['frac']:.1f}% HBM)",
              file=sys.stderr, flush=True)

    M_rows = wl.T * wl.k
    # FC1 is 2 M d n1 with n1 = 2n (gated) or n (sReLU); FC2, and each of the four backward
    # GEMMs, match FC1 or FC2
    fc1_flops = (4.0 if gated else 2.0) * M_rows * wl.d * wl.n
    flops = 3.0 * fc1_flops + 3.0 * 2.0 * M_rows * wl.d * wl.n
    fc1_tf = fc1_flops / (fc1_ms * 1e-3) / 1e12
    fc1_peak = PEAK_MXFP8_TFLOPS if mx_mode else PEAK_BF16_TFLOPS   # the FC1 launch's own dtype
    value = flops / (ms * 1e-3) / 1e12
    print(f"[bench] {ms:.3f} ms/step (wall {wall / args.steps * 1e3:.3f} ms), {value:.1f} TFLOP/s; "
          f"FC1+{glu} {fc1_ms:.3f} ms = {fc1_tf:.1f} TFLOP/s", file=sys.stderr, flush=True)

    # the same step captured once in a hipGraph and replayed: per-replay HIP events, median
    graph = None
    if args.graph_replays > 0:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()  # warm-up outside capture
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        times = []
        for _ in range(args.graph_replays):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        med = times[len(times) // 2]
        graph = {"replays": args.graph_replays, "ms_per_step_median": round(med, 4),
                 "ms_min": round(times[0], 4), "ms_max": round(times[-1], 4),
                 "value_median": round(flops / (med * 1e-3) / 1e12, 2)}
        assert int(buf.err.item()) == 0
        print(f"[bench] hipGraph replay: median {med:.3f} ms/step over {args.graph_replays} replays "
              f"({graph['value_median']:.1f} TFLOP/s)", file=sys.stderr, flush=True)
        del g

    if args.detail:
        buf.logits_for_detail = logits
        _detail(M, torch, wl, buf, x, w1, w2, dout, stream, mx, act=act, glu=glu, gather=args.gather,
                gated=gated)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = _cpu_baseline(wl, inp, act=args.act)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8" if mx_mode else "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: T={wl.T} tokens top-{wl.k} over E={wl.E} experts, d={wl.d}, "
                        f"n={wl.n} (FC1 N=2n={2 * wl.n}); route->permute->FC1+{glu}"
                        + ("+MXFP8 quant epilogue->MXFP8 FC2 (FC1 on MXFP8 X_perm and W1)" if mx_mode
                           else "->FC2")
                        + f"->combine + full backward with d{glu}, dS, ragged wgrads and the router "
                        "softmax backward"
                        + (" (every GEMM on MXFP8: dgrad2+dGLU with fused MXFP8 quantization of dH "
                           "and A', FC1 dgrad, both wgrads; element-wise and router work in bf16/fp32)"
                           if mx_mode else " (bf16)")
                        + ("; x and dO rows gathered inside the GEMMs (no permute)" if args.gather else ""),
            "T": wl.T, "k": wl.k, "E": wl.E, "d": wl.d, "n": wl.n,
            "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        },
        "roofline": {
            "kernel": f"grouped_gemm FC1+{glu}" + (" on MXFP8 operands" if mx_mode else ""),
            "bound": "mfma",
            "achieved": round(fc1_tf, 2),
            "peak": fc1_peak,
            "unit": "TFLOP/s",
            "frac": round(fc1_tf / fc1_peak, 4),
            "traffic": measured_traffic(wl.name) if act == M.MOE_ACT_SWIGLU else None,
            "traffic_unit": "bytes per launch",
        },
        "bandwidth": bandwidth,
        "graph": graph,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def _bandwidth(wl, buf, avg_ms, mx_mode):
    """Achieved HBM rate of the memory-bound launches of the step: algorithmic bytes (what
    the method must move for the T*k real pairs; padding rows and re-reads are overhead
    charged to the kernel) over the launch's average time from HIP events on its stream
    inside the timed steps."""
    T, k, d = wl.T, wl.k, wl.d
    P = T * k
    model = {
        # read x once and row_of, write k copies of each row
        "permute x": (2.0 * T * d + 4.0 * P + 2.0 * P * d, "gather x [T, d] -> X_perm; 2Td + 4Tk + 2Tkd"),
        "permute dO": (2.0 * T * d + 4.0 * P + 2.0 * P * d, "gather dO [T, d] -> dY_u; 2Td + 4Tk + 2Tkd"),
        # read the k rows, row_of and the weights of every token, write the token row
        "combine": (2.0 * P * d + 8.0 * P + 2.0 * T * d, "weighted sum of Y rows -> out; 2Tkd + 8Tk + 2Td"),
        "unpermute-sum dX": (2.0 * P * d + 4.0 * P + 2.0 * T * d, "sum of dX_perm rows -> dX; 2Tkd + 4Tk + 2Td"),
        # read x once and src_of, write row- and column-wise codes (1 B) plus scales (1 B / 32)
        "permute+quant x": (2.0 * T * d + 4.0 * P + 2.0 * P * d * 33 / 32,
                            "gather x + MXFP8 row and column copies; 2Td + 4Tk + 2Tkd(1 + 1/32)"),
        "permute+quant dO": (2.0 * T * d + 4.0 * P + 2.0 * P * d * 33 / 32,
                             "gather dO + MXFP8 row and column copies; 2Td + 4Tk + 2Tkd(1 + 1/32)"),
    }
    kernels = {}
    for name, ms in avg_ms.items():
        if name not in model:
            continue
        by, formula = model[name]
        gbs = by / (ms * 1e-3) / 1e9
        kernels[name] = {"bytes": by, "us": round(ms * 1e3, 2), "GBps": round(gbs, 1),
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_model": formula}
    return {"unit": "GB/s", "peak": PEAK_HBM_GBS, "timing": "HIP events on the launch stream, "
            "average over the timed steps", "kernels": kernels}


def _detail(M, torch, wl, buf, x, w1, w2, dout, stream, mx=None, reps=10, act=0, glu="SwiGLU",
            gather=False, gated=True):
    """Time each stage alone (stderr only)."""
    def timeit(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    Mr = wl.T * wl.k
    d, n = wl.d, wl.n
    g1 = 4.0 if gated else 2.0   # FC1-shaped GEMMs: 2 M d n1, n1 = 2n or n
    end = int(buf.offsets[-1].item())
    rows = [
        ("permute", lambda: M.moe_permute(x, buf.row_of, buf.src_of, buf.offsets, wl.k, wl.E, buf.x_perm),
         None, 2.0 * wl.T * d + 2.0 * end * d + 4.0 * end),
        (f"FC1+{glu}", lambda: M.moe_grouped_mlp_fwd(buf.x_perm, w1, w2, buf.offsets, buf.h, buf.a,
                                                     buf.y, M.MOE_STAGE_FC1, act=act),
         g1 * Mr * d * n, None),
        ("FC2", lambda: M.moe_grouped_mlp_fwd(buf.x_perm, w1, w2, buf.offsets, None, buf.a, buf.y,
                                              M.MOE_STAGE_FC2, act=act), 2.0 * Mr * d * n, None),
        ("combine", lambda: M.moe_combine(buf.y, buf.row_of, buf.topk_w, wl.k, buf.out), None,
         2.0 * Mr * d + 2.0 * wl.T * d + 8.0 * Mr),
    ]
    if mx is not None:
        # the standalone quantizer of A ([rows, n] bf16, 128 MB at the mxfp8 shape) cycles
        # through 4 copies of its input and outputs, so that no call finds its source in the
        # 256 MB last-level cache
        qsets = [(buf.a[:end].clone(), torch.empty(end, n, dtype=torch.uint8, device="cuda"),
                  torch.empty(end, n // 32, dtype=torch.uint8, device="cuda"),
                  torch.empty(n, end, dtype=torch.uint8, device="cuda"),
                  torch.empty(n, end // 32, dtype=torch.uint8, device="cuda")) for _ in range(4)]
        qturn = [0]

        def quant_a_rotated():
            src, qr, sr, qc, sc = qsets[qturn[0] % 4]
            qturn[0] += 1
            M.moe_quant_mxfp8(src, 3, qr, sr, qc, sc)
        rows += [
            (f"FC1+{glu}+MXq", lambda: M.moe_grouped_mlp_fwd(buf.x_perm, w1, w2, buf.offsets, buf.h,
                                                             buf.a, buf.y, M.MOE_STAGE_FC1,
                                                             mx=buf.mx_fwd(fc1=False, transposed_a=True),
                                                             act=act),
             4.0 * Mr * d * n, None),
            (f"MX FC1+{glu}+MXq", lambda: M.moe_grouped_mlp_fwd(buf.x_perm, w1, w2, buf.offsets, buf.h,
                                                                buf.a, buf.y, M.MOE_STAGE_FC1, mx=mx,
                                                                act=act),
             4.0 * Mr * d * n, None, PEAK_MXFP8_TFLOPS),
            ("quant X row+col", lambda: M.moe_quant_mxfp8(buf.x_perm, 3, buf.x_q, buf.x_s, buf.xt_q,
                                                          buf.xt_s),
             None, 2.0 * buf.M_cap * d + 2.0 * buf.M_cap * d * 33 / 32),
            ("permute+quant X", lambda: M.moe_permute_quant_mxfp8(x, buf.src_of, wl.k, wl.E, 3, buf.x_q,
                                                                  buf.x_s, buf.xt_q, buf.xt_s),
             None, 2.0 * end * d + 2.0 * buf.M_cap * d * 33 / 32),
            ("FC2 MXFP8", lambda: M.moe_grouped_mlp_fwd(buf.x_perm, w1, w2, buf.offsets, None, buf.a,
                                                        buf.y, M.MOE_STAGE_FC2, mx=mx),
             2.0 * Mr * d * n, None, PEAK_MXFP8_TFLOPS),
            ("quant A row+col", quant_a_rotated, None, 2.0 * end * n + 2.0 * (end * n + end * n // 32)),
        ]
    logits = buf.logits_for_detail
    rows.append(("route bwd", lambda: M.moe_route_bwd(logits, buf.topk_idx, buf.ds, buf.dlogits), None,
                 8.0 * wl.T * wl.E + 8.0 * Mr))
    for st, fl in ((M.MOE_STAGE_DGRAD2, 2.0 * Mr * d * n), (M.MOE_STAGE_WGRAD2, 2.0 * Mr * d * n),
                   (M.MOE_STAGE_DGRAD1, g1 * Mr * d * n), (M.MOE_STAGE_WGRAD1, g1 * Mr * d * n)):
        xa, da, gflag = (x, dout, M.MOE_GATHER_ROWS) if gather else (buf.x_perm, buf.dy_u, 0)
        rows.append((f"bwd stage 0x{st:02x}", (lambda s=st, xa=xa, da=da, gflag=gflag: M.moe_grouped_mlp_bwd(
            xa, w1, w2, buf.h, da, buf.topk_w, buf.src_of, buf.row_of, buf.offsets,
            buf.dh, buf.a_w, buf.ds, buf.dx_perm, buf.dw1, buf.dw2, buf.bwd_ws, s | gflag, act=act)),
            fl, None))
    if mx is not None:
        mxb = buf.mx_bwd()
        rows.append(("quant dY_u row+col", lambda: M.moe_quant_mxfp8(buf.dy_u, 3, buf.dy_q, buf.dy_s,
                                                                     buf.dyt_q, buf.dyt_s),
                     None, 2.0 * buf.M_cap * d + 2.0 * buf.M_cap * d * 33 / 32))
        rows.append(("MX bwd 0x04 bf16", (lambda: M.moe_grouped_mlp_bwd(
            buf.x_perm, w1, w2, buf.h, buf.dy_u, buf.topk_w, buf.src_of, buf.row_of, buf.offsets,
            buf.dh, buf.a_w, buf.ds, buf.dx_perm, buf.dw1, buf.dw2, buf.bwd_ws, M.MOE_STAGE_DGRAD2,
            act=act, mx=buf.mx_bwd(dgrad2=False))), 2.0 * Mr * d * n, None))
        for st, fl, pk in ((M.MOE_STAGE_DGRAD2, 2.0 * Mr * d * n, PEAK_MXFP8_TFLOPS),
                           (M.MOE_STAGE_WGRAD2, 2.0 * Mr * d * n, PEAK_MXFP8_TFLOPS),
                           (M.MOE_STAGE_DGRAD1, 4.0 * Mr * d * n, PEAK_MXFP8_TFLOPS),
                           (M.MOE_STAGE_WGRAD1, 4.0 * Mr * d * n, PEAK_MXFP8_TFLOPS)):
            rows.append((f"MX bwd 0x{st:02x}", (lambda s=st: M.moe_grouped_mlp_bwd(
                buf.x_perm, w1, w2, buf.h, buf.dy_u, buf.topk_w, buf.src_of, buf.row_of, buf.offsets,
                buf.dh, buf.a_w, buf.ds, buf.dx_perm, buf.dw1, buf.dw2, buf.bwd_ws, s, act=act, mx=mxb)),
                fl, None, pk))
    for row in rows:
        name, fn, fl, by = row[:4]
        peak = row[4] if len(row) > 4 else PEAK_BF16_TFLOPS
        ms = timeit(fn)
        msg = f"[detail] {name:16s} {ms * 1e3:9.1f} us"
        if fl:
            msg += f"  {fl / ms / 1e9:8.1f} TFLOP/s ({100 * fl / ms / 1e9 / peak:.1f}% of {peak:.0f})"
        if by:
            msg += f"  {by / ms / 1e6:8.1f} GB/s ({100 * by / ms / 1e6 / PEAK_HBM_GBS:.1f}% HBM)"
        print(msg, file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
