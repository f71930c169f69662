#!/usr/bin/env python3
"""Throughput of the attention backward hot path on one MI355X.

A step is one full backward of the workload: attn_bwd_preprocess (D =
rowsum(dO * O) and workspace clear) -> attn_bwd_full (dK, dV and dQ; the
dQ pass writes dQ in the I/O type), with Q, K, V, O, dO and LSE already
resident in HBM.  --api three times the three-call path instead
(attn_bwd_preprocess -> attn_bwd -> attn_bwd_dq_postprocess).  Inputs are seeded synthetic data of the
workload's shape; O and LSE come from the library's plain forward.

Prints ONE JSON line: whole-step TFLOP/s (10 * B * H * Sq * Sk * D FLOPs per
step, halved when causal), the main kernel's roofline figures measured with HIP
events on the stream the kernels run on, and the fp64 CPU oracle timed on a
bounded sample of the same workload.

Before the W warm-up steps the bench runs untimed steps for --settle seconds
(0.5 s by default): after idle the GPU needs about twenty calls to reach its
steady clock, and the first calls run up to 30% slower.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3] [--no-cpu] [--settle S] [--api full|three]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention-backward TFLOP/s (bf16, causal, S=4096, D=128) and % of MFMA peak"
# MI355X published dense peaks
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
TORCH_DT = {"bf16": "bfloat16", "f16": "float16", "f32": "float32"}
PEAK_HBM_GBS = 8000.0
# the sources the dK/dV and dQ kernels are compiled from: a change to any of
# them voids the committed HBM counter summary
MAIN_SRCS = [os.path.join(ROOT, "exact_attention_backward_amd", "csrc", f)
             for f in ("bwd_main.hip", "kv_kernel.h", "bwd_shared.h", "common.h", "launch.h", "bwd_dq.hip",
                       "bwd_dq_gemm.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_main_{}_{}.json")
KERNEL_DESC = {
    "stored_ds": "key-stationary dK/dV kernel storing dS + dQ = dS K pass",
    "separate": "key-stationary dK/dV kernel + query-stationary dQ kernel",
    "atomic": "key-stationary kernel with dQ atomics",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--deterministic", action="store_true")
    ap.add_argument("--dq-algo", default=None, choices=["stored_ds", "separate", "atomic"],
                    help="dQ from dS stored by the dK/dV kernel (default for bf16/fp16), by a query-stationary "
                         "pass that recomputes S and dP (default for fp32), or by fp32 atomics")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--dropout", type=float, default=0.0, metavar="P",
                    help="dropout of P with probability P (Philox4x32-10 keep mask, seed 1, offset 0)")
    ap.add_argument("--alibi", action="store_true", help="ALiBi slopes 2^(-8 (h + 1) / Hq) per q-head")
    ap.add_argument("--bias", action="store_true",
                    help="an elementwise bias [B, Hq, Sq, Sk] (seeded normal x 2) and its gradient dBias")
    ap.add_argument("--max-workspace-mib", type=int, default=0, metavar="MIB",
                    help="cap the stored-dS workspace (kv-head groups in chunks whose dS fits; 0 = no cap)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB, 5 times (HBM counter calibration)")
    ap.add_argument("--cpu-pairs", type=int, default=64, help="(sequence, head) pairs in the CPU oracle sample")
    ap.add_argument("--api", default="full", choices=["full", "three"],
                    help="full: attn_bwd_preprocess + attn_bwd_full (default); three: attn_bwd_preprocess + "
                         "attn_bwd + attn_bwd_dq_postprocess")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as replays of one HIP graph that holds a step's launches (for small "
                         "problems, where the host's launch cost per step exceeds the kernels'); the per-launch "
                         "HIP-event timing behind the roofline still runs on its own eager steps first")
    ap.add_argument("--settle", type=float, default=0.5, metavar="SECONDS",
                    help="untimed steps before the warm-up, until this much time has passed: after idle the GPU "
                         "takes about 20 calls (~25 ms) to reach its steady clock")
    return ap.parse_args()


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_entry(dq_algo, workload, api):
    """HBM bytes per attn_bwd_full call from the committed counter summary of
    this dQ algorithm on this workload, or None when there is none, a kernel
    source changed since the counters were taken, or the three-call path is
    timed (its counters are not kept)."""
    if api != "full":
        return None
    path = TRAFFIC_FILE.format(workload, dq_algo)
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("kernel_source_sha256_16") != "+".join(source_hash(p) for p in MAIN_SRCS):
        return None
    return t.get("hbm_bytes_per_launch")


def device_peak(dtype):
    """The dense MFMA peak from this device's own compute-unit count and
    peak clock (hipDeviceGetAttribute), reported beside the published figure
    the roofline uses; None where the runtime cannot be asked."""
    import ctypes
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return None
    khz = ctypes.c_int(0)
    HIP_DEVICE_ATTRIBUTE_CLOCK_RATE = 5   # hipDeviceAttributeClockRate: peak clock in kHz
    if hip.hipDeviceGetAttribute(ctypes.byref(khz), HIP_DEVICE_ATTRIBUTE_CLOCK_RATE,
                                 torch.cuda.current_device()) != 0 or khz.value <= 0:
        return None
    per_clock = {"bf16": 4096, "f16": 4096, "f32": 256}[dtype]   # dense FLOP per clock per CU
    return {"tflops": round(cus * khz.value * 1e3 * per_clock / 1e12, 1), "compute_units": cus,
            "peak_clock_mhz": round(khz.value / 1e3, 1), "flop_per_clock_per_cu": per_clock}


def cpu_baseline(p, x, n_pairs):
    """The fp64 oracle backward on the first n_pairs (sequence, q-head) pairs
    of the workload (sequence-major), each at full length, given O and LSE
    from the oracle forward (not timed)."""
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    host_cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    total = p.batch * p.heads_q
    n_pairs = max(1, min(n_pairs, total))
    g = p.heads_q // p.heads_kv
    cq, _ = p.cu_seqlens()
    elapsed, flops = 0.0, 0.0
    for idx in range(n_pairs):
        b, h = divmod(idx, p.heads_q)
        if p.varlen:
            q0, q1 = int(cq[b]), int(cq[b + 1])
            q, do = x["q"][q0:q1, h], x["do"][q0:q1, h]
            k, v = x["k"][q0:q1, h // g], x["v"][q0:q1, h // g]
            sq = sk = q1 - q0
        else:
            q, do = x["q"][b, :, h], x["do"][b, :, h]
            k, v = x["k"][b, :, h // g], x["v"][b, :, h // g]
            sq, sk = p.seqlen_q, p.seqlen_k
        o, lse = oracle.head_forward(q, k, v, p.scale, p.causal)
        t0 = time.perf_counter()
        oracle.head_backward(q, k, v, o, do, lse, p.scale, p.causal)
        elapsed += time.perf_counter() - t0
        f = 10.0 * sq * sk * p.head_dim
        flops += f / 2 if p.causal else f
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "host_cores": host_cores,
        "cpu_model": model,
        "kind": "oracle",
        "sample": f"fp64 numpy oracle backward of {n_pairs} of the workload's {total} (sequence, head) pairs "
                  f"at full length (O, LSE from the oracle forward, untimed); {elapsed:.1f} s wall time on "
                  f"{threads} BLAS threads ({host_cores} host cores available)",
        "seconds": elapsed,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the path shards by whole (batch, kv-head) groups, see the design notes)"}))
        sys.exit(2)

    import numpy as np
    import torch
    import datagen
    from exact_attention_backward_amd import api

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return
    p = datagen.workload(args.workload, deterministic=args.deterministic)
    if args.dq_algo is None:
        args.dq_algo = "separate" if p.dtype == "f32" else "stored_ds"
    dt = getattr(torch, TORCH_DT[p.dtype])
    x = datagen.draw(p)
    dev = {k: torch.from_numpy(v).to(dt).cuda() for k, v in x.items()}
    kw = {}
    if p.varlen:
        cq, ck = p.cu_seqlens()
        kw = dict(cu_seqlens_q=torch.from_numpy(cq).cuda(), cu_seqlens_k=torch.from_numpy(ck).cuda(),
                  max_seqlen_q=p.seqlen_q, max_seqlen_k=p.seqlen_k)
    bias = dbias = None
    if args.bias:
        gen = torch.Generator(device="cuda").manual_seed(91)
        bshape = (p.batch, p.heads_q, p.seqlen_q, p.seqlen_k)
        bias = (2 * torch.randn(bshape, generator=gen, device="cuda")).to(dt)
        dbias = torch.empty_like(bias)
    drop = (args.dropout, 1, 0) if args.dropout > 0 else None
    slopes = None
    if args.alibi:
        slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / p.heads_q) for h in range(p.heads_q)],
                              dtype=torch.float32, device="cuda")
    o, lse = api.forward(dev["q"], dev["k"], dev["v"], p.scale, p.causal, bias=bias, dropout=drop,
                         alibi_slopes=slopes, **kw)
    plan = api.BackwardPlan(dev["q"], dev["k"], p.scale, p.causal, p.deterministic, dq_algo=args.dq_algo,
                            bias=bias, dbias=dbias, dropout=drop, alibi_slopes=slopes,
                            max_workspace_bytes=args.max_workspace_mib << 20, **kw)
    dq, dk, dv = torch.empty_like(dev["q"]), torch.empty_like(dev["k"]), torch.empty_like(dev["v"])
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    torch.cuda.synchronize()

    three = args.api == "three"
    run = plan.run if three else plan.run_full
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(10):
            run(q, k, v, o, do, lse, dq, dk, dv)
        settle_steps += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        run(q, k, v, o, do, lse, dq, dk, dv)
    torch.cuda.synchronize()

    # the preprocess alone, 20 calls back to back between two events (the
    # launch of each overlaps the previous one's execution): its HBM rate
    st = torch.cuda.current_stream()
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(st)
    for _ in range(20):
        plan.preprocess(o, do)
    b1.record(st)
    torch.cuda.synchronize()
    pre_b2b_ms = b0.elapsed_time(b1) / 20

    # per-call HIP events on the stream the kernels are launched on
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        e = ev[s]
        e[0].record(st)
        plan.preprocess(o, do)
        e[1].record(st)
        if three:
            plan.main(q, k, v, do, lse, dk, dv)
            e[2].record(st)
            plan.postprocess(dq)
        else:
            plan.main_full(q, k, v, do, lse, dq, dk, dv)
            e[2].record(st)
        e[3].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eager_ms_per_step = wall * 1e3 / args.steps

    if args.graph:
        # one step (the same calls as run above) captured once, then replayed:
        # the host issues one graph launch per step instead of every kernel's
        side = torch.cuda.Stream()
        side.wait_stream(st)
        with torch.cuda.stream(side):   # a step on a non-default stream before the capture
            run(q, k, v, o, do, lse, dq, dk, dv)
        st.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run(q, k, v, o, do, lse, dq, dk, dv)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

    pre_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    main_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    post_ms = np.array([e[2].elapsed_time(e[3]) for e in ev])
    step_ms = np.array([e[0].elapsed_time(e[3]) for e in ev])
    flops = p.flops()
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    main_avg = float(main_ms.mean())
    achieved = flops / (main_avg * 1e-3) / 1e12
    peak = PEAK_TFLOPS[p.dtype]

    rows_q = p.total_q
    elem = 4 if p.dtype == "f32" else 2
    # preprocess: read O and dO, write D; the dQ accumulator is cleared only
    # in the atomic dQ mode (the other modes overwrite it)
    accum = rows_q * p.heads_q * p.head_dim * 4
    pre_bytes = 2 * rows_q * p.heads_q * p.head_dim * elem + rows_q * p.heads_q * 4 + \
        (accum if args.dq_algo == "atomic" else 0)
    post_bytes = rows_q * p.heads_q * p.head_dim * (4 + elem)

    out = {
        "metric": METRIC if args.workload == "c3" and not (args.bias or args.dropout or args.alibi) else
        f"attention-backward TFLOP/s ({p.dtype}, {p.name}{', elementwise bias and dBias' if args.bias else ''}"
        f"{f', dropout {args.dropout}' if args.dropout else ''}{', ALiBi' if args.alibi else ''}) "
        "and % of MFMA peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 4),
        "launch": "hip_graph" if args.graph else "eager",
        "ms_per_step_eager": round(eager_ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic (seeded normal Q, K, V, dO; O and LSE from the library forward)",
        "config": {
            "workload": f"{p.name}: B={p.batch} Hq={p.heads_q} Hkv={p.heads_kv} Sq={p.seqlen_q} "
                        f"Sk={p.seqlen_k} D={p.head_dim} {'causal' if p.causal else 'non-causal'}"
                        f"{' deterministic' if p.deterministic else ''}",
            "batch": p.batch, "heads_q": p.heads_q, "heads_kv": p.heads_kv, "seqlen_q": p.seqlen_q,
            "seqlen_k": p.seqlen_k, "head_dim": p.head_dim, "causal": p.causal,
            "deterministic": p.deterministic, "dq_algo": args.dq_algo, "flops_per_step": flops,
            "bias": bool(args.bias), "dropout": args.dropout, "alibi": bool(args.alibi),
            "max_workspace_mib": args.max_workspace_mib,
        },
        "roofline": {
            "kernel": ("attn_bwd (" if three else "attn_bwd_full (") + KERNEL_DESC[args.dq_algo] +
                      ("" if three or args.dq_algo != "atomic" else " + dQ postprocess") + ")",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "peak_from_device": device_peak(p.dtype),
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": None if args.bias or args.dropout or args.alibi or args.max_workspace_mib
            else traffic_entry(args.dq_algo, args.workload, args.api),
            "avg_launch_ms": round(main_avg, 5),
            "algorithmic_flops_per_launch": flops,
        },
        "api": "attn_bwd_preprocess + attn_bwd + attn_bwd_dq_postprocess" if three else
               "attn_bwd_preprocess + attn_bwd_full",
        "kernels_ms": {
            "preprocess": round(float(pre_ms.mean()), 5),
            "main": round(main_avg, 5),
            "postprocess": round(float(post_ms.mean()), 5) if three else None,
            "step_events": round(float(step_ms.mean()), 5),
        },
        "hbm_GBps": {
            "preprocess": round(pre_bytes / (pre_b2b_ms * 1e-3) / 1e9, 1),
            "preprocess_method": "20 preprocess calls back to back between two HIP events, before the timed steps",
            "preprocess_in_step": round(pre_bytes / (pre_ms.mean() * 1e-3) / 1e9, 1),
            "postprocess": round(post_bytes / (post_ms.mean() * 1e-3) / 1e9, 1) if three else None,
            "peak": PEAK_HBM_GBS,
        },
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(p, x, args.cpu_pairs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
