#!/usr/bin/env python3
"""Benchmark of the Lighthouse attention layer on one MI355X.

One step = lh_forward + lh_backward (the whole hot path: pool+score, top-K,
gather, attention forward, scatter, scatter adjoint, attention backward, pool
adjoint) on synthetic inputs already resident in HBM.  Default workload: the
512K-token kernel-level case (N=524288, H=16, d=128, bf16, p=4, L=5, K=128).

Prints one JSON line with the metric, per-stage times (HIP events on the
launch stream), the roofline position of the dominant kernel, the CPU oracle
timed on a bounded sample, and the dense causal attention comparison at the
same N.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]

With --block it instead times the attention block around the layer at the
530M model's shape (x W_QKV projections, the layer, the W_O projection,
forward and backward; N=98304, d_model=2048, H=16, d=128, p=4, L=4, K=128) and
prints that measurement's own JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Lighthouse layer fwd+bwd tokens/s at 512K ctx; speedup vs dense causal attn"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # dense bf16/fp16 MFMA, vendor figure


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stage_bytes(w, S, pk=False):
    """Algorithmic HBM bytes of one launch of each streaming stage (each kernel's compulsory reads
    and writes: inputs read once, outputs written once).  With the
    parent-kept selection the scatter and the pool adjoint read fp32 rows of the sub-sequence."""
    N, H, d, p, L = w["N"], w["H"], w["d"], w["p"], w["L"]
    e = 2 if w["dtype"] == "bf16" else 4
    row = N * H * d * e                         # one [N, H, d] tensor
    top = (N // p ** (L - 1)) * H * d * 4
    m = 0
    while m + 1 <= L - 1 and p ** (m + 1) <= 256 and p ** (m + 1) * H <= 8192:
        m += 1
    # the pooling pass stores the scores of levels 1..m (level 0 too when it is the top level
    # or the pass ends there: the selection never ranks leaves)
    nscore = sum(N // p ** l for l in range(0 if (L == 1 or m == 0) else 1, m + 1)) * H * 4
    pool_m = (N // p ** m) * H * d * 4 * 3
    sub32 = S * H * d * 4
    out = {
        "pool_score": 3 * row + nscore + pool_m,      # read q, k, v; write scores and level-m means
        "scatter_bwd": row + sub32,                   # read dO; write dO~ once
    }
    if pk:   # summed copies from the fp32 sub-sequence rows
        out["scatter_fwd"] = row + sub32              # write o; read the rows of O~ once
        out["pool_bwd"] = 3 * row + 3 * sub32         # write dq, dk, dv; read their sub-sequence rows once
    elif e == 2:
        # the attention kernels write the token rows themselves (o; dk, dv and dq from
        # the two roles of the one backward launch)
        out["attn_fwd"] = row
        out["attn_bwd"] = 3 * row
    else:
        out["scatter_fwd"] = row + sub32
        out["pool_bwd"] = 3 * row + 3 * sub32
    return out


def attn_flops(w, S):
    """Algorithmic flops of causal attention on the sub-sequence (per launch)."""
    H, d = w["H"], w["d"]
    unit = S * S * d * H                          # one causal S x S x d product
    return {"attn_fwd": 2 * unit, "attn_bwd": 5 * unit}


# the kernel each stage launches (one launch per stage and step)
STAGE_KERNEL = {"pool_score": "k_pool_score", "pool_up": "k_pool_up", "topk": "k_topk", "gather": "k_gather",
                "attn_fwd": "k_attn_fwd", "scatter_fwd": "k_scatter_fwd", "scatter_bwd": "k_scatter_bwd",
                "attn_bwd": "k_attn_bwd", "pool_bwd": "k_pool_bwd"}
# MFMA products each attention launch issues per algorithmic one (split operands:
# hi*hi + hi*lo + lo*hi; the backward recomputes S and dP in both roles: 7 products
# for the 5 of the gradient)
SPLIT_PRODUCTS = {"attn_fwd": 3.0, "attn_bwd": 3.0 * 7.0 / 5.0}


def measured_traffic(workload, stage):
    """HBM bytes per launch of `stage` from the committed rocprofv3 counter summary, or None
    when there is none or the kernel's source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("kernels", {}).get(stage)
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def achievable_peaks(lh, torch, stream):
    """What plain in-repo kernels reach on this GPU (lh_peak_probe): 2 GiB read, write and
    copy streams, 2 GiB written in the token-row pattern of the attention kernels' scatter
    (one head's 256-byte pieces, 4 KiB apart), and a register-only bf16 MFMA loop.
    Reported beside the vendor peaks."""
    nbytes = 2 << 30
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    acc = torch.zeros(4 * max(nbytes >> 20, 1024), dtype=torch.int32, device="cuda")   # per-workgroup folds
    src.fill_(1)
    iters = 10000
    mfma_flops = 4096 * iters * 4 * 32768
    out = {}
    for kind, name, moved in ((0, "read_GBs", nbytes), (1, "write_GBs", nbytes), (2, "copy_GBs", 2 * nbytes),
                              (5, "token_write_GBs", nbytes), (3, "mfma_bf16_TFLOPs", mfma_flops)):
        a = src if kind in (0, 2) else None
        b = acc if kind in (0, 3) else dst
        n = iters if kind == 3 else nbytes
        lh.peak_probe(kind, a, b, n, stream)            # warm-up
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(5):
            lh.peak_probe(kind, a, b, n, stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        sec = ev[0].elapsed_time(ev[1]) / 5 / 1e3
        out[name] = round(moved / sec / (1e12 if kind == 3 else 1e9), 1)
    del src, dst, acc
    return out


def cpu_threads():
    """Host threads this process may use: its CPU affinity, capped by OMP_NUM_THREADS when set
    (the GPU machine's share of host cores)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_baseline(w, x, heads, score_mode=0, select_mode=0):
    """The oracle (fwd+bwd) on the first `heads` heads of the same inputs, on every host thread
    this process may use (OpenMP over heads and over the sub-sequence's rows), scaled to all
    heads when heads < H."""
    import numpy as np
    import oracle
    sub = {n: np.ascontiguousarray(x[n][:, :heads]) for n in ("q", "k", "v", "dout")}
    p, L, K, dt = w["p"], w["L"], w["K"], w["dtype"]
    threads = cpu_threads()
    t0 = time.perf_counter()
    r = oracle.forward(sub["q"], sub["k"], sub["v"], p, L, K, dt, want=("sel", "o"), nthreads=threads,
                       score_mode=score_mode, select_mode=select_mode)
    oracle.backward(sub["q"], sub["k"], sub["v"], sub["dout"], p, L, K, (r["start"], r["level"]), dt,
                    want=("full",), nthreads=threads, select_mode=select_mode)
    t = time.perf_counter() - t0
    full = t * w["H"] / heads
    scaled = "" if heads == w["H"] else f", scaled by {w['H']}/{heads} heads (heads are independent)"
    return {"value": w["N"] / full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fwd+bwd on {heads} of {w['H']} heads (all {w['N']} tokens), {t:.1f} s on {threads} "
                      f"threads (nproc {os.cpu_count()}){scaled}"}


BLOCK_METRIC = ("Lighthouse attention block (QKV projections + layer + output projection) "
                "fwd+bwd tokens/s at 98K, 530M-model shape")


def block_gemm_flops(N, dm, hd):
    """Flops of one launch of each projection GEMM of the block."""
    one = 2 * N * dm * hd
    return {"proj_qkv": 3 * one, "proj_out": one, "proj_out_dx": one, "proj_out_dw": one,
            "proj_qkv_dx": 3 * one, "proj_qkv_dw": 3 * one}


def bench_block(args, lh, torch, np, si):
    w = si.BLOCK_WORKLOAD
    N, dm, H, d, p, L, K = w["N"], w["dm"], w["H"], w["d"], w["p"], w["L"], w["K"]
    hd = H * d
    S = int(lh.lh_subseq_len(N, p, L, K))
    log(f"block workload {w['name']}: N={N} dm={dm} H={H} d={d} p={p} L={L} K={K} S={S}")
    t0 = time.perf_counter()
    b = si.block_inputs(with_dy=True, threads=16)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    x, wqkv, wo, dy = dev(b["x"]), dev(b["w_qkv"]), dev(b["w_o"]), dev(b["dy"])
    ws = lh.block_workspace(N, H, d, dm, p, L, K)
    o = torch.empty((N, H, d), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    grads = (torch.empty_like(x), torch.empty((dm, 3 * hd), dtype=torch.float32, device="cuda"),
             torch.empty((hd, dm), dtype=torch.float32, device="cuda"))
    stream = torch.cuda.current_stream()

    def step():
        lh.block_forward(x, wqkv, wo, H, d, p, L, K, ws=ws, o=o, y=y, stream=stream)
        lh.block_backward(x, wqkv, wo, o, dy, H, d, p, L, K, ws, mode=args.mode, grads=grads, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")

    lh.lh_stage_timing(1)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    stages = lh.lh_stage_timing_read(32)
    lh.lh_stage_timing(0)
    fl = block_gemm_flops(N, dm, hd)
    stage_rep = {}
    for name, (ms, cnt) in stages.items():
        avg = ms / cnt
        rec = {"ms": round(avg, 4), "launches": cnt}
        if name in fl:
            rec["TFLOP/s"] = round(fl[name] / (avg / 1e3) / 1e12, 1)
            rec["frac_mfma_bf16"] = round(rec["TFLOP/s"] / BF16_PEAK_TFLOPS, 4)
        stage_rep[name] = rec
    gemm_ms = sum(stages[s][0] for s in stages if s in fl) / args.steps
    gemm_flops = sum(fl[s] * stages[s][1] for s in stages if s in fl) / args.steps
    layer_ms = sum(stages[s][0] for s in stages if s not in fl) / args.steps
    dominant = max((s for s in stages if s in fl), key=lambda s: stages[s][0])
    dom_ms = stages[dominant][0] / stages[dominant][1]
    ach = fl[dominant] / (dom_ms / 1e3) / 1e12
    roof = {"bound": "mfma", "kernel": dominant, "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(w["name"], dominant),
            "algorithmic_flops_per_launch": fl[dominant], "avg_launch_ms": round(dom_ms, 4),
            "all_gemms": {"ms_per_step": round(gemm_ms, 3), "TFLOP/s": round(gemm_flops / (gemm_ms / 1e3) / 1e12, 1)}}

    dense = None
    if not args.no_dense:
        log("dense causal attention at the same N ...")
        q = torch.empty((N, H, d), dtype=torch.bfloat16, device="cuda").normal_()
        kk, vv, do = torch.randn_like(q), torch.randn_like(q), torch.randn_like(q)
        dws = torch.empty(lh.lh_dense_workspace_bytes(N, H, d, 0), dtype=torch.uint8, device="cuda")
        od = torch.empty_like(q)
        lse = torch.empty((H, N), dtype=torch.float32, device="cuda")
        dg = tuple(torch.empty_like(q) for _ in range(3))
        lh.dense_forward(q, kk, vv, ws=dws, out=od, lse=lse, stream=stream)
        lh.dense_backward(q, kk, vv, od, lse, do, dws, grads=dg, stream=stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        reps = 3
        ev[0].record(stream)
        for _ in range(reps):
            lh.dense_forward(q, kk, vv, ws=dws, out=od, lse=lse, stream=stream)
            lh.dense_backward(q, kk, vv, od, lse, do, dws, grads=dg, stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        dense_ms = ev[0].elapsed_time(ev[1]) / reps
        dense = {"dense_attention_fwd_bwd_ms": round(dense_ms, 2), "reps": reps,
                 "block_with_dense_attention_ms_derived": round(gemm_ms + dense_ms, 2),
                 "speedup_block_derived": round((gemm_ms + dense_ms) / ms_per_step, 2),
                 "note": "derived: the block's measured GEMM time plus dense causal attention fwd+bwd "
                         "(same MFMA kernels) at the same N, against the measured Lighthouse block step"}
        del dws, od, lse, dg, q, kk, vv, do
        log(f"dense attention fwd+bwd {dense_ms:.1f} ms")

    cpu = None
    if not args.no_cpu:
        import oracle
        threads = cpu_threads()
        log(f"CPU oracle block fwd+bwd on {threads} threads ...")
        t0 = time.perf_counter()
        f = oracle.block_forward(b["x"], b["w_qkv"], b["w_o"], H, d, p, L, K, nthreads=threads)
        oracle.block_backward(f, b["x"], b["w_qkv"], b["w_o"], b["dy"], H, d, p, L, K, nthreads=threads)
        t = time.perf_counter() - t0
        cpu = {"value": N / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"the whole block fwd+bwd ({N} tokens), {t:.1f} s (fp64 numpy GEMMs and the layer oracle)"}

    out = {
        "metric": BLOCK_METRIC,
        "value": round(N / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, inputs resident in HBM)",
        "config": {"workload": w["name"], "N": N, "d_model": dm, "H": H, "d": d, "p": p, "L": L, "K": K, "S": S,
                   "scatter_mode": "deterministic" if args.mode else "fp_atomic"},
        "layer_ms_per_step": round(layer_ms, 3),
        "roofline": roof,
        "cpu_baseline": cpu,
        "dense_comparison": dense,
        "stages": stage_rep,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--mode", type=int, default=0, help="scatter adjoint: 0 fp-atomic, 1 deterministic (partial sums added in a fixed order)")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense attention comparison")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-heads", type=int, default=0, help="heads in the CPU oracle sample (0: all)")
    ap.add_argument("--select", choices=("partition", "parent_kept"), default="partition",
                    help="selection reading (default: partition; parent_kept prints its own line)")
    ap.add_argument("--score", choices=("qk", "k", "q", "qk_product"), default="qk",
                    help="score reading (default: qk)")
    ap.add_argument("--block", action="store_true",
                    help="time the attention block (projections + layer) at the 530M shape instead")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the layer runs on a single MI355X here; --gpus {args.gpus} "
              "is not supported (heads or sequence blocks would be sharded across GPUs).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "copies": 3}), flush=True)
        return
    import hierarchical_selection_attention_amd as lh
    import synth_inputs as si
    if args.block:
        bench_block(args, lh, torch, np, si)
        return

    w = si.WORKLOADS[args.workload]
    N, H, d, p, L, K = w["N"], w["H"], w["d"], w["p"], w["L"], w["K"]
    code = 0 if w["dtype"] == "bf16" else 1
    sel_mode = 1 if args.select == "parent_kept" else 0
    score_mode = {"qk": 0, "k": 1, "q": 2, "qk_product": 3}[args.score]
    S = int(lh.lh_subseq_len_sel(N, p, L, K, sel_mode))
    log(f"workload {w['name']}: N={N} H={H} d={d} {w['dtype']} p={p} L={L} K={K} S={S}")
    t0 = time.perf_counter()
    x = si.workload_inputs(args.workload, with_dout=True, threads=16)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")

    def dev(a):
        if w["dtype"] == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    q, k, v, do = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["dout"])
    ws = lh.alloc_workspace(N, H, d, p, L, K, code, select_mode=sel_mode)
    o = torch.empty_like(q)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    stream = torch.cuda.current_stream()

    def step():
        lh.forward(q, k, v, p, L, K, ws=ws, out=o, stream=stream, score_mode=score_mode, select_mode=sel_mode)
        lh.backward(do, p, L, K, ws, mode=args.mode, grads=grads, stream=stream, select_mode=sel_mode)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")

    # the measurement: exactly K steps, synchronised on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    tokens_per_s = N / (ms_per_step / 1e3)
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")

    # per-stage times: a second pass of K steps with HIP events around every stage
    # (diagnostic only; the events add a little time, so it does not enter `value`)
    lh.lh_stage_timing(1)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    stages = lh.lh_stage_timing_read(32)
    lh.lh_stage_timing(0)

    sb = stage_bytes(w, S, pk=bool(sel_mode))
    # counter summaries are per workload and kernel set: the variants have none
    prof_name = w["name"] + (f"_{args.select}" if sel_mode else "") + (f"_score_{args.score}" if score_mode else "")
    fl = attn_flops(w, S)
    stage_rep = {}
    for name, (ms, cnt) in stages.items():
        avg = ms / cnt
        rec = {"ms": round(avg, 4), "launches": cnt}
        if name in sb:
            rec["GB/s"] = round(sb[name] / (avg / 1e3) / 1e9, 1)
            rec["frac_hbm"] = round(rec["GB/s"] / HBM_PEAK_GBS, 3)
        if name in fl:
            rec["TFLOP/s"] = round(fl[name] / (avg / 1e3) / 1e12, 2)
            rec["frac_mfma_bf16"] = round(rec["TFLOP/s"] / BF16_PEAK_TFLOPS, 4)
        stage_rep[name] = rec
    dominant = max(stages, key=lambda s: stages[s][0])
    dom_ms = stages[dominant][0] / stages[dominant][1]
    # a kernel with both HBM bytes and MFMA flops (the attention kernels that write the
    # token rows) is placed against the resource it uses the larger fraction of
    f_hbm = sb.get(dominant, 0) / (dom_ms / 1e3) / 1e9 / HBM_PEAK_GBS
    f_mfma = fl.get(dominant, 0) / (dom_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS
    if dominant in sb and f_hbm >= f_mfma:
        ach = sb[dominant] / (dom_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "kernel": STAGE_KERNEL.get(dominant, dominant), "stage": dominant,
                "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(prof_name, dominant),
                "algorithmic_bytes_per_launch": sb[dominant], "avg_launch_ms": round(dom_ms, 4)}
    else:
        ach = fl.get(dominant, 0) / (dom_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "kernel": STAGE_KERNEL.get(dominant, dominant), "stage": dominant,
                "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(prof_name, dominant), "avg_launch_ms": round(dom_ms, 4)}

    # the attention kernels against bf16 MFMA peak, in algorithmic flops (S^2 d per causal
    # product) and in the MFMA work they issue; with every product split in three,
    # the algorithmic fraction can reach at most 1/3 (forward) and 5/21 (backward)
    mfma = {}
    for name in ("attn_fwd", "attn_bwd"):
        if name in stages and name in fl:
            t = stages[name][0] / stages[name][1] / 1e3
            mfma[STAGE_KERNEL[name]] = {
                "algorithmic_TFLOPs": round(fl[name] / t / 1e12, 2),
                "frac_bf16_peak": round(fl[name] / t / 1e12 / BF16_PEAK_TFLOPS, 4),
                "issued_TFLOPs": round(fl[name] * SPLIT_PRODUCTS[name] / t / 1e12, 2),
                "ceiling_frac_of_split": round(1.0 / SPLIT_PRODUCTS[name], 4)}
    roof["attention_mfma"] = mfma
    roof["achievable"] = achievable_peaks(lh, torch, stream)
    log(f"achievable on this GPU: {roof['achievable']}")

    dense = None
    if not args.no_dense and w["dtype"] == "bf16" and N % 64 == 0:
        log("dense causal attention at the same N ...")
        dws = torch.empty(lh.lh_dense_workspace_bytes(N, H, d, 0), dtype=torch.uint8, device="cuda")
        od = torch.empty_like(q)
        lse = torch.empty((H, N), dtype=torch.float32, device="cuda")
        dg = tuple(torch.empty_like(q) for _ in range(3))
        lh.dense_forward(q, k, v, ws=dws, out=od, lse=lse, stream=stream)          # warm-up
        lh.dense_backward(q, k, v, od, lse, do, dws, grads=dg, stream=stream)
        torch.cuda.synchronize()
        reps = 3
        f_all, b_all = [], []
        for _ in range(reps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record(stream)
            lh.dense_forward(q, k, v, ws=dws, out=od, lse=lse, stream=stream)
            ev[1].record(stream)
            lh.dense_backward(q, k, v, od, lse, do, dws, grads=dg, stream=stream)
            ev[2].record(stream)
            torch.cuda.synchronize()
            f_all.append(ev[0].elapsed_time(ev[1]))
            b_all.append(ev[1].elapsed_time(ev[2]))
        f_ms, bw_ms = sorted(f_all)[reps // 2], sorted(b_all)[reps // 2]
        fb_ms = f_ms + bw_ms
        lh_f = sum(stages[s][0] / stages[s][1] for s in stages
                   if s in ("pool_score", "pool_up", "topk", "gather", "sub_prep", "attn_fwd", "scatter_fwd"))
        unit = N * N * d * H                       # one causal N x N x d product
        dense = {"fwd_ms": round(f_ms, 2), "fwd_bwd_ms": round(fb_ms, 2),
                 "speedup_fwd": round(f_ms / lh_f, 1), "speedup_fwd_bwd": round(fb_ms / ms_per_step, 1),
                 "reps": reps, "fwd_ms_each": [round(t, 1) for t in f_all],
                 "bwd_ms_each": [round(t, 1) for t in b_all],
                 "fwd_TFLOPs": round(2 * unit / (f_ms / 1e3) / 1e12, 1),
                 "bwd_TFLOPs": round(5 * unit / (bw_ms / 1e3) / 1e12, 1),
                 "fwd_frac_bf16_peak": round(2 * unit / (f_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 3),
                 "bwd_frac_bf16_peak": round(5 * unit / (bw_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 3)}
        del dws, od, lse, dg
        log(f"dense: fwd {f_ms:.1f} ms, fwd+bwd {fb_ms:.1f} ms (median of {reps})")

    cpu = None
    if not args.no_cpu:
        heads = H if args.cpu_heads <= 0 else max(1, min(H, args.cpu_heads))
        log(f"CPU oracle on {heads} heads, {cpu_threads()} threads ...")
        cpu = cpu_baseline(w, x, heads, score_mode, sel_mode)

    variant = []
    if sel_mode:
        variant.append("parent-kept selection")
    if score_mode:
        variant.append(f"score {args.score}")
    out = {
        "metric": METRIC + (f" ({', '.join(variant)})" if variant else ""),
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic (seeded, inputs resident in HBM)",
        "config": {"workload": w["name"], "N": N, "H": H, "d": d, "p": p, "L": L, "K": K, "S": S,
                   "scatter_mode": "deterministic" if args.mode else "fp_atomic",
                   "select": args.select, "score": args.score},
        "roofline": roof,
        "cpu_baseline": cpu,
        "dense_causal_attention": dense,
        "stages": stage_rep,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
