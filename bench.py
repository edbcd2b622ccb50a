#!/usr/bin/env python3
"""Benchmark of the fused chunked-KL hot path on one MI355X.

One step = kd_fwd + kd_bwd (reverse KL, beta = 1, tau = 2) over one batch of
the 152k-vocabulary, 32k-token workload (N = 32768 tokens, V = 151936,
d_s = 2560, d_t = 4096, bf16 inputs, fp32 accumulation), inputs resident in
HBM. Prints one JSON line with whole-job tokens/s, the MFMA fraction of the
step, the roofline of the dominant kernel (the forward sweep, timed with HIP
events on its own stream) and the fp64 CPU oracle timed on a bounded sample
of the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--chunk-v C] [--beta B] [--with-dw] [--no-cpu]

--with-dw adds dL/dW_s to the backward (one more GEMM sweep per chunk); the
default step is the loss and dL/dh_s. --workload 2 or 4 runs the same step on
the 152k-vocabulary 4k-token or the 248k-vocabulary heavy-head workload.

  python bench.py --path topk|tail [--k K] [--beta B] [--support S] ...

times the top-k paths instead, on the 248k-vocabulary 16k-token top-k
workload: one step = kd_topk_fwd + kd_topk_bwd (three terms, all weights 1,
labels given), or kd_tail_fwd + kd_tail_bwd (tail-bucket divergence; the
support defaults to the beta rule); their CPU baseline is the oracle on 48 tokens.
--teacher-dim 256 gives the teacher the shapes of its rank-256 factorisation
([N, 256] hidden states, [V, 256] unembedding): the sweep's work depends on the
shapes only, so the factors are drawn with the workload's recipe instead of
being computed by an SVD.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
WORKLOAD = 3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--chunk-v", type=int, default=0,
                    help="backward recompute chunk (0: the library's default for the shape, kd_default_chunk)")
    ap.add_argument("--beta", type=float, default=1.0)
    ap.add_argument("--with-dw", action="store_true",
                    help="also compute dL/dW_s in the backward (the step then runs three GEMM sweeps)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=None,
                    help="tokens in the CPU oracle sample (default 1024; 48 for the top-k paths)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"))
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--workload", type=int, choices=(2, 3, 4), default=WORKLOAD,
                    help="the full-vocabulary workload (3: the headline; 2 and 4: the other bf16 shapes)")
    ap.add_argument("--small-n", action="store_true",
                    help="time kd_fwd alone on the 4k-token workload's shapes at N = 64 .. 1024 tokens, where the "
                         "sweep streams W from HBM, against the HBM roofline")
    ap.add_argument("--path", choices=("kd", "topk", "tail"), default="kd",
                    help="kd: the full-vocabulary divergence (default); topk / tail: the top-k paths")
    ap.add_argument("--k", type=int, default=64, help="top-k size for --path topk / tail")
    ap.add_argument("--support", type=int, default=None, help="KD_SUPPORT_* bits for --path tail")
    ap.add_argument("--teacher-dim", type=int, default=None,
                    help="teacher hidden size for --path topk / tail (256: the shapes of a rank-256 factorised "
                         "teacher, drawn with the same recipe)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of a "
                         "'--calibrate-copy' run into the traffic record and exit")
    return ap.parse_args()


COPY_BYTES = 1 << 30


def summarize_traffic(fetch_csv, write_csv, out_path):
    """Per-launch HBM bytes of the forward sweep kernel from two rocprofv3
    counter runs (FETCH_SIZE, then WRITE_SIZE, both in KiB per dispatch),
    each scaled by what the same counter reads for the 1 GiB copy kernel."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
            vals[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        return {k: statistics.median(v.values()) for k, v in vals.items()}

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    copy = [k for k in f if "elementwise" in k or "copy" in k.lower()]
    fwd = [k for k in f if "fwd_kernel" in k]
    if not copy or not fwd:
        raise SystemExit(f"kernels not found: copy={copy} fwd={fwd}")
    ck = max(copy, key=lambda k: f[k])
    ff = COPY_BYTES / (f[ck] * 1024.0)
    fw = COPY_BYTES / (w[ck] * 1024.0)
    fk = fwd[0]
    rec = {"kernel": fk, "copy_kernel": ck, "fetch_kib": f[fk], "write_kib": w.get(fk, 0.0),
           "copy_fetch_kib": f[ck], "copy_write_kib": w[ck], "fetch_scale": ff, "write_scale": fw,
           "bytes_per_launch": f[fk] * 1024.0 * ff + w.get(fk, 0.0) * 1024.0 * fw,
           "kernel_source_hash": kernel_hash()}
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def cpu_baseline(w, beta, rows_n, path="kd", with_dw=False, k=64, support=None):
    """The fp64 oracle (as it stands) on a bounded row sample of the same
    workload and the same step: for the full-vocabulary path the forward loss
    plus dL/dh_s (and dL/dW_s's share of the sampled rows with ``with_dw``);
    for the top-k paths their forward and backward."""
    import numpy as np

    import kdsynth
    from oracle import kd_oracle as O
    rows = kdsynth.sample_rows(w.N, rows_n, seed=99)
    hs, ht = w.h_s[rows], w.h_t[rows]
    t0 = time.perf_counter()
    if path == "kd":
        O.kd_fwd(hs, w.W_s, ht, w.W_t, beta, w.tau)
        O.kd_bwd(hs, w.W_s, ht, w.W_t, beta, w.tau)
        if with_dw:
            O.kd_bwd_w(hs, w.W_s, ht, w.W_t, beta, w.tau)
        what = "fwd loss + dL/dh_s" + (" + dL/dW_s" if with_dw else "")
    elif path == "topk":
        lab = w.labels[rows]
        one = np.ones(len(rows))
        out = O.kd_topk_fwd(hs, w.W_s, ht, w.W_t, k, w.tau, labels=lab)
        O.kd_topk_bwd(hs, w.W_s, ht, w.W_t, k, w.tau, lab, one, one, one, sel=out["idx"])
        what = f"top-{k} three terms + their dL/dh_s"
    else:
        lab = w.labels[rows]
        out = O.kd_tail_fwd(hs, w.W_s, ht, w.W_t, k, beta, w.tau, support=support, labels=lab)
        O.kd_tail_bwd(hs, w.W_s, ht, w.W_t, k, beta, w.tau, sup=out["sup"])
        what = f"tail-bucket divergence (k={k}, beta={beta}) + its dL/dh_s"
    dt = time.perf_counter() - t0
    host = host_info()
    # the oracle's arithmetic runs in BLAS (the GEMMs) and numpy's elementwise
    # loops (one thread): the threads it used are the BLAS pool's
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": host["blas_threads"], "kind": "oracle",
            "sample": f"{len(rows)} of {w.N} tokens of the same workload ({what}, fp64 numpy/BLAS), {dt:.1f} s",
            "host": host}


def host_info():
    """Host cores available to this process, CPU model and BLAS library and
    threads numpy uses (threadpoolctl)."""
    info = {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": None, "blas": None, "blas_threads": 1}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            info["blas_threads"] = max(int(i.get("num_threads", 1)) for i in blas)
    except Exception:  # pragma: no cover
        info["blas_threads"] = info["affinity_cores"]
    return info


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1], args.traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path is single-GPU: "
              "no sharding or collectives are built)", file=sys.stderr)
        sys.exit(2)
    if args.cpu_rows is None:
        args.cpu_rows = (256 if args.workload == 4 else 1024) if args.path == "kd" else 48
    if args.small_n:
        bench_small_n(args)
        return
    if args.path != "kd":
        bench_topk(args)
        return
    import numpy as np
    import torch

    import kdsynth
    import vocab_chunked_kl_amd as kd

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    kd.load_library()
    torch.cuda.set_device(0)
    w = kdsynth.make(args.workload)
    N, V, ds, dt_, tau, beta = w.N, w.V, w.d_s, w.d_t, w.tau, args.beta
    args.chunk_v = args.chunk_v or kd.default_chunk(N, V)
    dev = [to_dev(x) for x in (w.h_s, w.W_s, w.h_t, w.W_t)]
    stream = torch.cuda.Stream()
    fws = kd.workspace_size(kd.KD_OP_FWD, N, V, ds, dt_, kd.KD_BF16, beta=0.5)  # covers every beta
    bop = kd.KD_OP_BWD_W if args.with_dw else kd.KD_OP_BWD
    bws = kd.workspace_size(bop, N, V, ds, dt_, kd.KD_BF16, beta=beta, chunk_V=args.chunk_v)
    with torch.cuda.stream(stream):
        ws_f = torch.empty(fws, dtype=torch.uint8, device="cuda")
        ws_b = torch.empty(bws, dtype=torch.uint8, device="cuda")
        dh = torch.empty(N, ds, dtype=torch.float32, device="cuda")
        dW = torch.empty(V, ds, dtype=torch.float32, device="cuda") if args.with_dw else None
    torch.cuda.synchronize()
    base_mem = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        loss, lse_s, lse_t, aux = kd.kd_fwd(*dev, beta, tau, workspace=ws_f, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        kd.kd_bwd(*dev, beta, tau, lse_s, lse_t, aux, chunk_V=args.chunk_v, workspace=ws_b, stream=stream, dh=dh,
                  dW=dW, want_dW=args.with_dw)
        return loss

    if args.calibrate_copy:  # a plain copy of known size for scaling the byte counters
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    with torch.cuda.stream(stream):
        t_start.record(stream)
        for i in range(args.steps):
            loss = step(evs[i])
        t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    fwd_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    peak_extra = torch.cuda.max_memory_allocated() - base_mem

    # the other points of the beta sweep of this workload, one warm step then two timed steps each
    # (reported beside the headline step, which is the configured beta)
    sweep_ms = {}
    for b in w.betas:
        bws_b = kd.workspace_size(bop, N, V, ds, dt_, kd.KD_BF16, beta=b, chunk_V=args.chunk_v)
        fws_b = kd.workspace_size(kd.KD_OP_FWD, N, V, ds, dt_, kd.KD_BF16, beta=b)
        if bws_b > ws_b.numel() or fws_b > ws_f.numel():
            continue
        with torch.cuda.stream(stream):
            def one():
                l, a1, a2, a3 = kd.kd_fwd(*dev, b, tau, workspace=ws_f, stream=stream)
                kd.kd_bwd(*dev, b, tau, a1, a2, a3, chunk_V=args.chunk_v, workspace=ws_b, stream=stream, dh=dh,
                          dW=dW, want_dW=args.with_dw)
            one()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            one()
            one()
            e1.record(stream)
        torch.cuda.synchronize()
        sweep_ms[str(b)] = round(e0.elapsed_time(e1) / 2, 3)
    assert np.isfinite(loss.float().cpu().numpy()).all()

    fwd_flops = 2.0 * N * V * (ds + dt_)
    bwd_flops = 2.0 * N * V * (ds + dt_) + 2.0 * N * V * ds * (2 if args.with_dw else 1)
    jsd = 0.0 < beta < 1.0
    step_flops = fwd_flops * (2 if jsd else 1) + bwd_flops
    tok_s = N / (ms_step / 1e3)
    achieved = fwd_flops * (2 if jsd else 1) / (fwd_ms / 1e3) / 1e12
    traffic = recorded_traffic(args.traffic)
    out = {
        "metric": ("tokens/s + MFMA % of peak for fused chunked KL fwd+bwd, V=151936, N=32k" if args.workload == 3
                   else f"tokens/s + MFMA % of peak for fused chunked KL fwd+bwd, V={V}, N={N}"),
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: N={N} tokens, V={V}, d_s={ds}, d_t={dt_}, "
                               f"beta={beta}, tau={tau}, fwd+bwd (dL/dh_s{', dL/dW_s' if args.with_dw else ''}), "
                               f"chunk_V={args.chunk_v}",
                   "global_batch": N, "parallelism": "single GPU"},
        "mfma_frac_step": round(step_flops / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "step_tflops": round(step_flops / (ms_step / 1e3) / 1e12, 1),
        "fwd_ms": round(fwd_ms, 3),
        "bwd_ms": round(ms_step - fwd_ms, 3),
        "workspace_bytes": {"fwd": fws, "bwd": bws, "peak_alloc_delta": int(peak_extra)},
        "wall_s_timed": round(wall, 3),
        "beta_sweep_ms_per_step": sweep_ms,
        "roofline": {"kernel": "fwd_kernel (forward sweep: both logit GEMMs + online LSE/KL)",
                     "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
    }
    if not args.no_cpu:
        del dev
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(w, beta, args.cpu_rows, with_dw=args.with_dw)
    print(json.dumps(out), flush=True)


def bench_small_n(args):
    """kd_fwd (reverse KL) on the 4k-token workload's shapes (V = 151936, d_s = 1024,
    d_t = 2560) at N = 64 .. 1024 tokens: the sweep reads both unembeddings once
    (1.09 GB) and does 2 N V (d_s + d_t) flops, so below ~315 tokens it is
    bound by HBM. Median of ``steps`` timed calls per N (HIP events on the
    call's stream)."""
    import numpy as np
    import torch

    import kdsynth
    import vocab_chunked_kl_amd as kd

    kd.load_library()
    torch.cuda.set_device(0)
    w = kdsynth.make(2)
    dev = [torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for a in (w.h_s, w.W_s, w.h_t, w.W_t)]
    stream = torch.cuda.Stream()
    w_bytes = 2.0 * w.V * (w.d_s + w.d_t)
    points = []
    for n in (64, 128, 256, 512, 1024):
        hs, ht = dev[0][:n].contiguous(), dev[2][:n].contiguous()
        ws = torch.empty(kd.workspace_size(kd.KD_OP_FWD, n, w.V, w.d_s, w.d_t, kd.KD_BF16, beta=1.0),
                         dtype=torch.uint8, device="cuda")
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                kd.kd_fwd(hs, dev[1], ht, dev[3], 1.0, w.tau, workspace=ws, stream=stream)
            times = []
            for _ in range(args.steps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                kd.kd_fwd(hs, dev[1], ht, dev[3], 1.0, w.tau, workspace=ws, stream=stream)
                e1.record(stream)
                times.append((e0, e1))
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in times]))
        gbs = (w_bytes + 2.0 * n * (w.d_s + w.d_t)) / (ms / 1e3) / 1e9
        # the backward at the same N (beside the forward line; chunk_V as given, else the default for n)
        cv = args.chunk_v or kd.default_chunk(n, w.V)
        loss, lse_s, lse_t, aux = kd.kd_fwd(hs, dev[1], ht, dev[3], 1.0, w.tau)
        dh = torch.empty(n, w.d_s, dtype=torch.float32, device="cuda")
        kd.kd_bwd(hs, dev[1], ht, dev[3], 1.0, w.tau, lse_s, lse_t, aux, chunk_V=cv, dh=dh)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            kd.kd_bwd(hs, dev[1], ht, dev[3], 1.0, w.tau, lse_s, lse_t, aux, chunk_V=cv, dh=dh)
        e1.record()
        torch.cuda.synchronize()
        points.append({"N": n, "ms": round(ms, 4), "GB/s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                       "TFLOP/s": round(2.0 * n * w.V * (w.d_s + w.d_t) / (ms / 1e3) / 1e12, 1),
                       "bwd_ms": round(e0.elapsed_time(e1) / 5, 4), "bwd_chunk_V": cv})
    first = points[0]
    print(json.dumps({
        "metric": f"kd_fwd time at small N, V={w.V}, d_s={w.d_s}, d_t={w.d_t}", "value": first["ms"], "unit": "ms",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False, "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name} shapes, N in {[p['N'] for p in points]}, reverse KL, tau={w.tau}"},
        "points": points,
        "roofline": {"kernel": "fwd_kernel + merge at N = 64 (HIP events around kd_fwd)", "bound": "hbm",
                     "achieved": first["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": first["hbm_frac"],
                     "traffic": None},
    }), flush=True)


def bench_topk(args):
    """Top-k three-term or tail-bucket step on the 248k-vocabulary workload."""
    import numpy as np
    import torch

    import kdsynth
    import vocab_chunked_kl_amd as kd

    kd.load_library()
    torch.cuda.set_device(0)
    w = kdsynth.make(5, d_t=args.teacher_dim)
    N, V, ds, dt_, tau, k, beta = w.N, w.V, w.d_s, w.d_t, w.tau, args.k, args.beta
    args.chunk_v = args.chunk_v or kd.default_chunk(N, V)
    dev = [torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for a in (w.h_s, w.W_s, w.h_t, w.W_t)]
    lab = torch.from_numpy(w.labels.astype(np.int32)).cuda()
    stream = torch.cuda.Stream()
    tail = args.path == "tail"
    support = args.support if args.support is not None else kd.tail_default_support(k, beta, True)
    with torch.cuda.stream(stream):
        if tail:
            ws_f = torch.empty(kd.workspace_size(kd.KD_OP_TAIL, N, V, ds, dt_, kd.KD_BF16, k=k), dtype=torch.uint8,
                               device="cuda")
            ws_b = torch.empty(kd.workspace_size(kd.KD_OP_TAIL_BWD, N, V, ds, ds, kd.KD_BF16, chunk_V=args.chunk_v,
                                                 k=k), dtype=torch.uint8, device="cuda")
        else:
            ws_f = torch.empty(kd.workspace_size(kd.KD_OP_TOPK, N, V, ds, dt_, kd.KD_BF16, k=k), dtype=torch.uint8,
                               device="cuda")
            ws_b = torch.empty(kd.workspace_size(kd.KD_OP_TOPK_BWD, N, V, ds, ds, kd.KD_BF16, chunk_V=args.chunk_v,
                                                 k=k), dtype=torch.uint8, device="cuda")
        dh = torch.empty(N, ds, dtype=torch.float32, device="cuda")
        one = torch.ones(N, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if tail:
            out = kd.kd_tail_fwd(*dev, k, beta, tau, support, labels=lab, workspace=ws_f, stream=stream)
        else:
            out = kd.kd_topk_fwd(*dev, k, tau, labels=lab, workspace=ws_f, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        if tail:
            kd.kd_tail_bwd(dev[0], dev[1], out, k, beta, tau, support, chunk_V=args.chunk_v, workspace=ws_b,
                           stream=stream, dh=dh)
        else:
            kd.kd_topk_bwd(dev[0], dev[1], out, k, tau, labels=lab, grad_binary=one, grad_cond=one, grad_ce=one,
                           chunk_V=args.chunk_v, workspace=ws_b, stream=stream, dh=dh)
        return out

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        t0.record(stream)
        for i in range(args.steps):
            out = step(evs[i])
        t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    fwd_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    assert np.isfinite(out["loss" if tail else "binary"].cpu().numpy()).all()
    fwd_flops = 2.0 * N * V * (ds + dt_)  # one top-k sweep (it ranks one model or both)
    bwd_flops = 2.0 * N * V * ds * 2  # student recompute + dh GEMM
    achieved = fwd_flops / (fwd_ms / 1e3) / 1e12
    what = (f"tail-bucket divergence, k={k}, beta={beta}, support bits {support}" if tail
            else f"top-k three terms, k={k}, labels, all weights 1")
    res = {
        "metric": f"tokens/s for {args.path} fwd+bwd, V={V}, N={N}",
        "value": round(N / (ms_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}: N={N}, V={V}, d_s={ds}, d_t={dt_}, tau={tau}, {what}, "
                               f"chunk_V={args.chunk_v}"},
        "fwd_ms": round(fwd_ms, 3), "bwd_ms": round(ms_step - fwd_ms, 3),
        "step_tflops": round((fwd_flops + bwd_flops) / (ms_step / 1e3) / 1e12, 1),
        "roofline": {"kernel": f"{'tail' if tail else 'topk'} forward (top-k sweep + merge, HIP events around "
                               "the call)",
                     "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None},
    }
    if not args.no_cpu:
        del dev
        torch.cuda.empty_cache()
        res["cpu_baseline"] = cpu_baseline(w, beta, args.cpu_rows, path=args.path, k=k, support=support)
    print(json.dumps(res), flush=True)


def recorded_traffic(path):
    """The forward sweep's HBM bytes per launch from a traffic record, or
    None when there is none or it was taken on other kernel sources."""
    try:
        with open(path) as f:
            tr = json.load(f)
    except (OSError, ValueError):
        return None
    return tr.get("bytes_per_launch") if tr.get("kernel_source_hash") == kernel_hash() else None


def kernel_hash() -> str:
    """Hash of the kernel sources; traffic counters are only valid for the
    sources they were taken on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "vocab_chunked_kl_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
