#!/usr/bin/env python3
"""Benchmark: QuoKA chunked prefill (select + attend) on one MI355X.

One step = one whole prompt of the Llama-3-8B-shaped layer (L=32768 tokens in
16 chunks of 2048, H_q=32, H_kv=8, d=128, N_q=256, B=4096, bf16) pushed
through kvsel_prefill_chunk: query sub-selection, key scan, top-B,
compaction, attention and cache append for every chunk.  Inputs are resident
in HBM before timing starts.  Prints one JSON line:

  value      prefill tokens/s/layer = L / (time of one step)
  roofline   the attention kernel (the dominant one): algorithmic FLOP per
             launch / its average launch time, against bf16 dense MFMA peak;
             launch times come from HIP events recorded on the launch stream
             (kvsel_trace_*) over a second pass of the same K steps
  cpu_baseline  the CPU oracle timed on this host on the same inputs (the
             whole prompt of the 32K layer; the whole decode step), with the
             threads it may use and the CPU model

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

METRIC = "prefill tokens/s/layer (select+attend) at 32K ctx; % of HBM/MFMA roofline"
MFMA_BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0               # MI355X HBM3E
FP32_VECTOR_PEAK_TFLOPS = 157.3     # MI355X fp32 vector (the fp32 path's attention runs on the VALU)


def attn_kernel_name(wl) -> str:
    """The attention kernel the library launches for this shape (the same rule as
    its launcher: the 8-wave ping-pong kernel for bf16, d = 128, more than one
    128-row block per KV head, unless the grid of 256-row blocks holds between
    one and two workgroups per CU)."""
    if wl.dtype != "bf16":
        return f"attn_valu_kernel<{wl.d}> (fp32 VALU)"
    wgs = wl.H_kv * -(-wl.G * wl.C // 256)
    if wl.d == 128 and wl.G * wl.C > 128 and (wgs < 256 or wgs >= 512):
        return "attn_pp_kernel<128, bf16 out> (8 waves, ping-pong)"
    return f"attn_mfma_kernel<{wl.d}, bf16 out, 64, 4> (4 waves)"


def measured_traffic(kernel_src: str, summary: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when
    the kernel source has changed since those counters were taken."""
    import hashlib
    import re
    try:
        text = open(summary).read()
        want = re.search(r"kernel_source_sha256_16: (\w+)", text).group(1)
        have = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()[:16]
        if want != have:
            return None
        return float(re.search(r"traffic_bytes_per_launch: (\d+)", text).group(1))
    except (OSError, AttributeError):
        return None


def algorithmic_work(wl, starts, lens, pooling="head"):
    """Per-chunk algorithmic work of the method (see the design notes):
    attention: 4*d FLOP per (query row, visible key) pair, H_q*(C*B_eff + C(C+1)/2) pairs;
    scan: 2*d FLOP per (kept query, prior key) pair, H_q*min(N_q,C)*T pairs (H_kv*min(N_q,C)*T
    pooled rows with the group-first order), only when T > B;
    scan bytes: the prior keys read once, H_kv*T*d*2."""
    heads = wl.H_kv if pooling == "group" and wl.C > 1 else wl.H_q
    att_flop, scan_flop, scan_bytes, att_bytes = [], [], [], []
    for T, C in zip(starts, lens):
        beff = min(wl.B, T)
        att_flop.append(4.0 * wl.d * wl.H_q * (C * beff + C * (C + 1) / 2))
        esz = 2 if wl.dtype == "bf16" else 4
        att_bytes.append(esz * wl.d * (2 * wl.H_q * C + 2 * wl.H_kv * (beff + C)))
        if T > wl.B:
            scan_flop.append(2.0 * wl.d * heads * min(wl.n_q, C) * T)
            scan_bytes.append(esz * wl.H_kv * T * wl.d)
        else:
            scan_flop.append(0.0)
            scan_bytes.append(0.0)
    return att_flop, att_bytes, scan_flop, scan_bytes


def host_cpu():
    """(threads this process may run on, CPU model name) of the host."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return cores, model


def cpu_baseline(wl, chunks, pooling="head"):
    """The oracle, as it stands, on the same inputs: the whole prompt for prompts of
    up to 16 chunks (the 32K layer: about 40 s of host work), else every 8th chunk
    (the last of each group of 8; every 16th when a chunk holds more than 2048 x 32
    query rows) over the full prior cache."""
    from chunked_prefill_kv_amd import gen
    from oracle import quoka
    cores, model = host_cpu()
    c64 = [tuple(gen.to_f64(x) for x in c) for c in chunks]
    if len(chunks) <= 16:
        t0 = time.perf_counter()
        quoka.prefill(c64, wl.n_q, wl.B, pooling=pooling)
        t_total = time.perf_counter() - t0
        tokens = sum(c[0].shape[1] for c in c64)
        what = f"the whole {len(chunks)}-chunk prompt"
    else:
        every = 16 if wl.C * wl.H_q > 2048 * 32 else 8
        ks = list(range(every - 1, len(chunks), every))
        tokens, t_total = 0, 0.0
        for k in ks:
            Qc, Kc, Vc = c64[k]
            Kp = np.concatenate([c[1] for c in c64[:k]], axis=1)
            Vp = np.concatenate([c[2] for c in c64[:k]], axis=1)
            t0 = time.perf_counter()
            quoka.prefill_chunk(Qc, Kc, Vc, Kp, Vp, wl.n_q, wl.B, pooling=pooling)
            t_total += time.perf_counter() - t0
            tokens += Qc.shape[1]
        what = f"chunks {ks} of the {len(chunks)}-chunk prompt"
    return {"value": tokens / t_total, "unit": "tokens/s/layer", "cores": cores, "kind": "oracle",
            "cpu": model,
            "sample": f"{what} (all heads, fp64 numpy), {tokens} tokens in {t_total:.1f} s"}


def cpu_baseline_decode(wl, di):
    """The oracle on the whole ragged decode step (every sequence: select over its
    prior cache, attend), inputs read back from the paged pool beforehand."""
    from chunked_prefill_kv_amd import gen
    from oracle import quoka
    cores, model = host_cpu()
    t_total = 0.0
    for b in range(wl.batch):
        kp, vp = di.logical_kv(b, wl.block_size)
        Kp, Vp, Qc = gen.to_f64(kp), gen.to_f64(vp), gen.to_f64(di.q[b])
        Kn, Vn = gen.to_f64(di.k_new[b]), gen.to_f64(di.v_new[b])
        t0 = time.perf_counter()
        quoka.prefill_chunk(Qc, Kn, Vn, Kp, Vp, wl.n_q, wl.B)
        t_total += time.perf_counter() - t0
    return {"value": wl.batch / t_total, "unit": "tokens/s/layer", "cores": cores, "kind": "oracle", "cpu": model,
            "sample": f"the whole decode step ({wl.batch} sequences, all heads, fp64 numpy) in {t_total:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=8,
                    help="decode workload: consecutive steps of the reuse measurement")
    ap.add_argument("--lib", default=None, help="path of an alternative libkvsel.so build")
    ap.add_argument("--pooling", choices=["head", "group"], default="head",
                    help="order of the score poolings: per-head max then group mean (default), or group-pooled rows first")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (the reference kernel for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the kernels shard by KV head "
              f"with no exchange, and multi-GPU execution is not implemented", file=sys.stderr)
        sys.exit(2)

    import torch
    from chunked_prefill_kv_amd import gen, runner
    from chunked_prefill_kv_amd import kvsel as K

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return
    if gen.WORKLOADS[args.workload].L == 0:
        return bench_decode(args)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    K.load(args.lib) if args.lib else K.load()
    wl = gen.WORKLOADS[args.workload]
    print(f"[bench] generating {wl.name} inputs", file=sys.stderr, flush=True)
    chunks = [gen.chunk_inputs(wl, k) for k in range(wl.n_chunks)]
    r = runner.PromptRunner(wl, out_dtype=torch.bfloat16,
                            pooling=K.KVSEL_POOL_GROUP if args.pooling == "group" else K.KVSEL_POOL_HEAD)
    r.load(chunks)
    torch.cuda.synchronize()

    print(f"[bench] warmup {args.warmup}, timing {args.steps} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        r.run()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # the attention launches of the last timed step are bracketed by HIP events
    # on their own stream (the library's trace hook): the roofline's launch
    # time (one step's 16 launches; events around every step's launches would
    # add about 1% to the timed region)
    t0 = time.perf_counter()
    e0.record(st)
    for i in range(args.steps):
        if i == args.steps - 1:
            K.trace_start(["attn"])
        r.run()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    K.trace_stop()
    n_att, ms_att = K.trace_read()["attn"]
    att_steps = 1
    ms_step = e0.elapsed_time(e1) / args.steps
    value = wl.L / (ms_step / 1e3)

    # every kernel's launch times: the same K steps again with every launch bracketed by events
    K.trace_start()
    for _ in range(args.steps):
        r.run()
    torch.cuda.synchronize()
    K.trace_stop()
    tr = K.trace_read()
    att_flop, att_bytes, scan_flop, scan_bytes = algorithmic_work(wl, r.starts, r.lens, args.pooling)
    att_tflops = sum(att_flop) * att_steps / (ms_att * 1e-3) / 1e12
    bf16 = wl.dtype == "bf16"
    peak = MFMA_BF16_PEAK_TFLOPS if bf16 else FP32_VECTOR_PEAK_TFLOPS
    roofline = {"bound": "mfma" if bf16 else "alu", "achieved": round(att_tflops, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(att_tflops / peak, 4),
                "traffic": measured_traffic(os.path.join(ROOT, "chunked_prefill_kv_amd", "csrc", "attn.hip"),
                                            os.path.join(ROOT, "profiles", "attn_mfma_llama8b_32k_traffic.md"))
                if wl.name == "llama8b_32k" else None,
                "algorithmic_bytes_per_launch": sum(att_bytes) / len(att_bytes),
                "kernel": attn_kernel_name(wl),
                "launches": n_att, "avg_launch_us": round(ms_att * 1e3 / n_att, 2),
                "algorithmic_flop_per_launch": sum(att_flop) / len(att_flop)}
    kernels = {k: {"ms_per_step": round(v[1] / args.steps, 4), "launches_per_step": v[0] // args.steps}
               for k, v in tr.items()}
    if "scan" in tr:
        n_sc, ms_sc = tr["scan"]
        kernels["scan"]["tflops"] = round(sum(scan_flop) * args.steps / (ms_sc * 1e-3) / 1e12, 1)
        kernels["scan"]["mfma_frac"] = round(kernels["scan"]["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)
        kernels["scan"]["hbm_gbs"] = round(sum(scan_bytes) * args.steps / (ms_sc * 1e-3) / 1e9, 1)
    kernels["attn"]["hbm_gbs"] = round(sum(att_bytes) * args.steps / (tr["attn"][1] * 1e-3) / 1e9, 1)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s/layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded shared-direction generator, sinks x4)",
        "config": {"workload": wl.name, "L": wl.L, "C": wl.C, "H_q": wl.H_q, "H_kv": wl.H_kv, "d": wl.d,
                   "n_q": wl.n_q, "B": wl.B, "chunks": wl.n_chunks, "out": "bf16", "pooling": args.pooling},
        "roofline": roofline,
        "kernels": kernels,
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, chunks, pooling=args.pooling)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def bench_decode(args):
    """One ragged paged decode step (chunk of 1 per sequence) of the decode workload."""
    import torch
    from chunked_prefill_kv_amd import gen, runner
    from chunked_prefill_kv_amd import kvsel as K
    K.load(args.lib) if args.lib else K.load()
    wl = gen.WORKLOADS[args.workload]
    print(f"[bench] generating {wl.name} inputs", file=sys.stderr, flush=True)
    di = gen.decode_inputs(wl, steps=args.decode_steps)
    dr = runner.DecodeRunner(wl, di, out_dtype=torch.bfloat16)
    for _ in range(args.warmup):
        dr.run()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(args.steps):
        if i == args.steps - 1:
            K.trace_start(["scan"])              # the scan launch of the last timed step
        dr.run()
    e1.record(st)
    torch.cuda.synchronize()
    K.trace_stop()
    n_sc, ms_sc = K.trace_read().get("scan", (1, float("nan")))
    ms_step = e0.elapsed_time(e1) / args.steps
    K.trace_start()
    for _ in range(args.steps):
        dr.run()
    torch.cuda.synchronize()
    K.trace_stop()
    tr = K.trace_read()
    T = di.prior_len.astype(np.float64)
    scan_bytes = float((T[T > wl.B] * wl.H_kv * wl.d * 2).sum())      # every prior key read once
    gbs = scan_bytes * n_sc / (ms_sc * 1e-3) / 1e9
    out = {"metric": "decode tokens/s/layer (select+attend), ragged paged batch", "value": round(wl.batch / (ms_step / 1e3), 1),
           "unit": "tokens/s/layer", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": wl.name, "batch": wl.batch, "prior_len_mean": float(T.mean()), "B": wl.B,
                      "H_q": wl.H_q, "H_kv": wl.H_kv, "d": wl.d, "block_size": wl.block_size},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "scan (one query per head)",
                        "launches": n_sc, "avg_launch_us": round(ms_sc * 1e3 / n_sc, 2)},
           "kernels": {k: {"ms_per_step": round(v[1] / args.steps, 4)} for k, v in tr.items()},
           "cpu_baseline": None}
    del dr
    out["reuse"] = bench_decode_reuse(wl, di, args.decode_steps)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on the decode step", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_decode(wl, di)
    print(json.dumps(out), flush=True)


def bench_decode_reuse(wl, di, S):
    """S consecutive decode steps (the generator's tokens at T_b .. T_b + S - 1), plain and
    with the selected-entry cache (kvsel_decode_reuse; its first step fills the cache):
    time per step over steps 1 .. S-1 of each, and the hit rate of those steps."""
    import torch
    from chunked_prefill_kv_amd import runner
    sr = runner.DecodeStepsRunner(wl, di)
    st = torch.cuda.current_stream()
    ms = {}
    for reuse in (False, True):
        for _ in range(2):                       # the second pass is timed
            sr.reset()
            sr.step(0, reuse)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for t in range(1, S):
                sr.step(t, reuse)
            e1.record(st)
            torch.cuda.synchronize()
        ms["reuse" if reuse else "plain"] = e0.elapsed_time(e1) / (S - 1)
    sr.reset()
    hits = kept = 0
    for t in range(S):
        sr.step(t, True)
        torch.cuda.synchronize()
        if t:
            c = sr.counts.cpu().numpy()
            hits += int(c[..., 0].sum())
            kept += int(c.sum())
    return {"steps": S, "ms_per_step_plain": round(ms["plain"], 4), "ms_per_step_reuse": round(ms["reuse"], 4),
            "hit_rate": round(hits / max(kept, 1), 4),
            "what": "steps 1..S-1 of S consecutive decode steps; hit = a kept entry already in the "
                    "selected-entry cache from the previous step (its rows are not fetched again)"}


if __name__ == "__main__":
    main()
