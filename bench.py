"""Benchmark of the fused attention forward on one MI355X.

One step is one call of the library on the headline workload (exact bf16
causal prefill, B=4 H=32 N=4096 d=128), with inputs resident in HBM.  W
untimed warm-up steps, then K timed steps between two events on the launch
stream (torch's current stream), synchronised on both sides.  The library's
own per-kernel HIP events (attn_profiler_*) time the dominant kernel inside
the same timed region for the roofline figure.

The same JSON line also carries the split-KV decode workload (HBM bound,
GB/s; contiguous caches, and the same caches spread over a pool of 16-row
pages), the backward of the headline workload, a packed batch of
variable-length sequences, and the quantised prefill workload, each with its own roofline object,
and the fp64 CPU oracle timed on a bounded sample of the headline workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                  [--only prefill|bwd|varlen|decode|sage] [--calibrate-copy]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_FP8_TFLOPS = 5033.2    # fp8 / int8 dense
PEAK_HBM_GBS = 8000.0       # HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
UTIL_FILE = os.path.join(ROOT, "profiles", "mfma_util.json")
CSRC = os.path.join(ROOT, "softmax_attention_attn_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, files):
    """HBM bytes per launch from the committed counter runs, or None when the
    kernel sources changed since the counters were taken."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = data.get(kernel)
    if not ent or ent.get("source_hash") != kernel_source_hash(files):
        return None
    return ent.get("bytes_per_launch")


def measured_util(kernel: str, files):
    """Counter-derived busy fractions of a kernel (MFMA, VALU, LDS bank
    conflicts; rocprofv3 --pmc, in the kernel's own clock cycles) and the
    FLOPs its MFMAs executed, from the committed counter run, or None when
    the kernel's sources changed since."""
    try:
        data = json.load(open(UTIL_FILE))
    except (OSError, ValueError):
        return None
    ent = data.get(kernel)
    if not ent or ent.get("source_hash") != kernel_source_hash(files):
        return None
    return {k: ent[k] for k in ("mfma_busy", "valu_busy", "lds_bank_conflict", "executed_flop")}


def time_calls(fn, steps, warmup, stream):
    import softmax_attention_attn_amd as A
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    A.attn_profiler_enable(True)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    kern = A.attn_profiler_read()
    A.attn_profiler_enable(False)
    per_kernel = {k: (t / n if n else 0.0, n) for k, (t, n) in kern.items()}
    return total_ms / steps, per_kernel


def bench_prefill(args, stream):
    import softmax_attention_attn_amd as A
    w = workloads.WORKLOADS["llm_prefill"]
    inp = workloads.make(w)
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")

    def step():
        A.fwd(q, k, v, causal=w.causal, o=o, lse=lse, stream=stream)

    ms, per_kernel = time_calls(step, args.steps, args.warmup, stream)
    flops = w.flops()
    kms = per_kernel["prefill_exact"][0]
    achieved = flops / (kms * 1e-3) / 1e12
    res = {
        "workload": w, "ms_per_step": ms, "value": flops / (ms * 1e-3) / 1e12,
        "roofline": {"bound": "mfma", "kernel": "prefill_exact", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS,
                     "kernel_ms": kms,
                     "traffic": measured_traffic("prefill_exact",
                                                 ["prefill_exact.hip", "cdna4.hpp"]),
                     "counters": measured_util("prefill_exact",
                                               ["prefill_exact.hip", "cdna4.hpp"])},
        "inputs": (inp["q"], inp["k"], inp["v"]),
    }
    return res


def bench_bwd(args, stream):
    """Backward of the headline workload: dQ, dK, dV for a random dO, with O
    and LSE from the forward (outside the timed region)."""
    import softmax_attention_attn_amd as A
    w = workloads.WORKLOADS["llm_prefill"]
    inp = workloads.make(w)
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    do = workloads.make_prefill(w.B, w.H, w.Hkv, w.N, w.d, seed=1)[0].cuda()
    o, lse = A.fwd(q, k, v, causal=w.causal)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws = torch.empty((A.attn_bwd_workspace_size(w.B, w.H, w.N),), dtype=torch.uint8,
                     device="cuda")

    def step():
        A.bwd(q, k, v, o, lse, do, causal=w.causal, dq=dq, dk=dk, dv=dv, workspace=ws,
              stream=stream)

    ms, per_kernel = time_calls(step, args.steps, args.warmup, stream)
    # five products of the forward's size (S, dP, dV, dK, dQ): 2.5x the
    # forward's FLOPs; the recomputation of S and dP in the dQ kernel is not
    # counted
    flops = 2.5 * w.flops()
    kms = sum(t for t, _ in per_kernel.values())
    achieved = flops / (kms * 1e-3) / 1e12
    return {
        "workload": w.name + "_bwd", "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
        "ms_per_step": ms, "flops": flops,
        "kernels_ms": {k_: t for k_, (t, _) in per_kernel.items()},
        "roofline": {"bound": "mfma", "kernel": "bwd_delta + bwd_dq + bwd_dkv",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "kernel_ms": kms,
                     "traffic": bwd_traffic(),
                     "counters": {k: measured_util(k, ["bwd.hip", "cdna4.hpp"])
                                  for k in ("bwd_dq", "bwd_dkv")}},
    }


def bwd_traffic():
    """HBM bytes of one backward call (its three kernels), or None when any
    of them has no counter run for its current source."""
    parts = [measured_traffic(k, ["bwd.hip", "cdna4.hpp"])
             for k in ("bwd_delta", "bwd_dq", "bwd_dkv")]
    return None if any(p is None for p in parts) else sum(parts)


def bench_varlen(args, stream):
    import softmax_attention_attn_amd as A
    w = workloads.WORKLOADS["varlen_prefill"]
    inp = workloads.make(w)
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    cu = inp["cu_seqlens"].cuda()
    o = torch.empty_like(q)
    lse = torch.empty((w.H, q.shape[0]), dtype=torch.float32, device="cuda")

    def step():
        A.fwd_varlen(q, k, v, cu, w.N, causal=w.causal, o=o, lse=lse, stream=stream)

    ms, per_kernel = time_calls(step, args.steps, args.warmup, stream)
    flops = w.flops(inp["seqlens"].numpy())
    kms = per_kernel["prefill_exact_varlen"][0]
    achieved = flops / (kms * 1e-3) / 1e12
    return {
        "workload": w.name, "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
        "ms_per_step": ms, "seqlens": inp["seqlens"].tolist(), "H": w.H, "Hkv": w.Hkv,
        "d": w.d, "causal": w.causal,
        "roofline": {"bound": "mfma", "kernel": "prefill_exact_varlen", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "kernel_ms": kms,
                     "traffic": measured_traffic("prefill_exact_varlen",
                                                 ["prefill_exact.hip", "cdna4.hpp"])},
    }


def bench_decode(args, stream):
    import softmax_attention_attn_amd as A
    w = workloads.WORKLOADS["gqa_decode"]
    inp = workloads.make(w)
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    seqlens = inp["seqlens"].cuda()
    sum_len = int(inp["seqlens"].sum())
    del inp
    o = torch.empty((w.B, w.H, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    ws = torch.empty((A.attn_decode_workspace_size(w.B, w.H, w.N, w.d, w.split_tokens),),
                     dtype=torch.uint8, device="cuda")

    def step():
        A.decode(q, k, v, seqlens, split_tokens=w.split_tokens, o=o, lse=lse, workspace=ws,
                 stream=stream)

    ms, per_kernel = time_calls(step, max(args.steps, 20), args.warmup, stream)
    # algorithmic bytes: every valid K and V row once, q, o (bf16) and lse (fp32)
    alg_bytes = sum_len * w.Hkv * w.d * 2 * 2 + w.B * w.H * w.d * 2 * 2 + w.B * w.H * 4

    def result(ms, per_kernel, kernel, name, extra):
        kms = per_kernel[kernel][0]
        achieved = alg_bytes / (kms * 1e-3) / 1e9
        r = {
            "workload": name, "value": alg_bytes / (ms * 1e-3) / 1e9, "unit": "GB/s",
            "ms_per_step": ms, "sum_seqlen": sum_len, "algorithmic_bytes": alg_bytes,
            "kernels_ms": {k_: t for k_, (t, _) in per_kernel.items()},
            "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": achieved / PEAK_HBM_GBS, "kernel_ms": kms,
                         "traffic": measured_traffic(kernel, ["decode.hip", "cdna4.hpp"]),
                         "counters": measured_util(kernel, ["decode.hip", "cdna4.hpp"])},
        }
        r.update(extra)
        return r

    res = result(ms, per_kernel, "decode_split", w.name, {})
    # the same caches spread over a pool of 16-row pages in a random order
    ps = 16
    table, num_pages = workloads.make_page_table(seqlens.cpu(), ps, seed=77, spare_pages=0,
                                                 max_pages=w.N // ps)
    kp = workloads.paginate(k, table, num_pages, ps)
    vp = workloads.paginate(v, table, num_pages, ps)
    del k, v
    torch.cuda.empty_cache()
    table = table.cuda()

    def step_paged():
        A.decode_paged(q, kp, vp, table, seqlens, split_tokens=w.split_tokens, o=o, lse=lse,
                       workspace=ws, stream=stream)

    ms_p, per_kernel_p = time_calls(step_paged, max(args.steps, 20), args.warmup, stream)
    res["paged"] = result(ms_p, per_kernel_p, "decode_split_paged", w.name + "_paged16",
                          {"page_size": ps, "num_pages": num_pages})
    return res


def bench_sage(args, stream):
    import softmax_attention_attn_amd as A
    w = workloads.WORKLOADS["sage_prefill"]
    inp = workloads.make(w)
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    del inp
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    ws = torch.empty((A.attn_fwd_workspace_size(w.B, w.H, w.Hkv, w.N, w.d, A.MODES["sage"]),),
                     dtype=torch.uint8, device="cuda")

    def step():
        A.fwd(q, k, v, causal=w.causal, mode="sage", o=o, lse=lse, workspace=ws, stream=stream)

    ms, per_kernel = time_calls(step, max(5, args.steps // 2), args.warmup, stream)
    ops = w.flops()
    kms = per_kernel["sage_attn"][0]
    achieved = ops / (kms * 1e-3) / 1e12
    return {
        "workload": w.name, "value": ops / (ms * 1e-3) / 1e12, "unit": "TOP/s",
        "ms_per_step": ms, "note": "INT8 QK^T + FP8 PV MFMA; value includes the quantisation "
                                   "prologue kernels, the roofline the fused attention kernel",
        "kernels_ms": {k_: t for k_, (t, _) in per_kernel.items()},
        "roofline": {"bound": "mfma", "kernel": "sage_attn", "achieved": achieved,
                     "peak": PEAK_FP8_TFLOPS, "unit": "TOP/s", "frac": achieved / PEAK_FP8_TFLOPS,
                     "kernel_ms": kms,
                     "traffic": measured_traffic("sage_attn", ["sage.hip", "cdna4.hpp"]),
                     "counters": measured_util("sage_attn", ["sage.hip", "cdna4.hpp"])},
    }


def cpu_baseline(w, q, k, v):
    """fp64 oracle over the headline workload, every query row of every (b,h)
    slice (about 10 s on 16 host cores), reported in the headline's unit."""
    import oracle
    oracle.build(force=False)
    slices = np.arange(0, w.B * w.H, 1, dtype=np.int64)
    rows = (slices[:, None] * w.N + np.arange(w.N, dtype=np.int64)[None, :]).reshape(-1)
    i = rows % w.N
    flops = float(np.sum(4.0 * w.d * (i + 1 if w.causal else w.N)))
    threads = oracle.default_threads()
    qb, kb, vb = (workloads.bf16_bits(t) for t in (q, k, v))
    t0 = time.perf_counter()
    oracle.attn_rows(qb, kb, vb, causal=w.causal, scale=w.scale, rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "fp64 C oracle, every query row of %d of the %d (b,h) slices of %s "
                      "(%d rows, %.3g FLOP) in %.1f s" % (len(slices), w.B * w.H, w.name,
                                                         len(rows), flops, dt)}


def calibrate_copy():
    """A plain device-to-device copy of a known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters of a rocprofv3 --pmc run."""
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "launches": 3}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "bwd", "varlen", "decode", "sage"],
                    default=None)
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    stream = torch.cuda.current_stream()
    out = {}
    pre = None
    if args.only in (None, "prefill"):
        log("prefill: llm_prefill")
        pre = bench_prefill(args, stream)
        log("prefill %.3f ms/step, %.1f TFLOP/s" % (pre["ms_per_step"], pre["value"]))
    if args.only in (None, "bwd"):
        log("bwd: llm_prefill backward")
        bw = bench_bwd(args, stream)
        log("bwd %.3f ms/step, %.1f TFLOP/s" % (bw["ms_per_step"], bw["value"]))
        out["bwd"] = bw
        torch.cuda.empty_cache()
    if args.only in (None, "varlen"):
        log("varlen: varlen_prefill")
        vl = bench_varlen(args, stream)
        log("varlen %.3f ms/step, %.1f TFLOP/s" % (vl["ms_per_step"], vl["value"]))
        out["varlen"] = vl
    if args.only in (None, "sage"):
        log("sage: sage_prefill")
        sg = bench_sage(args, stream)
        log("sage %.3f ms/step, %.1f TOP/s (attention kernel %.1f TOP/s)" % (
            sg["ms_per_step"], sg["value"], sg["roofline"]["achieved"]))
        out["sage"] = sg
        torch.cuda.empty_cache()
    if args.only in (None, "decode"):
        log("decode: gqa_decode")
        dec = bench_decode(args, stream)
        log("decode %.3f ms/step, %.1f GB/s; paged (16-row pages) %.3f ms/step, %.1f GB/s" % (
            dec["ms_per_step"], dec["value"], dec["paged"]["ms_per_step"],
            dec["paged"]["value"]))
        out["decode"] = dec
        torch.cuda.empty_cache()
    if pre is None:
        print(json.dumps(out))
        return
    w = pre["workload"]
    line = {
        "metric": "attn fwd TFLOPS & % MFMA peak (prefill); decode HBM GB/s & % peak",
        "value": round(pre["value"], 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "out": "bf16 O + fp32 LSE"},
        "roofline": pre["roofline"],
    }
    line.update(out)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(w, *pre["inputs"])
    print(json.dumps(line))


if __name__ == "__main__":
    main()
