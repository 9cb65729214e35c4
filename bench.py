"""Benchmark of the fused attention forward on one MI355X.

One step is one call of the library on the headline workload (exact bf16
causal prefill, B=4 H=32 N=4096 d=128), with inputs resident in HBM.  W
untimed warm-up steps, then K timed steps between two events on the launch
stream (torch's current stream), synchronised on both sides; an event between
consecutive steps gives the per-step times, reported as mean, median, p10 and
p90.  The library's own per-launch HIP events (attn_profiler_*, recorded on
the launch stream from a pool created before the timed region) time every
kernel inside the same region for the roofline figures.

The same JSON line also carries, each with its own roofline object where the
workload has a bound worth stating:
  noncausal  the headline shape without the mask;
  tiny       B1 H2 N256 d64 fp32 O (a latency figure: two workgroups);
  long       B1 H16 N65536 d128 causal with outlier keys;
  bwd        the backward of the headline workload;
  varlen     a packed batch of variable-length sequences;
  sage       the quantised prefill B2 H24 N16384 d128, with its quantisation
             statistics read back from the workspace;
  mxfp4      the same inputs in the MXFP4 mode (FP4 MFMA);
  mxfp6      the same inputs in the MXFP6 mode (FP6 MFMA, the FP4 rate);
  decode     GQA split-KV decode, contiguous caches and 16-row pages;
and the fp64 CPU oracle timed on a bounded sample of the headline workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                  [--only prefill|noncausal|tiny|long|bwd|varlen|sage|mxfp4|mxfp6|decode]
                  [--calibrate-copy]
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
PEAK_FP4_TFLOPS = 10066.3   # fp4 / fp6 dense (MX, scaled MFMA)
PEAK_HBM_GBS = 8000.0       # HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
UTIL_FILE = os.path.join(ROOT, "profiles", "mfma_util.json")
CSRC = os.path.join(ROOT, "softmax_attention_attn_amd", "csrc")
LEGS = ("prefill", "noncausal", "tiny", "long", "bwd", "varlen", "sage", "mxfp4", "mxfp6",
        "decode")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _profile_entry(path, key, files):
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = data.get(key)
    if not ent or ent.get("source_hash") != kernel_source_hash(files):
        return None
    return ent


def measured_traffic(key: str, files):
    """HBM bytes per launch from the committed counter runs (``key`` names the
    kernel and workload), or None when the kernel sources changed since the
    counters were taken."""
    ent = _profile_entry(TRAFFIC_FILE, key, files)
    return None if ent is None else ent.get("bytes_per_launch")


def measured_util(key: str, files):
    """Counter-derived busy fractions of a kernel (MFMA, VALU, LDS bank
    conflicts; rocprofv3 --pmc, in the kernel's own clock cycles), the FLOPs
    its MFMAs executed and its L2 hit rate, from the committed counter runs,
    or None when the kernel's sources changed since."""
    ent = _profile_entry(UTIL_FILE, key, files)
    if ent is None:
        return None
    return {k: ent[k] for k in ("mfma_busy", "valu_busy", "lds_bank_conflict", "executed_flop",
                                "l2_hit") if k in ent}


def summed_traffic(keys, files):
    """HBM bytes of one call made of several kernels (the sum of their
    per-launch traffic), or None when any of them has no counter run for its
    current source."""
    parts = [measured_traffic(k, files) for k in keys]
    return None if any(p is None for p in parts) else sum(parts)


# the backward's kernels, in launch order (the dQ kernel also writes the
# per-row -D and -lse/scale the dK/dV kernel reads)
BWD_KERNELS = ("bwd_dq", "bwd_dkv")


def bwd_traffic():
    return summed_traffic(BWD_KERNELS, ["bwd.hip", "cdna4.hpp"])


def stats(xs):
    a = np.asarray(xs, dtype=np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)),
            "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "n": int(a.size)}


def time_calls(fn, steps, warmup, stream):
    """Run ``fn`` warmup times, then time ``steps`` calls back to back.

    Returns (per-step stats in ms, {kernel: per-launch stats in ms}).  The
    per-step times come from events recorded between consecutive calls on the
    launch stream; the kernel times from the library's per-launch events."""
    import softmax_attention_attn_amd as A
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    A.attn_profiler_enable(True)
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(steps):
        fn()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    total_ms = evs[0].elapsed_time(evs[-1])
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    launches = A.attn_profiler_launches()
    A.attn_profiler_enable(False)
    per_kernel = {}
    for name, ms in launches:
        per_kernel.setdefault(name, []).append(ms)
    st = stats(per_step)
    st["mean"] = total_ms / steps  # the whole timed region, K steps
    return st, {k: stats(v) for k, v in per_kernel.items()}


def roofline(bound, kernel, work, kstats, peak, unit, traffic=None, counters=None, **extra):
    """Roofline object of one kernel: algorithmic work per launch over the
    kernel's mean launch time (the median-based figure alongside)."""
    scale = 1e12 if unit in ("TFLOP/s", "TOP/s") else 1e9
    ach = work / (kstats["mean"] * 1e-3) / scale
    r = {"bound": bound, "kernel": kernel, "achieved": ach, "peak": peak, "unit": unit,
         "frac": ach / peak, "traffic": traffic, "kernel_ms": kstats,
         "achieved_median": work / (kstats["median"] * 1e-3) / scale, "work": work}
    if counters is not None:
        r["counters"] = counters
    r.update(extra)
    return r


def _prefill_inputs(w):
    inp = workloads.make(w)
    return inp, inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()


def bench_exact(args, stream, wname, key, causal=None, out_dtype=torch.bfloat16):
    """Exact prefill on a named workload (causal as the workload says unless
    given); roofline for prefill_exact."""
    import softmax_attention_attn_amd as A
    w = workloads.WORKLOADS[wname]
    causal = w.causal if causal is None else causal
    inp, q, k, v = _prefill_inputs(w)
    o = torch.empty(q.shape, dtype=out_dtype, device="cuda")
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")

    def step():
        A.fwd(q, k, v, causal=causal, o=o, lse=lse, out_dtype=out_dtype, stream=stream)

    st, per_kernel = time_calls(step, args.steps, args.warmup, stream)
    flops = 4.0 * w.B * w.H * w.N * w.N * w.d / (2 if causal else 1)
    files = ["prefill_exact.hip", "cdna4.hpp"]
    res = {
        "workload": w.name, "causal": causal, "B": w.B, "H": w.H, "Hkv": w.Hkv, "N": w.N,
        "d": w.d, "out": "%s O + fp32 LSE" % ("bf16" if out_dtype == torch.bfloat16 else "fp32"),
        "ms_per_step": st["mean"], "step_ms": st, "flops": flops,
        "value": flops / (st["mean"] * 1e-3) / 1e12, "unit": "TFLOP/s",
        "roofline": roofline("mfma", "prefill_exact", flops, per_kernel["prefill_exact"],
                             PEAK_BF16_TFLOPS, "TFLOP/s",
                             traffic=measured_traffic(key, files),
                             counters=measured_util(key, files)),
    }
    return res, inp


def bench_tiny(args, stream):
    """B1 H2 N256 d64 non-causal, fp32 O: two workgroups on a 256-CU chip, so
    a latency figure (launch to completion), not a roofline claim."""
    import softmax_attention_attn_amd as A
    w = workloads.WORKLOADS["tiny_exact"]
    _, q, k, v = _prefill_inputs(w)
    o = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")

    def step():
        A.fwd(q, k, v, causal=w.causal, o=o, lse=lse, out_dtype=torch.float32, stream=stream)

    st, per_kernel = time_calls(step, max(args.steps, 100), args.warmup, stream)
    flops = w.flops()
    ks = per_kernel["prefill_exact"]
    return {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
            "out": "fp32 O + fp32 LSE", "step_ms": st, "kernel_ms": ks,
            "latency_us_median": st["median"] * 1e3, "kernel_us_median": ks["median"] * 1e3,
            "value": flops / (st["median"] * 1e-3) / 1e12, "unit": "TFLOP/s",
            "note": "latency bound: 2 workgroups (one 256-query tile per head) on 256 CUs; "
                    "value is FLOPs over the median step time"}


def bench_bwd(args, stream):
    """Backward of the headline workload: dQ, dK, dV for a random dO, with O
    and LSE from the forward (outside the timed region)."""
    import softmax_attention_attn_amd as A
    w = workloads.WORKLOADS["llm_prefill"]
    _, q, k, v = _prefill_inputs(w)
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

    st, per_kernel = time_calls(step, args.steps, args.warmup, stream)
    # five products of the forward's size (S, dP, dV, dK, dQ): 2.5x the
    # forward's FLOPs; the recomputation of S and dP in the dQ kernel is not
    # counted
    flops = 2.5 * w.flops()
    names = BWD_KERNELS
    ksum = {"mean": sum(per_kernel[n]["mean"] for n in names),
            "median": sum(per_kernel[n]["median"] for n in names)}
    files = ["bwd.hip", "cdna4.hpp"]
    return {
        "workload": w.name + "_bwd", "value": flops / (st["mean"] * 1e-3) / 1e12,
        "unit": "TFLOP/s", "ms_per_step": st["mean"], "step_ms": st, "flops": flops,
        "kernels_ms": per_kernel,
        "roofline": roofline("mfma", " + ".join(names), flops, ksum,
                             PEAK_BF16_TFLOPS, "TFLOP/s",
                             traffic=summed_traffic(names, files),
                             counters={n: measured_util(n, files) for n in ("bwd_dq", "bwd_dkv")}),
    }


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

    st, per_kernel = time_calls(step, args.steps, args.warmup, stream)
    flops = w.flops(inp["seqlens"].numpy())
    files = ["prefill_exact.hip", "cdna4.hpp"]
    return {
        "workload": w.name, "value": flops / (st["mean"] * 1e-3) / 1e12, "unit": "TFLOP/s",
        "ms_per_step": st["mean"], "step_ms": st, "seqlens": inp["seqlens"].tolist(),
        "H": w.H, "Hkv": w.Hkv, "d": w.d, "causal": w.causal,
        "roofline": roofline("mfma", "prefill_exact_varlen", flops,
                             per_kernel["prefill_exact_varlen"], PEAK_BF16_TFLOPS, "TFLOP/s",
                             traffic=measured_traffic("prefill_exact_varlen", files),
                             counters=measured_util("prefill_exact_varlen", files)),
    }


def sage_quant_stats(A, ws, w):
    """Scale ranges and code counts of the quantisation state one quantised
    call left in its workspace (read back after the timed region)."""
    lay = A.attn_sage_workspace_layout(w.B, w.H, w.Hkv, w.N, w.d)
    nblk = (w.N + 63) // 64
    npad = nblk * 64
    BH, BG = w.B * w.H, w.B * w.Hkv

    def f32(name, n):
        off = lay[name]
        return ws[off:off + 4 * n].view(torch.float32)

    def u8(name, n):
        off = lay[name]
        return ws[off:off + n]

    def rng(t):
        return {"min": float(t.min()), "max": float(t.max()), "median": float(t.median())}

    qd, kd = f32("qdelta", BH * nblk), f32("kdelta", BG * nblk)
    vs, km = f32("vscale", BG * w.d), f32("kmean", BG * w.d)
    qh = u8("qhat", BH * npad * w.d).view(torch.int8).view(BH, npad, w.d)[:, :w.N]
    kh = u8("khat", BG * npad * w.d).view(torch.int8).view(BG, npad, w.d)[:, :w.N]
    vh = u8("vhatT", BG * w.d * npad).view(BG, w.d, npad)[:, :, :w.N]
    mag = vh & 0x7F  # E4M3 magnitude code: 0x7E is 448, codes below 8 subnormal
    nv = vh.numel()
    return {
        "q_scale": rng(qd), "k_scale": rng(kd), "v_scale": rng(vs), "k_mean": rng(km),
        "int8_q_at_127": int((qh.abs() == 127).sum()), "int8_q_codes": qh.numel(),
        "int8_k_at_127": int((kh.abs() == 127).sum()), "int8_k_codes": kh.numel(),
        "fp8_v_at_448": int((mag == 0x7E).sum()), "fp8_v_nan_codes": int((mag == 0x7F).sum()),
        "fp8_v_subnormal": int(((mag > 0) & (mag < 8)).sum()),
        "fp8_v_zero": int((mag == 0).sum()), "fp8_v_codes": nv,
        "note": "a code at +-127 / +-448 is a value at its block's or channel's max|x| (the "
                "scale maps it there): none beyond the range by construction; P codes are "
                "E4M3(448 p) with p <= 1 against the exact running max, so P never saturates",
    }


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

    st, per_kernel = time_calls(step, args.steps, args.warmup, stream)
    ops = w.flops()
    files = ["sage.hip", "cdna4.hpp"]
    return {
        "workload": w.name, "value": ops / (st["mean"] * 1e-3) / 1e12, "unit": "TOP/s",
        "ms_per_step": st["mean"], "step_ms": st,
        "note": "INT8 QK^T + FP8 PV MFMA; value includes the quantisation prologue kernels, "
                "the roofline the fused attention kernel",
        "kernels_ms": per_kernel,
        "quant_stats": sage_quant_stats(A, ws, w),
        "error_budget": sage_error_budget(),
        "roofline": roofline("mfma", "sage_attn", ops, per_kernel["sage_attn"],
                             PEAK_FP8_TFLOPS, "TOP/s",
                             traffic=measured_traffic("sage_attn", files),
                             counters=measured_util("sage_attn", files)),
    }


def mx_quant_stats(A, ws, w, mode):
    """Block-scale exponents of Q, K - kmean and V that one MX call left in
    its workspace (read back after the timed region)."""
    lay = A.attn_mx_workspace_layout(w.B, w.H, w.Hkv, w.N, w.d, mode)
    npad = (w.N + 63) // 64 * 64
    nb = w.d // 32
    BH, BG = w.B * w.H, w.B * w.Hkv

    def u8(name, n):
        off = lay[name]
        return ws[off:off + n]

    def rng(t):
        t = t.to(torch.int32) - 127
        return {"min": int(t.min()), "max": int(t.max()), "median": int(t.median())}

    qs = u8("qsc", BH * npad * nb).view(BH, npad, nb)[:, :w.N]
    ks = u8("ksc", BG * npad * nb).view(BG, npad, nb)[:, :w.N]
    vs = u8("vscT", BG * (npad // 32) * w.d).view(BG, npad // 32, w.d)[:, :(w.N + 31) // 32]
    km = ws[lay["kmean"]:lay["kmean"] + 4 * BG * w.d].view(torch.float32)
    return {
        "q_block_exp": rng(qs), "k_block_exp": rng(ks), "v_block_exp": rng(vs),
        "k_mean": {"min": float(km.min()), "max": float(km.max())},
        "blocks": {"q": qs.numel(), "k": ks.numel(), "v": vs.numel()},
        "note": "a block of 32 elements has the scale 2^e with e the smallest exponent that "
                "keeps its max|x| within the element format's largest magnitude (6 for E2M1, "
                "7.5 for E2M3), so no element saturates; P's block exponents live in "
                "registers only",
    }


def bench_mx(args, stream, mode):
    """The quantised-prefill inputs (B2 H24 N16384 d128) in an MX mode
    ("mxfp4": E2M1, "mxfp6": E2M3): roofline for the fused kernel against the
    dense FP4/FP6 peak (the scaled MFMA runs both at one rate)."""
    import softmax_attention_attn_amd as A
    w = workloads.WORKLOADS["sage_prefill"]
    inp = workloads.make(w)
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    del inp
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    ws = torch.empty((A.attn_fwd_workspace_size(w.B, w.H, w.Hkv, w.N, w.d, A.MODES[mode]),),
                     dtype=torch.uint8, device="cuda")

    def step():
        A.fwd(q, k, v, causal=w.causal, mode=mode, o=o, lse=lse, workspace=ws, stream=stream)

    st, per_kernel = time_calls(step, args.steps, args.warmup, stream)
    ops = w.flops()
    files = ["mx.hip", "cdna4.hpp"]
    kern = "mx_attn" if mode == "mxfp4" else "mx6_attn"
    elem = "FP4 (E2M1)" if mode == "mxfp4" else "FP6 (E2M3)"
    return {
        "workload": w.name + "_" + mode, "value": ops / (st["mean"] * 1e-3) / 1e12,
        "unit": "TOP/s", "ms_per_step": st["mean"], "step_ms": st,
        "note": "MX %s Q/K/V/P on the scaled MFMA; value includes the quantisation prologue "
                "kernels, the roofline the fused attention kernel" % elem,
        "kernels_ms": per_kernel,
        "quant_stats": mx_quant_stats(A, ws, w, mode),
        "roofline": roofline("mfma", kern, ops, per_kernel[kern], PEAK_FP4_TFLOPS,
                             "TOP/s", traffic=measured_traffic(kern, files),
                             counters=measured_util(kern, files)),
    }


def sage_error_budget():
    """The quantised recipe's error against exact attention split by source,
    as stored by tests/golden/make_sage_error_budget.py (oracle runs on the
    CPU; no value here comes from the GPU)."""
    path = os.path.join(ROOT, "tests", "golden", "sage_error_budget.json")
    try:
        return json.load(open(path))
    except (OSError, ValueError):
        return None


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
    ws = torch.empty((A.attn_decode_workspace_size(w.B, w.H, w.Hkv, w.d),),
                     dtype=torch.uint8, device="cuda")

    def step():
        A.decode(q, k, v, seqlens, split_tokens=w.split_tokens, o=o, lse=lse, workspace=ws,
                 stream=stream)

    st, per_kernel = time_calls(step, args.steps, args.warmup, stream)
    # algorithmic bytes: every valid K and V row once, q, o (bf16) and lse (fp32)
    alg_bytes = sum_len * w.Hkv * w.d * 2 * 2 + w.B * w.H * w.d * 2 * 2 + w.B * w.H * 4
    files = ["decode.hip", "cdna4.hpp"]

    def result(st, per_kernel, split, name, extra):
        merge = "decode_merge"
        call = {"mean": per_kernel[split]["mean"] + per_kernel[merge]["mean"],
                "median": per_kernel[split]["median"] + per_kernel[merge]["median"]}
        split_only = alg_bytes / (per_kernel[split]["mean"] * 1e-3) / 1e9
        r = {
            "workload": name, "value": alg_bytes / (st["mean"] * 1e-3) / 1e9, "unit": "GB/s",
            "ms_per_step": st["mean"], "step_ms": st, "sum_seqlen": sum_len,
            "algorithmic_bytes": alg_bytes, "kernels_ms": per_kernel,
            "roofline": roofline(
                "hbm", "%s + %s" % (split, merge), alg_bytes, call, PEAK_HBM_GBS, "GB/s",
                traffic=summed_traffic((split, merge), files),
                counters=measured_util(split, files),
                split_kernel_only={"achieved": split_only, "frac": split_only / PEAK_HBM_GBS}),
        }
        r.update(extra)
        return r

    res = result(st, per_kernel, "decode_split", w.name, {})
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

    st_p, per_kernel_p = time_calls(step_paged, args.steps, args.warmup, stream)
    res["paged"] = result(st_p, per_kernel_p, "decode_split_paged", w.name + "_paged16",
                          {"page_size": ps, "num_pages": num_pages})
    return res


def host_cores():
    return {"affinity": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


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
    hc = host_cores()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "host_cores": hc,
            "sample": "fp64 C oracle, every query row of %d of the %d (b,h) slices of %s "
                      "(%d rows, %.3g FLOP) in %.1f s on %d threads (OpenMP over rows; the host "
                      "has %s logical CPUs, %d in this process's affinity mask, and the thread "
                      "count is capped by OMP_NUM_THREADS=%s)" % (
                          len(slices), w.B * w.H, w.name, len(rows), flops, dt, threads,
                          hc["os_cpu_count"], hc["affinity"], hc["omp_num_threads"])}


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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=LEGS, default=None)
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    stream = torch.cuda.current_stream()
    out = {}
    pre = pre_inp = None

    def want(leg):
        return args.only in (None, leg)

    if want("prefill"):
        log("prefill: llm_prefill causal")
        pre, pre_inp = bench_exact(args, stream, "llm_prefill", "prefill_exact")
        log("prefill %.4f ms/step (median %.4f), %.1f TFLOP/s, kernel frac %.3f" % (
            pre["ms_per_step"], pre["step_ms"]["median"], pre["value"],
            pre["roofline"]["frac"]))
    if want("noncausal"):
        log("noncausal: llm_prefill without the mask")
        nc, _ = bench_exact(args, stream, "llm_prefill", "prefill_exact_noncausal", causal=False)
        log("noncausal %.4f ms/step, %.1f TFLOP/s" % (nc["ms_per_step"], nc["value"]))
        out["noncausal"] = nc
    if want("tiny"):
        log("tiny: tiny_exact")
        tn = bench_tiny(args, stream)
        log("tiny median %.1f us per call (kernel %.1f us)" % (tn["latency_us_median"],
                                                               tn["kernel_us_median"]))
        out["tiny"] = tn
    if want("long"):
        log("long: long_prefill causal with outliers")
        lg, _ = bench_exact(args, stream, "long_prefill", "prefill_exact_long")
        lg["target_ms"] = 1.76e13 / (0.6 * PEAK_BF16_TFLOPS * 1e12) * 1e3
        log("long %.3f ms/step, %.1f TFLOP/s (frac %.3f)" % (lg["ms_per_step"], lg["value"],
                                                              lg["roofline"]["frac"]))
        out["long"] = lg
        torch.cuda.empty_cache()
    if want("bwd"):
        log("bwd: llm_prefill backward")
        bw = bench_bwd(args, stream)
        log("bwd %.3f ms/step, %.1f TFLOP/s" % (bw["ms_per_step"], bw["value"]))
        out["bwd"] = bw
        torch.cuda.empty_cache()
    if want("varlen"):
        log("varlen: varlen_prefill")
        vl = bench_varlen(args, stream)
        log("varlen %.3f ms/step, %.1f TFLOP/s" % (vl["ms_per_step"], vl["value"]))
        out["varlen"] = vl
    if want("sage"):
        log("sage: sage_prefill")
        sg = bench_sage(args, stream)
        log("sage %.3f ms/step, %.1f TOP/s (attention kernel %.1f TOP/s)" % (
            sg["ms_per_step"], sg["value"], sg["roofline"]["achieved"]))
        out["sage"] = sg
        torch.cuda.empty_cache()
    for mode in ("mxfp4", "mxfp6"):
        if want(mode):
            log("%s: sage_prefill inputs, %s mode" % (mode, mode.upper()))
            mx = bench_mx(args, stream, mode)
            log("%s %.3f ms/step, %.1f TOP/s (attention kernel %.1f TOP/s)" % (
                mode, mx["ms_per_step"], mx["value"], mx["roofline"]["achieved"]))
            out[mode] = mx
            torch.cuda.empty_cache()
    if want("decode"):
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
    line = {
        "metric": "attn fwd TFLOPS & % MFMA peak (prefill); decode HBM GB/s & % peak",
        "value": round(pre["value"], 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(pre["ms_per_step"], 4),
        "step_ms": pre["step_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": pre["workload"], "B": pre["B"], "H": pre["H"], "Hkv": pre["Hkv"],
                   "N": pre["N"], "d": pre["d"], "causal": pre["causal"], "out": pre["out"]},
        "roofline": pre["roofline"],
    }
    line.update(out)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        w = workloads.WORKLOADS["llm_prefill"]
        line["cpu_baseline"] = cpu_baseline(w, pre_inp["q"], pre_inp["k"], pre_inp["v"])
    print(json.dumps(line))


if __name__ == "__main__":
    main()
