"""Writes sage_error_budget.json: the quantised recipe's error against exact
attention on the B2 H24 N16384 d128 quantised-prefill workload, attributed to
its sources by switching single steps of the oracle's step-by-step emulator
off ("GPU kernel overview" page, SageAttention chain: Smooth-K, INT8 per-block
Q/K for QK^T, E4M3 P and V for PV).  Only the oracle and the seeded input
generator are called; nothing here runs on or reads from a GPU.

    python tests/golden/make_sage_error_budget.py [--rows 2048]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

# emulator switches of each variant: which steps of the recipe are applied
VARIANTS = {
    "int8_qk_only": dict(quant_qk=True, quant_p=False, quant_v=False),
    "int8_qk_no_smooth_k": dict(quant_qk=True, quant_p=False, quant_v=False, smooth_k=False),
    "fp8_p_only": dict(quant_qk=False, quant_p=True, quant_v=False),
    "fp8_v_only": dict(quant_qk=False, quant_p=False, quant_v=True),
    "int8_qk_fp8_p": dict(quant_qk=True, quant_p=True, quant_v=False),
    "full_recipe": dict(),
    "full_recipe_no_smooth_k": dict(smooth_k=False),
    "full_recipe_l_from_quantised_p": dict(l_from_quantised_p=True),
}


def metrics(o, ref):
    o = o.reshape(-1)
    ref = ref.reshape(-1)
    cos = float(o @ ref / (np.linalg.norm(o) * np.linalg.norm(ref)))
    rel = float(np.abs(o - ref).sum() / np.abs(ref).sum())
    return cos, rel


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--rows", type=int, default=2048)
    ap.add_argument("--out", default=os.path.join(HERE, "sage_error_budget.json"))
    args = ap.parse_args()
    w = workloads.WORKLOADS["sage_prefill"]
    inp = workloads.make(w)
    qb, kb, vb = (workloads.bf16_bits(inp[x]) for x in ("q", "k", "v"))
    rng = np.random.default_rng(2024)
    rows = np.sort(rng.choice(w.B * w.H * w.N, size=args.rows, replace=False)).astype(np.int64)
    t0 = time.time()
    o_ex, _, _ = oracle.attn_rows(qb, kb, vb, causal=w.causal, scale=w.scale, rows=rows)
    out = {"workload": w.name, "rows": int(args.rows), "row_seed": 2024,
           "reference": "exact attention (fp64 oracle) on the same bf16 inputs",
           "metrics": "cos and rel-L1 = sum|dO| / sum|O_exact| over the sampled rows",
           "variants": {}}
    for name, kw in VARIANTS.items():
        o, _ = oracle.sage_rows(qb, kb, vb, causal=w.causal, scale=w.scale, rows=rows, **kw)
        cos, rel = metrics(o, o_ex)
        out["variants"][name] = {"switches": kw, "cos": cos, "rel_l1": rel}
        print("%-32s cos %.6f rel-L1 %.4f" % (name, cos, rel), flush=True)
    out["seconds"] = round(time.time() - t0, 1)
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
