"""GPU parity of the MXFP4 quantised prefill (SageAttention3-style FP4
microscaling on MX block formats) against the oracle's step-by-step
emulator of the recipe: Smooth-K, MXFP4 Q/K' per 32 channels, V per 32
tokens and P per 32 keys against the running max of 64-key tiles.

The kernel and the emulator take every Q, K', V code decision on the same
values (bit-exact); they differ only where the kernel's fp32 exponential
(against the emulator's fp64) moves a p across an E2M1 rounding boundary or
the block maximum across a scale boundary, and in the fp32 accumulation
order.  The gates are those of the INT8/FP8 mode: cos >= 0.99999, rel-L1 <=
2e-3 and |dlse| <= 1e-3 with the fp32 store, and a per-row bound at
workload size.  Against exact attention the recipe's own error (FP4 has a
one-bit mantissa) is recorded, not gated: the pages state no tolerance for
this mode.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._compare import cos_rel_l1

pytestmark = pytest.mark.gpu

EMU_COS, EMU_REL, EMU_LSE = 0.99999, 2e-3, 1e-3


@pytest.fixture(scope="module")
def attn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import softmax_attention_attn_amd as A
    return A


def _bits(*ts):
    return [workloads.bf16_bits(t) for t in ts]


def _run(attn, q, k, v, causal, out_dtype=torch.float32):
    o, lse = attn.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, mode="mxfp4",
                      out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _check(o, lse, o_emu, lse_emu, what, rel_tol=EMU_REL):
    assert np.isfinite(o).all() and np.isfinite(lse).all(), what
    cos, rel = cos_rel_l1(o, o_emu)
    dl = float(np.abs(lse - lse_emu).max())
    assert cos >= EMU_COS and rel <= rel_tol and dl <= EMU_LSE, (what, cos, rel, dl)
    return cos, rel, dl


CASES = [
    # B, H, Hkv, N, d, causal
    (1, 2, 2, 64, 128, False),
    (1, 4, 2, 384, 64, False),
    (1, 2, 1, 200, 128, False),
    (2, 4, 2, 300, 64, False),
    (1, 2, 2, 257, 128, True),
    (1, 4, 4, 512, 128, True),
    (2, 8, 2, 1000, 128, True),
    (1, 6, 2, 333, 64, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dKV%dN%dd%d-%s" % (
    c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full"))
def test_small_vs_emulator(attn, case):
    B, H, Hkv, N, d, causal = case
    q, k, v, _ = workloads.make_prefill(B, H, Hkv, N, d, seed=N + d + 1, k_bias_std=3.0)
    o, lse = _run(attn, q, k, v, causal)
    qb, kb, vb = _bits(q, k, v)
    o_emu, lse_emu = oracle.mxfp4_rows(qb, kb, vb, causal=causal, scale=1 / math.sqrt(d))
    res = _check(o, lse, o_emu, lse_emu, str(case))
    o_ex, _, _ = oracle.attn_rows(qb, kb, vb, causal=causal, scale=1 / math.sqrt(d))
    print(case, "vs emulator", res, "vs exact cos %.5f rel-L1 %.4f" % cos_rel_l1(o, o_ex))


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_rising_scores_vs_emulator(attn, causal):
    """Scores that rise from key to key move the running max on almost every
    tile (P is quantised against it)."""
    from tests.test_gpu_prefill import _rising_keys
    B, H, N, d = 1, 2, 600, 128
    q, k, v = _rising_keys(B, H, H, N, d, seed=78, top=25.0)
    o, lse = _run(attn, q, k, v, causal)
    qb, kb, vb = _bits(q, k, v)
    o_emu, lse_emu = oracle.mxfp4_rows(qb, kb, vb, causal=causal, scale=1 / math.sqrt(d))
    _check(o, lse, o_emu, lse_emu, "rising scores causal=%s" % causal)


def test_bf16_store(attn):
    B, H, N, d = 1, 2, 256, 128
    q, k, v, _ = workloads.make_prefill(B, H, H, N, d, seed=32, k_bias_std=10.0)
    o, lse = _run(attn, q, k, v, False, out_dtype=torch.bfloat16)
    qb, kb, vb = _bits(q, k, v)
    o_emu, lse_emu = oracle.mxfp4_rows(qb, kb, vb, causal=False, scale=1 / math.sqrt(d))
    _check(o, lse, o_emu, lse_emu, "bf16 store", rel_tol=5e-3)  # plus bf16 rounding of O


# Per-row rel-L1 against the emulator at workload size: as in the INT8/FP8
# mode, a flip of one key's P^ moves a near-uniform row by a per-cent; the
# bound is that mode's 2^-5.
EMU_ROW_REL = 2.0 ** -5


def test_workload_sampled(attn):
    """The B2 H24 N16384 d128 inputs of the quantised-prefill workload in the
    MXFP4 mode, fp32 store, on a declared sample: one whole (b, h) slice, the
    tile-edge and last rows of every slice, 2048 seeded random rows."""
    w = workloads.WORKLOADS["sage_prefill"]
    inp = workloads.make(w)
    q, k, v = inp["q"], inp["k"], inp["v"]
    rows = workloads.sample_rows(w.B, w.H, w.N, n_random=2048, whole_slices=((w.B - 1, 5),))
    o, lse = attn.fwd(q.cuda(), k.cuda(), v.cuda(), causal=w.causal, mode="mxfp4",
                      out_dtype=torch.float32)
    torch.cuda.synchronize()
    o = o.cpu().numpy().reshape(-1, w.d)[rows]
    lse = lse.cpu().numpy().reshape(-1)[rows]
    qb, kb, vb = _bits(q, k, v)
    o_emu, lse_emu = oracle.mxfp4_rows(qb, kb, vb, causal=w.causal, scale=w.scale, rows=rows)
    cos, rel, dl = _check(o, lse, o_emu, lse_emu, "mxfp4 workload")
    row = np.abs(o - o_emu).sum(axis=1) / np.abs(o_emu).sum(axis=1)
    o_ex, _, _ = oracle.attn_rows(qb, kb, vb, causal=w.causal, scale=w.scale, rows=rows)
    cos_x, rel_x = cos_rel_l1(o, o_ex)
    print("mxfp4 %d rows: vs emulator cos %.7f rel-L1 %.2e max |dlse| %.2e per-row max %.2e; "
          "vs exact cos %.5f rel-L1 %.4f" % (len(rows), cos, rel, dl, row.max(), cos_x, rel_x))
    assert row.max() <= EMU_ROW_REL, row.max()


def test_without_lse(attn):
    """lse is optional: O is the same with and without it."""
    B, H, N, d = 1, 2, 200, 128
    q, k, v, _ = workloads.make_prefill(B, H, H, N, d, seed=40, k_bias_std=3.0)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    o1, _ = attn.fwd(q, k, v, causal=True, mode="mxfp4", out_dtype=torch.float32)
    o2 = torch.empty_like(o1)
    attn.fwd(q, k, v, causal=True, mode="mxfp4", o=o2, with_lse=False, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
