"""GPU parity of the MXFP6 quantised prefill (the MX recipe with OCP E2M3
elements: Smooth-K, MXFP6 Q/K' per 32 channels, V per 32 tokens and P per
32 keys against the running max of 64-key tiles) against the oracle's
step-by-step emulator.

As in the MXFP4 mode, the kernel and the emulator take every Q, K', V code
decision on the same values; they differ where the kernel's fp32
exponential moves a p across an E2M3 rounding boundary or a block maximum
across a scale boundary, and in the fp32 accumulation order.  The gates are
the MXFP4 mode's.  One case puts every Q, K and V element that is not a
block maximum on an exact midpoint between two E2M3 values, so that a
conversion that did not round ties to even would move every score.
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
EMU_ROW_REL = 2.0 ** -5


@pytest.fixture(scope="module")
def attn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import softmax_attention_attn_amd as A
    return A


def _bits(*ts):
    return [workloads.bf16_bits(t) for t in ts]


def _run(attn, q, k, v, causal, out_dtype=torch.float32):
    o, lse = attn.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, mode="mxfp6",
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
    (1, 2, 2, 1, 64, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dKV%dN%dd%d-%s" % (
    c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full"))
def test_small_vs_emulator(attn, case):
    B, H, Hkv, N, d, causal = case
    q, k, v, _ = workloads.make_prefill(B, H, Hkv, N, d, seed=N + d + 7, k_bias_std=3.0)
    o, lse = _run(attn, q, k, v, causal)
    qb, kb, vb = _bits(q, k, v)
    o_emu, lse_emu = oracle.mxfp6_rows(qb, kb, vb, causal=causal, scale=1 / math.sqrt(d))
    res = _check(o, lse, o_emu, lse_emu, str(case))
    o_ex, _, _ = oracle.attn_rows(qb, kb, vb, causal=causal, scale=1 / math.sqrt(d))
    print(case, "vs emulator", res, "vs exact cos %.5f rel-L1 %.4f" % cos_rel_l1(o, o_ex))


def _midpoint_tensor(shape, rng):
    """Every block of 32 along the last axis holds one 7.5 (its maximum, so
    its scale is 2^0) and otherwise exact midpoints between neighbouring
    E2M3 magnitudes, with random signs; all are bf16 values."""
    pos = np.concatenate([np.arange(16) / 8, 2 + np.arange(8) / 4, 4 + np.arange(8) / 2])
    mids = (pos[1:] + pos[:-1]) / 2
    x = rng.choice(mids, shape) * rng.choice([-1.0, 1.0], shape)
    x[..., ::32] = 7.5
    return x


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_ties_round_to_even(attn, causal):
    """Q, K and V made of exact E2M3 midpoints (K rows in +- pairs, so the
    Smooth-K mean is exactly 0 and K' = K; V's blocks run along tokens, so
    V is built token-major with its maxima on tokens 0, 32, ...)."""
    rng = np.random.default_rng(21)
    B, H, N, d = 1, 2, 128, 128
    q = _midpoint_tensor((B, H, N, d), rng) * 0.25
    khalf = _midpoint_tensor((B, H, N // 2, d), rng) * 0.125
    k = np.concatenate([khalf, -khalf], axis=2)
    v = np.ascontiguousarray(np.swapaxes(_midpoint_tensor((B, H, d, N), rng), 2, 3)) * 0.5
    src = (q, k, v)
    q, k, v = (torch.tensor(t, dtype=torch.bfloat16) for t in src)
    for t, x in zip((q, k, v), src):  # every value is a bf16 value
        assert np.array_equal(t.double().numpy(), x)
    qb, kb, vb = _bits(q, k, v)
    o, lse = _run(attn, q, k, v, causal)
    o_emu, lse_emu = oracle.mxfp6_rows(qb, kb, vb, causal=causal, scale=1 / math.sqrt(d))
    _check(o, lse, o_emu, lse_emu, "midpoints causal=%s" % causal)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_rising_scores_vs_emulator(attn, causal):
    """Scores that rise from key to key move the running max on almost every
    tile (P is quantised against it)."""
    from tests.test_gpu_prefill import _rising_keys
    B, H, N, d = 1, 2, 600, 128
    q, k, v = _rising_keys(B, H, H, N, d, seed=79, top=25.0)
    o, lse = _run(attn, q, k, v, causal)
    qb, kb, vb = _bits(q, k, v)
    o_emu, lse_emu = oracle.mxfp6_rows(qb, kb, vb, causal=causal, scale=1 / math.sqrt(d))
    _check(o, lse, o_emu, lse_emu, "rising scores causal=%s" % causal)


def test_bf16_store(attn):
    B, H, N, d = 1, 2, 256, 128
    q, k, v, _ = workloads.make_prefill(B, H, H, N, d, seed=33, k_bias_std=10.0)
    o, lse = _run(attn, q, k, v, False, out_dtype=torch.bfloat16)
    qb, kb, vb = _bits(q, k, v)
    o_emu, lse_emu = oracle.mxfp6_rows(qb, kb, vb, causal=False, scale=1 / math.sqrt(d))
    _check(o, lse, o_emu, lse_emu, "bf16 store", rel_tol=5e-3)  # plus bf16 rounding of O


def test_more_accurate_than_mxfp4(attn):
    """The same inputs in both MX modes: against exact attention the FP6
    recipe's rel-L1 is several times below the FP4 recipe's."""
    B, H, N, d = 1, 4, 1024, 128
    q, k, v, _ = workloads.make_prefill(B, H, H, N, d, seed=5, k_bias_std=3.0)
    qb, kb, vb = _bits(q, k, v)
    o_ex, _, _ = oracle.attn_rows(qb, kb, vb, causal=True, scale=1 / math.sqrt(d))
    o6, _ = _run(attn, q, k, v, True)
    o4, _ = attn.fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, mode="mxfp4",
                     out_dtype=torch.float32)
    rel6 = cos_rel_l1(o6, o_ex)[1]
    rel4 = cos_rel_l1(o4.cpu().numpy(), o_ex)[1]
    print("rel-L1 vs exact: mxfp6 %.4f mxfp4 %.4f" % (rel6, rel4))
    assert rel6 < 0.1 and rel4 > 3 * rel6, (rel6, rel4)


def test_workload_sampled(attn):
    """The B2 H24 N16384 d128 inputs of the quantised-prefill workload in the
    MXFP6 mode, fp32 store, on a declared sample: one whole (b, h) slice, the
    tile-edge and last rows of every slice, 2048 seeded random rows."""
    w = workloads.WORKLOADS["sage_prefill"]
    inp = workloads.make(w)
    q, k, v = inp["q"], inp["k"], inp["v"]
    rows = workloads.sample_rows(w.B, w.H, w.N, n_random=2048, whole_slices=((w.B - 1, 5),))
    o, lse = attn.fwd(q.cuda(), k.cuda(), v.cuda(), causal=w.causal, mode="mxfp6",
                      out_dtype=torch.float32)
    torch.cuda.synchronize()
    o = o.cpu().numpy().reshape(-1, w.d)[rows]
    lse = lse.cpu().numpy().reshape(-1)[rows]
    qb, kb, vb = _bits(q, k, v)
    o_emu, lse_emu = oracle.mxfp6_rows(qb, kb, vb, causal=w.causal, scale=w.scale, rows=rows)
    cos, rel, dl = _check(o, lse, o_emu, lse_emu, "mxfp6 workload")
    row = np.abs(o - o_emu).sum(axis=1) / np.abs(o_emu).sum(axis=1)
    o_ex, _, _ = oracle.attn_rows(qb, kb, vb, causal=w.causal, scale=w.scale, rows=rows)
    cos_x, rel_x = cos_rel_l1(o, o_ex)
    print("mxfp6 %d rows: vs emulator cos %.7f rel-L1 %.2e max |dlse| %.2e per-row max %.2e; "
          "vs exact cos %.5f rel-L1 %.4f" % (len(rows), cos, rel, dl, row.max(), cos_x, rel_x))
    assert row.max() <= EMU_ROW_REL, row.max()


@pytest.mark.parametrize("mode", ["sage", "mxfp4", "mxfp6"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_quantised_modes_deterministic_and_in_bounds(attn, mode, causal):
    """Every quantised mode gives bitwise the same result on a second call,
    and on inputs embedded in NaN-filled storage (a read past a tensor's end
    would poison the output)."""
    B, H, Hkv, N, d = 1, 4, 2, 333, 128
    q, k, v, _ = workloads.make_prefill(B, H, Hkv, N, d, seed=17, k_bias_std=3.0)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = attn.fwd(q, k, v, causal=causal, mode=mode, out_dtype=torch.float32)
    o2, l2 = attn.fwd(q, k, v, causal=causal, mode=mode, out_dtype=torch.float32)
    dev = []
    for t in (q, k, v):
        buf = torch.full((t.numel() + 8192,), float("nan"), dtype=torch.bfloat16, device="cuda")
        buf[: t.numel()] = t.reshape(-1)
        dev.append(buf[: t.numel()].view(t.shape))
    o3, l3 = attn.fwd(*dev, causal=causal, mode=mode, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all() and torch.isfinite(l1).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_without_lse(attn):
    """lse is optional: O is the same with and without it."""
    B, H, N, d = 1, 2, 200, 128
    q, k, v, _ = workloads.make_prefill(B, H, H, N, d, seed=40, k_bias_std=3.0)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    o1, _ = attn.fwd(q, k, v, causal=True, mode="mxfp6", out_dtype=torch.float32)
    o2 = torch.empty_like(o1)
    attn.fwd(q, k, v, causal=True, mode="mxfp6", o=o2, with_lse=False, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
