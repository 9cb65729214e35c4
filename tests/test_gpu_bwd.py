"""GPU parity of the attention backward (dQ, dK, dV) against the fp64 oracle.

The oracle differentiates the exact definition on the same bf16 Q, K, V, dO;
the GPU recomputes P from the LSE its own forward wrote and takes D = dO . O
from its bf16 O, with bf16 products (P and dS rounded to bf16) and fp32
accumulation."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import softmax_attention_attn_amd as A
    return A


def grad_errors(got, ref, floor):
    """Max and L2 error relative to max(|ref|, floor) and max(||ref||, floor)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), "non-finite gradient"
    err = np.abs(got - ref)
    rmax = max(float(np.abs(ref).max()), floor)
    rl2 = max(float(np.linalg.norm(ref)), floor)
    return {"max_abs": float(err.max()), "ref_max": float(np.abs(ref).max()),
            "rel_max": float(err.max()) / rmax, "rel_l2": float(np.linalg.norm(err)) / rl2}


# Each gradient goes through at most three bf16 roundings the exact math does
# not have (one product operand: P or dS; D from the bf16 O; a bf16 output),
# each within 2^-9 relative: the tolerance is 2^-7 (four half-ulps) on the
# L2 error and 2^-6 on the largest error, both relative to the reference's
# own scale.  A gradient that is exactly zero (one visible key) is measured
# against 1e-2 of the largest reference gradient instead.
REL_MAX = 2.0 ** -6
REL_L2 = 2.0 ** -7


def check_grads(dq, dk, dv, ref, what):
    out = {}
    floor = 1e-2 * max(float(np.abs(r).max()) for r in ref)
    for name, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        e = grad_errors(got.float().cpu().numpy(), r, floor)
        out[name] = e
        assert e["rel_max"] <= REL_MAX and e["rel_l2"] <= REL_L2, "%s %s: %s" % (what, name, e)
    return out


def _run(attn, q, k, v, do, causal, grad_dtype=torch.float32, scale=None):
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = attn.fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = attn.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale,
                          grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return dq, dk, dv


def _ref(q, k, v, do, causal, scale):
    b = workloads.bf16_bits
    return oracle.attn_bwd(b(q), b(k), b(v), b(do), causal=causal, scale=scale)


CASES = [
    # B, H, Hkv, N, d
    (1, 2, 2, 256, 64),
    (2, 4, 2, 300, 128),
    (1, 8, 1, 200, 128),
    (1, 4, 4, 1000, 128),
    (2, 2, 1, 17, 64),
    (1, 2, 2, 1, 128),
    (1, 4, 2, 129, 128),
]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dKV%dN%dd%d" % c)
def test_bwd_small(attn, case, causal):
    B, H, Hkv, N, d = case
    q, k, v, _ = workloads.make_prefill(B, H, Hkv, N, d, seed=N + H)
    do = workloads.make_prefill(B, H, Hkv, N, d, seed=N + H + 1)[0]
    scale = 1 / math.sqrt(d)
    dq, dk, dv = _run(attn, q, k, v, do, causal)
    res = check_grads(dq, dk, dv, _ref(q, k, v, do, causal, scale), str(case))
    print(case, causal, res)


def test_bwd_bf16_grads_and_scale(attn):
    B, H, Hkv, N, d = 1, 4, 2, 333, 128
    q, k, v, _ = workloads.make_prefill(B, H, Hkv, N, d, seed=5)
    do = workloads.make_prefill(B, H, Hkv, N, d, seed=6)[0]
    dq, dk, dv = _run(attn, q, k, v, do, True, grad_dtype=torch.bfloat16, scale=0.3)
    assert dq.dtype == torch.bfloat16
    res = check_grads(dq, dk, dv, _ref(q, k, v, do, True, 0.3), "bf16 grads")
    print("bf16", res)


def test_bwd_llm_prefill_slices(attn):
    """The headline shape (B4 H32 N4096 d128, causal, bf16 gradients); the
    oracle checks eight whole (b, h) slices spread over the batch and heads
    (each self-contained: Hkv = H), stacked into one oracle call."""
    w = workloads.WORKLOADS["llm_prefill"]
    inp = workloads.make(w)
    q, k, v = inp["q"], inp["k"], inp["v"]
    do = workloads.make_prefill(w.B, w.H, w.Hkv, w.N, w.d, seed=1)[0]
    dq, dk, dv = _run(attn, q, k, v, do, True, grad_dtype=torch.bfloat16)
    slices = ((0, 0), (0, 17), (1, 5), (1, 31), (2, 9), (2, 22), (3, 0), (3, 31))
    st = lambda t: torch.cat([t[b:b + 1, h:h + 1] for b, h in slices]).contiguous()
    ref = _ref(st(q), st(k), st(v), st(do), True, w.scale)
    for i, (b, h) in enumerate(slices):
        one = tuple(r[i:i + 1] for r in ref)
        res = check_grads(dq[b:b + 1, h:h + 1], dk[b:b + 1, h:h + 1], dv[b:b + 1, h:h + 1],
                          one, "llm_prefill slice %d,%d" % (b, h))
        print("llm_prefill", b, h, res)


def test_bwd_noncausal_headline_slices(attn):
    """The headline shape without the mask (every query sees every key, so
    no tile of either kernel skips or masks anything), fp32 gradients: two
    whole (b, h) slices against the oracle."""
    w = workloads.WORKLOADS["llm_prefill"]
    inp = workloads.make(w)
    q, k, v = inp["q"], inp["k"], inp["v"]
    do = workloads.make_prefill(w.B, w.H, w.Hkv, w.N, w.d, seed=2)[0]
    dq, dk, dv = _run(attn, q, k, v, do, False)
    slices = ((1, 3), (2, 30))
    st = lambda t: torch.cat([t[b:b + 1, h:h + 1] for b, h in slices]).contiguous()
    ref = _ref(st(q), st(k), st(v), st(do), False, w.scale)
    for i, (b, h) in enumerate(slices):
        one = tuple(r[i:i + 1] for r in ref)
        res = check_grads(dq[b:b + 1, h:h + 1], dk[b:b + 1, h:h + 1], dv[b:b + 1, h:h + 1],
                          one, "llm_prefill non-causal slice %d,%d" % (b, h))
        print("llm_prefill non-causal", b, h, res)


def test_bwd_gqa_headline_size(attn):
    """GQA at the headline size (B4 H32 Hkv8 N4096 d128 causal, bf16
    gradients): a kv head's dK/dV sum the gradients of its 4 query heads.
    Two whole groups, (b, kv head) = (0, 0) and (3, 7), against the oracle."""
    B, H, Hkv, N, d = 4, 32, 8, 4096, 128
    q, k, v, _ = workloads.make_prefill(B, H, Hkv, N, d, seed=11)
    do = workloads.make_prefill(B, H, Hkv, N, d, seed=12)[0]
    dq, dk, dv = _run(attn, q, k, v, do, True, grad_dtype=torch.bfloat16)
    G = H // Hkv
    groups = ((0, 0), (3, 7))
    stq = lambda t: torch.cat([t[b:b + 1, g * G:(g + 1) * G] for b, g in groups]).contiguous()
    stk = lambda t: torch.cat([t[b:b + 1, g:g + 1] for b, g in groups]).contiguous()
    ref = _ref(stq(q), stk(k), stk(v), stq(do), True, 1 / math.sqrt(d))
    for i, (b, g) in enumerate(groups):
        one = tuple(r[i:i + 1] for r in ref)
        res = check_grads(dq[b:b + 1, g * G:(g + 1) * G], dk[b:b + 1, g:g + 1],
                          dv[b:b + 1, g:g + 1], one, "gqa group %d,%d" % (b, g))
        print("gqa headline", b, g, res)


def test_bwd_deterministic(attn):
    """Every gradient element has one writer and a fixed accumulation order
    (no atomics), so two calls on the same inputs agree bit for bit: the
    headline shape with GQA (H32 Hkv8) and both gradient dtypes."""
    B, H, Hkv, N, d = 4, 32, 8, 4096, 128
    q, k, v, _ = workloads.make_prefill(B, H, Hkv, N, d, seed=13)
    do = workloads.make_prefill(B, H, Hkv, N, d, seed=14)[0]
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = attn.fwd(qd, kd, vd, causal=True)
    for gd in (torch.bfloat16, torch.float32):
        first = attn.bwd(qd, kd, vd, o, lse, dod, causal=True, grad_dtype=gd)
        first = [t.clone() for t in first]
        for _ in range(2):
            again = attn.bwd(qd, kd, vd, o, lse, dod, causal=True, grad_dtype=gd)
            torch.cuda.synchronize()
            for a, b_, name in zip(first, again, ("dq", "dk", "dv")):
                assert torch.equal(a, b_), (gd, name)
