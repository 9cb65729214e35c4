"""Comparison helpers shared by the parity tests (no attention arithmetic)."""
from __future__ import annotations

import numpy as np

# Exact mode: max |dO| <= 1e-2 and relative LSE error <= 1e-3.
#  * literal=True (the five stated workloads, where the gate is stated): every
#    element within 1e-2, and |dlse| / |lse_ref| <= 1e-3; rows whose reference
#    LSE is within 1e-2 of zero, where a relative error means nothing, get
#    |dlse| <= 1e-5 instead (the fp32 LSE's own rounding is ~1e-6 there).
#  * literal=False (small shapes and stress cases): a bf16 output additionally
#    gets half a bf16 ulp of the reference value, the rounding any bf16 store
#    must make, and the LSE error is |dlse| / max(|lse_ref|, 1).
O_ABS_TOL = 1e-2
LSE_REL_TOL = 1e-3
LSE_NEAR_ZERO, LSE_ABS_TOL_NEAR_ZERO = 1e-2, 1e-5


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 0.5 * 2.0 ** (e - 7)


def check_exact(o_gpu: np.ndarray, o_ref: np.ndarray, lse_gpu, lse_ref, *, bf16_out: bool,
                what: str = "", literal: bool = False):
    """Assert the exact-mode tolerances; returns a dict of the measured errors."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.isfinite(o_gpu).all(), "%s: non-finite output" % what
    err = np.abs(o_gpu - o_ref)
    bound = O_ABS_TOL + (bf16_half_ulp(o_ref) if bf16_out and not literal else 0.0)
    bad = err > bound
    res = {"max_abs_dO": float(err.max()), "n_over_1e-2": int((err > O_ABS_TOL).sum()),
           "n_over_bound": int(bad.sum())}
    assert not bad.any(), "%s: %d elements over tolerance, max |dO| %.4g at %s" % (
        what, int(bad.sum()), err.max(), np.unravel_index(err.argmax(), err.shape))
    if lse_gpu is not None:
        lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
        lse_ref = np.asarray(lse_ref, dtype=np.float64)
        assert np.isfinite(lse_gpu).all(), "%s: non-finite lse" % what
        dl = np.abs(lse_gpu - lse_ref)
        if literal:
            near0 = np.abs(lse_ref) < LSE_NEAR_ZERO
            rel = dl[~near0] / np.abs(lse_ref[~near0])
            res["max_rel_dlse"] = float(rel.max()) if rel.size else 0.0
            res["n_lse_near_zero"] = int(near0.sum())
            if near0.any():
                res["max_abs_dlse_near_zero"] = float(dl[near0].max())
                assert dl[near0].max() <= LSE_ABS_TOL_NEAR_ZERO, (
                    "%s: |dlse| %.3g where |lse| < %g" % (what, dl[near0].max(), LSE_NEAR_ZERO))
        else:
            rel = dl / np.maximum(np.abs(lse_ref), 1.0)
            res["max_rel_dlse"] = float(rel.max())
        assert res["max_rel_dlse"] <= LSE_REL_TOL, "%s: lse rel err %.3g" % (
            what, res["max_rel_dlse"])
    return res


def cos_rel_l1(o: np.ndarray, ref: np.ndarray):
    o = np.asarray(o, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    cos = float(o @ ref / (np.linalg.norm(o) * np.linalg.norm(ref)))
    rel = float(np.abs(o - ref).sum() / np.abs(ref).sum())
    return cos, rel
