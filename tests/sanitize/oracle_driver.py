"""Run every oracle routine on small inputs against a sanitizer build of
oracle.c (ASan + UBSan).  Run by tests/test_sanitizers.py in a child process
with the sanitizer runtimes preloaded; argv[1] is the sanitizer build of
liboracle.so.  Exits 0 when every routine ran and returned finite values; a
sanitizer report aborts the process with a non-zero status."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle  # noqa: E402

oracle._LIB_PATH = sys.argv[1]
oracle._lib = None

rng = np.random.default_rng(0)


def bf16(shape, scale=1.0):
    """bf16 bit patterns of N(0, scale^2) values (truncated fp32)."""
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def finite(*arrs):
    for a in arrs:
        assert np.isfinite(np.asarray(a, dtype=np.float64)).all()


B, H, Hkv, N, d = 2, 4, 2, 70, 64
q, k, v = bf16((B, H, N, d)), bf16((B, Hkv, N, d)), bf16((B, Hkv, N, d))
for causal in (False, True):
    finite(*oracle.attn_rows(q, k, v, causal=causal, scale=0.125)[:2])
    finite(*oracle.attn_rows(q, k, v, causal=causal, scale=0.125, rows=[0, 5, 279, 559])[:2])
    finite(*oracle.sage_rows(q, k, v, causal=causal, scale=0.125))
    finite(*oracle.mxfp4_rows(q, k, v, causal=causal, scale=0.125))
    do = bf16((B, H, N, d))
    finite(*oracle.attn_bwd(q, k, v, do, causal=causal, scale=0.125))
finite(*oracle.sage_quantise(q, k, v).values())
finite(*oracle.attn_rows(q, k, v, causal=False, scale=0.125, k_range=(10, 50))[:2])
# decode: one query row per (b, h) over kv_len valid keys
qd = bf16((B, H, 1, d))
finite(*oracle.attn_rows(qd, k, v, causal=False, scale=0.125, kv_len=[70, 3])[:2])
# packed batch with an empty and a one-token sequence
cu = np.array([0, 0, 1, 40, 90], dtype=np.int32)
qp, kp, vp = bf16((90, H, d)), bf16((90, Hkv, d)), bf16((90, Hkv, d))
finite(*oracle.attn_varlen(qp, kp, vp, cu, causal=True, scale=0.125)[:2])
# merge of partials
o_parts = rng.standard_normal((3, 5, d))
lse_parts = rng.standard_normal((3, 5))
finite(*oracle.lse_merge(o_parts, lse_parts))
# element formats over their whole range
oracle.e4m3_decode(np.arange(256))  # two of the codes are NaN
oracle.e4m3_encode(np.linspace(-600, 600, 2001))
finite(oracle.e2m1_decode(np.arange(16)))
oracle.e2m1_encode(np.linspace(-10, 10, 2001))
oracle.mx_scale_exp(np.array([0.0, 1e-40, 1e-3, 1.0, 6.0, 7.0, 1e30, 3e38]))
oracle.quant_i8(np.linspace(-300, 300, 601), 1.0)
print("oracle driver: every routine ran")
