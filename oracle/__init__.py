"""fp64 CPU oracle for softmax attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never calls it and it
imports nothing from the product package: the two share no code.

Everything is computed in double precision by the plain C routines in
``oracle.c`` (explicit score and probability rows, no tiling), wrapped here
with ctypes over numpy arrays.  Inputs are bf16 bit patterns held in numpy
``uint16`` arrays; outputs are float64.

What each routine follows:

* ``attn_rows`` -- exact attention O = softmax(Q K^T * scale + mask) V and its
  natural-log LSE ("flashattention-kernels" page, §0/§1: tiling and online
  softmax preserve exact attention; "cuda-kernel-pretrain" page, §2).  Also the
  decode case (one query row, ``kv_len`` valid keys) and partial attention over
  a key range (Flash-Decoding's chunks, "flashattention-kernels" page, §3).
* ``attn_bwd`` -- the gradients of exact attention (dQ, dK, dV for an
  upstream dO), by the chain rule through the explicit softmax row by row
  (the backward pass the training kernels of the pages compute: "GPU kernel
  overview" page, SageBwd; "flashattention-kernels" page §0, FA2/FA3).
* ``attn_varlen`` -- the same over a packed batch of variable-length
  sequences, each attending only to its own tokens (packing without padding,
  "flashattention-kernels" page, recommendation table and §3).
* ``lse_merge`` -- the reduction that combines per-chunk partial results
  (same page, §3; the pages give no formula, the log-sum-exp weighting used
  here is the unique one that reproduces the unsplit softmax).
* ``sage_rows`` / ``sage_quantise`` -- the quantised recipe (Smooth-K, INT8
  Q/K per 64-token block, E4M3 P and per-channel E4M3 V, fp32 accumulation)
  emulated step by step ("GPU kernel overview" page, SageAttention chain and
  its insight that QK suits INT8 while PV suits FP8).
* ``mxfp4_rows`` -- the MXFP4 variant of the quantised recipe (SageAttention3's
  FP4 microscaling on CDNA4's MX formats: E2M1 elements with a power-of-two
  E8M0 scale per block of 32, for Q, K, V and P; "gpu-kernel-porting-with-ai-agents"
  page, SageAttention 3 section; "GPU kernel overview" page, insights on FP4).
* ``mx_rows`` -- the same recipe with the element format as a parameter:
  E2M1 (``mxfp4_rows``) or the MX FP6 format E2M3 (``mxfp6_rows``); the
  "GPU kernel overview" page's insights name FP4 and FP6 as the low-bit
  formats of CDNA4's matrix cores.
* ``e4m3_decode`` / ``e4m3_encode`` -- the OCP E4M3 ("fn") format;
  ``e2m1_decode`` / ``e2m1_encode`` / ``mx_scale_exp`` -- the MX FP4 element
  format and the choice of a block's scale; ``e2m3_decode`` /
  ``e2m3_encode`` / ``mx_scale_exp_max`` -- the MX FP6 element format and the
  scale rule for a format of any largest magnitude.
* ``gather_pages`` -- the paged KV layout (a pool of fixed-size pages named by
  a per-sequence page table) turned back into contiguous caches, so that
  paged decode is checked against ``attn_rows`` ("flashattention-kernels"
  page, §3: paged KV among the layouts a decode library covers).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_f64p = ctypes.POINTER(ctypes.c_double)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i8p = ctypes.POINTER(ctypes.c_int8)


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_attn_rows.restype = ctypes.c_double
    lib.oracle_attn_rows.argtypes = [
        _u16p, _u16p, _u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_double, _i64p, ctypes.c_int64, _f64p, _f64p, ctypes.c_int]
    lib.oracle_attn_bwd.restype = ctypes.c_int
    lib.oracle_attn_bwd.argtypes = [_u16p, _u16p, _u16p, _u16p] + [ctypes.c_int] * 6 + [
        ctypes.c_double, _f64p, _f64p, _f64p, ctypes.c_int]
    lib.oracle_lse_merge.restype = None
    lib.oracle_lse_merge.argtypes = [_f64p, _f64p, ctypes.c_int, ctypes.c_int64,
                                     ctypes.c_int, _f64p, _f64p]
    lib.oracle_sage_rows.restype = ctypes.c_double
    lib.oracle_sage_rows.argtypes = [
        _u16p, _u16p, _u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
        ctypes.c_int, _i64p, ctypes.c_int64, _f64p, _f64p, ctypes.c_int]
    lib.oracle_sage_quantise.restype = ctypes.c_int
    lib.oracle_sage_quantise.argtypes = [
        _u16p, _u16p, _u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64p, _i8p, _f64p, _i8p, _f64p,
        _f64p, _f64p]
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_quant_i8.restype = ctypes.c_int
    lib.oracle_quant_i8.argtypes = [ctypes.c_double, ctypes.c_double]
    lib.oracle_e2m1_decode.restype = ctypes.c_double
    lib.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_encode.restype = ctypes.c_uint8
    lib.oracle_e2m1_encode.argtypes = [ctypes.c_double]
    lib.oracle_mx_scale_exp.restype = ctypes.c_int
    lib.oracle_mx_scale_exp.argtypes = [ctypes.c_double]
    lib.oracle_e2m3_decode.restype = ctypes.c_double
    lib.oracle_e2m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m3_encode.restype = ctypes.c_uint8
    lib.oracle_e2m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_mx_scale_exp_max.restype = ctypes.c_int
    lib.oracle_mx_scale_exp_max.argtypes = [ctypes.c_double, ctypes.c_double]
    lib.oracle_mx_rows.restype = ctypes.c_double
    lib.oracle_mx_rows.argtypes = [
        _u16p, _u16p, _u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64p, ctypes.c_int64, _f64p, _f64p,
        ctypes.c_int]
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are bf16 bit patterns (numpy uint16), got %s" % a.dtype)
    return a


def _ptr(a, t):
    return a.ctypes.data_as(t)


def default_threads() -> int:
    """Host threads for the oracle: the affinity mask, capped by
    OMP_NUM_THREADS (else 16) so that a shared host is not oversubscribed."""
    n = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "16"))
    except ValueError:
        cap = 16
    return max(1, min(n, cap if cap > 0 else 16))


def attn_rows(q, k, v, *, causal: bool, scale: float, rows=None, kv_len=None,
              k_range=None, threads: int | None = None):
    """Exact attention rows in fp64.

    q: [B,H,Nq,d]; k, v: [B,Hkv,Nk,d] (uint16 bf16 bits).  ``rows`` lists
    flattened (b*H + h)*Nq + i indices (None: all rows, returned as
    [B,H,Nq,d] / [B,H,Nq]).  ``kv_len`` [B] limits the visible keys per batch.
    ``k_range`` (lo, hi) restricts the keys to [lo, hi).
    Returns (o, lse, max |1 - sum P|).
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, H, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, dk) != (B, d) or v.shape != k.shape:
        raise ValueError("shape mismatch")
    lib = _load()
    if rows is None:
        nrows = B * H * Nq
        rows_p = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows.size
        rows_p = _ptr(rows, _i64p)
    o = np.empty((nrows, d), dtype=np.float64)
    lse = np.empty((nrows,), dtype=np.float64)
    kl = None
    if kv_len is not None:
        kv_len = np.ascontiguousarray(kv_len, dtype=np.int32)
        kl = _ptr(kv_len, _i32p)
    lo, hi = (0, Nk) if k_range is None else k_range
    err = lib.oracle_attn_rows(_ptr(q, _u16p), _ptr(k, _u16p), _ptr(v, _u16p), B, H, Hkv,
                               Nq, Nk, d, int(bool(causal)), kl, int(lo), int(hi),
                               float(scale), rows_p, nrows, _ptr(o, _f64p),
                               _ptr(lse, _f64p), int(threads or default_threads()))
    if err < 0:
        raise ValueError("oracle_attn_rows rejected its arguments")
    if rows is None:
        o = o.reshape(B, H, Nq, d)
        lse = lse.reshape(B, H, Nq)
    return o, lse, err


def attn_bwd(q, k, v, dout, *, causal: bool, scale: float, threads: int | None = None):
    """Gradients (dq, dk, dv) of exact attention for the upstream gradient
    ``dout``, in fp64 (chain rule through the explicit softmax, row by row;
    a kv head's gradients sum over its query heads).

    q, dout [B,H,N,d]; k, v [B,Hkv,N,d] (uint16 bf16 bits).
    """
    q, k, v, dout = _u16(q), _u16(k), _u16(v), _u16(dout)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch")
    dq = np.empty((B, H, N, d), dtype=np.float64)
    dk = np.empty((B, Hkv, N, d), dtype=np.float64)
    dv = np.empty((B, Hkv, N, d), dtype=np.float64)
    err = _load().oracle_attn_bwd(_ptr(q, _u16p), _ptr(k, _u16p), _ptr(v, _u16p),
                                  _ptr(dout, _u16p), B, H, Hkv, N, d, int(bool(causal)),
                                  float(scale), _ptr(dq, _f64p), _ptr(dk, _f64p), _ptr(dv, _f64p),
                                  int(threads or default_threads()))
    if err < 0:
        raise ValueError("oracle_attn_bwd rejected its arguments")
    return dq, dk, dv


def attn_varlen(q, k, v, cu_seqlens, *, causal: bool, scale: float,
                threads: int | None = None):
    """Exact attention over a packed batch: each sequence attends only to its
    own tokens (sequence b holds tokens [cu_seqlens[b], cu_seqlens[b+1])).

    q [total,H,d], k/v [total,Hkv,d] (uint16 bf16 bits), token-major.
    Returns (o [total,H,d], lse [H,total]) in float64, computed sequence by
    sequence with ``attn_rows``; empty sequences contribute nothing.
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    total, H, d = q.shape
    cu = [int(x) for x in np.asarray(cu_seqlens)]
    o = np.zeros((total, H, d), dtype=np.float64)
    lse = np.zeros((H, total), dtype=np.float64)
    for t0, t1 in zip(cu[:-1], cu[1:]):
        if t1 <= t0:
            continue
        qs = np.ascontiguousarray(q[t0:t1].transpose(1, 0, 2))[None]
        ks = np.ascontiguousarray(k[t0:t1].transpose(1, 0, 2))[None]
        vs = np.ascontiguousarray(v[t0:t1].transpose(1, 0, 2))[None]
        os_, ls, _ = attn_rows(qs, ks, vs, causal=causal, scale=scale, threads=threads)
        o[t0:t1] = os_[0].transpose(1, 0, 2)
        lse[:, t0:t1] = ls[0]
    return o, lse


def lse_merge(o_parts, lse_parts):
    """Merge partial (O_s, lse_s) over disjoint key sets.

    o_parts [S, R, d], lse_parts [S, R] (float64).  Returns (o [R,d], lse [R]).
    """
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    S, R, d = o_parts.shape
    o = np.empty((R, d), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64)
    _load().oracle_lse_merge(_ptr(o_parts, _f64p), _ptr(lse_parts, _f64p), S, R, d,
                             _ptr(o, _f64p), _ptr(lse, _f64p))
    return o, lse


def sage_rows(q, k, v, *, causal: bool, scale: float, rows=None, blk: int = 64,
              tile_n: int = 64, smooth_k: bool = True, quant_qk: bool = True,
              quant_p: bool = True, quant_v: bool = True, p_scale: float = 448.0,
              l_from_quantised_p: bool = False, threads: int | None = None):
    """Quantised (SageAttention-style) attention emulated step by step in fp64.

    Same shapes and ``rows`` convention as :func:`attn_rows` (Nq == Nk == N).
    ``tile_n`` is the key-tile width of the online softmax, which decides the
    running max that P is quantised against.  ``smooth_k``, ``quant_qk``,
    ``quant_p`` and ``quant_v`` switch single steps of the recipe off (for
    attributing its error to its sources); ``l_from_quantised_p`` sums the
    quantised P instead of the unrounded one into the row sum (an alternative
    reading).  Returns (o, lse).
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape:
        raise ValueError("shape mismatch")
    if rows is None:
        nrows = B * H * N
        rows_p = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows.size
        rows_p = _ptr(rows, _i64p)
    o = np.empty((nrows, d), dtype=np.float64)
    lse = np.empty((nrows,), dtype=np.float64)
    r = _load().oracle_sage_rows(_ptr(q, _u16p), _ptr(k, _u16p), _ptr(v, _u16p), B, H, Hkv, N,
                                 d, int(bool(causal)), float(scale), int(blk), int(tile_n),
                                 int(smooth_k), int(quant_qk), int(quant_p), int(quant_v),
                                 float(p_scale), int(bool(l_from_quantised_p)), rows_p,
                                 nrows, _ptr(o, _f64p),
                                 _ptr(lse, _f64p), int(threads or default_threads()))
    if r < 0:
        raise ValueError("oracle_sage_rows rejected its arguments")
    if rows is None:
        o = o.reshape(B, H, N, d)
        lse = lse.reshape(B, H, N)
    return o, lse


def sage_quantise(q, k, v, *, blk: int = 64, smooth_k: bool = True):
    """Quantisation state of the recipe (see ``oracle_sage_quantise`` in oracle.c)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    nb = (N + blk - 1) // blk
    out = dict(
        kmean=np.empty((B, Hkv, d)), qhat=np.empty((B, H, N, d), dtype=np.int8),
        qdelta=np.empty((B, H, nb)), khat=np.empty((B, Hkv, N, d), dtype=np.int8),
        kdelta=np.empty((B, Hkv, nb)), vq=np.empty((B, Hkv, N, d)),
        vdelta=np.empty((B, Hkv, d)))
    r = _load().oracle_sage_quantise(
        _ptr(q, _u16p), _ptr(k, _u16p), _ptr(v, _u16p), B, H, Hkv, N, d, int(blk),
        int(smooth_k), _ptr(out["kmean"], _f64p), _ptr(out["qhat"], _i8p),
        _ptr(out["qdelta"], _f64p), _ptr(out["khat"], _i8p), _ptr(out["kdelta"], _f64p),
        _ptr(out["vq"], _f64p), _ptr(out["vdelta"], _f64p))
    if r < 0:
        raise ValueError("oracle_sage_quantise rejected its arguments")
    return out


MX_ELEMS = {"e2m1": 0, "e2m3": 1}


def mx_rows(q, k, v, *, causal: bool, scale: float, elem: str, rows=None, tile_n: int = 64,
            smooth_k: bool = True, quant_qk: bool = True, quant_p: bool = True,
            quant_v: bool = True, threads: int | None = None):
    """MX quantised attention (SageAttention3-style, MX block formats) with
    elements ``elem`` ("e2m1": MXFP4, "e2m3": MXFP6), emulated step by step in
    fp64; see ``oracle_mx_rows`` in oracle.c.  Same shapes and ``rows``
    convention as :func:`sage_rows`.  Returns (o, lse)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape:
        raise ValueError("shape mismatch")
    if rows is None:
        nrows = B * H * N
        rows_p = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows.size
        rows_p = _ptr(rows, _i64p)
    o = np.empty((nrows, d), dtype=np.float64)
    lse = np.empty((nrows,), dtype=np.float64)
    r = _load().oracle_mx_rows(_ptr(q, _u16p), _ptr(k, _u16p), _ptr(v, _u16p), B, H, Hkv, N,
                               d, int(bool(causal)), float(scale), int(tile_n), MX_ELEMS[elem],
                               int(smooth_k), int(quant_qk), int(quant_p), int(quant_v),
                               rows_p, nrows, _ptr(o, _f64p), _ptr(lse, _f64p),
                               int(threads or default_threads()))
    if r < 0:
        raise ValueError("oracle_mx_rows rejected its arguments")
    if rows is None:
        o = o.reshape(B, H, N, d)
        lse = lse.reshape(B, H, N)
    return o, lse


def mxfp4_rows(q, k, v, **kw):
    """:func:`mx_rows` with E2M1 elements (the MXFP4 recipe)."""
    return mx_rows(q, k, v, elem="e2m1", **kw)


def mxfp6_rows(q, k, v, **kw):
    """:func:`mx_rows` with E2M3 elements (the MXFP6 recipe)."""
    return mx_rows(q, k, v, elem="e2m3", **kw)


def e2m1_decode(codes) -> np.ndarray:
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e2m1_decode(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def e2m1_encode(x) -> np.ndarray:
    lib = _load()
    x = np.asarray(x, dtype=np.float64)
    return np.array([lib.oracle_e2m1_encode(float(t)) for t in x.ravel()],
                    dtype=np.uint8).reshape(x.shape)


def mx_scale_exp(amax) -> np.ndarray:
    lib = _load()
    a = np.asarray(amax, dtype=np.float64)
    return np.array([lib.oracle_mx_scale_exp(float(t)) for t in a.ravel()],
                    dtype=np.int64).reshape(a.shape)


def e2m3_decode(codes) -> np.ndarray:
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e2m3_decode(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def e2m3_encode(x) -> np.ndarray:
    lib = _load()
    x = np.asarray(x, dtype=np.float64)
    return np.array([lib.oracle_e2m3_encode(float(t)) for t in x.ravel()],
                    dtype=np.uint8).reshape(x.shape)


def mx_scale_exp_max(amax, emax: float) -> np.ndarray:
    lib = _load()
    a = np.asarray(amax, dtype=np.float64)
    return np.array([lib.oracle_mx_scale_exp_max(float(t), float(emax)) for t in a.ravel()],
                    dtype=np.int64).reshape(a.shape)


def e4m3_decode(codes) -> np.ndarray:
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e4m3_decode(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def e4m3_encode(x) -> np.ndarray:
    lib = _load()
    x = np.asarray(x, dtype=np.float64)
    return np.array([lib.oracle_e4m3_encode(float(t)) for t in x.ravel()],
                    dtype=np.uint8).reshape(x.shape)


def quant_i8(x, delta) -> np.ndarray:
    lib = _load()
    x = np.asarray(x, dtype=np.float64)
    return np.array([lib.oracle_quant_i8(float(t), float(delta)) for t in x.ravel()],
                    dtype=np.int64).reshape(x.shape)


def gather_pages(pages, block_table, seqlens, page_size: int):
    """Contiguous caches from a paged pool, by the paged layout's definition.

    pages [num_pages, Hkv, page_size, d] (any dtype); block_table [B, max_pages]
    (int); seqlens [B].  Key position n of sequence b is row n % page_size of
    page block_table[b, n // page_size] ("flashattention-kernels" page, §3:
    the paged KV layouts a decode library covers).  Returns
    [B, Hkv, max_pages * page_size, d] with positions >= seqlens[b] zero.
    Plain loops over positions: this is the definition, not a fast path.
    """
    pages = np.asarray(pages)
    block_table = np.asarray(block_table)
    seqlens = np.asarray(seqlens)
    P, Hkv, ps, d = pages.shape
    if ps != page_size:
        raise ValueError("page_size does not match the pool")
    B, max_pages = block_table.shape
    out = np.zeros((B, Hkv, max_pages * page_size, d), dtype=pages.dtype)
    for b in range(B):
        for n in range(int(seqlens[b])):
            out[b, :, n, :] = pages[int(block_table[b, n // page_size]), :, n % page_size, :]
    return out


def num_threads() -> int:
    return _load().oracle_num_threads()
