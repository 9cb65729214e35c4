"""Python binding of the MI355X fused-attention library (``libattn.so``).

This module only marshals arguments: it checks torch tensors (device, dtype,
shape, contiguity), allocates outputs and workspaces with torch when the
caller does not pass them, and calls the C ABI of ``include/attn.h`` through
ctypes on torch's current HIP stream.  Every step of the computation runs in
the library's HIP kernels; there is no fallback.  Importing this package
fails loudly when the library has not been built.

The functions carry the C names (``attn_fwd``, ``attn_decode``, ...); the
convenience wrappers ``fwd``, ``fwd_varlen``, ``bwd``, ``decode`` and
``decode_paged`` allocate what the caller omits.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch  # loaded first so that the library binds to torch's HIP runtime

from . import _abi

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = -1
ATTN_ERR_UNSUPPORTED = -2
ATTN_ERR_WORKSPACE = -3
ATTN_ERR_HIP = -4

ATTN_MODE_EXACT_BF16 = 0
ATTN_MODE_SAGE_QK_I8_BLK64_PV_FP8_E4M3 = 1
ATTN_MODE_SAGE3_QK_MXFP4_PV_MXFP4 = 2
ATTN_MODE_SAGE3_QK_MXFP6_PV_MXFP6 = 3
ATTN_OUT_BF16 = 0
ATTN_OUT_FP32 = 1

MODES = {"exact": ATTN_MODE_EXACT_BF16, "sage": ATTN_MODE_SAGE_QK_I8_BLK64_PV_FP8_E4M3,
         "mxfp4": ATTN_MODE_SAGE3_QK_MXFP4_PV_MXFP4, "mxfp6": ATTN_MODE_SAGE3_QK_MXFP6_PV_MXFP6}

EXPORTS = ("attn_fwd", "attn_fwd_workspace_size", "attn_fwd_varlen", "attn_bwd",
           "attn_bwd_workspace_size", "attn_decode", "attn_decode_workspace_size",
           "attn_decode_paged", "attn_status_string", "attn_last_error",
           "attn_profiler_enable", "attn_profiler_read", "attn_profiler_launches",
           "attn_sage_workspace_layout", "attn_mx_workspace_layout", "attn_decode_noalloc")


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (status %d): %s" % (_status_name(status), status, message))
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libattn.so is not built (%s); run __graft_entry__.build() or "
                          "python softmax_attention_attn_amd/_build.py" % LIB_PATH)
    return _abi.declare(ctypes.CDLL(LIB_PATH))


_lib = _load()


def _status_name(status: int) -> str:
    return _lib.attn_status_string(int(status)).decode()


def attn_status_string(status: int) -> str:
    return _status_name(status)


def attn_last_error() -> str:
    return _lib.attn_last_error().decode()


def _check(status: int):
    if status != ATTN_OK:
        raise AttnError(status, attn_last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ----------------------------------------------------------------- raw C ABI

def attn_fwd_workspace_size(B, H, Hkv, N, d, mode) -> int:
    return int(_lib.attn_fwd_workspace_size(B, H, Hkv, N, d, mode))


def attn_decode_workspace_size(B, H, Hkv, d) -> int:
    return int(_lib.attn_decode_workspace_size(B, H, Hkv, d))


def attn_fwd(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale, mode, o_dtype, workspace,
             workspace_bytes, stream) -> int:
    """Direct call of the C function with raw pointers (ints or None)."""
    return int(_lib.attn_fwd(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale, mode, o_dtype,
                             workspace, workspace_bytes, stream))


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, H, Hkv, total, max_seqlen, d, causal, scale,
                    mode, o_dtype, stream) -> int:
    return int(_lib.attn_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, H, Hkv, total, max_seqlen, d,
                                    causal, scale, mode, o_dtype, stream))


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, d, causal, scale, grad_dtype,
             workspace, workspace_bytes, stream) -> int:
    return int(_lib.attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, d, causal, scale,
                             grad_dtype, workspace, workspace_bytes, stream))


def attn_bwd_workspace_size(B, H, N) -> int:
    return int(_lib.attn_bwd_workspace_size(B, H, N))


def attn_decode(q, k_cache, v_cache, seqlens, o, lse, B, H, Hkv, N_max, d, scale, mode,
                o_dtype, split_tokens, workspace, workspace_bytes, stream) -> int:
    return int(_lib.attn_decode(q, k_cache, v_cache, seqlens, o, lse, B, H, Hkv, N_max, d,
                                scale, mode, o_dtype, split_tokens, workspace,
                                workspace_bytes, stream))


def attn_decode_noalloc(q, k_cache, v_cache, seqlens, o, lse, B, H, Hkv, N_max, d, scale, mode,
                        o_dtype, split_tokens, stream) -> int:
    return int(_lib.attn_decode_noalloc(q, k_cache, v_cache, seqlens, o, lse, B, H, Hkv, N_max,
                                        d, scale, mode, o_dtype, split_tokens, stream))


# the size of the library's fixed decode array (ATTN_DECODE_SCRATCH_BYTES)
DECODE_SCRATCH_BYTES = 16 << 20


def attn_decode_paged(q, k_pages, v_pages, block_table, seqlens, o, lse, B, H, Hkv, num_pages,
                      page_size, max_pages, d, scale, mode, o_dtype, split_tokens, workspace,
                      workspace_bytes, stream) -> int:
    return int(_lib.attn_decode_paged(q, k_pages, v_pages, block_table, seqlens, o, lse, B, H,
                                      Hkv, num_pages, page_size, max_pages, d, scale, mode,
                                      o_dtype, split_tokens, workspace, workspace_bytes, stream))


def attn_profiler_enable(enable: bool) -> None:
    _check(_lib.attn_profiler_enable(int(bool(enable))))


def attn_profiler_read(cap: int = 16, name_len: int = 64) -> dict:
    """{kernel name: (total_ms, launches)} since the profiler was enabled/read."""
    names = ctypes.create_string_buffer(cap * name_len)
    tot = (ctypes.c_double * cap)()
    cnt = (ctypes.c_int * cap)()
    n = _lib.attn_profiler_read(names, name_len, tot, cnt, cap)
    if n < 0:
        _check(n)
    out = {}
    for j in range(n):
        nm = names.raw[j * name_len:(j + 1) * name_len].split(b"\0", 1)[0].decode()
        out[nm] = (tot[j], cnt[j])
    return out


def attn_profiler_launches(cap: int = 4096, name_len: int = 64) -> list:
    """[(kernel name, ms)] of the launches recorded since the profiler was
    enabled or last read, in launch order."""
    names = ctypes.create_string_buffer(cap * name_len)
    ms = (ctypes.c_float * cap)()
    n = _lib.attn_profiler_launches(names, name_len, ms, cap)
    if n < 0:
        _check(n)
    return [(names.raw[j * name_len:(j + 1) * name_len].split(b"\0", 1)[0].decode(), ms[j])
            for j in range(n)]


SAGE_WS_PIECES = ("ksum_part", "vmax_part", "kmean", "vscale", "vinv", "qdelta", "kdelta",
                  "qkdot", "qhat", "khat", "vhatT")


def attn_sage_workspace_layout(B, H, Hkv, N, d) -> dict:
    """{piece name: byte offset} of the quantised mode's workspace."""
    off = (ctypes.c_size_t * len(SAGE_WS_PIECES))()
    _check(_lib.attn_sage_workspace_layout(B, H, Hkv, N, d, off))
    return dict(zip(SAGE_WS_PIECES, off))


MX_WS_PIECES = ("ksum_part", "kmean", "qkdot", "qhat", "qsc", "khat", "ksc", "vhatT", "vscT")


def attn_mx_workspace_layout(B, H, Hkv, N, d, mode) -> dict:
    """{piece name: byte offset} of an MX mode's workspace (mode "mxfp4" or
    "mxfp6", or its attn_mode value)."""
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    off = (ctypes.c_size_t * len(MX_WS_PIECES))()
    _check(_lib.attn_mx_workspace_layout(B, H, Hkv, N, d, m, off))
    return dict(zip(MX_WS_PIECES, off))


# ----------------------------------------------------------------- tensor API

def _need(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _need_out(t, name, dtype, shape, device):
    """A caller-supplied output: a contiguous tensor of exactly this dtype and
    shape on the inputs' GPU (the kernels write it in full)."""
    _need(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.device != device:
        raise ValueError("%s is on %s, the inputs on %s" % (name, t.device, device))


def _workspace(ws, need, device):
    """(pointer, size in bytes) of a workspace: the caller's tensor, checked to
    be a contiguous tensor on the inputs' GPU of at least ``need`` bytes, or a
    new uint8 tensor of that size."""
    if ws is None:
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=device)
    else:
        if not isinstance(ws, torch.Tensor):
            raise TypeError("workspace must be a torch tensor")
        if ws.device != device:
            raise ValueError("workspace is on %s, the inputs on %s" % (ws.device, device))
        if not ws.is_contiguous():
            raise ValueError("workspace must be contiguous")
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError("workspace of %d bytes needed, %d given" % (need, nbytes))
    return ws, nbytes


def _out_code(dtype, what="out_dtype"):
    try:
        return {torch.bfloat16: ATTN_OUT_BF16, torch.float32: ATTN_OUT_FP32}[dtype]
    except KeyError:
        raise TypeError("%s must be torch.bfloat16 or torch.float32, got %s" % (what, dtype))


def fwd(q, k, v, *, causal: bool = False, scale: float | None = None, mode: str = "exact",
        out_dtype=torch.bfloat16, o=None, lse=None, with_lse: bool = True, workspace=None,
        stream=None):
    """Attention forward.  q [B,H,N,d], k/v [B,Hkv,N,d] bf16 GPU tensors.

    Returns (o, lse) with o [B,H,N,d] of ``out_dtype`` and lse fp32 [B,H,N]
    (None when ``with_lse`` is False).
    """
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k/v shape %s does not match q %s" % (tuple(k.shape), tuple(q.shape)))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if mode not in MODES:
        raise ValueError("mode must be one of %s" % sorted(MODES))
    m = MODES[mode]
    o_code = _out_code(out_dtype)
    dev = q.device
    if k.device != dev or v.device != dev:
        raise ValueError("q, k and v must be on one GPU")
    if o is None:
        o = torch.empty((B, H, N, d), dtype=out_dtype, device=dev)
    else:
        _need_out(o, "o", out_dtype, (B, H, N, d), dev)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    elif lse is not None:
        _need_out(lse, "lse", torch.float32, (B, H, N), dev)
    ws_bytes = attn_fwd_workspace_size(B, H, Hkv, N, d, m)
    ws_ptr, ws_len = None, 0
    if ws_bytes or workspace is not None:
        workspace, ws_len = _workspace(workspace, ws_bytes, dev)
        ws_ptr = _ptr(workspace)
    st = _lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                       int(bool(causal)), float(scale), m, o_code, ws_ptr, ws_len,
                       _stream(stream))
    _check(st)
    return o, lse


def bwd(q, k, v, o, lse, dout, *, causal: bool = False, scale: float | None = None,
        grad_dtype=torch.bfloat16, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients of the exact forward.  q/o/dout [B,H,N,d], k/v [B,Hkv,N,d] bf16,
    lse fp32 [B,H,N] from ``fwd``.  Returns (dq, dk, dv) of ``grad_dtype``."""
    for t, name in ((q, "q"), (o, "o"), (dout, "dout")):
        _need(t, name, torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != tuple(k.shape) or \
            tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape) or \
            tuple(lse.shape) != (B, H, N):
        raise ValueError("shapes do not agree")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    g_code = _out_code(grad_dtype, "grad_dtype")
    dev = q.device
    for t, name in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (lse, "lse")):
        if t.device != dev:
            raise ValueError("%s is on %s, q on %s" % (name, t.device, dev))
    if dq is None:
        dq = torch.empty((B, H, N, d), dtype=grad_dtype, device=dev)
    else:
        _need_out(dq, "dq", grad_dtype, (B, H, N, d), dev)
    if dk is None:
        dk = torch.empty((B, Hkv, N, d), dtype=grad_dtype, device=dev)
    else:
        _need_out(dk, "dk", grad_dtype, (B, Hkv, N, d), dev)
    if dv is None:
        dv = torch.empty((B, Hkv, N, d), dtype=grad_dtype, device=dev)
    else:
        _need_out(dv, "dv", grad_dtype, (B, Hkv, N, d), dev)
    workspace, ws_len = _workspace(workspace, attn_bwd_workspace_size(B, H, N), dev)
    st = _lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                       _ptr(dk), _ptr(dv), B, H, Hkv, N, d, int(bool(causal)), float(scale),
                       g_code, _ptr(workspace), ws_len, _stream(stream))
    _check(st)
    return dq, dk, dv


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen: int, *, causal: bool = False,
               scale: float | None = None, out_dtype=torch.bfloat16, o=None, lse=None,
               with_lse: bool = True, stream=None):
    """Attention over a packed batch of variable-length sequences (exact mode).

    q [total,H,d], k/v [total,Hkv,d] bf16; cu_seqlens int32 [B+1] on the GPU;
    ``max_seqlen`` bounds the sequence lengths.  Returns (o [total,H,d] of
    ``out_dtype``, lse fp32 [H,total] or None).
    """
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    total, H, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (total, Hkv, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k/v shape %s does not match q %s" % (tuple(k.shape), tuple(q.shape)))
    B = cu_seqlens.shape[0] - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o_code = _out_code(out_dtype)
    dev = q.device
    for t, name in ((k, "k"), (v, "v"), (cu_seqlens, "cu_seqlens")):
        if t.device != dev:
            raise ValueError("%s is on %s, q on %s" % (name, t.device, dev))
    if o is None:
        o = torch.empty((total, H, d), dtype=out_dtype, device=dev)
    else:
        _need_out(o, "o", out_dtype, (total, H, d), dev)
    if lse is None and with_lse:
        lse = torch.empty((H, total), dtype=torch.float32, device=dev)
    elif lse is not None:
        _need_out(lse, "lse", torch.float32, (H, total), dev)
    st = _lib.attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens),
                              B, H, Hkv, total, int(max_seqlen), d, int(bool(causal)),
                              float(scale), ATTN_MODE_EXACT_BF16, o_code, _stream(stream))
    _check(st)
    return o, lse


def _decode_outputs(o, lse, with_lse, out_dtype, B, H, d, dev):
    if o is None:
        o = torch.empty((B, H, d), dtype=out_dtype, device=dev)
    else:
        _need_out(o, "o", out_dtype, (B, H, d), dev)
    if lse is None and with_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    elif lse is not None:
        _need_out(lse, "lse", torch.float32, (B, H), dev)
    return o, lse


def decode(q, k_cache, v_cache, seqlens, *, scale: float | None = None,
           split_tokens: int = 512, out_dtype=torch.bfloat16, o=None, lse=None,
           with_lse: bool = True, workspace=None, stream=None):
    """Split-KV decode.  q [B,H,d]; caches [B,Hkv,N_max,d] bf16; seqlens int32 [B]."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(seqlens, "seqlens", torch.int32, 1)
    B, H, d = q.shape
    _, Hkv, N_max, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, Hkv, N_max, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    if seqlens.shape[0] != B:
        raise ValueError("seqlens must have B entries")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o_code = _out_code(out_dtype)
    dev = q.device
    for t, name in ((k_cache, "k_cache"), (v_cache, "v_cache"), (seqlens, "seqlens")):
        if t.device != dev:
            raise ValueError("%s is on %s, q on %s" % (name, t.device, dev))
    o, lse = _decode_outputs(o, lse, with_lse, out_dtype, B, H, d, dev)
    workspace, ws_len = _workspace(workspace, attn_decode_workspace_size(B, H, Hkv, d), dev)
    st = _lib.attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o),
                          _ptr(lse), B, H, Hkv, N_max, d, float(scale), ATTN_MODE_EXACT_BF16,
                          o_code, int(split_tokens), _ptr(workspace), ws_len,
                          _stream(stream))
    _check(st)
    return o, lse


def decode_noalloc(q, k_cache, v_cache, seqlens, o, lse=None, *, scale: float | None = None,
                   split_tokens: int = 512, stream=None):
    """``decode`` without a workspace: the partials live in the library's
    fixed array on the GPU (see ``attn_decode_noalloc`` in attn.h), so the
    call allocates nothing.  The caller passes o (bf16 or fp32 [B,H,d]) and,
    optionally, lse (fp32 [B,H]); returns (o, lse)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(seqlens, "seqlens", torch.int32, 1)
    B, H, d = q.shape
    _, Hkv, N_max, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, Hkv, N_max, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    if seqlens.shape[0] != B:
        raise ValueError("seqlens must have B entries")
    if not isinstance(o, torch.Tensor):
        raise TypeError("o must be a torch tensor")
    o_code = _out_code(o.dtype, "o.dtype")
    dev = q.device
    for t, name in ((k_cache, "k_cache"), (v_cache, "v_cache"), (seqlens, "seqlens")):
        if t.device != dev:
            raise ValueError("%s is on %s, q on %s" % (name, t.device, dev))
    _need_out(o, "o", o.dtype, (B, H, d), dev)
    if lse is not None:
        _need_out(lse, "lse", torch.float32, (B, H), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = _lib.attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o),
                                  _ptr(lse), B, H, Hkv, N_max, d, float(scale),
                                  ATTN_MODE_EXACT_BF16, o_code, int(split_tokens),
                                  _stream(stream))
    _check(st)
    return o, lse


def decode_paged(q, k_pages, v_pages, block_table, seqlens, *, scale: float | None = None,
                 split_tokens: int = 512, out_dtype=torch.bfloat16, o=None, lse=None,
                 with_lse: bool = True, workspace=None, stream=None):
    """Split-KV decode over paged caches.  q [B,H,d]; k_pages/v_pages
    [num_pages,Hkv,page_size,d] bf16; block_table int32 [B,max_pages];
    seqlens int32 [B]."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_pages, "k_pages", torch.bfloat16, 4)
    _need(v_pages, "v_pages", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seqlens, "seqlens", torch.int32, 1)
    B, H, d = q.shape
    num_pages, Hkv, page_size, _ = k_pages.shape
    if tuple(k_pages.shape) != (num_pages, Hkv, page_size, d) or \
            tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("page pool shapes do not match q")
    if block_table.shape[0] != B or seqlens.shape[0] != B:
        raise ValueError("block_table and seqlens must have B rows")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o_code = _out_code(out_dtype)
    dev = q.device
    for t, name in ((k_pages, "k_pages"), (v_pages, "v_pages"), (block_table, "block_table"),
                    (seqlens, "seqlens")):
        if t.device != dev:
            raise ValueError("%s is on %s, q on %s" % (name, t.device, dev))
    o, lse = _decode_outputs(o, lse, with_lse, out_dtype, B, H, d, dev)
    workspace, ws_len = _workspace(workspace, attn_decode_workspace_size(B, H, Hkv, d), dev)
    st = _lib.attn_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                _ptr(seqlens), _ptr(o), _ptr(lse), B, H, Hkv, num_pages,
                                page_size, max_pages, d, float(scale), ATTN_MODE_EXACT_BF16,
                                o_code, int(split_tokens), _ptr(workspace), ws_len,
                                _stream(stream))
    _check(st)
    return o, lse
