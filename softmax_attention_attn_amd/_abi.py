"""ctypes declarations of the C ABI in ``include/attn.h``.

Kept free of torch and of the package's other modules, so that a test can
apply the same declarations to another build of the library (a host-code
sanitizer build) without importing torch.
"""
from __future__ import annotations

import ctypes


def declare(lib):
    """Set ``restype`` and ``argtypes`` of every exported entry point of
    ``lib`` (a ``ctypes.CDLL`` of libattn) and return it."""
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.restype = i
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.attn_fwd_workspace_size.restype = sz
    lib.attn_fwd_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.attn_bwd.restype = i
    lib.attn_bwd.argtypes = [vp] * 9 + [i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.attn_bwd_workspace_size.restype = sz
    lib.attn_bwd_workspace_size.argtypes = [i, i, i]
    lib.attn_fwd_varlen.restype = i
    lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp]
    lib.attn_decode.restype = i
    lib.attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    lib.attn_decode_noalloc.restype = i
    lib.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
    lib.attn_decode_workspace_size.restype = sz
    lib.attn_decode_workspace_size.argtypes = [i, i, i, i]
    lib.attn_decode_paged.restype = i
    lib.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i,
                                      i, vp, sz, vp]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [i]
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_profiler_enable.restype = i
    lib.attn_profiler_enable.argtypes = [i]
    lib.attn_profiler_read.restype = i
    lib.attn_profiler_read.argtypes = [ctypes.c_char_p, i, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int), i]
    lib.attn_profiler_launches.restype = i
    lib.attn_profiler_launches.argtypes = [ctypes.c_char_p, i, ctypes.POINTER(ctypes.c_float), i]
    lib.attn_sage_workspace_layout.restype = i
    lib.attn_sage_workspace_layout.argtypes = [i, i, i, i, i, ctypes.POINTER(sz)]
    lib.attn_mx_workspace_layout.restype = i
    lib.attn_mx_workspace_layout.argtypes = [i, i, i, i, i, i, ctypes.POINTER(sz)]
    return lib
