"""The C-ABI library loads, exports every entry point that include/attn.h
declares, and rejects invalid arguments before touching the GPU (these calls
pass dummy non-null pointers: validation must fail before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def A():
    import softmax_attention_attn_amd as A
    return A


def test_header_declares_expected(A):
    assert set(_declared()) == set(A.EXPORTS)


def test_library_exports_every_symbol(A):
    lib = ctypes.CDLL(A.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
        assert hasattr(A, name), "binding lacks %s" % name


P = ctypes.c_void_p(256)  # dummy non-null device pointer; never dereferenced


def _fwd(A, **kw):
    args = dict(q=P, k=P, v=P, o=P, lse=None, B=1, H=4, Hkv=2, N=16, d=128, causal=0,
                scale=0.1, mode=0, o_dtype=0, workspace=None, workspace_bytes=0, stream=None)
    args.update(kw)
    return A.attn_fwd(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(B=0), -1), (dict(N=-3), -1),
    (dict(H=3), -1), (dict(Hkv=0), -1), (dict(scale=0.0), -1), (dict(scale=float("nan")), -1),
    (dict(scale=float("inf")), -1), (dict(o_dtype=7), -1), (dict(mode=9), -1),
    (dict(d=96), -2), (dict(d=256), -2),
])
def test_fwd_validation(A, kw, status):
    assert _fwd(A, **kw) == status
    assert A.attn_last_error() != ""


def test_mxfp4_mode(A):
    need = A.attn_fwd_workspace_size(1, 4, 2, 100, 128, A.ATTN_MODE_SAGE3_QK_MXFP4_PV_MXFP4)
    # FP4 Q^, K^, V^^T (half a byte per value) and one scale byte per 32
    # values, padded to 64 tokens, plus the K-mean partials and q . kmean
    assert need > (4 + 2 + 2) * 128 * 128 // 2
    assert _fwd(A, mode=2, N=100, workspace=None, workspace_bytes=0) == -3
    assert _fwd(A, mode=2, N=100, workspace=P, workspace_bytes=need - 1) == -3
    assert _fwd(A, mode=2, d=96) == -2
    assert _dec(A, mode=2) == -2


def test_mxfp6_mode(A):
    need4 = A.attn_fwd_workspace_size(1, 4, 2, 100, 128, A.ATTN_MODE_SAGE3_QK_MXFP4_PV_MXFP4)
    need = A.attn_fwd_workspace_size(1, 4, 2, 100, 128, A.ATTN_MODE_SAGE3_QK_MXFP6_PV_MXFP6)
    # FP6 codes take 3/4 of a byte per value against FP4's 1/2: the Q^, K^,
    # V^^T pieces (8 * 128 * 128 values at 64-token padding) grow by 1/4 byte each
    assert need >= need4 + (4 + 2 + 2) * 128 * 128 // 4
    assert _fwd(A, mode=3, N=100, workspace=None, workspace_bytes=0) == -3
    assert _fwd(A, mode=3, N=100, workspace=P, workspace_bytes=need - 1) == -3
    assert _fwd(A, mode=3, d=96) == -2
    assert _dec(A, mode=3) == -2
    assert _fwd(A, mode=4) == -1


def test_mx_workspace_layout(A):
    for mode, bits in (("mxfp4", 4), ("mxfp6", 6)):
        B, H, Hkv, N, d = 2, 4, 2, 100, 128
        lay = A.attn_mx_workspace_layout(B, H, Hkv, N, d, mode)
        off = list(lay.values())
        npad = 128
        sizes = {"ksum_part": 8 * B * Hkv * 16 * d, "kmean": 4 * B * Hkv * d,
                 "qkdot": 4 * B * H * N, "qhat": B * H * npad * d * bits // 8,
                 "qsc": B * H * npad * d // 32, "khat": B * Hkv * npad * d * bits // 8,
                 "ksc": B * Hkv * npad * d // 32, "vhatT": B * Hkv * d * npad * bits // 8,
                 "vscT": B * Hkv * npad // 32 * d}
        assert off == sorted(off) and all(o % 256 == 0 for o in off)
        names = list(lay)
        for a, b in zip(names, names[1:]):  # pieces in order, each large enough
            assert lay[b] - lay[a] >= sizes[a], (mode, a)
        need = A.attn_fwd_workspace_size(B, H, Hkv, N, d, A.MODES[mode])
        assert need - lay["vscT"] >= sizes["vscT"]
    with pytest.raises(A.AttnError):
        A.attn_mx_workspace_layout(1, 2, 2, 10, 128, "sage")
    with pytest.raises(A.AttnError):
        A.attn_mx_workspace_layout(1, 2, 2, 10, 96, "mxfp4")


def test_fwd_sage_workspace_required(A):
    need = A.attn_fwd_workspace_size(1, 4, 2, 16, 128, A.ATTN_MODE_SAGE_QK_I8_BLK64_PV_FP8_E4M3)
    if need == 0:
        pytest.skip("quantised mode needs no workspace in this build")
    assert _fwd(A, mode=1) == A.ATTN_ERR_WORKSPACE
    assert _fwd(A, mode=1, workspace=P, workspace_bytes=need - 1) == A.ATTN_ERR_WORKSPACE


def _fwdv(A, **kw):
    args = dict(q=P, k=P, v=P, o=P, lse=None, cu_seqlens=P, B=3, H=4, Hkv=2, total=100,
                max_seqlen=64, d=128, causal=1, scale=0.1, mode=0, o_dtype=0, stream=None)
    args.update(kw)
    return A.attn_fwd_varlen(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(cu_seqlens=None), -1), (dict(q=None), -1), (dict(o=None), -1), (dict(B=0), -1),
    (dict(total=0), -1), (dict(max_seqlen=0), -1), (dict(H=3), -1), (dict(scale=0.0), -1),
    (dict(o_dtype=2), -1), (dict(mode=7), -1),
    (dict(mode=1), -2), (dict(mode=2), -2), (dict(mode=3), -2), (dict(d=96), -2),
    (dict(max_seqlen=1 << 25), -2),
    (dict(B=1 << 20, H=1 << 10, Hkv=1 << 10, d=64, max_seqlen=4096), -2),
])
def test_fwd_varlen_validation(A, kw, status):
    assert _fwdv(A, **kw) == status
    assert A.attn_last_error() != ""


def _bwd(A, **kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, B=1, H=4, Hkv=2, N=16,
                d=128, causal=1, scale=0.1, grad_dtype=0, workspace=P, workspace_bytes=1 << 20,
                stream=None)
    args.update(kw)
    return A.attn_bwd(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(lse=None), -1), (dict(dout=None), -1), (dict(dk=None), -1), (dict(B=0), -1),
    (dict(N=0), -1), (dict(H=3), -1), (dict(scale=-2.0), -1), (dict(grad_dtype=5), -1),
    (dict(scale=2.0 ** -65), -1), (dict(d=32), -2), (dict(workspace=None), -3),
    (dict(workspace_bytes=10), -3),
])
def test_bwd_validation(A, kw, status):
    assert _bwd(A, **kw) == status
    assert A.attn_last_error() != ""


def test_bwd_workspace_size(A):
    # fp32 -D and -lse/scale per row, each head's rows padded to a multiple of 64
    assert A.attn_bwd_workspace_size(2, 4, 100) == 2 * (((4 * 2 * 4 * 128) + 255) // 256 * 256)
    assert A.attn_bwd_workspace_size(1, 1, 64) == 2 * 256
    assert A.attn_bwd_workspace_size(0, 4, 100) == 0


def _dec(A, **kw):
    args = dict(q=P, k_cache=P, v_cache=P, seqlens=P, o=P, lse=None, B=2, H=8, Hkv=2,
                N_max=1024, d=128, scale=0.1, mode=0, o_dtype=0, split_tokens=512,
                workspace=P, workspace_bytes=1 << 30, stream=None)
    args.update(kw)
    return A.attn_decode(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(seqlens=None), -1), (dict(k_cache=None), -1), (dict(B=0), -1), (dict(H=7), -1),
    (dict(H=6), -2),
    (dict(scale=-1.0), -1), (dict(split_tokens=0), -1), (dict(split_tokens=100), -1),
    (dict(mode=1), -2), (dict(mode=5), -1), (dict(d=80), -2), (dict(H=24, Hkv=2), -2), (dict(H=64, Hkv=2), -2),
    (dict(workspace=None), -3),
    (dict(workspace_bytes=1000), -3),
])
def test_decode_validation(A, kw, status):
    assert _dec(A, **kw) == status


def _decn(A, **kw):
    args = dict(q=P, k_cache=P, v_cache=P, seqlens=P, o=P, lse=None, B=2, H=8, Hkv=2,
                N_max=1024, d=128, scale=0.1, mode=0, o_dtype=0, split_tokens=512, stream=None)
    args.update(kw)
    return A.attn_decode_noalloc(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(seqlens=None), -1), (dict(o=None), -1), (dict(B=0), -1), (dict(H=7), -1),
    (dict(H=6), -2), (dict(scale=-1.0), -1), (dict(split_tokens=100), -1), (dict(mode=1), -2),
    (dict(d=80), -2),
    # the partials of B1024 H64 Hkv8 d128 need 37.7 MB, beyond the 16 MiB array
    (dict(B=1024, H=64, Hkv=8), -2),
])
def test_decode_noalloc_validation(A, kw, status):
    assert _decn(A, **kw) == status
    assert A.attn_last_error() != ""


def test_decode_noalloc_rejects_beyond_the_array(A):
    # the first B at H32 Hkv8 d128 whose partials exceed the fixed array is
    # rejected before any HIP call (the GPU test runs the largest that fits)
    lim = A.DECODE_SCRATCH_BYTES
    B = 1
    while A.attn_decode_workspace_size(B + 1, 32, 8, 128) <= lim:
        B += 1
    assert _decn(A, B=B + 1, H=32, Hkv=8) == -2
    assert "fixed array" in A.attn_last_error()


def _decp(A, **kw):
    args = dict(q=P, k_pages=P, v_pages=P, block_table=P, seqlens=P, o=P, lse=None, B=2, H=8,
                Hkv=2, num_pages=40, page_size=16, max_pages=64, d=128, scale=0.1, mode=0,
                o_dtype=0, split_tokens=512, workspace=P, workspace_bytes=1 << 30, stream=None)
    args.update(kw)
    return A.attn_decode_paged(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(block_table=None), -1), (dict(k_pages=None), -1), (dict(seqlens=None), -1),
    (dict(num_pages=0), -1), (dict(max_pages=-1), -1),
    (dict(page_size=0), -1), (dict(page_size=24), -1), (dict(page_size=-16), -1),
    (dict(page_size=8), -2),                                   # below 16
    (dict(page_size=1 << 20, max_pages=4096), -2),             # 2^32 positions
    (dict(H=7), -1), (dict(split_tokens=100), -1), (dict(mode=1), -2), (dict(mode=2), -2),
    (dict(mode=3), -2), (dict(mode=4), -1), (dict(d=80), -2),
    (dict(workspace=None), -3), (dict(workspace_bytes=1000), -3),
])
def test_decode_paged_validation(A, kw, status):
    assert _decp(A, **kw) == status
    assert A.attn_last_error() != ""


def test_decode_paged_workspace_is_decode_workspace(A):
    # the paged call needs exactly the contiguous call's workspace
    need = A.attn_decode_workspace_size(2, 8, 2, 128)
    assert _decp(A, workspace_bytes=need - 1) == -3
    assert _dec(A, workspace_bytes=need - 1) == -3


def test_workspace_sizes(A):
    # one partial per (wave, sequence, kv head) piece: B*Hkv + 1024 slots of
    # G = H/Hkv rows, partial O fp32 [slots, G, d] + partial lse fp32
    # [slots, G], each 256-B aligned; independent of N_max and split_tokens
    B, H, Hkv, d = 64, 32, 8, 128
    slots = B * Hkv + 1024
    G = H // Hkv
    o_b = 4 * slots * G * d
    l_b = 4 * slots * G
    r = lambda x: (x + 255) // 256 * 256
    assert A.attn_decode_workspace_size(B, H, Hkv, d) == r(o_b) + r(l_b)
    assert A.attn_decode_workspace_size(0, H, Hkv, d) == 0
    assert A.attn_decode_workspace_size(B, H, 5, d) == 0
    assert A.attn_fwd_workspace_size(1, 4, 2, 16, 128, 0) == 0


def test_status_strings(A):
    for st in (0, -1, -2, -3, -4):
        assert A.attn_status_string(st)
    assert A.attn_status_string(123) == "unknown status"
