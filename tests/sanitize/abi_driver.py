"""Exercise the host code of a sanitizer build of libattn (ASan + UBSan).

Run by tests/test_sanitizers.py in a child process with the sanitizer
runtime preloaded; argv[1] is the library, argv[2] the binding's torch-free
ctypes declarations (softmax_attention_attn_amd/_abi.py).  Every call either
fails validation before any HIP call or is a host-side size or layout query,
so nothing here touches a GPU.  Exits 0 when every status is the expected
one; a sanitizer report aborts the process with a non-zero status.
"""
import ctypes
import importlib.util
import sys

spec = importlib.util.spec_from_file_location("attn_abi", sys.argv[2])
abi = importlib.util.module_from_spec(spec)
spec.loader.exec_module(abi)
lib = abi.declare(ctypes.CDLL(sys.argv[1]))

P = ctypes.c_void_p(256)  # dummy non-null device pointer; never dereferenced
BIG = 1 << 40
IMAX = 2 ** 31 - 1
failures = []


def expect(what, got, want):
    if got != want:
        failures.append("%s: status %d, expected %d (%s)" %
                        (what, got, want, lib.attn_last_error().decode()))


def call(fn, order, base, kw):
    args = dict(base)
    args.update(kw)
    return fn(*[args[k] for k in order])


FWD = ("q k v o lse B H Hkv N d causal scale mode o_dtype workspace workspace_bytes "
       "stream").split()
fwd0 = dict(q=P, k=P, v=P, o=P, lse=None, B=1, H=4, Hkv=2, N=16, d=128, causal=0, scale=0.1,
            mode=0, o_dtype=0, workspace=None, workspace_bytes=0, stream=None)
for kw, st in [(dict(q=None), -1), (dict(o=None), -1), (dict(B=0), -1), (dict(N=-3), -1),
               (dict(H=3), -1), (dict(Hkv=0), -1), (dict(scale=0.0), -1),
               (dict(scale=float("nan")), -1), (dict(scale=float("inf")), -1),
               (dict(o_dtype=7), -1), (dict(mode=9), -1), (dict(d=96), -2), (dict(d=256), -2),
               (dict(mode=1), -3), (dict(mode=2), -3),
               (dict(B=IMAX, H=IMAX, Hkv=IMAX, N=IMAX), -2),
               (dict(mode=1, B=IMAX, H=IMAX, Hkv=1, N=IMAX, workspace=P,
                     workspace_bytes=BIG), -2)]:
    expect("attn_fwd %s" % kw, call(lib.attn_fwd, FWD, fwd0, kw), st)

VAR = ("q k v o lse cu_seqlens B H Hkv total max_seqlen d causal scale mode o_dtype "
       "stream").split()
var0 = dict(q=P, k=P, v=P, o=P, lse=None, cu_seqlens=P, B=3, H=4, Hkv=2, total=100,
            max_seqlen=64, d=128, causal=1, scale=0.1, mode=0, o_dtype=0, stream=None)
for kw, st in [(dict(cu_seqlens=None), -1), (dict(B=0), -1), (dict(total=0), -1),
               (dict(max_seqlen=0), -1), (dict(H=3), -1), (dict(mode=1), -2),
               (dict(d=96), -2), (dict(max_seqlen=1 << 25), -2),
               (dict(B=1 << 20, H=1 << 10, Hkv=1 << 10, d=64, max_seqlen=4096), -2),
               (dict(B=IMAX, H=IMAX, Hkv=IMAX, total=IMAX, max_seqlen=IMAX), -2)]:
    expect("attn_fwd_varlen %s" % kw, call(lib.attn_fwd_varlen, VAR, var0, kw), st)

BWD = ("q k v o lse dout dq dk dv B H Hkv N d causal scale grad_dtype workspace "
       "workspace_bytes stream").split()
bwd0 = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, B=1, H=4, Hkv=2, N=16,
            d=128, causal=1, scale=0.1, grad_dtype=0, workspace=P, workspace_bytes=1 << 20,
            stream=None)
for kw, st in [(dict(lse=None), -1), (dict(dout=None), -1), (dict(B=0), -1), (dict(N=0), -1),
               (dict(H=3), -1), (dict(scale=-2.0), -1), (dict(grad_dtype=5), -1),
               (dict(d=32), -2), (dict(workspace=None), -3), (dict(workspace_bytes=10), -3),
               (dict(B=IMAX, H=IMAX, Hkv=IMAX, N=IMAX, workspace_bytes=BIG), -2)]:
    expect("attn_bwd %s" % kw, call(lib.attn_bwd, BWD, bwd0, kw), st)

DEC = ("q k_cache v_cache seqlens o lse B H Hkv N_max d scale mode o_dtype split_tokens "
       "workspace workspace_bytes stream").split()
dec0 = dict(q=P, k_cache=P, v_cache=P, seqlens=P, o=P, lse=None, B=2, H=8, Hkv=2, N_max=1024,
            d=128, scale=0.1, mode=0, o_dtype=0, split_tokens=512, workspace=P,
            workspace_bytes=1 << 30, stream=None)
dec_cases = [(dict(seqlens=None), -1), (dict(B=0), -1), (dict(H=7), -1), (dict(H=6), -2),
             (dict(scale=-1.0), -1), (dict(split_tokens=0), -1), (dict(split_tokens=100), -1),
             (dict(mode=1), -2), (dict(mode=5), -1), (dict(d=80), -2),
             (dict(H=64, Hkv=2), -2), (dict(workspace=None), -3),
             (dict(workspace_bytes=1000), -3),
             (dict(B=IMAX, H=IMAX, Hkv=IMAX, N_max=IMAX, workspace_bytes=BIG), -2)]
for kw, st in dec_cases:
    expect("attn_decode %s" % kw, call(lib.attn_decode, DEC, dec0, kw), st)

DECN = ("q k_cache v_cache seqlens o lse B H Hkv N_max d scale mode o_dtype split_tokens "
        "stream").split()
for kw, st in [(dict(seqlens=None), -1), (dict(B=0), -1), (dict(H=6), -2), (dict(mode=1), -2),
               (dict(B=1024, H=64, Hkv=8), -2),
               (dict(B=IMAX, H=IMAX, Hkv=IMAX, N_max=IMAX), -2)]:
    expect("attn_decode_noalloc %s" % kw, call(lib.attn_decode_noalloc, DECN, dec0, kw), st)

PAG = ("q k_pages v_pages block_table seqlens o lse B H Hkv num_pages page_size max_pages d "
       "scale mode o_dtype split_tokens workspace workspace_bytes stream").split()
pag0 = dict(q=P, k_pages=P, v_pages=P, block_table=P, seqlens=P, o=P, lse=None, B=2, H=8,
            Hkv=2, num_pages=40, page_size=16, max_pages=64, d=128, scale=0.1, mode=0,
            o_dtype=0, split_tokens=512, workspace=P, workspace_bytes=1 << 30, stream=None)
for kw, st in [(dict(block_table=None), -1), (dict(num_pages=0), -1), (dict(max_pages=-1), -1),
               (dict(page_size=0), -1), (dict(page_size=24), -1), (dict(page_size=-16), -1),
               (dict(page_size=8), -2), (dict(page_size=1 << 20, max_pages=4096), -2),
               (dict(page_size=1 << 30, max_pages=IMAX), -2),
               (dict(workspace=None), -3), (dict(workspace_bytes=1000), -3)]:
    expect("attn_decode_paged %s" % kw, call(lib.attn_decode_paged, PAG, pag0, kw), st)

# size and layout queries over ordinary, degenerate and extreme shapes
for B, H, Hkv, N, d in [(1, 4, 2, 16, 128), (2, 24, 24, 16384, 128), (0, 4, 2, 16, 128),
                        (1, 4, 3, 16, 64), (IMAX, IMAX, IMAX, IMAX, 128), (-1, -1, -1, -1, -1)]:
    for mode in (0, 1, 2, 7):
        lib.attn_fwd_workspace_size(B, H, Hkv, N, d, mode)
    offs = (ctypes.c_size_t * 16)()
    lib.attn_sage_workspace_layout(B, H, Hkv, N, d, offs)
    lib.attn_bwd_workspace_size(B, H, N)
    lib.attn_decode_workspace_size(B, H, Hkv, d)
for st in (0, -1, -2, -3, -4, 123, -IMAX - 1):
    lib.attn_status_string(st)
lib.attn_last_error()

if failures:
    print("\n".join(failures))
    sys.exit(1)
print("abi driver: all statuses as expected")
