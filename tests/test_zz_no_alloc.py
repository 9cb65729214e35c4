"""The decode entry point that allocates nothing (attn_decode_noalloc): its
partials live in the library's fixed array on the GPU.  Called through the C
ABI, it must return exactly what attn_decode returns on the same inputs (the
same kernels over a caller's workspace): on two calls in a row, the second
smaller than the first, and again after that with the first shape, so that
the array's contents left by an earlier call cannot leak into a later one.
The first call uses the largest batch whose partials fit the array."""
import ctypes
import math

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import softmax_attention_attn_amd as A
    return A


def _inputs(B, H, Hkv, N, d, seed):
    # seeded on the GPU (both calls read the same device tensors; no oracle)
    g = torch.Generator(device="cuda").manual_seed(seed)
    lens = torch.randint(1, N + 1, (B,), generator=g, device="cuda").to(torch.int32)
    q = torch.randn((B, H, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((B, Hkv, N, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, Hkv, N, d), generator=g, device="cuda").to(torch.bfloat16)
    return q, k, v, lens


def _largest_batch(attn, H, Hkv, d):
    B = 1
    while attn.attn_decode_workspace_size(B + 1, H, Hkv, d) <= attn.DECODE_SCRATCH_BYTES:
        B += 1
    return B


def _noalloc_raw(attn, q, k, v, lens, o, lse, split):
    """attn_decode_noalloc through the raw C ABI (pointers and sizes)."""
    B, H, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = attn.attn_decode_noalloc(ptr(q), ptr(k), ptr(v), ptr(lens), ptr(o), ptr(lse), B, H, Hkv,
                                  N, d, 1 / math.sqrt(d), attn.ATTN_MODE_EXACT_BF16,
                                  attn.ATTN_OUT_FP32 if o.dtype == torch.float32 else
                                  attn.ATTN_OUT_BF16, split,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == attn.ATTN_OK, attn.attn_last_error()


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_noalloc_matches_decode(attn, out_dtype):
    H, Hkv, d = 32, 8, 128
    Bmax = _largest_batch(attn, H, Hkv, d)
    shapes = [(Bmax, 600, 512, 1), (3, 2000, 64, 2), (Bmax, 600, 512, 3)]
    for B, N, split, seed in shapes:
        q, k, v, lens = _inputs(B, H, Hkv, N, d, seed)
        o = torch.full((B, H, d), float("nan"), dtype=out_dtype, device="cuda")
        lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
        _noalloc_raw(attn, q, k, v, lens, o, lse, split)
        o_ref, lse_ref = attn.decode(q, k, v, lens, split_tokens=split, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), (B, N, split)
        # the tensor wrapper makes the same call
        o2 = torch.empty_like(o)
        attn.decode_noalloc(q, k, v, lens, o2, split_tokens=split)
        torch.cuda.synchronize()
        assert torch.equal(o2, o_ref)


def test_noalloc_rejects_beyond_the_array(attn):
    H, Hkv, d = 32, 8, 128
    B = _largest_batch(attn, H, Hkv, d) + 1
    q = torch.zeros((B, H, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, 64, d), dtype=torch.bfloat16, device="cuda")
    lens = torch.ones((B,), dtype=torch.int32, device="cuda")
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(attn.AttnError) as e:
        attn.decode_noalloc(q, k, k, lens, o)
    assert e.value.status == attn.ATTN_ERR_UNSUPPORTED
