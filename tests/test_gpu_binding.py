"""The binding's checks of caller-supplied outputs and workspaces, and the
kernels' independence from what a workspace holds on entry.

* An output or workspace of the wrong dtype, shape or device, or a
  workspace too small or not contiguous, raises TypeError / ValueError in the
  binding before anything is launched (the output tensor is left untouched).
* The kernels write every workspace byte they later read: a workspace filled
  with NaN bytes on entry gives bit-identical results to a zeroed one
  (quantised prefill, decode, backward).
"""
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


def _prefill(B=1, H=4, Hkv=2, N=200, d=128, seed=3):
    q, k, v, _ = workloads.make_prefill(B, H, Hkv, N, d, seed=seed)
    return q.cuda(), k.cuda(), v.cuda()


def _sentinel(t):
    t.fill_(7)
    return t


@pytest.mark.parametrize("bad", ["o_dtype", "o_shape", "o_cpu", "o_noncontig", "lse_dtype",
                                 "lse_shape", "lse_cpu", "out_dtype"])
def test_fwd_rejects_bad_outputs(attn, bad):
    q, k, v = _prefill()
    B, H, N, d = q.shape
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    kw = {}
    if bad == "o_dtype":
        kw["o"] = _sentinel(torch.empty((B, H, N, d), dtype=torch.float32, device="cuda"))
    elif bad == "o_shape":
        kw["o"] = _sentinel(torch.empty((B, H, N - 1, d), dtype=torch.bfloat16, device="cuda"))
    elif bad == "o_cpu":
        kw["o"] = torch.empty((B, H, N, d), dtype=torch.bfloat16)
    elif bad == "o_noncontig":
        kw["o"] = _sentinel(torch.empty((B, H, d, N), dtype=torch.bfloat16,
                                        device="cuda").transpose(2, 3))
    elif bad == "lse_dtype":
        kw["lse"] = torch.empty((B, H, N), dtype=torch.bfloat16, device="cuda")
    elif bad == "lse_shape":
        kw["lse"] = torch.empty((B, H, N + 1), dtype=torch.float32, device="cuda")
    elif bad == "lse_cpu":
        kw["lse"] = torch.empty((B, H, N), dtype=torch.float32)
    elif bad == "out_dtype":
        kw["out_dtype"] = torch.float16
    kw.setdefault("o", o)
    kw.setdefault("lse", lse)
    with pytest.raises((TypeError, ValueError)):
        attn.fwd(q, k, v, causal=True, **kw)
    torch.cuda.synchronize()
    if bad in ("o_dtype", "o_shape", "o_noncontig"):
        assert bool((kw["o"] == 7).all()), "rejected output was written"


@pytest.mark.parametrize("bad", ["small", "cpu", "noncontig"])
def test_sage_rejects_bad_workspace(attn, bad):
    q, k, v = _prefill()
    B, H, N, d = q.shape
    need = attn.attn_fwd_workspace_size(B, H, k.shape[1], N, d, attn.MODES["sage"])
    if bad == "small":
        ws = torch.empty((need - 1,), dtype=torch.uint8, device="cuda")
    elif bad == "cpu":
        ws = torch.empty((need,), dtype=torch.uint8)
    else:
        ws = torch.empty((2, need), dtype=torch.uint8, device="cuda")[:, 0]
    with pytest.raises(ValueError):
        attn.fwd(q, k, v, mode="sage", workspace=ws)


def test_workspace_size_counts_bytes_not_elements(attn):
    """A float32 workspace of need/4 elements is exactly big enough."""
    q, k, v = _prefill()
    B, H, N, d = q.shape
    need = attn.attn_fwd_workspace_size(B, H, k.shape[1], N, d, attn.MODES["sage"])
    ws = torch.empty(((need + 3) // 4,), dtype=torch.float32, device="cuda")
    o1, _ = attn.fwd(q, k, v, mode="sage", workspace=ws)
    o2, _ = attn.fwd(q, k, v, mode="sage")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    with pytest.raises(ValueError):
        attn.fwd(q, k, v, mode="sage", workspace=ws[:-1])


def test_decode_rejects_bad_outputs(attn):
    B, H, Hkv, N, d = 2, 8, 2, 300, 128
    q = torch.zeros((B, H, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, Hkv, N, d), dtype=torch.bfloat16, device="cuda")
    sl = torch.full((B,), N, dtype=torch.int32, device="cuda")
    with pytest.raises(TypeError):
        attn.decode(q, kc, kc, sl, o=torch.empty((B, H, d), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        attn.decode(q, kc, kc, sl, o=torch.empty((B, H + 1, d), dtype=torch.bfloat16,
                                                 device="cuda"))
    with pytest.raises(ValueError):
        attn.decode(q, kc, kc, sl, lse=torch.empty((B, H), dtype=torch.float32))
    need = attn.attn_decode_workspace_size(B, H, Hkv, d)
    with pytest.raises(ValueError):
        attn.decode(q, kc, kc, sl, split_tokens=64,
                    workspace=torch.empty((need - 1,), dtype=torch.uint8, device="cuda"))


def test_bwd_rejects_bad_outputs(attn):
    q, k, v = _prefill()
    o, lse = attn.fwd(q, k, v, causal=True)
    with pytest.raises(TypeError):
        attn.bwd(q, k, v, o, lse, o, causal=True, grad_dtype=torch.float32,
                 dq=torch.empty(q.shape, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        attn.bwd(q, k, v, o, lse, o, causal=True,
                 dk=torch.empty(q.shape, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        attn.bwd(q, k, v, o, lse, o, causal=True,
                 workspace=torch.empty((16,), dtype=torch.uint8, device="cuda"))


def _poisoned(nbytes):
    return torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN in fp32/fp64


def test_sage_workspace_contents_do_not_matter(attn):
    q, k, v = _prefill(B=1, H=4, Hkv=2, N=333, d=128, seed=9)
    B, H, N, d = q.shape
    need = attn.attn_fwd_workspace_size(B, H, k.shape[1], N, d, attn.MODES["sage"])
    for causal in (False, True):
        a = attn.fwd(q, k, v, causal=causal, mode="sage", out_dtype=torch.float32,
                     workspace=torch.zeros((need,), dtype=torch.uint8, device="cuda"))
        b = attn.fwd(q, k, v, causal=causal, mode="sage", out_dtype=torch.float32,
                     workspace=_poisoned(need))
        torch.cuda.synchronize()
        assert torch.isfinite(b[0]).all() and torch.isfinite(b[1]).all()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), causal


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp6"])
def test_mx_workspace_contents_do_not_matter(attn, mode):
    q, k, v = _prefill(B=1, H=4, Hkv=2, N=333, d=128, seed=12)
    B, H, N, d = q.shape
    need = attn.attn_fwd_workspace_size(B, H, k.shape[1], N, d, attn.MODES[mode])
    for causal in (False, True):
        a = attn.fwd(q, k, v, causal=causal, mode=mode, out_dtype=torch.float32,
                     workspace=torch.zeros((need,), dtype=torch.uint8, device="cuda"))
        b = attn.fwd(q, k, v, causal=causal, mode=mode, out_dtype=torch.float32,
                     workspace=_poisoned(need))
        torch.cuda.synchronize()
        assert torch.isfinite(b[0]).all() and torch.isfinite(b[1]).all()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), causal


def test_decode_workspace_contents_do_not_matter(attn):
    B, H, Hkv, N, d = 3, 8, 2, 2000, 128
    g = torch.Generator().manual_seed(4)
    q = torch.randn((B, H, d), generator=g).to(torch.bfloat16).cuda()
    kc = torch.randn((B, Hkv, N, d), generator=g).to(torch.bfloat16).cuda()
    vc = torch.randn((B, Hkv, N, d), generator=g).to(torch.bfloat16).cuda()
    sl = torch.tensor([1, 777, 2000], dtype=torch.int32, device="cuda")
    for split in (64, 512):
        need = attn.attn_decode_workspace_size(B, H, Hkv, d)
        a = attn.decode(q, kc, vc, sl, split_tokens=split, out_dtype=torch.float32,
                        workspace=torch.zeros((need,), dtype=torch.uint8, device="cuda"))
        b = attn.decode(q, kc, vc, sl, split_tokens=split, out_dtype=torch.float32,
                        workspace=_poisoned(need))
        torch.cuda.synchronize()
        assert torch.isfinite(b[0]).all() and torch.isfinite(b[1]).all()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), split


def test_bwd_workspace_contents_do_not_matter(attn):
    q, k, v = _prefill(B=1, H=4, Hkv=2, N=300, d=128, seed=10)
    do = workloads.make_prefill(1, 4, 2, 300, 128, seed=11)[0].cuda()
    o, lse = attn.fwd(q, k, v, causal=True)
    need = attn.attn_bwd_workspace_size(1, 4, 300)
    a = attn.bwd(q, k, v, o, lse, do, causal=True, grad_dtype=torch.float32,
                 workspace=torch.zeros((need,), dtype=torch.uint8, device="cuda"))
    b = attn.bwd(q, k, v, o, lse, do, causal=True, grad_dtype=torch.float32,
                 workspace=_poisoned(need))
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.isfinite(y).all() and torch.equal(x, y)
