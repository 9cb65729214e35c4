"""GPU parity of the packed variable-length prefill (exact mode) against the
fp64 oracle run sequence by sequence, and against the fixed-layout call on
equal-length batches (same tiles, same arithmetic: bit-identical)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._compare import check_exact

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import softmax_attention_attn_amd as A
    return A


def _oracle(q, k, v, cu, causal, scale):
    return oracle.attn_varlen(workloads.bf16_bits(q), workloads.bf16_bits(k),
                              workloads.bf16_bits(v), cu.numpy(), causal=causal, scale=scale)


CASES = [
    # H, Hkv, d, lengths
    (4, 2, 128, (1, 255, 256, 257, 0, 700)),
    (8, 8, 128, (513,)),
    (8, 1, 64, (64, 3, 1000, 17)),
    (16, 4, 128, (300, 1, 1, 2, 299)),
]


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "H%dKV%dd%d-%s" % (
    c[0], c[1], c[2], "_".join(map(str, c[3]))))
def test_varlen_small(attn, case, causal, out_dtype):
    H, Hkv, d, lens = case
    q, k, v, cu = workloads.make_varlen(lens, H, Hkv, d, seed=sum(lens) + H)
    scale = 1 / math.sqrt(d)
    o, lse = attn.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), max(lens), causal=causal,
                             out_dtype=out_dtype)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(q, k, v, cu, causal, scale)
    check_exact(o.float().cpu().numpy(), o_ref, lse.cpu().numpy(), lse_ref,
                bf16_out=out_dtype == torch.bfloat16, what="varlen %s" % (case,))


@pytest.mark.parametrize("nseq", [64, 70], ids=["B64", "B70"])
def test_varlen_many_sequences(attn, nseq):
    """Up to 64 sequences are dispatched longest first (ranked in a wave,
    ties by index); beyond 64 they keep their order.  Both sides of that
    bound, with repeated and zero lengths, every row against the oracle."""
    g = torch.Generator().manual_seed(nseq)
    lens = tuple(int(x) for x in torch.randint(0, 160, (nseq,), generator=g))
    lens = lens[:5] + (lens[5],) * 3 + (0,) + lens[9:]
    H, Hkv, d = 2, 1, 64
    q, k, v, cu = workloads.make_varlen(lens, H, Hkv, d, seed=nseq)
    o, lse = attn.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), max(lens), causal=True,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(q, k, v, cu, True, 1 / math.sqrt(d))
    check_exact(o.float().cpu().numpy(), o_ref, lse.cpu().numpy(), lse_ref, bf16_out=False,
                what="varlen %d sequences" % nseq)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_varlen_equal_lengths_match_fixed_layout(attn, causal):
    B, H, Hkv, N, d = 3, 8, 2, 700, 128
    q, k, v, _ = workloads.make_prefill(B, H, Hkv, N, d, seed=31)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse = attn.fwd(qd, kd, vd, causal=causal, out_dtype=torch.float32)
    pack = lambda t: t.transpose(1, 2).reshape(B * N, t.shape[1], d).contiguous()
    cu = torch.arange(0, B * N + 1, N, dtype=torch.int32, device="cuda")
    ov, lsev = attn.fwd_varlen(pack(qd), pack(kd), pack(vd), cu, N, causal=causal,
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(ov, pack(o))
    assert torch.equal(lsev, lse.permute(1, 0, 2).reshape(H, B * N))


def test_varlen_workload(attn):
    """The packed workload (8 sequences, lengths uniform on [256, 4096]),
    every row compared with the oracle."""
    w = workloads.WORKLOADS["varlen_prefill"]
    inp = workloads.make(w)
    q, k, v, cu = inp["q"], inp["k"], inp["v"], inp["cu_seqlens"]
    o, lse = attn.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), w.N, causal=w.causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(q, k, v, cu, w.causal, w.scale)
    res = check_exact(o.float().cpu().numpy(), o_ref, lse.cpu().numpy(), lse_ref,
                      bf16_out=True, what=w.name)
    print(w.name, res)


def test_varlen_truncates_to_max_seqlen(attn):
    """A sequence longer than max_seqlen is cut to its first max_seqlen
    queries and keys; the others are computed in full."""
    lens = (600, 200)
    q, k, v, cu = workloads.make_varlen(lens, 4, 4, 128, seed=8)
    o = torch.zeros((800, 4, 128), dtype=torch.float32, device="cuda")
    attn.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), 300, causal=True,
                    out_dtype=torch.float32, o=o, with_lse=False)
    torch.cuda.synchronize()
    cut = torch.tensor([0, 300], dtype=torch.int32)
    o_ref0, _ = _oracle(q[:300], k[:300], v[:300], cut, True, 1 / math.sqrt(128))
    o_ref1, _ = _oracle(q[600:], k[600:], v[600:], torch.tensor([0, 200], dtype=torch.int32),
                        True, 1 / math.sqrt(128))
    oc = o.cpu().numpy()
    check_exact(oc[:300], o_ref0, None, None, bf16_out=False, what="truncated sequence")
    assert (oc[300:600] == 0).all()
    check_exact(oc[600:], o_ref1, None, None, bf16_out=False, what="sequence after it")


def test_varlen_clamps_malformed_offsets(attn):
    """Offsets out of order or past the end are clamped into [0, total]: the
    call completes, and rows owned by one well-formed sequence are right."""
    q, k, v, _ = workloads.make_varlen((300,), 4, 2, 128, seed=4)
    cu = torch.tensor([0, 100, 50, 300, 1 << 30], dtype=torch.int32)
    o, lse = attn.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), 300, causal=True,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(q[:100], k[:100], v[:100], torch.tensor([0, 100], dtype=torch.int32),
                             True, 1 / math.sqrt(128))
    # rows 0..49 belong to the first sequence only (the third starts at 50)
    check_exact(o[:50].cpu().numpy(), o_ref[:50], lse[:, :50].cpu().numpy(), lse_ref[:, :50],
                bf16_out=False, what="clamped offsets")
