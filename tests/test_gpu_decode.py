"""GPU parity of the split-KV GQA decode (split kernel + LSE merge) against the
fp64 oracle, which computes each query row over its valid keys without any
splitting.  Cache positions beyond each sequence length hold NaN, so any
over-read poisons the output."""
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


def _oracle(q, k, v, seqlens, scale):
    B, H, d = q.shape
    o, lse, err = oracle.attn_rows(workloads.bf16_bits(q.reshape(B, H, 1, d)),
                                   workloads.bf16_bits(k), workloads.bf16_bits(v),
                                   causal=False, scale=scale, kv_len=seqlens.numpy())
    assert err <= 1e-12
    return o.reshape(B, H, d), lse.reshape(B, H)


CASES = [
    # B, H, Hkv, N_max, d, lengths, split
    (3, 8, 2, 1000, 128, (1, 513, 1000), 512),
    (3, 8, 2, 1000, 128, (64, 65, 999), 64),
    (2, 4, 4, 700, 64, (700, 129), 128),
    (2, 16, 2, 300, 128, (300, 17), 256),
    (4, 2, 1, 2048, 128, (2048, 1, 1536, 777), 512),
    (2, 32, 2, 1100, 128, (1100, 31), 128),
]


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dKV%dN%dd%d-%s-s%d" % (
    c[0], c[1], c[2], c[3], c[4], "_".join(map(str, c[5])), c[6]))
def test_small_decode(attn, case, out_dtype):
    B, H, Hkv, N, d, lens, split = case
    q, k, v, _ = workloads.make_prefill(B, H, Hkv, N, d, seed=B + H + N)
    q = q[:, :, 0].contiguous()
    seqlens = torch.tensor(lens, dtype=torch.int32)
    for b, L in enumerate(lens):
        k[b, :, L:] = float("nan")
        v[b, :, L:] = float("nan")
    scale = 1 / math.sqrt(d)
    o, lse = attn.decode(q.cuda(), k.cuda(), v.cuda(), seqlens.cuda(), split_tokens=split,
                         out_dtype=out_dtype)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(q, k, v, seqlens, scale)
    check_exact(o.float().cpu().numpy(), o_ref, lse.cpu().numpy(), lse_ref,
                bf16_out=out_dtype == torch.bfloat16, what=str(case))


def test_rising_scores_decode(attn):
    """Scores rising from key to key move each chunk's running max on every
    sub-tile (the decode kernel's rescale path)."""
    from tests.test_gpu_prefill import _rising_keys
    B, H, Hkv, N, d = 2, 8, 2, 1500, 128
    qf, k, v = _rising_keys(B, H, Hkv, N, d, seed=5, top=40.0)
    q = qf[:, :, 0].contiguous()
    seqlens = torch.tensor((1500, 901), dtype=torch.int32)
    k[1, :, 901:] = float("nan")
    v[1, :, 901:] = float("nan")
    o, lse = attn.decode(q.cuda(), k.cuda(), v.cuda(), seqlens.cuda(), split_tokens=256,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(q, k, v, seqlens, 1 / math.sqrt(d))
    check_exact(o.float().cpu().numpy(), o_ref, lse.cpu().numpy(), lse_ref, bf16_out=False,
                what="rising scores decode")


def test_split_size_invariance(attn):
    B, H, Hkv, N, d = 2, 8, 2, 2000, 128
    q, k, v, seqlens = workloads.make_decode(B, H, Hkv, N, d, len_lo=1500, len_hi=2000, seed=9)
    outs = []
    for split in (64, 256, 512):
        o, lse = attn.decode(q.cuda(), k.cuda(), v.cuda(), seqlens.cuda(), split_tokens=split,
                             out_dtype=torch.float32)
        torch.cuda.synchronize()
        outs.append((o.cpu().numpy(), lse.cpu().numpy()))
    # P is rounded to bf16 relative to each chunk's own max before the PV
    # product, so chunkings agree to bf16 precision (each is checked against
    # the oracle elsewhere); the LSE does not see that rounding
    for o, lse in outs[1:]:
        assert np.abs(o - outs[0][0]).max() < 2e-3
        assert np.abs(lse - outs[0][1]).max() < 1e-5


def test_gqa_decode_workload_full(attn):
    """The full decode workload, every (b, h) row compared."""
    w = workloads.WORKLOADS["gqa_decode"]
    inp = workloads.make(w)
    q, k, v, seqlens = inp["q"], inp["k"], inp["v"], inp["seqlens"]
    o, lse = attn.decode(q.cuda(), k.cuda(), v.cuda(), seqlens.cuda(),
                         split_tokens=w.split_tokens)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(q, k, v, seqlens, w.scale)
    res = check_exact(o.float().cpu().numpy(), o_ref, lse.cpu().numpy(), lse_ref,
                      bf16_out=True, what=w.name, literal=True)
    print(w.name, res)


def test_decode_rejects_unsupported(attn):
    q = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16, device="cuda")
    sl = torch.ones((1,), dtype=torch.int32, device="cuda")
    with pytest.raises(attn.AttnError) as e:
        attn.decode(q, kc, kc, sl, split_tokens=100)
    assert e.value.status == attn.ATTN_ERR_INVALID_ARG


# ------------------------------------------------------------------ paged KV

PAGED_CASES = [
    # B, H, Hkv, d, lengths, page_size, split, spare pages
    (3, 8, 2, 128, (1, 513, 1000), 16, 512, 5),
    (3, 8, 2, 128, (64, 65, 999), 32, 64, 0),
    (2, 4, 4, 64, (700, 129), 64, 128, 3),
    (2, 16, 2, 128, (300, 17), 128, 256, 1),
    (4, 2, 1, 128, (2048, 1, 1536, 777), 1024, 512, 2),
    (2, 32, 2, 128, (1100, 31), 16, 1024, 4),
]


def _paged_inputs(B, H, Hkv, d, lens, ps, spare, seed):
    max_pages = (max(lens) + ps - 1) // ps
    N = max_pages * ps
    q, k, v, _ = workloads.make_prefill(B, H, Hkv, N, d, seed=seed)
    q = q[:, :, 0].contiguous()
    seqlens = torch.tensor(lens, dtype=torch.int32)
    for b, L in enumerate(lens):
        k[b, :, L:] = float("nan")
        v[b, :, L:] = float("nan")
    table, num_pages = workloads.make_page_table(lens, ps, seed=seed + 1, spare_pages=spare,
                                                 max_pages=max_pages)
    kp = workloads.paginate(k, table, num_pages, ps)
    vp = workloads.paginate(v, table, num_pages, ps)
    return q, k, v, seqlens, table, kp, vp


@pytest.mark.parametrize("case", PAGED_CASES, ids=lambda c: "B%dH%dKV%dd%d-%s-p%d-s%d" % (
    c[0], c[1], c[2], c[3], "_".join(map(str, c[4])), c[5], c[6]))
def test_paged_decode(attn, case):
    """Paged caches give bit-identical results to the same keys held
    contiguously (the chunking and arithmetic do not change), and match the
    oracle run on caches gathered back from the page pool."""
    B, H, Hkv, d, lens, ps, split, spare = case
    q, k, v, seqlens, table, kp, vp = _paged_inputs(B, H, Hkv, d, lens, ps, spare,
                                                    seed=B * 7 + ps)
    o_p, lse_p = attn.decode_paged(q.cuda(), kp.cuda(), vp.cuda(), table.cuda(), seqlens.cuda(),
                                   split_tokens=split, out_dtype=torch.float32)
    o_c, lse_c = attn.decode(q.cuda(), k.cuda(), v.cuda(), seqlens.cuda(), split_tokens=split,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_c) and torch.equal(lse_p, lse_c)
    kg = oracle.gather_pages(workloads.bf16_bits(kp), table.numpy(), seqlens.numpy(), ps)
    vg = oracle.gather_pages(workloads.bf16_bits(vp), table.numpy(), seqlens.numpy(), ps)
    o_ref, lse_ref, err = oracle.attn_rows(workloads.bf16_bits(q.reshape(B, H, 1, d)), kg, vg,
                                           causal=False, scale=1 / math.sqrt(d),
                                           kv_len=seqlens.numpy())
    assert err <= 1e-12
    check_exact(o_p.cpu().numpy(), o_ref.reshape(B, H, d), lse_p.cpu().numpy(),
                lse_ref.reshape(B, H), bf16_out=False, what="paged " + str(case))


def test_paged_decode_workload(attn):
    """The decode workload's caches spread over 16-row pages in a random
    order: bit-identical to the contiguous call on every row, and within the
    exact-mode tolerance of the oracle on the gathered caches of 8 sequences."""
    w = workloads.WORKLOADS["gqa_decode"]
    inp = workloads.make(w)
    q, k, v, seqlens = inp["q"], inp["k"], inp["v"], inp["seqlens"]
    ps = 16
    table, num_pages = workloads.make_page_table(seqlens, ps, seed=77, spare_pages=100,
                                                 max_pages=w.N // ps)
    kd, vd = k.cuda(), v.cuda()
    kp = workloads.paginate(kd, table, num_pages, ps)
    vp = workloads.paginate(vd, table, num_pages, ps)
    o_c, lse_c = attn.decode(q.cuda(), kd, vd, seqlens.cuda(), split_tokens=w.split_tokens)
    del kd, vd
    o_p, lse_p = attn.decode_paged(q.cuda(), kp, vp, table.cuda(), seqlens.cuda(),
                                   split_tokens=w.split_tokens)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_c) and torch.equal(lse_p, lse_c)
    sel = [0, 5, 17, 28, 33, 41, 50, 63]
    tab_s = table[sel].numpy()
    sl_s = seqlens[sel].numpy()
    kg = oracle.gather_pages(workloads.bf16_bits(kp.cpu()), tab_s, sl_s, ps)
    vg = oracle.gather_pages(workloads.bf16_bits(vp.cpu()), tab_s, sl_s, ps)
    B, H, d = len(sel), w.H, w.d
    o_ref, lse_ref, err = oracle.attn_rows(
        workloads.bf16_bits(q[sel].reshape(B, H, 1, d)), kg, vg, causal=False, scale=w.scale,
        kv_len=sl_s)
    assert err <= 1e-12
    res = check_exact(o_p[sel].float().cpu().numpy(), o_ref.reshape(B, H, d),
                      lse_p[sel].cpu().numpy(), lse_ref.reshape(B, H), bf16_out=True,
                      what="paged " + w.name)
    print("paged", w.name, res)


def test_paged_decode_clamps_bad_page_numbers(attn):
    """Page numbers outside the pool are clamped into it by the kernel: the
    call completes and returns finite values (which ones is unspecified)."""
    # whole pages only, so that no pool row is NaN
    q, k, v, seqlens, table, kp, vp = _paged_inputs(2, 8, 2, 128, (304, 208), 16, 0, seed=3)
    bad = table.clone()
    bad[0, 3] = 1 << 30
    bad[1, 0] = -5
    o, lse = attn.decode_paged(q.cuda(), kp.cuda(), vp.cuda(), bad.cuda(), seqlens.cuda(),
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    # the pool holds only real rows (no spare pages, no partial last page)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


# ------------------------------------------------- the work split's edge cases

def _decode_vs_oracle(attn, B, H, Hkv, N, d, lens, split, seed, what):
    q, k, v, _ = workloads.make_prefill(B, H, Hkv, N, d, seed=seed)
    q = q[:, :, 0].contiguous()
    seqlens = torch.tensor(lens, dtype=torch.int32)
    for b, L in enumerate(lens):
        k[b, :, L:] = float("nan")
        v[b, :, L:] = float("nan")
    o, lse = attn.decode(q.cuda(), k.cuda(), v.cuda(), seqlens.cuda(), split_tokens=split,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(q, k, v, seqlens, 1 / math.sqrt(d))
    return check_exact(o.cpu().numpy(), o_ref, lse.cpu().numpy(), lse_ref, bf16_out=False,
                       what=what)


def test_decode_many_short_sequences(attn):
    """300 sequences of 1 to 8 keys with one kv head: a wave's range crosses
    hundreds of sequences (its window of 64 sequence lengths is reloaded) and
    most pieces are shorter than a sub-tile."""
    g = torch.Generator().manual_seed(5)
    lens = torch.randint(1, 9, (300,), generator=g).tolist()
    res = _decode_vs_oracle(attn, 300, 4, 1, 8, 128, lens, 64, 41, "300 short sequences")
    print(res)


def test_decode_one_long_sequence(attn):
    """One sequence of 70000 keys over two kv heads: every wave's range lies in
    one segment, and each head merges hundreds of partials (the merge's
    64-at-a-time loop)."""
    res = _decode_vs_oracle(attn, 1, 8, 2, 70000, 128, (70000,), 512, 42, "one long sequence")
    print(res)


def test_decode_ragged_lengths_all_group_sizes(attn):
    """Lengths that are not multiples of the 32-key sub-tile, for every group
    size, at d 64 and 128."""
    for G in (1, 2, 4, 8, 16):
        for d in (64, 128):
            lens = (33, 1000, 4097, 31, 555)
            _decode_vs_oracle(attn, 5, 2 * G, 2, 4200, d, lens, 128, G + d,
                              "G%d d%d" % (G, d))
