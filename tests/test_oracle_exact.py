"""Pins of the exact-attention oracle against things other than itself.

Each test checks the oracle against brute force on tiny inputs, a library
routine (torch's scaled_dot_product_attention in fp64 on the CPU), a closed
form, or an invariant that exact softmax attention must satisfy.  Together
they are chosen so that a dropped term, a wrong sign or index, a transposed
operand, a wrong causal direction, a wrong GQA head map or a wrong LSE base
each fail at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits


def _bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def _rand(shape, gen, scale=1.0):
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * scale).to(torch.bfloat16)


def _brute(q, k, v, causal, scale, kv_len=None):
    """Materialised S and P with numpy, one (b, h) at a time."""
    q = q.to(torch.float64).numpy()
    k = k.to(torch.float64).numpy()
    v = v.to(torch.float64).numpy()
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    o = np.zeros((B, H, Nq, d))
    lse = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            g = h // (H // Hkv)
            S = q[b, h] @ k[b, g].T * scale
            mask = np.ones((Nq, Nk), dtype=bool)
            if causal:
                mask &= np.tril(np.ones((Nq, Nk), dtype=bool))
            if kv_len is not None:
                mask[:, kv_len[b]:] = False
            S = np.where(mask, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            P = E / E.sum(axis=1, keepdims=True)
            o[b, h] = P @ v[b, g]
            lse[b, h] = (m[:, 0] + np.log(E.sum(axis=1)))
    return o, lse


def _run(q, k, v, causal, scale, **kw):
    o, lse, err = oracle.attn_rows(bf16_bits(q), bf16_bits(k), bf16_bits(v), causal=causal,
                                   scale=scale, **kw)
    return o, lse, err


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 4), (2, 4, 2, 17, 16), (1, 6, 3, 64, 8),
                                   (1, 2, 1, 33, 5)])
def test_brute_force_tiny(oracle_lib, causal, shape):
    B, H, Hkv, N, d = shape
    g = torch.Generator().manual_seed(hash(shape) % 1000 + causal)
    q, k, v = _rand((B, H, N, d), g), _rand((B, Hkv, N, d), g), _rand((B, Hkv, N, d), g)
    scale = 1.0 / math.sqrt(d)
    o, lse, err = _run(q, k, v, causal, scale)
    ob, lseb = _brute(q, k, v, causal, scale)
    assert err <= 1e-12
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lseb, rtol=0, atol=1e-12)


def test_brute_force_adversarial(oracle_lib):
    """Large-magnitude scores (a naive exp would overflow) and ties."""
    g = torch.Generator().manual_seed(7)
    B, H, Hkv, N, d = 1, 2, 1, 24, 8
    q = _rand((B, H, N, d), g, scale=30.0)
    k = _rand((B, Hkv, N, d), g, scale=30.0)
    k[0, 0, 5] = k[0, 0, 9]  # tie between two keys
    v = _rand((B, Hkv, N, d), g)
    for causal in (False, True):
        o, lse, err = _run(q, k, v, causal, 1.0)
        ob, lseb = _brute(q, k, v, causal, 1.0)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-10)
        np.testing.assert_allclose(lse, lseb, rtol=1e-13, atol=1e-9)


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_sdpa_fp64(oracle_lib, causal):
    g = torch.Generator().manual_seed(11)
    B, H, Hkv, N, d = 2, 8, 2, 48, 32
    q, k, v = _rand((B, H, N, d), g), _rand((B, Hkv, N, d), g), _rand((B, Hkv, N, d), g)
    scale = 0.37
    o, lse, _ = _run(q, k, v, causal, scale)
    rep = H // Hkv
    kk = k.to(torch.float64).repeat_interleave(rep, dim=1)
    vv = v.to(torch.float64).repeat_interleave(rep, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.to(torch.float64), kk, vv, is_causal=causal, scale=scale)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    # LSE against torch.logsumexp of the masked scores
    S = (q.to(torch.float64) @ kk.transpose(-1, -2)) * scale
    if causal:
        S = S.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(S, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_rows_subset_matches_full(oracle_lib):
    g = torch.Generator().manual_seed(3)
    B, H, Hkv, N, d = 2, 4, 2, 40, 16
    q, k, v = _rand((B, H, N, d), g), _rand((B, Hkv, N, d), g), _rand((B, Hkv, N, d), g)
    o, lse, _ = _run(q, k, v, True, 0.25)
    rows = np.array([0, 5, 39, 40, 77, B * H * N - 1])
    os_, ls, _ = _run(q, k, v, True, 0.25, rows=rows)
    np.testing.assert_array_equal(os_, o.reshape(-1, d)[rows])
    np.testing.assert_array_equal(ls, lse.reshape(-1)[rows])


def test_identical_keys_give_mean_of_v(oracle_lib):
    """All keys equal -> uniform P -> O is the mean of the visible V rows and
    lse = s*q.k + ln(#visible)."""
    g = torch.Generator().manual_seed(5)
    B, H, N, d = 1, 2, 32, 16
    q = _rand((B, H, N, d), g)
    krow = _rand((d,), g)
    k = krow.expand(B, 1, N, d).contiguous()
    v = _rand((B, 1, N, d), g)
    scale = 0.5
    vd = v.to(torch.float64).numpy()[0, 0]
    qd = q.to(torch.float64).numpy()
    kd = krow.to(torch.float64).numpy()
    for causal in (False, True):
        o, lse, _ = _run(q, k, v, causal, scale)
        for i in range(N):
            nvis = i + 1 if causal else N
            np.testing.assert_allclose(o[0, :, i], np.broadcast_to(vd[:nvis].mean(0), (H, d)),
                                       rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[0, :, i], scale * qd[0, :, i] @ kd + math.log(nvis),
                                       rtol=0, atol=1e-12)


def test_zero_query_closed_form(oracle_lib):
    g = torch.Generator().manual_seed(6)
    B, H, N, d = 1, 1, 20, 8
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
    k, v = _rand((B, 1, N, d), g), _rand((B, 1, N, d), g)
    vd = v.to(torch.float64).numpy()[0, 0]
    o, lse, _ = _run(q, k, v, True, 1.0)
    for i in range(N):
        np.testing.assert_allclose(o[0, 0, i], vd[: i + 1].mean(0), atol=1e-14)
        assert abs(lse[0, 0, i] - math.log(i + 1)) < 1e-14
    o, lse, _ = _run(q, k, v, False, 1.0)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(vd.mean(0), (N, d)), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], math.log(N), atol=1e-14)


def test_causal_row0_and_single_key(oracle_lib):
    g = torch.Generator().manual_seed(8)
    q, k, v = _rand((1, 3, 9, 8), g), _rand((1, 3, 9, 8), g), _rand((1, 3, 9, 8), g)
    o, lse, _ = _run(q, k, v, True, 0.3)
    vd = v.to(torch.float64).numpy()
    np.testing.assert_array_equal(o[0, :, 0], vd[0, :, 0])
    s0 = 0.3 * np.einsum("hc,hc->h", q.to(torch.float64).numpy()[0, :, 0],
                         k.to(torch.float64).numpy()[0, :, 0])
    np.testing.assert_allclose(lse[0, :, 0], s0, atol=1e-14)
    # N = 1, non-causal: O = V0
    o1, _, _ = _run(q[:, :, :1], k[:, :, :1], v[:, :, :1], False, 0.3)
    np.testing.assert_array_equal(o1[0, :, 0], vd[0, :, 0])


def test_smooth_k_invariance(oracle_lib):
    """Subtracting any per-channel vector from every key leaves O unchanged and
    shifts lse_i by -s * q_i . kbar (the shift is a row constant)."""
    g = torch.Generator().manual_seed(9)
    B, H, N, d = 1, 2, 30, 16
    q = _rand((B, H, N, d), g)
    # keys on a 1/8 grid in [-4, 4] so that adding the shift is exact in bf16
    k2 = _bf16(torch.clamp(torch.round(torch.randn((B, 1, N, d), generator=g) * 8) / 8, -4, 4))
    v = _rand((B, 1, N, d), g)
    kbar = _bf16(torch.tensor([1.0, -2.0] * (d // 2)))
    k = _bf16(k2.to(torch.float32) + kbar.to(torch.float32))
    assert torch.equal(k.to(torch.float32) - kbar.to(torch.float32), k2.to(torch.float32))
    for causal in (False, True):
        o1, l1, _ = _run(q, k, v, causal, 0.2)
        o2, l2, _ = _run(q, k2, v, causal, 0.2)
        np.testing.assert_allclose(o2, o1, atol=1e-12)
        shift = 0.2 * q.to(torch.float64).numpy() @ kbar.to(torch.float64).numpy()
        np.testing.assert_allclose(l2, l1 - shift, atol=1e-12)


def test_affine_v_and_permutation(oracle_lib):
    g = torch.Generator().manual_seed(10)
    B, H, N, d = 1, 2, 26, 8
    q, k, v = _rand((B, H, N, d), g), _rand((B, 2, N, d), g), _rand((B, 2, N, d), g)
    o, lse, _ = _run(q, k, v, False, 0.4)
    # V -> 2 V + 1 c^T is exact in bf16 for these magnitudes only approximately,
    # so compare against the transformed oracle output in fp64.
    c = torch.linspace(-1, 1, d)
    v2 = (2 * v.to(torch.float32) + c).to(torch.bfloat16)
    o2, lse2, _ = _run(q, k, v2, False, 0.4)
    ov2, _ = _brute(q, k, v2, False, 0.4)
    np.testing.assert_allclose(o2, ov2, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=0)  # V does not enter the LSE
    # joint permutation of key/value rows (non-causal) leaves everything unchanged
    perm = torch.randperm(N, generator=g)
    o3, lse3, _ = _run(q, k[:, :, perm], v[:, :, perm], False, 0.4)
    np.testing.assert_allclose(o3, o, atol=1e-13)
    np.testing.assert_allclose(lse3, lse, atol=1e-13)


def test_dominant_key(oracle_lib):
    """A key whose score beats all others by >= 50 gives O = V_j (to ~1e-20)."""
    d, N = 8, 16
    q = torch.zeros((1, 1, 1, d), dtype=torch.bfloat16)
    q[0, 0, 0, 0] = 1.0
    k = torch.zeros((1, 1, N, d), dtype=torch.bfloat16)
    k[0, 0, 7, 0] = 64.0
    g = torch.Generator().manual_seed(12)
    v = _rand((1, 1, N, d), g)
    o, lse, _ = _run(q, k, v, False, 1.0)
    np.testing.assert_allclose(o[0, 0, 0], v.to(torch.float64).numpy()[0, 0, 7], atol=1e-20)
    assert abs(lse[0, 0, 0] - (64.0 + math.log1p((N - 1) * math.exp(-64.0)))) < 1e-12


def test_decode_kv_len_matches_brute(oracle_lib):
    g = torch.Generator().manual_seed(13)
    B, H, Hkv, Nmax, d = 3, 8, 2, 40, 16
    q = _rand((B, H, 1, d), g)
    k, v = _rand((B, Hkv, Nmax, d), g), _rand((B, Hkv, Nmax, d), g)
    kv_len = np.array([1, 17, 40], dtype=np.int32)
    # poison the positions beyond each length: the oracle must never read them
    for b, L in enumerate(kv_len):
        k[b, :, L:] = float("nan")
        v[b, :, L:] = float("nan")
    o, lse, _ = _run(q, k, v, False, 0.25, kv_len=kv_len)
    kc, vc = k.clone(), v.clone()
    for b, L in enumerate(kv_len):
        kc[b, :, L:] = 0
        vc[b, :, L:] = 0
    ob, lseb = _brute(q, kc, vc, False, 0.25, kv_len=kv_len)
    assert np.isfinite(o).all()
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(lse, lseb, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_is_block_diagonal_attention(oracle_lib, causal):
    """The packed batch against one softmax over all packed tokens whose mask
    keeps only same-sequence (and, causal, earlier-or-equal) keys."""
    g = torch.Generator().manual_seed(21)
    lens = [5, 0, 1, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, Hkv, d, scale = int(cu[-1]), 4, 2, 8, 0.3
    q, k, v = _rand((T, H, d), g), _rand((T, Hkv, d), g), _rand((T, Hkv, d), g)
    o, lse = oracle.attn_varlen(bf16_bits(q), bf16_bits(k), bf16_bits(v), cu, causal=causal,
                                scale=scale)
    seq = np.repeat(np.arange(len(lens)), lens)
    pos = np.arange(T) - cu[seq]
    mask = seq[:, None] == seq[None, :]
    if causal:
        mask &= pos[None, :] <= pos[:, None]
    qd, kd, vd = (x.to(torch.float64).numpy() for x in (q, k, v))
    for h in range(H):
        gh = h // (H // Hkv)
        S = np.where(mask, qd[:, h] @ kd[:, gh].T * scale, -np.inf)
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        np.testing.assert_allclose(o[:, h], (E / E.sum(1, keepdims=True)) @ vd[:, gh],
                                   atol=1e-12)
        np.testing.assert_allclose(lse[h], m[:, 0] + np.log(E.sum(1)), atol=1e-12)


def test_gather_pages_worked_example():
    # pool of 3 pages of 2 rows (1 kv head, d = 1); page p row j holds 10p + j.
    # Sequence 0 (3 keys) uses pages 2 then 0, sequence 1 (4 keys) pages 1 then 2:
    # its positions 0..3 are page 1 rows 0, 1 and page 2 rows 0, 1.
    pages = np.array([[[[0], [1]]], [[[10], [11]]], [[[20], [21]]]], dtype=np.int64)
    table = np.array([[2, 0], [1, 2]])
    out = oracle.gather_pages(pages, table, np.array([3, 4]), 2)
    assert out.shape == (2, 1, 4, 1)
    assert out[:, 0, :, 0].tolist() == [[20, 21, 0, 0], [10, 11, 20, 21]]


@pytest.mark.parametrize("page_size", [1, 4, 16])
def test_gather_pages_inverts_a_scatter(page_size):
    # scatter contiguous caches into a shuffled pool one whole page at a time
    # (slices, not positions), then gather them back
    rng = np.random.default_rng(page_size)
    B, Hkv, d, max_pages = 3, 2, 5, 6
    L = np.array([1, page_size * max_pages, page_size * 2 + 1])
    cont = rng.standard_normal((B, Hkv, max_pages * page_size, d))
    used = [(b, j) for b in range(B) for j in range((L[b] + page_size - 1) // page_size)]
    perm = rng.permutation(len(used) + 3)  # 3 spare pages stay NaN
    pool = np.full((len(used) + 3, Hkv, page_size, d), np.nan)
    table = np.full((B, max_pages), -1)
    for (b, j), p in zip(used, perm):
        table[b, j] = p
        pool[p] = cont[b, :, j * page_size:(j + 1) * page_size, :]
    out = oracle.gather_pages(pool, table, L, page_size)
    for b in range(B):
        np.testing.assert_array_equal(out[b, :, :L[b]], cont[b, :, :L[b]])
        assert (out[b, :, L[b]:] == 0).all()


@pytest.mark.parametrize("cuts", [(0, 40), (0, 1, 40), (0, 8, 16, 24, 32, 40), (0, 13, 29, 40)])
def test_split_and_merge_equals_unsplit(oracle_lib, cuts):
    g = torch.Generator().manual_seed(14)
    B, H, Hkv, N, d = 2, 4, 2, 40, 8
    q = _rand((B, H, 1, d), g)
    k, v = _rand((B, Hkv, N, d), g), _rand((B, Hkv, N, d), g)
    kv_len = np.array([40, 23], dtype=np.int32)
    o, lse, _ = _run(q, k, v, False, 0.3, kv_len=kv_len)
    parts_o, parts_l = [], []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        po, pl, _ = _run(q, k, v, False, 0.3, kv_len=kv_len, k_range=(lo, hi))
        parts_o.append(po.reshape(-1, d))
        parts_l.append(pl.reshape(-1))
    mo, ml = oracle.lse_merge(np.stack(parts_o), np.stack(parts_l))
    np.testing.assert_allclose(mo, o.reshape(-1, d), atol=1e-13)
    np.testing.assert_allclose(ml, lse.reshape(-1), atol=1e-13)
    # order invariance of the merge
    mo2, ml2 = oracle.lse_merge(np.stack(parts_o[::-1]), np.stack(parts_l[::-1]))
    np.testing.assert_allclose(mo2, mo, atol=1e-14)
    np.testing.assert_allclose(ml2, ml, atol=1e-14)


def test_softmax_rows_sum_to_one_reported(oracle_lib):
    g = torch.Generator().manual_seed(15)
    q, k, v = _rand((1, 2, 64, 16), g, 4.0), _rand((1, 2, 64, 16), g, 4.0), _rand((1, 2, 64, 16), g)
    _, _, err = _run(q, k, v, True, 1.0)
    assert 0 <= err <= 1e-12


def test_rejects_bad_shapes(oracle_lib):
    q = np.zeros((1, 3, 4, 8), dtype=np.uint16)
    k = np.zeros((1, 2, 4, 8), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.attn_rows(q, k, k, causal=False, scale=1.0)  # H % Hkv != 0
    with pytest.raises(TypeError):
        oracle.attn_rows(q.astype(np.float32), k, k, causal=False, scale=1.0)
