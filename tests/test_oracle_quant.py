"""Pins of the oracle's quantisation routines and of the quantised-attention
emulator.

* E4M3: all 256 codes against torch's float8_e4m3fn (an independent library
  implementation of the OCP format) and against the printed E4M3 maximum.
* INT8: against numpy's round-half-to-even.
* The emulator's steps: Smooth-K mean against numpy, block scales against
  their closed form, codes against numpy.
* The emulator as a whole: with quantisation switched off it must equal the
  exact oracle (this checks the tile loop, the 448 fold, the V-scale
  bookkeeping and the Smooth-K LSE correction); with quantisation on but every
  quantity exactly representable it must also equal the exact oracle; on
  Gaussian inputs its error must sit inside what E4M3's 3-bit mantissa allows,
  and Smooth-K must reduce the error when K carries a shared bias.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_facts.json")


def _rand(shape, gen, scale=1.0):
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * scale).to(torch.bfloat16)


def _bits(*ts):
    return [bf16_bits(t) for t in ts]


# --------------------------------------------------------------------------- E4M3

def test_e4m3_decode_all_codes_vs_torch(oracle_lib):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_e4m3_golden_facts(oracle_lib):
    facts = json.load(open(GOLDEN))
    assert oracle.e4m3_decode(np.array([0x7E]))[0] == facts["e4m3_max_finite"]
    for ex in facts["round_trip_examples"]:
        got = oracle.e4m3_decode(oracle.e4m3_encode(np.array([ex["x"]])))[0]
        assert got == ex["nearest_even"], ex
        got = oracle.e4m3_decode(oracle.e4m3_encode(np.array([-ex["x"]])))[0]
        assert got == -ex["nearest_even"], ex


def test_e4m3_encode_vs_torch_cast(oracle_lib):
    g = torch.Generator().manual_seed(0)
    x = torch.cat([
        torch.randn(20000, generator=g, dtype=torch.float64) * 50,
        torch.rand(20000, generator=g, dtype=torch.float64) * 1e-2,
        torch.linspace(-460, 460, 5001, dtype=torch.float64),
        # every midpoint between neighbouring codes (ties)
        torch.from_numpy(np.convolve(oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)),
                                     [0.5, 0.5], mode="valid")),
    ])
    ours = oracle.e4m3_decode(oracle.e4m3_encode(x.numpy()))
    # torch's cast rounds to nearest even but returns NaN above 464; clamp first
    ref = x.clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_saturates_and_nan(oracle_lib):
    enc = oracle.e4m3_encode(np.array([1e30, -1e30, np.inf, -np.inf, np.nan]))
    assert list(enc[:4]) == [0x7E, 0xFE, 0x7E, 0xFE]
    assert enc[4] in (0x7F, 0xFF)


# --------------------------------------------------------------------------- INT8

def test_int8_quant_vs_numpy_rint(oracle_lib):
    g = np.random.default_rng(1)
    x = np.concatenate([g.normal(size=5000) * 3, np.arange(-130, 131) + 0.5,
                        np.array([126.5, -126.5, 127.49, 200.0, -200.0])])
    delta = 1.0
    ref = np.clip(np.rint(x / delta), -127, 127)
    np.testing.assert_array_equal(oracle.quant_i8(x, delta), ref)
    delta = 0.037
    np.testing.assert_array_equal(oracle.quant_i8(x, delta), np.clip(np.rint(x / delta), -127, 127))


def test_sage_quantise_steps(oracle_lib):
    """Each quantisation step against numpy, with the codes decided in fp32
    (the kernel's precision): kmean = mean (fp64, rounded to fp32),
    delta = max|x| / 127, code = rint(x * (127 / max|x|)); V codes =
    E4M3(V * (448 / max|V|)) via torch's float8_e4m3fn cast."""
    g = torch.Generator().manual_seed(2)
    B, H, Hkv, N, d, blk = 1, 4, 2, 150, 16, 64  # ragged last block (150 = 2*64 + 22)
    q = _rand((B, H, N, d), g)
    k = _rand((B, Hkv, N, d), g) + torch.linspace(-5, 5, d).to(torch.bfloat16)
    v = _rand((B, Hkv, N, d), g)
    v[0, 1, :, 3] = 0  # an all-zero V channel uses delta = 1
    st = oracle.sage_quantise(*_bits(q, k, v), blk=blk)
    f32 = np.float32
    kd = k.to(torch.float32).numpy()
    qd = q.to(torch.float32).numpy()
    vd = v.to(torch.float32).numpy()
    kmean = k.to(torch.float64).numpy().mean(axis=2).astype(f32)
    np.testing.assert_array_equal(st["kmean"], kmean.astype(np.float64))
    ks = kd - kmean[:, :, None, :]  # fp32 subtraction
    nb = math.ceil(N / blk)
    for t in range(nb):
        sl = slice(t * blk, min((t + 1) * blk, N))
        aq = np.abs(qd[:, :, sl]).max(axis=(2, 3))
        ak = np.abs(ks[:, :, sl]).max(axis=(2, 3))
        np.testing.assert_array_equal(st["qdelta"][:, :, t], (aq / f32(127)).astype(np.float64))
        np.testing.assert_array_equal(st["kdelta"][:, :, t], (ak / f32(127)).astype(np.float64))
        iq = (f32(127) / aq)[:, :, None, None]
        ik = (f32(127) / ak)[:, :, None, None]
        np.testing.assert_array_equal(st["qhat"][:, :, sl],
                                      np.clip(np.rint(qd[:, :, sl] * iq), -127, 127))
        np.testing.assert_array_equal(st["khat"][:, :, sl],
                                      np.clip(np.rint(ks[:, :, sl] * ik), -127, 127))
    # each block's extreme value maps to +-127
    assert np.abs(st["qhat"]).max() == 127 and np.abs(st["khat"]).max() == 127
    av = np.abs(vd).max(axis=2)
    dv = np.where(av > 0, av / f32(448), f32(1))
    np.testing.assert_array_equal(st["vdelta"], dv.astype(np.float64))
    assert st["vdelta"][0, 1, 3] == 1.0
    iv = np.where(av > 0, f32(448) / np.where(av > 0, av, 1), f32(1))
    ref_vq = torch.from_numpy(vd * iv[:, :, None, :]).clamp(-448, 448).to(
        torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(st["vq"], ref_vq)


# --------------------------------------------------------------------------- emulator

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tile_n", [16, 64, 1000])
def test_emulator_without_quantisation_is_exact(oracle_lib, causal, tile_n):
    g = torch.Generator().manual_seed(3)
    B, H, Hkv, N, d = 1, 4, 2, 130, 32
    q = _rand((B, H, N, d), g)
    k = _rand((B, Hkv, N, d), g) + torch.linspace(-3, 3, d).to(torch.bfloat16)
    v = _rand((B, Hkv, N, d), g)
    qb, kb, vb = _bits(q, k, v)
    o, lse = oracle.sage_rows(qb, kb, vb, causal=causal, scale=0.2, tile_n=tile_n,
                              quant_qk=False, quant_p=False, quant_v=False)
    oe, lsee, _ = oracle.attn_rows(qb, kb, vb, causal=causal, scale=0.2)
    np.testing.assert_allclose(o, oe, atol=1e-12)
    np.testing.assert_allclose(lse, lsee, atol=1e-11)


def test_emulator_exact_on_representable_inputs(oracle_lib):
    """Every quantity on its quantisation grid: Q, K in {-1,0,1} with zero
    channel mean of K, scale = ln 2 (so P = 2^integer), V on the E4M3 grid
    with each channel reaching +-448.  The emulator must then be exact."""
    rng = np.random.default_rng(4)
    B, H, N, d = 1, 2, 128, 8

    def sparse_pm1(rows):
        x = np.zeros((rows, d))
        for r in range(rows):
            idx = rng.choice(d, size=3, replace=False)
            x[r, idx] = rng.choice([-1.0, 1.0], size=3)
        return x

    qv = sparse_pm1(B * H * N).reshape(B, H, N, d)
    kh = sparse_pm1(N // 2)
    kv = np.concatenate([kh, -kh])[rng.permutation(N)].reshape(B, 1, N, d)
    assert np.all(kv.mean(axis=2) == 0)
    for t in range(N // 64):  # every 64-token block reaches |1|
        assert np.abs(kv[..., t * 64:(t + 1) * 64, :]).max() == 1
        assert np.abs(qv[..., t * 64:(t + 1) * 64, :]).max(axis=(2, 3)).min() == 1
    grid = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    vv = rng.choice(np.concatenate([grid, -grid]), size=(B, 1, N, d))
    vv[0, 0, 0, :] = 448.0
    q = torch.from_numpy(qv).to(torch.bfloat16)
    k = torch.from_numpy(kv).to(torch.bfloat16)
    v = torch.from_numpy(vv).to(torch.bfloat16)
    assert np.array_equal(v.to(torch.float64).numpy(), vv)
    qb, kb, vb = _bits(q, k, v)
    for causal in (False, True):
        for tile_n in (32, 64):
            o, lse = oracle.sage_rows(qb, kb, vb, causal=causal, scale=math.log(2), tile_n=tile_n)
            oe, lsee, _ = oracle.attn_rows(qb, kb, vb, causal=causal, scale=math.log(2))
            # the scales are fp32 (1/127 is not exact): ~1e-7 relative
            np.testing.assert_allclose(o, oe, rtol=1e-6, atol=1e-6)
            np.testing.assert_allclose(lse, lsee, atol=1e-6)


def _cos_rel(o, ref):
    o, ref = o.ravel(), ref.ravel()
    cos = float(o @ ref / (np.linalg.norm(o) * np.linalg.norm(ref)))
    rel = float(np.abs(o - ref).sum() / np.abs(ref).sum())
    return cos, rel


def test_emulator_error_is_fp8_sized_and_smooth_k_helps(oracle_lib):
    g = torch.Generator().manual_seed(5)
    B, H, N, d = 1, 2, 1024, 64
    q = _rand((B, H, N, d), g)
    bias = torch.randn((d,), generator=g) * 3
    k = (torch.randn((B, H, N, d), generator=g) + bias).to(torch.bfloat16)
    v = _rand((B, H, N, d), g)
    qb, kb, vb = _bits(q, k, v)
    rows = np.arange(0, B * H * N, 7)
    scale = 1 / math.sqrt(d)
    oe, _, _ = oracle.attn_rows(qb, kb, vb, causal=False, scale=scale, rows=rows)
    o, _ = oracle.sage_rows(qb, kb, vb, causal=False, scale=scale, rows=rows)
    cos, rel = _cos_rel(o, oe)
    # E4M3 keeps 3 mantissa bits: relative RMS rounding error ~ 2^-4/sqrt(3) ~ 3.6%
    # per element; P and V errors do not cancel on i.i.d. zero-mean V.
    assert cos > 0.998 and 0.005 < rel < 0.08, (cos, rel)
    o_ns, _ = oracle.sage_rows(qb, kb, vb, causal=False, scale=scale, rows=rows, smooth_k=False)
    cos_ns, rel_ns = _cos_rel(o_ns, oe)
    assert cos_ns < cos and rel_ns > rel, (cos, cos_ns, rel, rel_ns)
    # only INT8 QK (P and V unquantised): far more accurate than the FP8 parts
    o_qk, _ = oracle.sage_rows(qb, kb, vb, causal=False, scale=scale, rows=rows,
                               quant_p=False, quant_v=False)
    cos_qk, rel_qk = _cos_rel(o_qk, oe)
    assert rel_qk < rel and cos_qk > cos


def test_emulator_lse_is_true_lse(oracle_lib):
    """The Smooth-K correction makes the emulator's LSE track the exact LSE."""
    g = torch.Generator().manual_seed(6)
    B, H, N, d = 1, 2, 256, 64
    q = _rand((B, H, N, d), g)
    k = (torch.randn((B, H, N, d), generator=g) + 4.0).to(torch.bfloat16)
    v = _rand((B, H, N, d), g)
    qb, kb, vb = _bits(q, k, v)
    _, lsee, _ = oracle.attn_rows(qb, kb, vb, causal=True, scale=0.125)
    _, lse = oracle.sage_rows(qb, kb, vb, causal=True, scale=0.125)
    assert np.abs(lse - lsee).max() < 0.05
    _, lse_raw = oracle.sage_rows(qb, kb, vb, causal=True, scale=0.125, quant_qk=False,
                                  quant_p=False, quant_v=False)
    np.testing.assert_allclose(lse_raw, lsee, atol=1e-11)


# ---------------------------------------------------- hand-computed running max

def _two_key_case(order):
    """q = (1, 0) for both query rows; K rows (-1/2, 0), (+1/2, 0) in the given
    order (their mean is 0, so Smooth-K leaves them); V rows (1, 2), (-1/2, 1).
    With scale 1 every quantity is exact in INT8 / E4M3: q^ = (127, 0) with
    dQ = 1/127, k^ = (-+127, 0) with dK = (1/2)/127, so the scores are -+1/2;
    V / dV = (448, 448), (-224, 224)."""
    q = torch.tensor([[[[1.0, 0.0], [1.0, 0.0]]]], dtype=torch.bfloat16)
    kr = [[-0.5, 0.0], [0.5, 0.0]]
    k = torch.tensor([[kr if order == "rising" else kr[::-1]]], dtype=torch.bfloat16)
    v = torch.tensor([[[[1.0, 2.0], [-0.5, 1.0]]]], dtype=torch.bfloat16)
    return _bits(q, k, v)


@pytest.mark.parametrize("case", ["rising_tile1", "falling_tile1", "rising_one_tile",
                                  "falling_tile1_lquant"])
def test_emulator_running_max_hand_computed(oracle_lib, case):
    """P^ = E4M3(448 exp(S - m)) against the running max of each key tile,
    fixed by hand on a two-key row (e = exp(-1), the score gap is 1):
    * rising scores, one key per tile: each key is its tile's max when it is
      quantised, so P^ = (448, 448) and, after the rescale by e, the weights
      are (e, 1) -- the exact softmax;
    * falling scores, one key per tile: the second key is quantised against
      the first key's max, 448 e = 164.8 -> P^ = 160 (E4M3 steps by 16 on
      [128, 256)), weights (1, 160/448);
    * rising scores in one tile of two keys: both quantised against the tile
      max, weights (160/448, 1);
    * the row sum l is the unrounded 1 + e in all three, so the LSE is
      1/2 + ln(1 + e); with the quantised-P row sum instead it is
      1/2 + ln(1 + 160/448) and O is normalised by that.
    A P quantised against the final row max, or a running max not rescaling
    the accumulator, gives other weights in at least one case."""
    order = "rising" if case.startswith("rising") else "falling"
    tile_n = 2 if case == "rising_one_tile" else 1
    lq = case.endswith("lquant")
    qb, kb, vb = _two_key_case(order)
    o, lse = oracle.sage_rows(qb, kb, vb, causal=False, scale=1.0, tile_n=tile_n, blk=64,
                              l_from_quantised_p=lq)
    e = math.exp(-1.0)
    v0, v1 = np.array([1.0, 2.0]), np.array([-0.5, 1.0])
    if order == "rising":  # key 0 scores -1/2, key 1 scores +1/2
        w0, w1 = (e, 1.0) if tile_n == 1 else (160 / 448, 1.0)
    else:                  # key 0 scores +1/2, key 1 scores -1/2
        w0, w1 = 1.0, 160 / 448
    l = (w0 + w1) if lq else (1.0 + e)
    o_hand = (w0 * v0 + w1 * v1) / l
    lse_hand = 0.5 + math.log(l)
    for row in range(2):
        np.testing.assert_allclose(o[0, 0, row], o_hand, rtol=1e-6, atol=1e-7)
        assert abs(lse[0, 0, row] - lse_hand) < 1e-6, (lse[0, 0, row], lse_hand)
