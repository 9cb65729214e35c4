"""Pins of the oracle's MXFP4 routines and of the MXFP4 quantised-attention
emulator (SageAttention3-style FP4 microscaling on MX block formats).

* E2M1: all 16 codes against the element table of the OCP MX format
  (tests/golden/e2m1_facts.json), the encoder against brute force over that
  table and the printed tie cases.
* The block scale: worked values of the rule "smallest power of two 2^e with
  max|x| <= 6 * 2^e", and torch's float8_e8m0fnu decoding of the scale byte.
* The emulator: with quantisation switched off it equals the exact oracle; on
  inputs whose quantisation is exact it equals the exact oracle; a
  hand-computed case fixes P^ quantised against the running max per tile and
  per 32-key block; on Gaussian inputs its error is FP4-sized.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "e2m1_facts.json")))


def test_e2m1_decode_all_codes(oracle_lib):
    got = oracle.e2m1_decode(np.arange(16))
    want = np.array(FACTS["values_by_code"])
    np.testing.assert_array_equal(got, want)
    assert np.signbit(got[8])  # code 8 is -0


def test_e2m1_encode_printed_ties(oracle_lib):
    for ex in FACTS["round_to_nearest_even_examples"]:
        assert int(oracle.e2m1_encode(ex["x"])) == ex["code"], ex


def test_e2m1_encode_is_nearest(oracle_lib):
    """Brute force over the table: the nearest value (ties to the even code),
    saturating at +-6; representable values encode to themselves."""
    vals = np.array(FACTS["values_by_code"])
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.uniform(-8, 8, 4000), vals, (vals[1:8] + vals[0:7]) / 2])
    for x in xs:
        d = np.abs(vals - x)
        best = [c for c in range(16) if d[c] == d.min()]
        if len(best) > 1:  # a tie (or +-0): prefer the even code of the right sign
            best = [c for c in best if c % 2 == 0 and (c >= 8) == (x < 0)] or best
        assert vals[oracle.e2m1_encode(x)] == vals[best[0]], x


def test_mx_scale_rule(oracle_lib):
    """2^e is the smallest power of two with max|x| <= 6 * 2^e (worked values)."""
    cases = {6.0: 0, 6.0 * (1 + 2 ** -20): 1, 3.0: -1, 3.0000001: 0, 1.0: -2, 0.75: -3,
             1.5: -2, 1.5000001: -1, 48.0: 3, 0.0: 0}
    for amax, e in cases.items():
        assert int(oracle.mx_scale_exp(amax)) == e, (amax, e)


def test_e8m0_scale_byte(oracle_lib):
    """The scale byte 127 + e decodes to 2^e (torch's float8_e8m0fnu)."""
    for ex in FACTS["e8m0_examples"]:
        t = torch.tensor([ex["code"]], dtype=torch.uint8).view(torch.float8_e8m0fnu).float()
        assert float(t[0]) == ex["value"]
    codes = torch.arange(1, 255, dtype=torch.uint8)
    dec = codes.view(torch.float8_e8m0fnu).double().numpy()
    np.testing.assert_array_equal(dec, np.ldexp(1.0, codes.numpy().astype(np.int64) - 127))


def _rand(shape, gen, scale=1.0):
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("causal", [False, True])
def test_emulator_without_quantisation_is_exact(oracle_lib, causal):
    g = torch.Generator().manual_seed(11)
    B, H, Hkv, N, d = 1, 4, 2, 150, 64
    q, k, v = _rand((B, H, N, d), g), _rand((B, Hkv, N, d), g), _rand((B, Hkv, N, d), g)
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    o, lse = oracle.mxfp4_rows(qb, kb, vb, causal=causal, scale=0.125, quant_qk=False,
                               quant_p=False, quant_v=False)
    o_ex, lse_ex, _ = oracle.attn_rows(qb, kb, vb, causal=causal, scale=0.125)
    np.testing.assert_allclose(o, o_ex, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ex, atol=1e-10)


def test_emulator_exact_on_representable_inputs(oracle_lib):
    """Q, K, V of MXFP4-representable values with identical K rows (Smooth-K
    then leaves zeros, every score is equal and every p is 1, which MXFP4
    holds exactly): the emulator's O is the mean of V, as the exact oracle's."""
    g = np.random.default_rng(5)
    vals = np.array(FACTS["values_by_code"][:8])
    B, H, N, d = 1, 2, 96, 64
    q = torch.tensor(g.choice(vals, (B, H, N, d)) * g.choice([-1, 1], (B, H, N, d)),
                     dtype=torch.bfloat16)
    krow = torch.tensor(g.choice(vals, d), dtype=torch.bfloat16)
    k = krow.expand(B, H, N, d).contiguous()
    v = torch.tensor(g.choice(vals, (B, H, N, d)) * 0.5, dtype=torch.bfloat16)
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    for causal in (False, True):
        o, lse = oracle.mxfp4_rows(qb, kb, vb, causal=causal, scale=0.1)
        o_ex, lse_ex, _ = oracle.attn_rows(qb, kb, vb, causal=causal, scale=0.1)
        np.testing.assert_allclose(o, o_ex, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ex, atol=1e-10)


def _two_key_case(order):
    """q = (1, 0, ...) (d = 32); K rows 0 and 32 are (1/2, 0, ...) and (3/2,
    0, ...) in the given order, every other K row (-48, 0, ...); V rows 0 and
    32 are (1, 2, 0, ...) and (-1/2, 1, 0, ...), the others zero.  Every value
    is exact in MXFP4 (Smooth-K off), so with scale 1 the scores are 1/2 and
    3/2 and the others -48 (their p < 1e-20)."""
    N, d = 64, 32
    q = torch.zeros((1, 1, N, d))
    q[..., 0] = 1.0
    k = torch.zeros((1, 1, N, d))
    k[..., 0] = -48.0
    a, b = (0.5, 1.5) if order == "rising" else (1.5, 0.5)
    k[0, 0, 0, 0], k[0, 0, 32, 0] = a, b
    v = torch.zeros((1, 1, N, d))
    v[0, 0, 0, :2] = torch.tensor([1.0, 2.0])
    v[0, 0, 32, :2] = torch.tensor([-0.5, 1.0])
    return [bf16_bits(t.to(torch.bfloat16)) for t in (q, k, v)]


@pytest.mark.parametrize("case", ["rising_two_tiles", "falling_two_tiles", "rising_one_tile"])
def test_emulator_running_max_hand_computed(oracle_lib, case):
    """P^ = MXFP4(exp(S - m_running)) per block of 32 keys, fixed by hand on a
    row whose visible weight sits on keys 0 and 32 (e = exp(-1)):
    * rising scores, 32-key tiles: each key is its tile's max when quantised,
      P^ = (1, 1), after the rescale the weights are (e, 1): exact softmax;
    * falling scores, 32-key tiles: key 32 (p = e) is quantised in its own
      block: scale 2^-4 (e <= 6/16), e / 2^-4 = 5.89 -> 6, P^ = 0.375;
    * rising scores, one 64-key tile: key 0 (p = e) is quantised against the
      tile max, P^ = 0.375, weights (0.375, 1).
    The row sum is the unrounded 1 + e, the LSE 3/2 + ln(1 + e)."""
    qb, kb, vb = _two_key_case("falling" if case.startswith("falling") else "rising")
    tile = 64 if case == "rising_one_tile" else 32
    o, lse = oracle.mxfp4_rows(qb, kb, vb, causal=False, scale=1.0, tile_n=tile,
                               smooth_k=False)
    e = math.exp(-1.0)
    v0, v1 = np.array([1.0, 2.0]), np.array([-0.5, 1.0])
    w = {"rising_two_tiles": (e, 1.0), "falling_two_tiles": (1.0, 0.375),
         "rising_one_tile": (0.375, 1.0)}[case]
    o_hand = (w[0] * v0 + w[1] * v1) / (1 + e)
    for row in range(64):
        np.testing.assert_allclose(o[0, 0, row, :2], o_hand, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(o[0, 0, row, 2:], 0.0, atol=1e-15)
        assert abs(lse[0, 0, row] - (1.5 + math.log(1 + e))) < 1e-12


def test_emulator_error_is_fp4_sized(oracle_lib):
    """On Gaussian inputs the recipe's error against exact attention is that
    of 2-bit-mantissa elements: well below 1 in cos distance but far above
    the FP8 recipe's; each of Q/K, P and V alone costs a part of it."""
    g = torch.Generator().manual_seed(9)
    B, H, N, d = 1, 2, 512, 128
    q, k, v = _rand((B, H, N, d), g), _rand((B, H, N, d), g), _rand((B, H, N, d), g)
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    o_ex, _, _ = oracle.attn_rows(qb, kb, vb, causal=False, scale=d ** -0.5)

    def cos(a):
        a, b = a.ravel(), o_ex.ravel()
        return float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))

    full = cos(oracle.mxfp4_rows(qb, kb, vb, causal=False, scale=d ** -0.5)[0])
    parts = [cos(oracle.mxfp4_rows(qb, kb, vb, causal=False, scale=d ** -0.5,
                                   quant_qk=a, quant_p=b, quant_v=c)[0])
             for a, b, c in ((True, False, False), (False, True, False), (False, False, True))]
    assert 0.95 < full < 0.999, full
    for p in parts:
        assert full < p < 0.9999, (full, parts)
