"""Pins of the oracle's MXFP6 routines (the MX FP6 element format E2M3) and of
the element-format parameter of the MX quantised-attention emulator.

* E2M3: all 64 codes against the element table of the OCP MX format
  (tests/golden/e2m3_facts.json), that table against the format's spacing
  rule and against torch's E4M3 (every E2M3 value is an E4M3 value), the
  encoder against brute force over the table and the listed tie cases.
* The block scale for a format of largest magnitude 7.5: worked values of
  "smallest power of two 2^e with max|x| <= 7.5 * 2^e"; with 6 the general
  rule is the MXFP4 one.
* The emulator with E2M3 elements: without quantisation it is exact; on
  inputs whose quantisation is exact it equals the exact oracle; a
  hand-computed row fixes P^ per 32-key block against the running max in
  both element formats (the E2M3 and E2M1 roundings of the same p differ);
  on Gaussian inputs its error is FP6-sized: several times below FP4's.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "e2m3_facts.json")))
VALS = np.array(FACTS["values_by_code"])


def test_table_follows_the_spacing_rule():
    """The positive E2M3 magnitudes are the multiples of 1/8 in [0, 2), of 1/4
    in [2, 4) and of 1/2 in [4, 7.5], in increasing code order; the negative
    codes mirror them (code 32 is -0)."""
    want = np.concatenate([np.arange(16) / 8, 2 + np.arange(8) / 4, 4 + np.arange(8) / 2])
    np.testing.assert_array_equal(VALS[:32], want)
    np.testing.assert_array_equal(VALS[32:], -want)
    for sv in FACTS["special_values"]:
        assert VALS[sv["code"]] == sv["value"], sv


def test_table_values_are_e4m3_values():
    """E2M3 has fewer exponent and mantissa bits than E4M3 and lies inside its
    range, so torch's E4M3 cast holds every E2M3 value exactly."""
    t = torch.tensor(VALS, dtype=torch.float64)
    back = t.to(torch.float8_e4m3fn).double()
    np.testing.assert_array_equal(back.numpy(), VALS)


def test_e2m3_decode_all_codes(oracle_lib):
    got = oracle.e2m3_decode(np.arange(64))
    np.testing.assert_array_equal(got, VALS)
    assert np.signbit(got[32])  # code 32 is -0


def test_e2m3_encode_listed_ties(oracle_lib):
    for ex in FACTS["round_to_nearest_even_examples"]:
        assert int(oracle.e2m3_encode(ex["x"])) == ex["code"], ex


def test_e2m3_encode_is_nearest(oracle_lib):
    """Brute force over the table: the nearest value (ties to the even code),
    saturating at +-7.5; representable values encode to themselves."""
    rng = np.random.default_rng(4)
    xs = np.concatenate([rng.uniform(-9, 9, 4000), VALS, (VALS[1:32] + VALS[0:31]) / 2,
                         -(VALS[1:32] + VALS[0:31]) / 2])
    for x in xs:
        d = np.abs(VALS - x)
        best = [c for c in range(64) if d[c] == d.min()]
        if len(best) > 1:  # a tie (or +-0): prefer the even code of the right sign
            best = [c for c in best if c % 2 == 0 and (c >= 32) == (x < 0)] or best
        assert VALS[oracle.e2m3_encode(x)] == VALS[best[0]], x
    codes = oracle.e2m3_encode(VALS[:32])
    np.testing.assert_array_equal(codes, np.arange(32))


def test_mx_scale_rule_fp6(oracle_lib):
    """2^e is the smallest power of two with max|x| <= 7.5 * 2^e (worked
    values: 7.5 * 2^-2 = 1.875, 7.5 * 2^3 = 60)."""
    cases = {7.5: 0, 7.5 * (1 + 2 ** -20): 1, 3.75: -1, 3.7500001: 0, 1.0: -2, 1.875: -2,
             1.8750001: -1, 0.9375: -3, 60.0: 3, 0.0: 0, 2.0 ** -130: -127}
    for amax, e in cases.items():
        assert int(oracle.mx_scale_exp_max(amax, 7.5)) == e, (amax, e)


def test_mx_scale_rule_general_matches_fp4(oracle_lib):
    rng = np.random.default_rng(6)
    a = np.concatenate([np.ldexp(rng.uniform(0.5, 1.0, 300), rng.integers(-20, 20, 300)),
                        [6.0, 3.0, 1.5, 0.0]])
    np.testing.assert_array_equal(oracle.mx_scale_exp_max(a, 6.0), oracle.mx_scale_exp(a))


def _rand(shape, gen, scale=1.0):
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("causal", [False, True])
def test_emulator_without_quantisation_is_exact(oracle_lib, causal):
    g = torch.Generator().manual_seed(12)
    B, H, Hkv, N, d = 1, 4, 2, 150, 64
    q, k, v = _rand((B, H, N, d), g), _rand((B, Hkv, N, d), g), _rand((B, Hkv, N, d), g)
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    o, lse = oracle.mxfp6_rows(qb, kb, vb, causal=causal, scale=0.125, quant_qk=False,
                               quant_p=False, quant_v=False)
    o_ex, lse_ex, _ = oracle.attn_rows(qb, kb, vb, causal=causal, scale=0.125)
    np.testing.assert_allclose(o, o_ex, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ex, atol=1e-10)


def test_emulator_exact_on_representable_inputs(oracle_lib):
    """Q, K, V of E2M3 values with identical K rows (Smooth-K then leaves
    zeros, every score is equal and every p is 1): a block scaled up by a
    power of two stays on the E2M3 grid (its spacing grows with the
    magnitude), so the emulator's O is the mean of V, as the exact oracle's."""
    g = np.random.default_rng(7)
    vals = VALS[:32]
    B, H, N, d = 1, 2, 96, 64
    q = torch.tensor(g.choice(vals, (B, H, N, d)) * g.choice([-1, 1], (B, H, N, d)),
                     dtype=torch.bfloat16)
    krow = torch.tensor(g.choice(vals, d), dtype=torch.bfloat16)
    k = krow.expand(B, H, N, d).contiguous()
    v = torch.tensor(g.choice(vals, (B, H, N, d)) * 0.5, dtype=torch.bfloat16)
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    for causal in (False, True):
        o, lse = oracle.mxfp6_rows(qb, kb, vb, causal=causal, scale=0.1)
        o_ex, lse_ex, _ = oracle.attn_rows(qb, kb, vb, causal=causal, scale=0.1)
        np.testing.assert_allclose(o, o_ex, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ex, atol=1e-10)


def _two_key_case(order):
    """q = (1, 0, ...) (d = 32); K rows 0 and 32 are (1, 0, ...) and (3/2, 0,
    ...) in the given order, every other K row (-48, 0, ...); V rows 0 and 32
    are (1, 2, 0, ...) and (-1/2, 1, 0, ...), the others zero.  Every value
    is exact in E2M1 and in E2M3 (Smooth-K off), so with scale 1 the scores
    are 1 and 3/2 and the others -48 (their p < 1e-20)."""
    N, d = 64, 32
    q = torch.zeros((1, 1, N, d))
    q[..., 0] = 1.0
    k = torch.zeros((1, 1, N, d))
    k[..., 0] = -48.0
    a, b = (1.0, 1.5) if order == "rising" else (1.5, 1.0)
    k[0, 0, 0, 0], k[0, 0, 32, 0] = a, b
    v = torch.zeros((1, 1, N, d))
    v[0, 0, 0, :2] = torch.tensor([1.0, 2.0])
    v[0, 0, 32, :2] = torch.tensor([-0.5, 1.0])
    return [bf16_bits(t.to(torch.bfloat16)) for t in (q, k, v)]


@pytest.mark.parametrize("elem", ["e2m1", "e2m3"])
@pytest.mark.parametrize("case", ["rising_two_tiles", "falling_two_tiles", "rising_one_tile"])
def test_emulator_running_max_hand_computed(oracle_lib, case, elem):
    """P^ = MX(exp(S - m_running)) per block of 32 keys, fixed by hand on a row
    whose visible weight sits on keys 0 and 32 (r = exp(-1/2) = 0.6065):
    * rising scores, 32-key tiles: each key is its tile's max when quantised,
      P^ = (1, 1); after the rescale the weights are (r, 1): exact softmax;
    * falling scores, 32-key tiles: key 32 (p = r) is quantised in its own
      block with scale 2^-3 (r <= 0.75 = 6/8 and r <= 0.9375 = 7.5/8, but
      above 6/16 and 7.5/16); r / 2^-3 = 4.85 rounds to 4 in E2M1 (codes 4,
      6) and to 5 in E2M3 (codes 4.5, 5): P^ = 0.5 or 0.625;
    * rising scores, one 64-key tile: key 0 (p = r) is quantised against the
      tile max the same way.
    The row sum is the unrounded 1 + r, the LSE 3/2 + ln(1 + r)."""
    qb, kb, vb = _two_key_case("falling" if case.startswith("falling") else "rising")
    tile = 64 if case == "rising_one_tile" else 32
    o, lse = oracle.mx_rows(qb, kb, vb, causal=False, scale=1.0, tile_n=tile, smooth_k=False,
                            elem=elem)
    r = math.exp(-0.5)
    ph = {"e2m1": 0.5, "e2m3": 0.625}[elem]
    v0, v1 = np.array([1.0, 2.0]), np.array([-0.5, 1.0])
    w = {"rising_two_tiles": (r, 1.0), "falling_two_tiles": (1.0, ph),
         "rising_one_tile": (ph, 1.0)}[case]
    o_hand = (w[0] * v0 + w[1] * v1) / (1 + r)
    for row in range(64):
        np.testing.assert_allclose(o[0, 0, row, :2], o_hand, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(o[0, 0, row, 2:], 0.0, atol=1e-15)
        assert abs(lse[0, 0, row] - (1.5 + math.log(1 + r))) < 1e-12


def test_emulator_error_is_fp6_sized(oracle_lib):
    """On Gaussian inputs (K with a per-channel bias, as the workloads have)
    the E2M3 recipe's error against exact attention is that of 4-bit
    significands: its rel-L1 several times below the E2M1 recipe's, and each
    of Q/K, P and V alone costs a part of it."""
    g = torch.Generator().manual_seed(10)
    B, H, N, d = 1, 2, 512, 128
    q, v = _rand((B, H, N, d), g), _rand((B, H, N, d), g)
    k = (torch.randn((B, H, N, d), generator=g) +
         3 * torch.randn((B, H, 1, d), generator=g)).to(torch.bfloat16)
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    o_ex, _, _ = oracle.attn_rows(qb, kb, vb, causal=False, scale=d ** -0.5)

    def rel(a):
        return float(np.abs(a - o_ex).sum() / np.abs(o_ex).sum())

    fp6 = rel(oracle.mxfp6_rows(qb, kb, vb, causal=False, scale=d ** -0.5)[0])
    fp4 = rel(oracle.mxfp4_rows(qb, kb, vb, causal=False, scale=d ** -0.5)[0])
    parts = [rel(oracle.mxfp6_rows(qb, kb, vb, causal=False, scale=d ** -0.5,
                                   quant_qk=a, quant_p=b, quant_v=c)[0])
             for a, b, c in ((True, False, False), (False, True, False), (False, False, True))]
    print("rel-L1 fp6 %.4f fp4 %.4f parts %s" % (fp6, fp4, parts))
    assert 0.01 < fp6 < 0.1 and fp4 > 3 * fp6, (fp6, fp4)
    for p in parts:
        assert 1e-3 < p < fp6, (fp6, parts)
