"""Pins for the oracle's element formats (e2m1, e4m3, NVFP4 dequant, e4m3 encoder)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from _golden import lines, table


def _e2m1_golden():
    rows = [ln.split() for ln in lines("e2m1_codes.txt")]
    return {int(c): float(v) for c, v in rows}


def _torch_e4m3(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_e2m1_matches_published_table():
    gold = _e2m1_golden()
    got = oracle.e2m1_decode(np.arange(16))
    for c in range(16):
        assert got[c] == gold[c]
        assert np.signbit(got[c]) == np.signbit(gold[c]), c


def test_e4m3_all_256_codes_match_torch():
    codes = np.arange(256)
    ours = oracle.e4m3_decode(codes)
    ref = _torch_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_page_facts():
    facts = {}
    for ln in lines("e4m3_facts.txt"):
        k, *v = ln.split()
        facts[k] = v
    dec = oracle.e4m3_decode
    assert dec(int(facts["max_finite_code"][0], 16)) == float(facts["max_finite"][0])
    finite = dec(np.arange(256))
    assert np.nanmax(finite) == float(facts["max_finite"][0])
    assert dec(int(facts["min_normal_code"][0], 16)) == float(facts["min_normal"][0])
    assert dec(int(facts["min_subnormal_code"][0], 16)) == float(facts["min_subnormal"][0])
    for c in facts["nan_codes"]:
        assert np.isnan(dec(int(c, 16)))
    assert np.isnan(finite).sum() == len(facts["nan_codes"])
    # saturation at +-448 and the page's "about 6 %" rounding bound in the normal range
    assert oracle.e4m3_encode_rne_sat(np.array([1e6, -1e6, 500.0])).tolist() == [0x7E, 0xFE, 0x7E]
    rng = np.random.default_rng(1)
    v = np.exp(rng.uniform(np.log(2.0 ** -6), np.log(448.0), 200000))
    q = dec(oracle.e4m3_encode_rne_sat(v))
    rel = np.abs(q - v) / v
    bound = float(facts["max_rel_rounding_normal"][0])
    assert rel.max() <= bound
    assert rel.max() > 0.9 * bound


def test_nvfp4_hand_worked_bytes():
    for code_hex, scale_hex, s2, vals in table("nvfp4_bytes.txt"):
        codes = np.array([int(b, 16) for b in code_hex.split()], dtype=np.uint8)[None, :]
        scales = np.array([[int(scale_hex, 16)]], dtype=np.uint8)
        got = oracle.dequant_nvfp4(codes, scales, float(s2))[0]
        want = np.array([float(v) for v in vals.split()])
        assert np.array_equal(got, want), (code_hex, scale_hex, got, want)
        assert np.array_equal(np.signbit(got), np.signbit(want))


def test_dequant_is_the_exact_rational_product():
    rng = np.random.default_rng(7)
    N, K = 6, 64
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (N, K // 16), dtype=np.uint8)  # every finite positive code
    s2 = np.float32(0.3)                                          # not a power of two
    got = oracle.dequant_nvfp4(codes, scales, s2)
    e2 = _e2m1_golden()
    sc = _torch_e4m3(scales)
    for n in range(N):
        for k in range(K):
            byte = int(codes[n, k // 2])
            c = byte & 0xF if k % 2 == 0 else byte >> 4
            exact = Fraction(e2[c]) * Fraction(float(sc[n, k // 16])) * Fraction(float(s2))
            assert Fraction(float(got[n, k])) == exact


def _brute_encode(v):
    codes = np.arange(0x7F)
    vals = _torch_e4m3(codes)
    out = []
    for x in v:
        a = min(abs(float(x)), 448.0)
        best = None
        for c, val in zip(codes, vals):
            d = abs(val - a)
            if best is None or d < best[0] or (d == best[0] and (c & 1) == 0 and (best[1] & 1) == 1):
                best = (d, int(c))
        c = best[1]
        if np.signbit(x):
            c |= 0x80
        out.append(c)
    return np.array(out, dtype=np.uint8)


def test_e4m3_encoder_brute_force_including_ties():
    rng = np.random.default_rng(3)
    vals = _torch_e4m3(np.arange(0x7F))
    mids = (vals[1:] + vals[:-1]) / 2            # exact ties between neighbours
    v = np.concatenate([
        rng.normal(0, 50, 3000), rng.uniform(-0.02, 0.02, 1000), mids, -mids,
        [0.0, -0.0, 448.0, 449.0, 463.9, 464.0, 465.0, 1e9, -1e9, 2.0 ** -10, 2.0 ** -11],
    ]).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode_rne_sat(v), _brute_encode(v))


def test_e4m3_encoder_matches_torch_cast_in_range():
    rng = np.random.default_rng(4)
    vals = _torch_e4m3(np.arange(0x7F))
    mids = (vals[1:] + vals[:-1]) / 2
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 0.01, 5000), mids, -mids,
                        [448.0, -448.0, 0.0]]).astype(np.float32)
    t = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode_rne_sat(v), t)


def test_encoder_rejects_nan():
    with pytest.raises(ValueError):
        oracle.e4m3_encode_rne_sat(np.array([np.nan]))
