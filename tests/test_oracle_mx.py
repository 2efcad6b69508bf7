"""Pins of the oracle's number formats: bf16 rounding, E4M3 coding and the MX
block quantizer.  References: the OCP OFP8 / MX v1.0 values stored in
tests/golden/e4m3_reference_values.json, torch's own bfloat16 and
float8_e4m3fn casts (an independent library), and a brute-force nearest-code
search over all 256 E4M3 codes for every bf16 bit pattern."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_decode_matches_spec_values():
    g = json.load(open(os.path.join(GOLD, "e4m3_reference_values.json")))
    for code, val in g["e4m3"].items():
        d = O.e4m3_decode(np.array([int(code, 16)], np.uint8))[0]
        assert d == val and math.copysign(1, d) == math.copysign(1, val), code
    for code in g["e4m3_nan_codes"]:
        assert np.isnan(O.e4m3_decode(np.array([int(code, 16)], np.uint8))[0])
    assert O.E4M3_MAX == g["e4m3_max_normal"] and O.E4M3_EMAX_ELEM == g["e4m3_emax"]


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(theirs)
    np.testing.assert_array_equal(ours[~both_nan], theirs[~both_nan])
    assert (np.isnan(ours) == np.isnan(theirs)).all()


def test_e4m3_encode_roundtrips_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    np.testing.assert_array_equal(O.e4m3_encode(O.e4m3_decode(codes)), codes)


def test_e4m3_round_matches_torch_cast_in_range():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(200000) * 50, rng.standard_normal(50000) * 0.01,
                        np.linspace(-448, 448, 100001)]).astype(np.float32)
    ours = O.e4m3_round(v.astype(np.float64))
    theirs = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, theirs)


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(300000), rng.standard_normal(1000) * 1e-39,
                        rng.standard_normal(1000) * 1e30]).astype(np.float32)
    ours = O.bf16_round(v.astype(np.float64))
    theirs = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, theirs)
    np.testing.assert_array_equal(O.bits_to_bf16(O.bf16_to_bits(ours)), ours)


def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = O.bits_to_bf16(bits)
    return vals[np.isfinite(vals)]


def _nearest_code(q):
    """Brute force: nearest finite E4M3 value to q (ties -> even code), with
    values above 448 in magnitude going to +-448."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = O.e4m3_decode(codes)
    d = np.abs(vals[None, :] - q[:, None])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # prefer the candidate whose sign matches q (only differs for 0 / -0), then even code
    sign_ok = np.signbit(vals)[None, :] == np.signbit(q)[:, None]
    even = (codes % 2 == 0)[None, :]
    score = cand * (4 + 2 * sign_ok + even)
    return codes[np.argmax(score, axis=1)]


def test_mx_block_max_exhaustive_over_bf16():
    """Every finite bf16 value as the maximum of a block: the scale byte is
    floor(log2|v|) - 8 + 127 clamped to [0, 254], and its code is the nearest
    E4M3 value to v / 2^E (brute force over all codes)."""
    vals = _all_finite_bf16()
    vals = vals[vals != 0]
    blocks = np.zeros((vals.size, 32))
    blocks[:, 5] = vals
    blocks[:, 6] = vals * 0.0
    codes, scales = O.mx_quantize_rows(blocks)
    for v, s in zip(vals[::97], scales[::97, 0]):
        E = max(min(math.frexp(abs(v))[1] - 1 - 8, 127), -127)
        assert s == E + 127
    E = scales[:, 0].astype(np.int64) - 127
    q = vals * np.ldexp(1.0, -E)
    np.testing.assert_array_equal(codes[:, 5], _nearest_code(q))


def test_mx_random_blocks_against_bruteforce():
    rng = np.random.default_rng(2)
    raw = rng.standard_normal((4000, 64)) * np.exp(rng.uniform(-30, 30, size=(4000, 1)))
    v = O.bf16_round(raw)
    codes, scales = O.mx_quantize_rows(v)
    E = scales.astype(np.int64) - 127
    q = v.reshape(4000, 2, 32) * np.ldexp(1.0, -E)[:, :, None]
    np.testing.assert_array_equal(codes.ravel(), _nearest_code(q.ravel()))
    # dequantization error: half an E4M3 step (relative 2^-4, or 2^-10 of the
    # scale in the subnormal range) plus what saturation at 448 * 2^E removes
    dq = O.mx_dequantize_rows(codes, scales)
    sc = np.ldexp(1.0, E).repeat(32, axis=1)
    bound = np.abs(v) * 2 ** -4 + sc * 2 ** -10 + np.maximum(0.0, np.abs(v) - 448 * sc)
    assert (np.abs(dq - v) <= bound).all()


def test_mx_special_blocks():
    ones = np.ones((1, 32))
    c, s = O.mx_quantize_rows(ones)
    assert s.tolist() == [[119]] and (c == 0x78).all()
    c, s = O.mx_quantize_rows(np.zeros((1, 32)))
    assert s.tolist() == [[0]] and (c == 0).all()
    neg0 = -np.zeros((1, 32))
    c, _ = O.mx_quantize_rows(neg0)
    assert (c == 0x80).all()
    for k in (-20, 0, 7):
        blk = np.zeros((1, 32))
        blk[0, 0] = O.bf16_round(1.9 * 2.0 ** k)
        blk[0, 1] = -blk[0, 0]
        c, s = O.mx_quantize_rows(blk)
        assert c[0, 0] == 0x7E and c[0, 1] == 0xFE and s[0, 0] == k - 8 + 127
    # values already on the E4M3 grid at the block scale come back exactly
    grid = O.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    blk = np.zeros((4, 32))
    blk.ravel()[: grid.size] = grid
    blk[:, 0] = 448.0
    c, s = O.mx_quantize_rows(blk)
    np.testing.assert_array_equal(O.mx_dequantize_rows(c, s), blk)


def test_mx_row_length_must_be_block_multiple():
    with pytest.raises(ValueError):
        O.mx_quantize_rows(np.zeros((2, 33)))
