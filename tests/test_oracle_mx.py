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


# ---------------------------------------------------------------------------
# MXFP4: E2M1 elements (OCP MX v1.0 FP4), same E8M0 block scale
# ---------------------------------------------------------------------------

def test_e2m1_decode_matches_spec_values():
    g = json.load(open(os.path.join(GOLD, "e2m1_reference_values.json")))
    for code, val in g["e2m1"].items():
        d = O.e2m1_decode(np.array([int(code, 16)], np.uint8))[0]
        assert d == val and math.copysign(1, d) == math.copysign(1, val), code
    assert O.E2M1_MAX == g["e2m1_max_normal"] and O.E2M1_EMAX_ELEM == g["e2m1_emax"]


def test_e2m1_encode_roundtrips_every_code():
    codes = np.arange(16, dtype=np.uint8)
    np.testing.assert_array_equal(O.e2m1_encode(O.e2m1_decode(codes)), codes)


def _nearest_e2m1(q):
    """Brute force: nearest E2M1 value to q over all 16 codes (ties -> even
    code, the sign of q kept for zeros), magnitudes above 6 going to +-6."""
    codes = np.arange(16, dtype=np.uint8)
    vals = O.e2m1_decode(codes)
    d = np.abs(vals[None, :] - np.clip(q, -6.0, 6.0)[:, None])
    cand = d == d.min(axis=1, keepdims=True)
    sign_ok = np.signbit(vals)[None, :] == np.signbit(q)[:, None]
    even = (codes % 2 == 0)[None, :]
    return codes[np.argmax(cand * (4 + 2 * sign_ok + even), axis=1)]


def test_e2m1_round_against_bruteforce():
    # every midpoint and grid value, dense values around them, beyond +-6
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    grid = O.e2m1_decode(np.arange(8, dtype=np.uint8))
    q = np.concatenate([mids, grid, np.linspace(0, 9, 90001), mids + 1e-9, mids - 1e-9,
                        [7.0, 100.0, 1e30]])
    q = np.concatenate([q, -q])
    np.testing.assert_array_equal(O.e2m1_encode(O.e2m1_round(q)), _nearest_e2m1(q))
    # the ties go to the even code: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2,
    # 2.5 -> 2, 3.5 -> 4, 5 -> 4
    np.testing.assert_array_equal(O.e2m1_round(mids), [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0])


def test_mx4_random_blocks_against_bruteforce():
    rng = np.random.default_rng(12)
    raw = rng.standard_normal((3000, 64)) * np.exp(rng.uniform(-30, 30, size=(3000, 1)))
    v = O.bf16_round(raw)
    codes, scales = O.mx4_quantize_rows(v)
    for row, blk in ((0, 0), (17, 1), (2999, 1)):
        amax = max(abs(float(t)) for t in v[row, 32 * blk:32 * blk + 32])
        assert scales[row, blk] == math.frexp(amax)[1] - 1 - 2 + 127
    E = scales.astype(np.int64) - 127
    q = v.reshape(3000, 2, 32) * np.ldexp(1.0, -E)[:, :, None]
    np.testing.assert_array_equal(codes.ravel(), _nearest_e2m1(q.ravel()))
    # every block's largest magnitude maps to 4 or 6 (amax / 2^E lies in [4, 8))
    mags = O.e2m1_decode(codes & 7).reshape(3000, 2, 32).max(axis=2)
    assert np.isin(mags, [4.0, 6.0]).all()
    # dequantization error: half a step (0.25 * 2^E below 2, 1 * 2^E at 4..6)
    # plus what saturation at 6 * 2^E removes
    dq = O.mx4_dequantize_rows(codes, scales)
    sc = np.ldexp(1.0, E).repeat(32, axis=1)
    bound = np.maximum(0.25 * sc, np.abs(v) / 4) + np.maximum(0.0, np.abs(v) - 6 * sc)
    assert (np.abs(dq - v) <= bound).all()


def test_mx4_special_blocks_and_packing():
    c, s = O.mx4_quantize_rows(np.ones((1, 32)))      # 1 = 1.0 * 2^-2 * 4: code 4 -> 4.0 at 2^-2
    assert s.tolist() == [[125]] and (c == 0x6).all()
    c, s = O.mx4_quantize_rows(np.zeros((1, 32)))
    assert s.tolist() == [[0]] and (c == 0).all()
    c, _ = O.mx4_quantize_rows(-np.zeros((1, 32)))
    assert (c == 0x8).all()
    blk = np.zeros((1, 32))
    blk[0, :4] = [7.5, -7.5, 5.0, 0.2]                  # E = 0: 7.5 saturates to 6, 5 ties to 4
    c, s = O.mx4_quantize_rows(blk)
    assert s[0, 0] == 127 and c[0, :4].tolist() == [0x7, 0xF, 0x6, 0x0]
    # values on the E2M1 grid at their block scale come back exactly
    grid = O.e2m1_decode(np.arange(16, dtype=np.uint8))
    blk = np.tile(grid, (3, 2)) * np.array([[2.0 ** -9], [1.0], [2.0 ** 20]])
    c, s = O.mx4_quantize_rows(blk)
    np.testing.assert_array_equal(O.mx4_dequantize_rows(c, s), blk)
    # packing: element 2i in the low nibble
    p = O.pack_fp4(np.array([[1, 2, 0xF, 0x3]], np.uint8))
    assert p.tolist() == [[0x21, 0x3F]]
    np.testing.assert_array_equal(O.unpack_fp4(p), [[1, 2, 0xF, 0x3]])


def test_columns_grouped_blocks_stay_inside_groups():
    """Column-wise, group-aware MX blocks: each group blocked on its own (zero
    rows pad it to a multiple of 128), a block's scale follows its own 32
    values only, and the blocks dequantize back to the group's rows."""
    rng = np.random.default_rng(5)
    counts = [40, 0, 130, 1]
    off = np.concatenate([[0], np.cumsum(counts)])
    C = 64
    v = O.bf16_round(rng.standard_normal((off[-1], C)) * np.exp(rng.uniform(-8, 8, (off[-1], 1))))
    pb, codes, scales = O.mx_quantize_columns_grouped(v, off)
    assert list(pb) == [0, 4, 4, 12, 16]
    for e, m in enumerate(counts):
        for j in range(pb[e + 1] - pb[e]):
            rows = v[off[e] + 32 * j: off[e] + min(m, 32 * j + 32)]
            blk = np.zeros((32, C))
            blk[:len(rows)] = rows
            for c in range(C):
                # the row quantizer on the block's column alone (a group's
                # neighbour never enters its scale)
                cc, ss = O.mx_quantize_rows(blk[:, c][None, :])
                assert (codes[pb[e] + j, c] == cc[0]).all() and scales[pb[e] + j, c] == ss[0, 0]
            deq = O.mx_dequantize_rows(codes[pb[e] + j].reshape(C, 32), scales[pb[e] + j][:, None]).T
            assert (deq[len(rows):] == 0).all()   # padding rows of the group stay zero
    # a zero padding block: scale byte 0, codes 0
    assert (scales[15] == 0).all() and (codes[15] == 0).all()
