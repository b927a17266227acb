"""Pins of the oracle's number-format codecs against the published format
definitions (golden fixtures) and against torch's own casts."""
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# --------------------------------------------------------------------------- bf16

def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        (rng.standard_normal(20000) * 1e-30).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38], np.float32),
    ])
    # exact midpoints between neighbouring bf16 values
    u = rng.integers(0, 0x7F7F, 5000, dtype=np.uint32) << 16   # finite only
    mids = (u | 0x8000).view(np.float32)
    x = np.concatenate([x, mids])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codecs.bf16_bits(x), ref)


def test_bf16_ties_to_even():
    one = np.float32(1.0)
    half_ulp = np.float32(2.0 ** -8)
    assert codecs.bf16_round(one + half_ulp) == 1.0                  # tie -> even (1.0)
    assert codecs.bf16_round(one + 3 * half_ulp) == 1.0 + 2.0 ** -6  # tie -> even


# --------------------------------------------------------------------------- e4m3fn

def test_e4m3_anchors_from_spec():
    for code_hex, val in _read_golden("ocp_e4m3fn_anchors.txt"):
        v = codecs.e4m3_decode(int(code_hex, 16))
        if val == "nan":
            assert np.isnan(v)
        else:
            assert v == float(val) and np.signbit(v) == val.startswith("-")


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = codecs.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(100000) * 40,
        rng.uniform(-448, 448, 100000),
        rng.standard_normal(20000) * 1e-3,
    ]).astype(np.float32)
    finite = codecs.E4M3_VALUES[:0x7F]
    mids = ((finite[1:] + finite[:-1]) / 2).astype(np.float32)     # all ties
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codecs.e4m3_encode(x), ref)


def test_e4m3_saturates():
    out = codecs.e4m3_encode(np.array([448.0, 449.0, 464.0, 500.0, 1e30, -1e30, np.nan]))
    assert list(out[:6]) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert out[6] == 0x7F


def test_e4m3_ties_go_to_even_code():
    # 1.0 (0x38) and 1.125 (0x39): the midpoint goes to the even code 0x38;
    # 1.125 and 1.25 (0x3A): the midpoint goes to 0x3A.
    assert codecs.e4m3_encode(1.0625) == 0x38
    assert codecs.e4m3_encode(1.1875) == 0x3A
    # subnormal grid: midpoint of 2^-9 and 2*2^-9 goes to 2*2^-9 (code 2)
    assert codecs.e4m3_encode(1.5 * 2.0 ** -9) == 0x02
    assert codecs.e4m3_encode(0.5 * 2.0 ** -9) == 0x00


# --------------------------------------------------------------------------- e8m0

def test_e8m0_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = codecs.e8m0_decode(b)
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])


# --------------------------------------------------------------------------- e2m1

def test_e2m1_values_from_spec():
    for code, val in _read_golden("ocp_e2m1_values.txt"):
        c = int(code)
        assert codecs.e2m1_decode(c) == float(val)
        assert codecs.e2m1_decode(c | 8) == -float(val)
        assert codecs.e2m1_encode(float(val)) == c


def test_e2m1_rounding_and_saturation():
    cases = {0.25: 0, 0.74: 1, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6,
             5.0: 6, 5.1: 7, 7.0: 7, 100.0: 7, -0.1: 8, -2.6: 13}
    for v, code in cases.items():
        assert codecs.e2m1_encode(v) == code, v


# --------------------------------------------------------------------------- mixed KV entry

def test_kv_scale_exponent_is_smallest_power():
    rng = np.random.default_rng(3)
    amax = np.abs(rng.standard_normal(20000)) * 10.0 ** rng.uniform(-20, 20, 20000)
    amax = np.concatenate([amax, 448.0 * 2.0 ** np.arange(-30, 30)])   # exact powers
    e = codecs.kv_scale_exponent(amax)
    assert np.all(amax <= 448.0 * np.ldexp(1.0, e))
    assert np.all(amax > 448.0 * np.ldexp(1.0, e - 1))
    assert codecs.kv_scale_exponent(0.0) == -127


def test_kv_mixed_roundtrip_and_bound():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((257, 512)).astype(np.float32)
    x[3, :128] = 0.0                               # an all-zero block
    nope, scale, rope = codecs.quantize_kv_mixed(x)
    assert nope.shape == (257, 448) and scale.shape == (257, 4) and rope.shape == (257, 64)
    assert scale[3, 0] == 0 and np.all(nope[3, :128] == 0)
    y = codecs.dequantize_kv_mixed(nope, scale, rope)
    # rope part: exactly bf16-rounded
    assert np.array_equal(y[:, 448:], codecs.bf16_round(x[:, 448:]).astype(np.float64))
    # non-rope part: e4m3 keeps 3 mantissa bits -> relative error <= 2^-4 for
    # normals, absolute <= half the subnormal step 2^-10 * scale below
    for b in range(4):
        lo, hi = b * 128, min(b * 128 + 128, 448)
        s = codecs.e8m0_decode(scale[:, b])[:, None]
        err = np.abs(y[:, lo:hi] - x[:, lo:hi])
        bound = np.maximum(np.abs(x[:, lo:hi]) * 2.0 ** -4, s * 2.0 ** -10)
        assert np.all(err <= bound)
        assert np.all(np.abs(x[:, lo:hi]) <= 448 * s)
    # values already on the grid survive exactly
    z = codecs.dequantize_kv_mixed(*codecs.quantize_kv_mixed(y.astype(np.float32)))
    assert np.array_equal(z, y)


def test_kv_entry_bytes_golden():
    rows = dict(_read_golden("kv_entry_bytes.txt"))
    assert int(rows["fp8_mixed"]) == codecs.KV_ENTRY_BYTES == 580
    assert int(rows["bf16"]) == 512 * 2
    assert codecs.KV_ENTRY_BYTES / 1024 < 0.6        # "about half"


# --------------------------------------------------------------------------- MXFP4

def test_mxfp4_worked_example():
    # block amax 3.0: floor(log2 3) = 1, X = 2^(1-2) = 0.5; 3.0/X = 6 -> code 7;
    # 0.3/X = 0.6 -> 0.5 (code 1); -1.1/X = -2.2 -> -2 (code 12); 1.4/X = 2.8 -> 3 (code 5)
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [3.0, 0.3, -1.1, 1.4]
    codes, scales = codecs.quantize_mxfp4(x)
    assert scales[0, 0] == 127 - 1
    el = codecs.unpack_e2m1(codes)[0]
    assert list(el[:4]) == [7, 1, 12, 5] and np.all(el[4:] == 0)
    y = codecs.dequantize_mxfp4(codes, scales)[0]
    assert list(y[:4]) == [3.0, 0.25, -1.0, 1.5]


def test_mxfp4_saturates_top_of_binade():
    # amax 1.75: X = 2^-2, 1.75/X = 7 -> saturates to 6 (code 7)
    x = np.zeros((1, 32), np.float32)
    x[0, 5] = 1.75
    codes, scales = codecs.quantize_mxfp4(x)
    assert scales[0, 0] == 125 and codecs.unpack_e2m1(codes)[0, 5] == 7


def test_mxfp4_nibble_order_and_roundtrip():
    rng = np.random.default_rng(5)
    el = rng.integers(0, 16, (64, 64)).astype(np.uint8)
    ex = rng.integers(-10, 10, (64, 2))
    vals = codecs.e2m1_decode(el).reshape(64, 2, 32) * np.ldexp(1.0, ex)[:, :, None]
    vals = vals.reshape(64, 64)
    # force each block's amax to 6*2^e so the spec's scale equals 2^e
    vals[:, 0] = 6.0 * np.ldexp(1.0, ex[:, 0])
    vals[:, 32] = 6.0 * np.ldexp(1.0, ex[:, 1])
    codes, scales = codecs.quantize_mxfp4(vals.astype(np.float32))
    assert np.array_equal(codecs.dequantize_mxfp4(codes, scales), vals)
    assert np.array_equal(scales.astype(np.int64) - 127, ex)
    assert np.all((codes[:, 0] & 0xF) == 7)           # element 0 in the low nibble


# --------------------------------------------------------------------------- FP4 -> FP8

def test_fp4_to_fp8_lossless_exhaustive():
    """All 16 e2m1 codes at every block-exponent offset: lossless iff the
    block exponents differ by at most 14 (scale ratio <= 2^14)."""
    all_codes = np.arange(16, dtype=np.uint8)
    el = np.tile(all_codes, 4)[None, :]             # 64 elements, two blocks of 32
    packed = (el[:, 0::2] | (el[:, 1::2] << 4)).astype(np.uint8)
    for e_hi in (-20, 0, 30):
        for diff in range(0, 18):
            for order in (0, 1):
                ex = [e_hi, e_hi - diff] if order == 0 else [e_hi - diff, e_hi]
                scales = (np.array([ex]) + 127).astype(np.uint8)
                fp8, g, ok = codecs.mxfp4_to_fp8(packed, scales)
                back = codecs.e4m3_decode(fp8) * np.ldexp(1.0, int(g[0]) - 127)
                exact = codecs.dequantize_mxfp4(packed, scales)
                if diff <= 14:
                    assert ok[0]
                    assert np.array_equal(back, exact)
                    assert np.array_equal(np.signbit(back), np.signbit(exact))
                else:
                    assert not ok[0]
                    assert not np.array_equal(back, exact)  # 0.5 * 2^-k is lost
