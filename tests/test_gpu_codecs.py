"""GPU codec kernels against the oracle codecs: bit-exact."""
import numpy as np
import pytest
import torch

from long_context_compressed_kv_amd import ops
from long_context_compressed_kv_amd.ops import BF16, F32, FP8_MIXED, KV, MXFP4
from oracle import codecs

from gpu_inputs import bits16, dev_f32

pytestmark = pytest.mark.gpu


def _hard_rows(rng, n, d):
    x = rng.standard_normal((n, d)).astype(np.float32)
    x[0] = 0.0                                             # all-zero row
    x[1] *= 1e-30                                          # tiny block values
    x[2] *= 1e20                                           # large
    x[3, :128] = 448.0 * 2.0 ** -3                          # amax exactly on a power boundary
    x[4, :] = np.float32(1.0625)                           # e4m3 midpoints after scaling
    x[5, ::2] *= -1
    x[6, 100] = 3e38                                       # near fp32 max
    return x


def test_kv_mixed_quantize_bitexact():
    rng = np.random.default_rng(11)
    x = _hard_rows(rng, 1031, 512)
    src = KV(F32, 512, dev_f32(x))
    dst = KV.empty(FP8_MIXED, x.shape[0], 512)
    ops.quantize(src, dst)
    nope, scale, rope = codecs.quantize_kv_mixed(x)
    assert np.array_equal(dst.data.cpu().numpy(), nope)
    assert np.array_equal(dst.scale.cpu().numpy(), scale)
    assert np.array_equal(bits16(dst.rope), rope)


def test_kv_mixed_quantize_from_bf16():
    rng = np.random.default_rng(12)
    x = codecs.bf16_round(rng.standard_normal((300, 512)).astype(np.float32))
    src = KV(BF16, 512, dev_f32(x).to(torch.bfloat16))
    dst = KV.empty(FP8_MIXED, 300, 512)
    ops.quantize(src, dst)
    nope, scale, rope = codecs.quantize_kv_mixed(x)
    assert np.array_equal(dst.data.cpu().numpy(), nope)
    assert np.array_equal(dst.scale.cpu().numpy(), scale)
    assert np.array_equal(bits16(dst.rope), rope)


def test_dequantize_every_e4m3_code():
    rng = np.random.default_rng(13)
    n = 64
    nope = np.tile(np.arange(256, dtype=np.uint8), (n, 2))[:, :448].copy()
    nope = np.roll(nope, 7, axis=0)
    scale = rng.integers(100, 160, (n, 4)).astype(np.uint8)
    rope = rng.integers(0, 0x7F7F, (n, 64)).astype(np.uint16)
    t = KV(FP8_MIXED, 512, torch.from_numpy(nope).cuda(), torch.from_numpy(scale).cuda(),
           torch.from_numpy(rope.view(np.int16)).cuda().view(torch.bfloat16))
    got = ops.dequantize(t).cpu().numpy().astype(np.float64)
    want = codecs.dequantize_kv_mixed(nope, scale, rope)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def test_mxfp4_quantize_bitexact():
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((777, 64)) * 0.125).astype(np.float32)
    x[0] = 0
    x[1, :32] = [3.0, 0.3, -1.1, 1.4] + [0.0] * 28
    x[2] *= 1e-35
    x[3, 5] = 1.75
    src = KV(F32, 64, dev_f32(x))
    dst = KV.empty(MXFP4, 777, 64)
    ops.quantize(src, dst)
    codes, scales = codecs.quantize_mxfp4(x)
    assert np.array_equal(dst.data.cpu().numpy(), codes)
    assert np.array_equal(dst.scale.cpu().numpy(), scales)


def test_mxfp4_dequantize_every_code():
    rng = np.random.default_rng(15)
    codes = rng.integers(0, 256, (50, 32)).astype(np.uint8)
    codes[0, :16] = np.arange(16) | (np.arange(16) << 4)
    scales = rng.integers(90, 160, (50, 2)).astype(np.uint8)
    t = KV(MXFP4, 64, torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda())
    got = ops.dequantize(t).cpu().numpy().astype(np.float64)
    assert np.array_equal(got, codecs.dequantize_mxfp4(codes, scales))


def test_mxfp4_to_fp8_exhaustive():
    el = np.tile(np.arange(16, dtype=np.uint8), 4)[None, :]
    packed = (el[:, 0::2] | (el[:, 1::2] << 4)).astype(np.uint8)
    rows_c, rows_s = [], []
    for e_hi in (-100, -20, 0, 30, 100):
        for diff in range(0, 18):
            for order in (0, 1):
                ex = [e_hi, e_hi - diff] if order == 0 else [e_hi - diff, e_hi]
                rows_c.append(packed[0])
                rows_s.append(np.array(ex) + 127)
    codes = np.stack(rows_c).astype(np.uint8)
    scales = np.stack(rows_s).astype(np.uint8)
    t = KV(MXFP4, 64, torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda())
    fp8, g, ok = ops.mxfp4_to_fp8(t)
    r_fp8, r_g, r_ok = codecs.mxfp4_to_fp8(codes, scales)
    assert np.array_equal(fp8.cpu().numpy(), r_fp8)
    assert np.array_equal(g.cpu().numpy(), r_g)
    assert np.array_equal(ok.cpu().numpy().astype(bool), r_ok)


def test_f32_to_bf16_bitexact():
    rng = np.random.default_rng(16)
    x = rng.standard_normal(100003).astype(np.float32)
    u = rng.integers(0, 0x7F7F, 5000, dtype=np.uint32) << 16
    x = np.concatenate([x, (u | 0x8000).view(np.float32)])[None, :]
    src = KV(F32, x.shape[1], dev_f32(x))
    dst = KV(BF16, x.shape[1], torch.empty(1, x.shape[1], dtype=torch.bfloat16, device="cuda"))
    ops.quantize(src, dst)
    assert np.array_equal(bits16(dst.data)[0], codecs.bf16_bits(x[0]))
