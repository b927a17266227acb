"""Shared by the GPU tests: the same float32 draws become device tensors (via
the library's own quantiser for the low-precision formats) and oracle values
(via the oracle's codecs).  Nothing computed on the GPU flows to the oracle."""
import numpy as np
import torch

from long_context_compressed_kv_amd import ops
from long_context_compressed_kv_amd.ops import BF16, F32, FP8_MIXED, KV, MXFP4
from oracle import codecs

FMT = {"f32": F32, "bf16": BF16, "fp8_mixed": FP8_MIXED, "mxfp4": MXFP4}


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_kv(a, fmt):
    """float32 draws [rows, dim] -> device KV tensor in `fmt` ('f32', 'bf16',
    'fp8_mixed', 'mxfp4')."""
    a = np.ascontiguousarray(a, dtype=np.float32).reshape(-1, a.shape[-1])
    t = dev_f32(a)
    if fmt == "f32":
        return KV(F32, a.shape[1], t)
    if fmt == "bf16":
        return KV(BF16, a.shape[1], t.to(torch.bfloat16))
    dst = KV.empty(FMT[fmt], a.shape[0], a.shape[1])
    ops.quantize(KV(F32, a.shape[1], t), dst)
    return dst


def ref_vals(a, fmt):
    """float32 draws -> the exact values the oracle sees for the stored format."""
    a = np.asarray(a, dtype=np.float32)
    shp = a.shape
    a2 = a.reshape(-1, shp[-1])
    if fmt == "f32":
        v = a2.astype(np.float64)
    elif fmt == "bf16":
        v = codecs.bf16_round(a2).astype(np.float64)
    elif fmt == "fp8_mixed":
        v = codecs.dequantize_kv_mixed(*codecs.quantize_kv_mixed(a2))
    elif fmt == "mxfp4":
        v = codecs.dequantize_mxfp4(*codecs.quantize_mxfp4(a2))
    else:
        raise ValueError(fmt)
    return v.reshape(shp)


def bf16_ulp(x):
    """Spacing of bf16 values at |x| (fp64)."""
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def to_np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def bits16(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def check_mixed(out, c64, cabs, rel=2.0 ** -20):
    """Mixed-format entries against the oracle's.

    c64  : exact entries; cabs: the same weighted sum of |x| (bounds the fp32
    accumulation error: |c_fp32 - c| <= cabs * rel, 2^-20 for the one-pass
    weighted sum over these window sizes).
    Scale bytes must match unless the block amax sits within that error of a
    power-of-two bound; an e4m3 code may differ by one step, or a bf16 RoPE value
    by one ulp, only where the exact value is within that error of the rounding
    midpoint.  Returns the number of differing codes."""
    err = cabs * rel
    nope_r, scale_r, rope_r = codecs.quantize_kv_mixed(c64.astype(np.float32))
    nope_g = out.data.cpu().numpy()
    scale_g = out.scale.cpu().numpy()
    rope_g = bits16(out.rope)
    gr = codecs.bf16_to_f32(rope_g).astype(np.float64)
    assert np.all(np.abs(gr - c64[:, 448:]) <= 0.5 * bf16_ulp(c64[:, 448:]) * 1.0001 + err[:, 448:])
    bad_scale = scale_g != scale_r
    for r, b in zip(*np.nonzero(bad_scale)):
        lo, hi = b * 128, min(b * 128 + 128, 448)
        amax = np.max(np.abs(c64[r, lo:hi]))
        bound = 448.0 * 2.0 ** np.round(np.log2(amax / 448.0))
        assert abs(amax - bound) <= np.max(err[r, lo:hi])
    diff = nope_g != nope_r
    for r, c in zip(*np.nonzero(diff)):
        b = c // 128
        if bad_scale[r, b]:
            continue
        s = codecs.e8m0_decode(scale_r[r, b])
        a, bb = codecs.e4m3_decode(nope_g[r, c]), codecs.e4m3_decode(nope_r[r, c])
        assert abs(int(nope_g[r, c] & 0x7F) - int(nope_r[r, c] & 0x7F)) == 1
        assert abs(c64[r, c] - (a + bb) / 2 * s) <= err[r, c]
    return int(diff.sum())


def check_attention(out, lse, qv, H, ent_rows, win_rows, tol=2e-2):
    """Attention outputs against the oracle, query by query.

    qv [n_q, H, D]: the oracle's query values; ent_rows[i] / win_rows[i]: the
    oracle's values of query i's compressed keys (selected or visible) and
    window rows.  Outputs and log-sum-exps within tol (bf16 compute)."""
    from oracle import csa as ref
    g, gl = to_np(out).reshape(len(qv), H, -1), to_np(lse).reshape(len(qv), H)
    sc = ref.default_scale(qv.shape[-1])
    err = lerr = 0.0
    for i in range(len(qv)):
        keys = np.concatenate([ent_rows[i], win_rows[i]])
        o, l = ref.attend(qv[i], keys, sc)
        err = max(err, float(np.max(np.abs(g[i] - o))))
        lerr = max(lerr, float(np.max(np.abs(gl[i] - l))))
    assert err <= tol and lerr <= tol, (err, lerr)
    return err, lerr
