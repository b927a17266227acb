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
