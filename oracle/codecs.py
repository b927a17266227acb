"""Number-format codecs of the CSA/HCA oracle (test infrastructure only).

TEST INFRASTRUCTURE. Nothing in the product path may import this module; only
the tests, the smoke check and the CPU-baseline leg of the benchmark use it.

Formats, each written from its published definition rather than from any
implementation:

* bfloat16: the upper 16 bits of an IEEE binary32, rounded to nearest-even.
* e4m3fn (OCP 8-bit Floating Point Specification, OFP8, E4M3 encoding):
  bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite
  magnitude 448, smallest subnormal 2^-9.  Conversion here is round to
  nearest-even with saturation to +-448.
* e8m0 (OCP Microscaling Formats (MX) v1.0, scale data type): an unsigned
  biased exponent, value 2^(byte-127), byte 255 is NaN.
* e2m1 (OCP MX v1.0, FP4 element type): bias 1, 1 mantissa bit, magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}; bit 3 is the sign.  Conversion saturates to
  +-6 and rounds to nearest-even.

The two cache layouts of the pages:

* Mixed-precision KV entry (page "DeepSeek V4 深度解析", section 2: the RoPE
  dimensions are kept in BF16 and the rest in FP8, about half the size of pure
  BF16).  Reading used here: a 512-dim entry is [448 non-RoPE | 64 RoPE]; the
  non-RoPE part is e4m3fn in blocks of 128 dims ([0,128), [128,256),
  [256,384), [384,448)), each block with a power-of-two e8m0 scale, the
  smallest 2^e with amax <= 448 * 2^e; the RoPE part is bf16.
* MXFP4 indexer operands (same page, FP4 quantisation-aware training: the
  indexer QK path is FP4 and FP4 -> FP8 is lossless while the in-block
  max/min ratio stays under a threshold).  OCP MX v1.0 block of 32 e2m1
  elements with one e8m0 scale X = 2^(floor(log2 amax) - 2).
"""
import numpy as np

# ----------------------------------------------------------------------------
# bfloat16
# ----------------------------------------------------------------------------


def bf16_bits(x):
    """fp32 values -> bf16 bit patterns (uint16), round to nearest-even.

    NaN maps to the quiet NaN 0x7FC0 (sign kept)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    nan = np.isnan(x)
    r = np.where(nan, ((u >> 16) & 0x8000) | 0x7FC0, r)
    return r.astype(np.uint16)


def bf16_to_f32(bits):
    """bf16 bit patterns -> fp32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def bf16_round(x):
    """Round values (any float dtype, first cast to fp32) to the nearest bf16;
    returns fp32."""
    return bf16_to_f32(bf16_bits(np.asarray(x, dtype=np.float32)))


# ----------------------------------------------------------------------------
# e4m3fn
# ----------------------------------------------------------------------------


def _e4m3_decode_table():
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        mnt = code & 0x7
        if e == 0xF and mnt == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * mnt * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
        else:
            vals[code] = s * (1.0 + mnt / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_decode_table()
E4M3_MAX = 448.0
# codes 0x00..0x7E are the non-negative finite values in increasing order
_E4M3_POS = E4M3_VALUES[:0x7F]


def _nearest_even(mag, grid):
    """Index into the increasing grid of representable magnitudes nearest to
    `mag` (already clipped into [0, grid[-1]]); ties go to the even index,
    which is the code with a zero last mantissa bit."""
    hi = np.searchsorted(grid, mag, side="left")
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    d_lo = mag - grid[lo]
    d_hi = grid[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


def e4m3_encode(x):
    """Values -> e4m3fn codes (uint8): round to nearest-even, saturate to
    +-448, NaN -> 0x7F (sign kept)."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), E4M3_MAX)
    idx = _nearest_even(np.nan_to_num(mag), _E4M3_POS)
    code = idx.astype(np.uint8) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    code = np.where(np.isnan(x), np.where(np.signbit(x), 0xFF, 0x7F), code)
    return code.astype(np.uint8)


def e4m3_decode(codes):
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


# ----------------------------------------------------------------------------
# e8m0
# ----------------------------------------------------------------------------


def e8m0_decode(b):
    b = np.asarray(b, dtype=np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


# ----------------------------------------------------------------------------
# e2m1
# ----------------------------------------------------------------------------

E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_VALUES = np.concatenate([E2M1_POS, -E2M1_POS])   # code 8..15 negative


def e2m1_encode(x):
    """Values -> e2m1 codes (uint8 in 0..15): nearest-even, saturate to +-6,
    sign kept (a negative value that rounds to zero gives -0, code 8)."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), 6.0)
    idx = _nearest_even(mag, E2M1_POS)
    return (idx | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def e2m1_decode(codes):
    return E2M1_VALUES[np.asarray(codes, dtype=np.uint8) & 0xF]


# ----------------------------------------------------------------------------
# Mixed-precision KV entry: [448 e4m3fn with 4 e8m0 block scales | 64 bf16]
# ----------------------------------------------------------------------------

KV_DIM = 512
KV_NOPE = 448
KV_ROPE = 64
KV_BLOCK = 128
KV_NBLK = 4                      # blocks [0,128) [128,256) [256,384) [384,448)
KV_ENTRY_BYTES = KV_NOPE + 2 * KV_ROPE + KV_NBLK


def kv_scale_exponent(amax):
    """Smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127].
    amax == 0 gives -127.  Computed exactly: amax = f * 2^ex with
    f in [0.5, 1) and 448 = 0.875 * 2^9, so e = ex - 9 + (f > 0.875)."""
    amax = np.asarray(amax, dtype=np.float64)
    f, ex = np.frexp(amax)
    e = ex - 9 + (f > 0.875)
    e = np.where(amax == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_kv_mixed(rows):
    """rows [N, 512] (fp32 values) -> (nope uint8 [N,448], scale uint8 [N,4],
    rope uint16 [N,64])."""
    rows = np.asarray(rows, dtype=np.float32)
    assert rows.ndim == 2 and rows.shape[1] == KV_DIM
    n = rows.shape[0]
    nope = np.empty((n, KV_NOPE), dtype=np.uint8)
    scale = np.empty((n, KV_NBLK), dtype=np.uint8)
    for b in range(KV_NBLK):
        lo, hi = b * KV_BLOCK, min((b + 1) * KV_BLOCK, KV_NOPE)
        blk = rows[:, lo:hi].astype(np.float64)
        e = kv_scale_exponent(np.max(np.abs(blk), axis=1))
        scale[:, b] = (e + 127).astype(np.uint8)
        nope[:, lo:hi] = e4m3_encode(np.ldexp(blk, -e[:, None]))
    rope = bf16_bits(rows[:, KV_NOPE:])
    return nope, scale, rope


def dequantize_kv_mixed(nope, scale, rope):
    """Inverse view of `quantize_kv_mixed`: fp64 [N, 512] (exact)."""
    nope = np.asarray(nope, dtype=np.uint8)
    n = nope.shape[0]
    out = np.empty((n, KV_DIM), dtype=np.float64)
    for b in range(KV_NBLK):
        lo, hi = b * KV_BLOCK, min((b + 1) * KV_BLOCK, KV_NOPE)
        out[:, lo:hi] = e4m3_decode(nope[:, lo:hi]) * e8m0_decode(scale[:, b])[:, None]
    out[:, KV_NOPE:] = bf16_to_f32(rope).astype(np.float64)
    return out


# ----------------------------------------------------------------------------
# MXFP4 (OCP MX v1.0): blocks of 32 e2m1 elements, one e8m0 scale per block
# ----------------------------------------------------------------------------

MX_BLOCK = 32
E2M1_EMAX = 2          # exponent of the largest e2m1 normal, 6 = 1.5 * 2^2


def mx_block_exponent(amax):
    """Shared exponent of an MX block: floor(log2(amax)) - emax_elem, clamped
    to [-127, 127]; amax == 0 gives -127."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)                    # amax = f * 2^ex, f in [0.5,1)
    e = (ex - 1) - E2M1_EMAX
    e = np.where(amax == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_mxfp4(x):
    """x [N, d] (fp32 values, d % 32 == 0) -> (codes uint8 [N, d/2],
    scales uint8 [N, d/32]).  Element 2i sits in the low nibble of byte i."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    n, d = x.shape
    assert d % MX_BLOCK == 0
    blocks = x.reshape(n, d // MX_BLOCK, MX_BLOCK)
    e = mx_block_exponent(np.max(np.abs(blocks), axis=2))
    q = e2m1_encode(np.ldexp(blocks, -e[:, :, None])).reshape(n, d)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return codes, (e + 127).astype(np.uint8)


def unpack_e2m1(codes):
    """uint8 [N, d/2] -> element codes uint8 [N, d]."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def dequantize_mxfp4(codes, scales):
    """-> fp64 [N, d] (exact)."""
    el = e2m1_decode(unpack_e2m1(codes))
    n, d = el.shape
    s = e8m0_decode(scales).reshape(n, d // MX_BLOCK, 1)
    return (el.reshape(n, d // MX_BLOCK, MX_BLOCK) * s).reshape(n, d)


def mxfp4_to_fp8(codes, scales):
    """Regroup MXFP4 rows into e4m3fn with one power-of-two scale per row.

    The row's group exponent is g = max_b(e_b) - 6, where e_b are the block
    exponents of its MX blocks.  Each element c * 2^e_b becomes the e4m3fn
    code of c * 2^(e_b - g).  e4m3fn holds every e2m1 magnitude times 2^k
    exactly iff k is in [-8, 6] (6 * 2^6 = 384 <= 448; 0.5 * 2^-8 = 2^-9 is the
    smallest subnormal), so the row is lossless iff max_b e_b - min_b e_b <= 14
    (a block-scale ratio of at most 2^14).  Rows outside the bound are still
    converted (rounded) and flagged.

    Returns (fp8 codes uint8 [N, d], group scale byte uint8 [N],
    lossless bool [N])."""
    el = unpack_e2m1(codes)
    n, d = el.shape
    e = np.asarray(scales, dtype=np.int64) - 127          # [N, nb]
    g = np.max(e, axis=1) - 6
    k = e - g[:, None]                                     # [N, nb] <= 6
    lossless = np.min(k, axis=1) >= -8
    vals = e2m1_decode(el).reshape(n, d // MX_BLOCK, MX_BLOCK)
    fp8 = e4m3_encode(np.ldexp(vals, k[:, :, None])).reshape(n, d)
    gbyte = np.clip(g + 127, 0, 254).astype(np.uint8)
    return fp8, gbyte, lossless
