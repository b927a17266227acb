"""The C ABI library loads, exports every call declared in include/csa.h, and
rejects bad arguments on the host before launching anything (no GPU needed:
validation fails before any HIP call)."""
import ctypes
import os
import re

import pytest

from long_context_compressed_kv_amd import _lib
from long_context_compressed_kv_amd._lib import CsaBatch, CsaTensor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

BAD_ARG, UNSUPPORTED = 1, 2
FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails first


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:csa_status|int|size_t|const char\*)\s+(csa_\w+)\s*\(",
                                 text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_calls():
    names = declared_symbols()
    for n in ("csa_kv_compress", "csa_indexer_score", "csa_topk_select",
              "csa_sparse_mqa_attn", "csa_swa_merge"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert set(declared_symbols()) == set(_lib.EXPORTED)


def test_version_and_strings(lib):
    assert lib.csa_abi_version() == 5
    assert lib.csa_status_string(0) == b"ok"
    assert lib.csa_status_string(3) == b"workspace too small"


def _t(fmt, dim, rows, data=FAKE, scale=None, rope=None):
    return CsaTensor(fmt, dim, rows, data, scale, rope)


def test_kv_compress_validation(lib):
    x = _t(0, 128, 64)
    out = _t(0, 128, 16)
    z = b = FAKE
    call = lambda xx, oo, m, w, e0, n, pos0=0: lib.csa_kv_compress(
        ctypes.byref(xx), z, pos0, b, m, w, e0, n, ctypes.byref(oo), None)
    assert call(x, out, 4, 2, 0, 4) == BAD_ARG              # w < m
    assert call(x, out, 4, 2000, 0, 4) == BAD_ARG           # w too large
    assert call(x, out, 4, 8, 0, 17) == BAD_ARG             # more entries than output rows
    assert call(x, out, 4, 8, 0, 16, pos0=1) == BAD_ARG     # raw rows miss position 0
    assert call(x, out, 4, 8, 0, 17) == BAD_ARG
    assert call(_t(0, 128, 64), _t(1, 64, 16), 4, 8, 0, 4) == BAD_ARG   # dim mismatch
    assert call(_t(2, 512, 64), _t(0, 512, 16), 4, 8, 0, 4) == BAD_ARG  # mixed without scales
    assert call(_t(2, 512, 64, scale=FAKE, rope=FAKE), _t(0, 512, 16), 4, 8, 0, 4) == UNSUPPORTED
    assert call(_t(0, 96, 64), _t(0, 96, 16), 4, 8, 0, 4) == UNSUPPORTED  # not a power of two
    assert call(x, out, 4, 8, 0, 0) == 0                    # nothing to do, nothing launched
    assert b"raw rows" in lib.csa_last_error() or lib.csa_last_error() == b""
    # the per-channel variant makes the same checks
    chan = lambda xx, oo, m, w, e0, n, pos0=0: lib.csa_kv_compress_channel(
        ctypes.byref(xx), z, pos0, b, m, w, e0, n, ctypes.byref(oo), None)
    assert chan(x, out, 4, 2, 0, 4) == BAD_ARG
    assert chan(x, out, 4, 8, 0, 16, pos0=1) == BAD_ARG
    assert b"csa_kv_compress_channel" in lib.csa_last_error()
    assert chan(_t(0, 96, 64), _t(0, 96, 16), 4, 8, 0, 4) == UNSUPPORTED
    assert chan(x, out, 4, 8, 0, 0) == 0
    # into a paged cache: block rows a power of two, a block list; the pool's
    # size does not bound the entry count
    paged = lambda xx, oo, m, w, e0, n, blk=FAKE, brows=32: lib.csa_kv_compress_paged(
        ctypes.byref(xx), z, 0, b, m, w, e0, n, blk, brows, ctypes.byref(oo), None)
    assert paged(x, out, 4, 8, 0, 4, brows=24) == BAD_ARG
    assert paged(x, out, 4, 8, 0, 4, brows=0) == BAD_ARG
    assert paged(x, out, 4, 8, 0, 4, blk=None) == BAD_ARG
    assert paged(x, out, 4, 2, 0, 4) == BAD_ARG
    assert paged(x, out, 4, 8, 0, 0) == 0


def _batch(n_q=4, n_req=1, max_kv=16):
    return CsaBatch(n_req, 0, n_q, max_kv, FAKE, FAKE, FAKE, FAKE, FAKE)


def test_kv_compress_batch_validation(lib):
    """The ragged compression call's host checks (no device needed)."""
    x, out = _t(0, 128, 64), _t(0, 128, 64)
    z = b = FAKE
    call = lambda bt, m=4, w=8, xx=x, oo=out: lib.csa_kv_compress_batch(
        ctypes.byref(xx), z, b, m, w, None if bt is None else ctypes.byref(bt), ctypes.byref(oo), None)
    assert call(None) == BAD_ARG                             # no batch
    assert call(_batch(), m=4, w=2) == BAD_ARG               # w < m
    assert call(_batch(), xx=_t(0, 64, 64)) == BAD_ARG       # dim mismatch
    ring = CsaBatch(1, 1, 4, 16, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert call(ring) == UNSUPPORTED                         # raw rows must be in order
    assert b"csa_kv_compress_batch" in lib.csa_last_error()
    no_raw = CsaBatch(1, 0, 4, 16, FAKE, FAKE, FAKE, None, None)
    assert call(no_raw) == BAD_ARG                           # raw offsets needed
    paged = CsaBatch(1, 0, 4, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 24, 0)
    assert call(paged) == BAD_ARG                            # block rows not a power of two
    assert call(CsaBatch(0, 0, 0, 0, None, None, None, None, None)) == 0   # empty batch, nothing launched


def test_kv_append_validation(lib):
    """Arguments the host refuses before any launch (no device needed)."""
    x, cache = _t(1, 128, 4), _t(1, 128, 64)
    f = lambda xx, cc, m=4, w=8, win=None, woff=FAKE, wrows=0, pos=FAKE, st=FAKE, eoff=FAKE, \
        table=None, stride=0, brows=0: \
        lib.csa_kv_compress_append(ctypes.byref(xx), FAKE, FAKE, m, w, pos, st, eoff, table, stride,
                                   brows, ctypes.byref(cc), ctypes.byref(win) if win is not None else None,
                                   woff, wrows, None)
    assert f(x, cache, w=9) == BAD_ARG                            # w > 2m
    assert f(x, cache, w=3) == BAD_ARG                            # w < m
    assert f(x, _t(1, 64, 64)) == BAD_ARG                         # dim mismatch
    assert f(_t(1, 32, 4), _t(1, 32, 64)) == UNSUPPORTED          # dim 32
    assert f(x, _t(2, 128, 64, scale=FAKE, rope=FAKE)) == BAD_ARG   # a mixed row has 512 dims
    assert f(x, _t(3, 128, 64, scale=FAKE)) == UNSUPPORTED        # MXFP4 entries
    assert f(x, cache, win=_t(1, 128, 256), wrows=0) == BAD_ARG   # ring without capacity
    assert f(x, cache, win=_t(1, 128, 256), woff=None, wrows=128) == BAD_ARG
    assert f(x, cache, pos=None) == BAD_ARG
    assert f(_t(1, 128, 0), cache, pos=None) == 0                 # no requests: nothing to do
    # a paged cache: block rows a power of two, a stride of at least one block
    assert f(x, cache, table=FAKE, stride=0, brows=32) == BAD_ARG
    assert f(x, cache, table=FAKE, stride=4, brows=24) == BAD_ARG
    assert f(x, cache, table=FAKE, stride=4, brows=0) == BAD_ARG
    assert f(x, cache, eoff=None) == BAD_ARG                       # neither rows nor blocks
    assert f(_t(1, 128, 0), cache, eoff=None, table=FAKE, stride=4, brows=32) == 0
    assert lib.csa_kv_append_state_size(3, 128) == 3 * 2 * 132 * 4


def test_attn_window_ring_flag_validated(lib):
    bt = _batch(n_q=2)
    bt.window_ring = 2
    q = _t(1, 128, 2 * 64)
    raw = _t(1, 128, 256)
    st = lib.csa_sparse_mqa_attn(ctypes.byref(q), 64, None, None, 0, ctypes.byref(raw), 128,
                                 ctypes.byref(bt), 4, 0.1, FAKE, 1, None, 0, None, 0, None)
    assert st == BAD_ARG


def test_indexer_validation(lib):
    qi, ki = _t(1, 64, 16), _t(1, 64, 32)
    bt = _batch()
    f = lambda qi_, h, ki_, b_, ld, sf=1: lib.csa_indexer_score(
        ctypes.byref(qi_), h, None, ctypes.byref(ki_), ctypes.byref(b_), 4, 1, FAKE, sf, ld, None)
    assert f(qi, 2, ki, bt, 16) == UNSUPPORTED               # 2 heads
    assert f(qi, 4, _t(0, 64, 32), bt, 16) == UNSUPPORTED    # format mismatch
    assert f(qi, 4, ki, bt, 8) == BAD_ARG                    # ld < max_kv
    assert f(_t(1, 64, 12), 4, ki, bt, 16) == BAD_ARG        # rows != n_q * heads
    assert f(qi, 4, ki, bt, 16, sf=2) == UNSUPPORTED         # score format
    assert f(_t(3, 64, 16, scale=None), 4, _t(3, 64, 32), bt, 16) == BAD_ARG  # MXFP4 without scales


def test_block_table_validation(lib):
    """A paged batch (kv_block_table) needs a stride of at least one block and
    a power-of-two block size; every call that reads entries checks it."""
    for stride, rows in ((0, 32), (4, 24), (4, 0), (4, 1 << 21)):
        bt = _batch(n_q=2)
        bt.kv_block_table, bt.kv_block_stride, bt.kv_block_rows = FAKE, stride, rows
        q, kv = _t(1, 128, 2 * 64), _t(1, 128, 100)
        assert lib.csa_sparse_mqa_attn(ctypes.byref(q), 64, ctypes.byref(kv), None, 0, None, 0,
                                       ctypes.byref(bt), 4, 0.1, FAKE, 1, None, 0, None, 0,
                                       None) == BAD_ARG
        qi, ki = _t(1, 64, 8), _t(1, 64, 32)
        assert lib.csa_indexer_score(ctypes.byref(qi), 4, None, ctypes.byref(ki), ctypes.byref(bt),
                                     4, 1, FAKE, 1, 16, None) == BAD_ARG
        assert lib.csa_indexer_topk(ctypes.byref(qi), 4, None, ctypes.byref(ki), ctypes.byref(bt),
                                    4, 1, 1, 8, FAKE, FAKE, 1 << 30, None) == BAD_ARG
        assert b"kv_block" in lib.csa_last_error()


def test_topk_validation(lib):
    bt = _batch()
    f = lambda k, ld, sf=1: lib.csa_topk_select(FAKE, sf, ld, ctypes.byref(bt), 4, k, FAKE, None)
    assert f(0, 16) == BAD_ARG
    assert f(5000, 16) == BAD_ARG
    assert f(8, 15) == BAD_ARG
    assert f(8, 16, sf=2) == UNSUPPORTED


def test_attn_validation(lib):
    bt = _batch(n_q=2)
    q = _t(1, 128, 2 * 64)
    kv = _t(1, 128, 100)
    f = lambda qq, h, kk, of=1, m=4, k=8, split=0, ws=None, wsb=0, sc=0.1: lib.csa_sparse_mqa_attn(
        ctypes.byref(qq), h, ctypes.byref(kk) if kk is not None else None, None, k, None, 0,
        ctypes.byref(bt), m, sc, FAKE, of, None, split, ws, wsb, None)
    assert f(q, 48, kv) == BAD_ARG                  # rows != n_q * heads
    assert f(_t(1, 128, 2 * 48), 48, kv) == UNSUPPORTED   # 48 heads
    assert f(q, 64, _t(1, 256, 100)) == BAD_ARG     # kv dim mismatch
    assert f(_t(1, 256, 128), 64, None) == UNSUPPORTED   # D = 256
    assert f(q, 64, kv, of=2) == UNSUPPORTED        # out format
    assert f(q, 64, kv, m=0) == BAD_ARG
    assert f(q, 64, _t(2, 128, 100, scale=FAKE, rope=FAKE)) == BAD_ARG  # mixed needs D 512
    assert f(_t(0, 128, 128), 64, kv) == UNSUPPORTED   # f32 q with bf16 kv
    assert f(q, 64, kv, sc=0.0) == BAD_ARG             # scale must be positive
    q8 = _t(2, 512, 2 * 64, scale=FAKE, rope=FAKE)     # fp8 queries
    assert f(q8, 64, _t(1, 512, 100)) == UNSUPPORTED    # need FP8_MIXED entries
    assert f(q8, 64, None) == UNSUPPORTED                # ... given
    assert f(_t(2, 512, 2 * 32, scale=FAKE, rope=FAKE), 32, _t(2, 512, 100, scale=FAKE, rope=FAKE)) == UNSUPPORTED
    assert f(q, 64, kv, split=64) == 3                 # split-K without workspace
    need = lib.csa_attn_workspace_size(2, 64, 128, 16, 64)
    assert need > 2 * 64 * 129 * 4
    assert f(q, 64, kv, split=64, ws=FAKE, wsb=need - 1) == 3
    assert f(_t(1, 128, 2 * 16), 16, kv, split=64, ws=FAKE, wsb=need) == UNSUPPORTED
    assert lib.csa_attn_workspace_size(2, 64, 128, 16, 0) == 0
    # D = 512 with 64 heads split over keys: a part may hold at most 4096 keys
    q5, kv5 = _t(1, 512, 2 * 64), _t(1, 512, 100)
    need5 = lib.csa_attn_workspace_size(2, 64, 512, 16, 5000)
    assert f(q5, 64, kv5, split=5000, ws=FAKE, wsb=need5) == UNSUPPORTED
    assert b"exceed 2048" in lib.csa_last_error()


@pytest.mark.parametrize("max_keys,split_keys", [(1152, 288), (640, 288), (8320, 288), (100000, 128),
                                                 (31, 32), (1, 1), (4224, 128), (1025, 32)])
def test_attn_workspace_follows_the_split_rule(lib, max_keys, split_keys):
    """The split-K workspace holds min(32, ceil(max_keys / split_keys)) parts of
    fp32 partials and lse per row (the parts rule the header states), plus the
    per-query bookkeeping."""
    n_q, H, D = 7, 64, 512
    parts = min(32, -(-max_keys // split_keys))
    expect = parts * n_q * H * (D + 1) * 4 + (n_q * (2 + parts) + 2) * 4 + 16 + n_q * 64 + 256
    assert lib.csa_attn_workspace_size(n_q, H, D, max_keys, split_keys) == expect


def test_projection_validation(lib):
    """Host checks of csa_linear and csa_grouped_out_proj (no device needed)."""
    A = ctypes.c_void_p(1 << 20)       # 16-byte aligned stand-in pointers
    f = lambda M=4, N=4, K=64, ldx=64, ldw=64, ldy=4, fmt=0, batch=1, x=A, sx=0: lib.csa_linear(
        x, ldx, sx, A, ldw, 0, A, fmt, ldy, 0, M, N, K, batch, None)
    assert f(K=0) == BAD_ARG
    assert f(K=96, ldx=96, ldw=96) == UNSUPPORTED          # K not a multiple of 64
    assert f(fmt=2) == UNSUPPORTED                          # y format
    assert f(ldx=32) == BAD_ARG                             # short leading dimension
    assert f(ldy=3) == BAD_ARG
    assert f(x=ctypes.c_void_p((1 << 20) + 8)) == BAD_ARG   # misaligned x
    assert f(ldx=68) == BAD_ARG                             # rows not 16-byte aligned
    assert f(x=None) == BAD_ARG
    assert f(batch=0) == BAD_ARG
    assert f(M=0) == 0 and f(N=0, x=None) == 0              # nothing to do
    g = lambda H=64, D=512, G=8, dg=256, ws=A, wsb=1 << 30: lib.csa_grouped_out_proj(
        A, 4, H, D, G, A, dg, A, 384, A, 0, ws, wsb, None)
    assert g(G=6) == BAD_ARG                                # groups must divide the heads
    assert g(H=8, D=8, G=8) == UNSUPPORTED                  # group inputs not a multiple of 64
    assert g(dg=36) == UNSUPPORTED                          # 8 * 36 not a multiple of 64
    assert g(ws=None) == 3
    assert g(wsb=lib.csa_grouped_out_proj_workspace_size(4, 8, 256) - 1) == 3
    assert lib.csa_grouped_out_proj_workspace_size(4, 8, 256) >= 4 * 8 * 256 * 2


def test_merge_and_codec_validation(lib):
    assert lib.csa_swa_merge(FAKE, FAKE, FAKE, FAKE, 4, 6, FAKE, 1, None, None) == BAD_ARG
    assert lib.csa_swa_merge(FAKE, FAKE, FAKE, FAKE, 4, 8, FAKE, 3, None, None) == UNSUPPORTED
    assert lib.csa_swa_merge(None, FAKE, FAKE, FAKE, 4, 8, FAKE, 1, None, None) == BAD_ARG
    assert lib.csa_swa_merge(None, None, None, None, 0, 8, None, 1, None, None) == 0
    src, dst = _t(0, 512, 4), _t(2, 512, 4, scale=FAKE, rope=FAKE)
    assert lib.csa_quantize(ctypes.byref(src), ctypes.byref(_t(2, 512, 5, scale=FAKE, rope=FAKE)), None) == BAD_ARG
    assert lib.csa_quantize(ctypes.byref(dst), ctypes.byref(src), None) == UNSUPPORTED
    assert lib.csa_quantize(ctypes.byref(_t(0, 40, 4)), ctypes.byref(_t(3, 40, 4, scale=FAKE)), None) == BAD_ARG
    assert lib.csa_mxfp4_to_fp8(ctypes.byref(src), FAKE, FAKE, FAKE, None) == BAD_ARG


def test_indexer_topk_validation(lib):
    qi, ki = _t(1, 64, 16), _t(1, 64, 32)
    bt = _batch()
    need = lib.csa_indexer_topk_workspace_size(4, 8)
    assert need >= 4 * 2 * 4 + 4 * 4096 * 8         # per-query state and candidate lists
    assert lib.csa_indexer_topk_workspace_size(0, 8) == 0
    f = lambda k=8, ws=FAKE, nbytes=need, b_=bt, sf=1, qi_=qi: lib.csa_indexer_topk(
        ctypes.byref(qi_), 4, None, ctypes.byref(ki), ctypes.byref(b_), 4, 1, sf, k, FAKE, ws,
        nbytes, None)
    WORKSPACE = 3
    assert f(ws=None) == WORKSPACE
    assert f(nbytes=need - 1) == WORKSPACE
    assert f(k=0) == BAD_ARG
    assert f(k=4097) == BAD_ARG
    assert f(sf=2) == UNSUPPORTED                       # scores are F32 or BF16
    assert f(qi_=_t(1, 64, 15)) == BAD_ARG               # rows != n_q * heads
    assert f(b_=_batch(max_kv=(1 << 20) + 1)) == UNSUPPORTED
    assert f(ws=ctypes.c_void_p(0x1008)) == BAD_ARG      # workspace not 16-byte aligned


def test_indexer_topk_noalloc_limit_checked_on_the_host(lib):
    """The entry point without a workspace refuses, before any HIP call, a call
    whose candidate lists exceed its static scratch; its other checks are
    those of csa_indexer_topk."""
    cap = lib.csa_indexer_topk_noalloc_max_bytes()
    assert cap == 16 << 20
    n_q = 4096                                    # 4096 queries at k = 1024: far above
    assert lib.csa_indexer_topk_workspace_size(n_q, 1024) > cap
    qi = CsaTensor(3, 64, n_q * 4, FAKE, FAKE, None)
    ki = CsaTensor(3, 64, 1000, FAKE, FAKE, None)
    bt = CsaBatch(n_q, 0, n_q, 1000, FAKE, FAKE, FAKE, None, None, None, 0, 0, 0)
    WORKSPACE = 3
    st = lib.csa_indexer_topk_noalloc(ctypes.byref(qi), 4, None, ctypes.byref(ki), ctypes.byref(bt),
                                      4, 1, 1, 1024, FAKE, None)
    assert st == WORKSPACE
    assert b"static scratch" in lib.csa_last_error()
    # the shared checks: wrong head count
    st = lib.csa_indexer_topk_noalloc(ctypes.byref(qi), 8, None, ctypes.byref(ki), ctypes.byref(bt),
                                      4, 1, 1, 1024, FAKE, None)
    assert st == UNSUPPORTED
