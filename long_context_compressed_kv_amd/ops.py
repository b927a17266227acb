"""Python binding of the CSA/HCA library: the C-ABI calls with torch tensors.

Argument marshalling only: every step runs in libcsa.so's HIP kernels, on the
current torch stream.  Torch provides device memory and streams.
"""
import ctypes
import math
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import CSA_BF16, CSA_F32, CSA_FP8_MIXED, CSA_MXFP4, CsaBatch, CsaTensor, check

F32, BF16, FP8_MIXED, MXFP4 = CSA_F32, CSA_BF16, CSA_FP8_MIXED, CSA_MXFP4


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _fmt_of(t):
    """Output format code of a float32 or bfloat16 tensor."""
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError("output must be float32 or bfloat16")


def _need_cuda(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


@dataclass
class KV:
    """A matrix of `rows` vectors of `dim` elements in one storage format.

    F32 / BF16 : data float32 / bfloat16 [rows, dim]
    FP8_MIXED  : data uint8 [rows, 448] (e4m3fn), scale uint8 [rows, 4] (e8m0),
                 rope bfloat16 [rows, 64]; dim 512
    MXFP4      : data uint8 [rows, dim/2] (two e2m1 per byte), scale uint8
                 [rows, dim/32] (e8m0)
    """
    fmt: int
    dim: int
    data: torch.Tensor
    scale: Optional[torch.Tensor] = None
    rope: Optional[torch.Tensor] = None

    @property
    def rows(self):
        return self.data.shape[0]

    def c(self):
        _need_cuda(self.data, self.scale, self.rope)
        return CsaTensor(self.fmt, self.dim, self.rows, _ptr(self.data), _ptr(self.scale),
                         _ptr(self.rope))

    def narrow(self, start, length):
        """Rows start .. start+length-1 (a view)."""
        f = lambda t: None if t is None else t.narrow(0, start, length)
        return KV(self.fmt, self.dim, f(self.data), f(self.scale), f(self.rope))

    @staticmethod
    def empty(fmt, rows, dim, device="cuda"):
        if fmt == F32:
            return KV(fmt, dim, torch.empty(rows, dim, dtype=torch.float32, device=device))
        if fmt == BF16:
            return KV(fmt, dim, torch.empty(rows, dim, dtype=torch.bfloat16, device=device))
        if fmt == FP8_MIXED:
            assert dim == 512
            return KV(fmt, dim, torch.empty(rows, 448, dtype=torch.uint8, device=device),
                      torch.empty(rows, 4, dtype=torch.uint8, device=device),
                      torch.empty(rows, 64, dtype=torch.bfloat16, device=device))
        if fmt == MXFP4:
            assert dim % 32 == 0
            return KV(fmt, dim, torch.empty(rows, dim // 2, dtype=torch.uint8, device=device),
                      torch.empty(rows, dim // 32, dtype=torch.uint8, device=device))
        raise ValueError(fmt)


def dense(t):
    """A float32 / bfloat16 tensor [..., dim] as a KV view of its rows."""
    fmt = {torch.float32: F32, torch.bfloat16: BF16}[t.dtype]
    return KV(fmt, t.shape[-1], t.reshape(-1, t.shape[-1]))


@dataclass
class Batch:
    """Requests of a call (see csa_batch in include/csa.h).  Offsets and
    positions are int64 device tensors; n_q and max_kv are host ints."""
    q_off: torch.Tensor
    q_pos: torch.Tensor
    kv_off: Optional[torch.Tensor]
    raw_off: Optional[torch.Tensor]
    raw_pos: Optional[torch.Tensor]
    n_q: int
    max_kv: int
    window_ring: bool = False   # raw rows of a request form a ring (see csa_batch)
    # paged entries (see csa_batch): int32 [n_req, stride] block ids, P entries a block
    kv_block_table: Optional[torch.Tensor] = None
    kv_block_rows: int = 0

    @property
    def n_req(self):
        return self.q_pos.shape[0]

    def c(self):
        for t in (self.q_off, self.q_pos, self.kv_off, self.raw_off, self.raw_pos):
            if t is not None:
                _need_cuda(t)
                assert t.dtype == torch.int64
        stride = 0
        if self.kv_block_table is not None:
            _need_cuda(self.kv_block_table)
            assert self.kv_block_table.dtype == torch.int32 and self.kv_block_table.dim() == 2
            assert self.kv_block_table.is_contiguous()
            stride = self.kv_block_table.shape[1]
        return CsaBatch(self.n_req, int(bool(self.window_ring)), self.n_q, self.max_kv,
                        _ptr(self.q_off), _ptr(self.q_pos),
                        _ptr(self.kv_off), _ptr(self.raw_off), _ptr(self.raw_pos),
                        _ptr(self.kv_block_table), stride, int(self.kv_block_rows), 0)

    @staticmethod
    def make(q_counts, q_pos, kv_counts=None, raw_counts=None, raw_pos=None, device="cuda"):
        """Build from per-request host lists."""
        def off(c):
            o = [0]
            for x in c:
                o.append(o[-1] + int(x))
            return torch.tensor(o, dtype=torch.int64, device=device)
        i64 = lambda v: torch.tensor([int(x) for x in v], dtype=torch.int64, device=device)
        return Batch(off(q_counts), i64(q_pos),
                     off(kv_counts) if kv_counts is not None else None,
                     off(raw_counts) if raw_counts is not None else None,
                     i64(raw_pos) if raw_pos is not None else None,
                     int(sum(int(x) for x in q_counts)),
                     int(max([int(x) for x in kv_counts] or [0])) if kv_counts is not None else 0)


# ----------------------------------------------------------------------------- calls


def kv_compress(x: KV, logits, x_pos0, slot_bias, m, w, entry_begin, n_entries, out: KV,
                blocks=None, block_rows=0):
    """CSA step 1: entries entry_begin .. +n_entries of one sequence into
    out[0:n], or with `blocks` (int32, the request's block ids) into the
    paged cache `out`: entry j at row blocks[j // block_rows] * block_rows +
    j % block_rows."""
    _need_cuda(logits, slot_bias, blocks)
    lib = _lib.load()
    xc, oc = x.c(), out.c()
    if blocks is not None:
        assert blocks.dtype == torch.int32 and blocks.is_contiguous()
        check(lib.csa_kv_compress_paged(ctypes.byref(xc), _ptr(logits), int(x_pos0), _ptr(slot_bias),
                                        int(m), int(w), int(entry_begin), int(n_entries),
                                        _ptr(blocks), int(block_rows), ctypes.byref(oc), _stream()),
              "csa_kv_compress_paged")
        return out
    check(lib.csa_kv_compress(ctypes.byref(xc), _ptr(logits), int(x_pos0), _ptr(slot_bias),
                              int(m), int(w), int(entry_begin), int(n_entries),
                              ctypes.byref(oc), _stream()), "csa_kv_compress")
    return out


def kv_compress_batch(x: KV, logits, slot_bias, m, w, batch, out: KV):
    """CSA step 1 for a batch of prefill chunks in one launch: for each
    request r, the entries its chunk completes (floor(q_pos/m) ..
    floor((q_pos+T_r)/m) - 1) from its raw rows (raw_off / raw_pos) into its
    cache rows (kv_off, or its blocks when the batch is paged)."""
    _need_cuda(logits, slot_bias)
    lib = _lib.load()
    xc, oc, bc = x.c(), out.c(), batch.c()
    check(lib.csa_kv_compress_batch(ctypes.byref(xc), _ptr(logits), _ptr(slot_bias), int(m), int(w),
                                    ctypes.byref(bc), ctypes.byref(oc), _stream()), "csa_kv_compress_batch")
    return out


def kv_compress_channel(x: KV, logits, x_pos0, slot_bias, m, w, entry_begin, n_entries, out: KV):
    """CSA step 1 with a logit per raw token and channel: logits float
    [x.rows, dim], slot_bias float [w, dim]; one softmax per channel."""
    _need_cuda(logits, slot_bias)
    assert logits.dtype == torch.float32 and logits.is_contiguous()
    assert slot_bias.dtype == torch.float32 and slot_bias.is_contiguous()
    assert tuple(logits.shape) == (x.rows, x.dim) and tuple(slot_bias.shape) == (int(w), x.dim)
    lib = _lib.load()
    xc, oc = x.c(), out.c()
    check(lib.csa_kv_compress_channel(ctypes.byref(xc), _ptr(logits), int(x_pos0), _ptr(slot_bias),
                                      int(m), int(w), int(entry_begin), int(n_entries),
                                      ctypes.byref(oc), _stream()), "csa_kv_compress_channel")
    return out


def kv_append_state_size(n_req, dim):
    """Bytes of the per-request compression state csa_kv_compress_append keeps."""
    return int(_lib.load().csa_kv_append_state_size(int(n_req), int(dim)))


def kv_compress_append(x: KV, logits, slot_bias, m, w, pos, state, entry_off, cache: KV,
                       window: Optional[KV] = None, window_off=None, window_rows=0,
                       block_table=None, block_rows=0):
    """Decode-time compression: appends row r of x (at position pos[r]) to
    request r's state; finished entries go to cache row entry_off[r] + i (or,
    with an int32 [n_req, stride] block table, to row
    block_table[r, i // block_rows] * block_rows + i % block_rows), and with a
    window the raw row to window_off[r] + pos[r] % window_rows."""
    _need_cuda(logits, slot_bias, pos, state, entry_off, window_off, block_table)
    stride = 0
    if block_table is not None:
        assert block_table.dtype == torch.int32 and block_table.dim() == 2
        assert block_table.is_contiguous()
        stride = block_table.shape[1]
    lib = _lib.load()
    xc, cc = x.c(), cache.c()
    wc = window.c() if window is not None else None
    check(lib.csa_kv_compress_append(ctypes.byref(xc), _ptr(logits), _ptr(slot_bias), int(m),
                                     int(w), _ptr(pos), _ptr(state), _ptr(entry_off),
                                     _ptr(block_table), stride, int(block_rows),
                                     ctypes.byref(cc), ctypes.byref(wc) if wc is not None else None,
                                     _ptr(window_off), int(window_rows), _stream()),
          "csa_kv_compress_append")
    return cache


def indexer_score(qi: KV, n_heads, ki: KV, batch: Batch, m, scores, score_fmt,
                  head_w=None, relu=True):
    """CSA step 2: indexer scores [n_q, ld] (columns beyond each row's visible
    entries are left untouched)."""
    _need_cuda(scores, head_w)
    lib = _lib.load()
    qc, kc, bc = qi.c(), ki.c(), batch.c()
    check(lib.csa_indexer_score(ctypes.byref(qc), int(n_heads), _ptr(head_w), ctypes.byref(kc),
                                ctypes.byref(bc), int(m), 1 if relu else 0, _ptr(scores),
                                int(score_fmt), int(scores.shape[1]), _stream()),
          "csa_indexer_score")
    return scores


def topk_select(scores, score_fmt, batch: Batch, m, k, idx=None):
    """CSA step 2: int32 [n_q, k] ascending entry indices, -1 padded."""
    _need_cuda(scores)
    if idx is None:
        idx = torch.empty(batch.n_q, k, dtype=torch.int32, device=scores.device)
    lib = _lib.load()
    bc = batch.c()
    check(lib.csa_topk_select(_ptr(scores), int(score_fmt), int(scores.shape[1]),
                              ctypes.byref(bc), int(m), int(k), _ptr(idx), _stream()),
          "csa_topk_select")
    return idx


def indexer_topk_workspace_size(n_q, k):
    return int(_lib.load().csa_indexer_topk_workspace_size(int(n_q), int(k)))


def indexer_topk(qi: KV, n_heads, ki: KV, batch: Batch, m, score_fmt, k, head_w=None,
                 relu=True, idx=None, workspace=None):
    """CSA step 2 fused: the top-k entries of each query by indexer score
    (score_fmt rounding), int32 [n_q, k] ascending, -1 padded, without a score
    matrix.  `workspace` is a uint8 device tensor of at least
    indexer_topk_workspace_size(n_q, k) bytes (allocated here when None)."""
    _need_cuda(head_w, idx, workspace)
    dev = qi.data.device
    if idx is None:
        idx = torch.empty(batch.n_q, k, dtype=torch.int32, device=dev)
    lib = _lib.load()
    need = indexer_topk_workspace_size(batch.n_q, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    qc, kc, bc = qi.c(), ki.c(), batch.c()
    check(lib.csa_indexer_topk(ctypes.byref(qc), int(n_heads), _ptr(head_w), ctypes.byref(kc),
                               ctypes.byref(bc), int(m), 1 if relu else 0, int(score_fmt), int(k),
                               _ptr(idx), _ptr(workspace), int(workspace.numel()), _stream()),
          "csa_indexer_topk")
    return idx


def indexer_topk_noalloc_max_bytes():
    return int(_lib.load().csa_indexer_topk_noalloc_max_bytes())


def indexer_topk_noalloc(qi: KV, n_heads, ki: KV, batch: Batch, m, score_fmt, k, idx,
                         head_w=None, relu=True):
    """indexer_topk without a workspace: the candidate lists live in the
    library's static device scratch (see csa_indexer_topk_noalloc); `idx`
    int32 [n_q, k] is written in place."""
    _need_cuda(head_w, idx)
    lib = _lib.load()
    qc, kc, bc = qi.c(), ki.c(), batch.c()
    check(lib.csa_indexer_topk_noalloc(ctypes.byref(qc), int(n_heads), _ptr(head_w),
                                       ctypes.byref(kc), ctypes.byref(bc), int(m),
                                       1 if relu else 0, int(score_fmt), int(k), _ptr(idx),
                                       _stream()),
          "csa_indexer_topk_noalloc")
    return idx


def attn_workspace_size(n_q, n_heads, dim, max_keys, split_keys):
    return int(_lib.load().csa_attn_workspace_size(int(n_q), int(n_heads), int(dim),
                                                   int(max_keys), int(split_keys)))


def sparse_mqa_attn(q: KV, n_heads, kv: Optional[KV], idx, k, raw: Optional[KV], window,
                    batch: Batch, m, out, out_fmt, lse=None, scale=None, split_keys=0,
                    workspace=None):
    """CSA step 3 / HCA: attention over selected (idx) or all visible entries
    (idx=None) plus the window; out [n_q*H, D], lse [n_q*H] (optional).
    split_keys > 0 cuts each query's keys into parallel chunks merged by
    log-sum-exp (decode); `workspace` is then a uint8 device tensor of at least
    attn_workspace_size(...) bytes (allocated here when None)."""
    _need_cuda(idx, out, lse, workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(q.dim)
    lib = _lib.load()
    if split_keys and workspace is None:
        max_keys = (k if idx is not None else batch.max_kv) + (window if raw is not None else 0)
        workspace = torch.empty(max(attn_workspace_size(batch.n_q, n_heads, q.dim, max_keys,
                                                        split_keys), 1),
                                dtype=torch.uint8, device=q.data.device)
    qc, bc = q.c(), batch.c()
    kvc = kv.c() if kv is not None else None
    rc = raw.c() if raw is not None else None
    check(lib.csa_sparse_mqa_attn(ctypes.byref(qc), int(n_heads),
                                  ctypes.byref(kvc) if kvc is not None else None,
                                  _ptr(idx), int(k),
                                  ctypes.byref(rc) if rc is not None else None, int(window),
                                  ctypes.byref(bc), int(m), float(scale), _ptr(out),
                                  int(out_fmt), _ptr(lse), int(split_keys), _ptr(workspace),
                                  int(workspace.numel()) if workspace is not None else 0,
                                  _stream()),
          "csa_sparse_mqa_attn")
    return out


def swa_merge(o_a, lse_a, o_b, lse_b, out, out_fmt, lse_out=None):
    """Log-sum-exp combination of two partial attentions."""
    _need_cuda(o_a, lse_a, o_b, lse_b, out, lse_out)
    lib = _lib.load()
    check(lib.csa_swa_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), int(o_a.shape[0]),
                            int(o_a.shape[1]), _ptr(out), int(out_fmt), _ptr(lse_out), _stream()),
          "csa_swa_merge")
    return out


def linear(x, w, y):
    """y = x W^T (the projections around the path): x bf16 [..., M, K],
    w bf16 [..., N, K] (weights stored [out, in]), y F32 or BF16 [..., M, N];
    a leading batch dimension (the same on all three, or absent) runs the
    batch in one launch.  Row strides and batch strides are taken from the
    tensors (the last dimension must be contiguous)."""
    if not (x.is_cuda and w.is_cuda and y.is_cuda):
        raise ValueError("tensors must live on the GPU")
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise ValueError("x and w must be bfloat16")
    batched = x.dim() == 3
    if batched != (w.dim() == 3) or batched != (y.dim() == 3):
        raise ValueError("x, w and y must all be batched or none")
    if x.stride(-1) != 1 or w.stride(-1) != 1 or y.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    M, K = x.shape[-2], x.shape[-1]
    N = w.shape[-2]
    if w.shape[-1] != K or y.shape[-2] != M or y.shape[-1] != N:
        raise ValueError("shape mismatch")
    batch = x.shape[0] if batched else 1
    bs = lambda t: t.stride(0) if batched else 0
    lib = _lib.load()
    check(lib.csa_linear(_ptr(x), x.stride(-2), bs(x), _ptr(w), w.stride(-2), bs(w), _ptr(y),
                         _fmt_of(y), y.stride(-2), bs(y), M, N, K, batch, _stream()), "csa_linear")
    return y


def grouped_out_proj_workspace_size(n_q, groups, d_group):
    return int(_lib.load().csa_grouped_out_proj_workspace_size(int(n_q), int(groups), int(d_group)))


def grouped_out_proj(o, n_heads, w_group, w_out, out, workspace=None):
    """Grouped output projection of attention outputs o bf16 [n_q*n_heads, D]
    (or [n_q, n_heads, D]): w_group bf16 [G, d_g, (n_heads/G)*D], w_out bf16
    [d_model, G*d_g], out F32 or BF16 [n_q, d_model]; `workspace` a uint8
    device tensor of grouped_out_proj_workspace_size(...) bytes (allocated
    here when None)."""
    _need_cuda(o, w_group, w_out, out, workspace)
    if o.dtype != torch.bfloat16 or w_group.dtype != torch.bfloat16 or w_out.dtype != torch.bfloat16:
        raise ValueError("o and the weights must be bfloat16")
    for t in (o, w_group, w_out, out):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    D = o.shape[-1]
    n_q = o.numel() // (n_heads * D)
    G, d_g = w_group.shape[0], w_group.shape[1]
    d_model = w_out.shape[0]
    if workspace is None:
        workspace = torch.empty(max(grouped_out_proj_workspace_size(n_q, G, d_g), 1),
                                dtype=torch.uint8, device=o.device)
    lib = _lib.load()
    check(lib.csa_grouped_out_proj(_ptr(o), n_q, int(n_heads), D, G, _ptr(w_group), d_g, _ptr(w_out),
                                   d_model, _ptr(out), _fmt_of(out), _ptr(workspace),
                                   workspace.numel(), _stream()), "csa_grouped_out_proj")
    return out


def quantize(src: KV, dst: KV):
    lib = _lib.load()
    sc, dc = src.c(), dst.c()
    check(lib.csa_quantize(ctypes.byref(sc), ctypes.byref(dc), _stream()), "csa_quantize")
    return dst


def dequantize(src: KV, out=None):
    lib = _lib.load()
    if out is None:
        out = torch.empty(src.rows, src.dim, dtype=torch.float32, device=src.data.device)
    _need_cuda(out)
    sc = src.c()
    check(lib.csa_dequantize(ctypes.byref(sc), _ptr(out), _stream()), "csa_dequantize")
    return out


def mxfp4_to_fp8(src: KV):
    lib = _lib.load()
    dev = src.data.device
    fp8 = torch.empty(src.rows, src.dim, dtype=torch.uint8, device=dev)
    g = torch.empty(src.rows, dtype=torch.uint8, device=dev)
    ok = torch.empty(src.rows, dtype=torch.uint8, device=dev)
    sc = src.c()
    check(lib.csa_mxfp4_to_fp8(ctypes.byref(sc), _ptr(fp8), _ptr(g), _ptr(ok), _stream()),
          "csa_mxfp4_to_fp8")
    return fp8, g, ok


def abi_version():
    return _lib.load().csa_abi_version()
