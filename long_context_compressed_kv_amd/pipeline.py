"""One CSA or HCA layer as a sequence of library calls (plumbing only).

Prefill (one sequence):
  CSA: kv_compress (new entries into the cache) -> indexer_topk (scores and
       selection fused; or indexer_score -> topk_select with fused=False)
       -> sparse_mqa_attn over the selected entries and the window, one softmax
  HCA: kv_compress -> sparse_mqa_attn over all visible entries and the window
Decode (a batch of requests, one query each):
  CSA: indexer_topk (or indexer_score -> topk_select) -> sparse_mqa_attn(selected
       entries and window, split into key chunks merged by log-sum-exp)
  HCA: sparse_mqa_attn(visible entries and window, split the same way)
(page "DeepSeek V4 深度解析", section 2: the three CSA steps and HCA).
"""
import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import torch

from . import ops
from .ops import BF16, F32, KV, Batch

INDEXER_HEADS = 4


def _score_dtype(fmt):
    return torch.bfloat16 if fmt == BF16 else torch.float32


def _out_dtype(fmt):
    return torch.bfloat16 if fmt == BF16 else torch.float32


@dataclass
class Buffers:
    """Reusable device buffers of a layer call (allocated on first use)."""
    store: dict = field(default_factory=dict)

    def get(self, name, shape, dtype, device="cuda"):
        t = self.store.get(name)
        if t is None or tuple(t.shape) != tuple(shape) or t.dtype != dtype:
            t = torch.empty(shape, dtype=dtype, device=device)
            self.store[name] = t
        return t


def _select(L, n_q, ld):
    """CSA step 2 for a layer L with n_q queries and rows of at most ld entries:
    the fused call, or the score matrix and the selection over it."""
    idx = L.buf.get("idx", (n_q, L.k), torch.int32)
    if L.fused:
        ws = L.buf.get("itk_ws", (max(ops.indexer_topk_workspace_size(n_q, L.k), 1),),
                       torch.uint8)
        ops.indexer_topk(L.qi, INDEXER_HEADS, L.ki, L.batch, L.m, L.score_fmt, L.k, idx=idx,
                         workspace=ws)
        return None, idx
    scores = L.buf.get("scores", (n_q, ld), _score_dtype(L.score_fmt))
    ops.indexer_score(L.qi, INDEXER_HEADS, L.ki, L.batch, L.m, scores, L.score_fmt)
    ops.topk_select(scores, L.score_fmt, L.batch, L.m, L.k, idx)
    return scores, idx


# ---------------------------------------------------------------- prefill


@dataclass
class PrefillLayer:
    """A prefill of T query tokens at positions pos0 .. pos0+T-1 of one sequence.

    raw   : raw KV rows for positions raw_pos0 .. pos0+T-1 (history + chunk)
    z     : compression logits aligned with raw; bias: slot biases [w]
    cache : entry tensor with room for all entries up to pos0+T (rows
            0 .. n_cached-1 already filled)
    q     : [T*H, D] attention queries; qi: [T*4, 64] indexer queries;
            ki: [>= n_entries, 64] indexer keys (CSA only)
    """
    csa: bool
    H: int
    m: int
    w: int
    k: int
    window: int
    raw: KV
    z: torch.Tensor
    bias: torch.Tensor
    raw_pos0: int
    pos0: int
    T: int
    cache: KV
    n_cached: int
    q: KV
    qi: Optional[KV] = None
    ki: Optional[KV] = None
    score_fmt: int = F32
    out_fmt: int = F32
    fused: bool = True
    buf: Buffers = field(default_factory=Buffers)

    def __post_init__(self):
        dev = self.q.data.device
        self.n_entries = (self.pos0 + self.T) // self.m
        self.first_new = self.pos0 // self.m
        assert self.first_new == self.n_cached, "cache must hold every entry before the chunk"
        assert self.cache.rows >= self.n_entries
        self.batch = Batch.make([self.T], [self.pos0], kv_counts=[self.n_entries],
                                raw_counts=[self.raw.rows], raw_pos=[self.raw_pos0], device=dev)

    def compress(self):
        n_new = self.n_entries - self.first_new
        ops.kv_compress(self.raw, self.z, self.raw_pos0, self.bias, self.m, self.w,
                        self.first_new, n_new, self.cache.narrow(self.first_new, max(n_new, 0)))

    def select(self):
        """(scores, or None when fused; idx [T, k])"""
        return _select(self, self.T, self.n_entries)

    def attend(self, idx):
        out = self.buf.get("out", (self.T * self.H, self.q.dim), _out_dtype(self.out_fmt))
        lse = self.buf.get("lse", (self.T * self.H,), torch.float32)
        ops.sparse_mqa_attn(self.q, self.H, self.cache, idx, self.k if idx is not None else 0,
                            self.raw, self.window, self.batch, self.m, out, self.out_fmt, lse)
        return out, lse

    def run(self):
        self.compress()
        scores = idx = None
        if self.csa:
            scores, idx = self.select()
        out, lse = self.attend(idx)
        return {"out": out, "lse": lse, "idx": idx, "scores": scores}


# ---------------------------------------------------------------- decode


@dataclass
class DecodeLayer:
    """One decode step of a batch: request r has one query at position ctx[r],
    entries kv_off[r] .. of `cache`, and window rows swa_off[r] .. of `swa`
    holding positions swa_pos[r] .. ctx[r]."""
    csa: bool
    H: int
    m: int
    k: int
    window: int
    ctx: list
    n_entries: list
    swa_len: list
    cache: KV
    swa: KV
    q: KV
    qi: Optional[KV] = None
    ki: Optional[KV] = None
    score_fmt: int = BF16
    out_fmt: int = BF16
    # keys per split-K part: None = a quarter of a CSA query's k + window
    # (at least 128), 288 for HCA; a layer constant, so a request's parts
    # depend on its own key count only
    split_keys: Optional[int] = None
    fused: bool = True
    # paged compressed cache: int32 [B, stride] block ids, block_rows entries a block
    kv_block_table: Optional[torch.Tensor] = None
    kv_block_rows: int = 0
    buf: Buffers = field(default_factory=Buffers)

    def __post_init__(self):
        dev = self.q.data.device
        B = len(self.ctx)
        self.B = B
        swa_pos = [int(c) - int(s) + 1 for c, s in zip(self.ctx, self.swa_len)]
        self.batch = Batch.make([1] * B, self.ctx, kv_counts=self.n_entries,
                                raw_counts=self.swa_len, raw_pos=swa_pos, device=dev)
        if self.kv_block_table is not None:
            self.batch = dataclasses.replace(self.batch, kv_block_table=self.kv_block_table,
                                             kv_block_rows=self.kv_block_rows)
        self.ld = max(int(x) for x in self.n_entries)
        if self.split_keys is None:
            self.split_keys = max(128, -(-(self.k + self.window) // 4)) if self.csa else 288

    def select(self):
        """(scores, or None when fused; idx [B, k])"""
        return _select(self, self.B, self.ld)

    def attend(self, idx):
        """One attention call over entries and window together, its keys cut
        into chunks of `split_keys` run in parallel and merged by log-sum-exp."""
        rows, D = self.B * self.H, self.q.dim
        out = self.buf.get("out", (rows, D), _out_dtype(self.out_fmt))
        lse = self.buf.get("lse", (rows,), torch.float32)
        max_keys = (self.k if idx is not None else self.ld) + self.window
        ws = self.buf.get("ws", (max(ops.attn_workspace_size(self.B, self.H, D, max_keys,
                                                               self.split_keys), 1),),
                          torch.uint8)
        ops.sparse_mqa_attn(self.q, self.H, self.cache, idx, self.k if idx is not None else 0,
                            self.swa, self.window, self.batch, self.m, out, self.out_fmt, lse,
                            split_keys=self.split_keys, workspace=ws)
        return out, lse

    def run(self):
        scores = idx = None
        if self.csa:
            scores, idx = self.select()
        out, lse = self.attend(idx)
        return {"out": out, "lse": lse, "idx": idx, "scores": scores}
