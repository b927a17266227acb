"""Seeded synthetic inputs for the CSA/HCA compressed-attention workloads.

This module only draws random numbers and lays out shapes and positions; it
holds none of the method's arithmetic (no compression, scoring, selection,
attention or number-format conversion).  Values are drawn in float32; each
consumer converts them to its storage format with its own codec.

Every tensor has its own substream, keyed by
SeedSequence([2026, workload, tensor, layer, request]), so any tensor (or one
request's part of it) can be regenerated alone and requests can be reordered.
"""
from dataclasses import dataclass, field

import numpy as np

ROOT_SEED = 2026

# tensor ids of the substreams
X, Z, BIAS, Q, QI, KI, CACHE, SWA, HEADW, LEN, HIST = range(1, 12)


def rng(workload, tensor, layer=0, request=0):
    return np.random.default_rng(
        np.random.SeedSequence([ROOT_SEED, workload, tensor, layer, request]))


def normal(workload, tensor, shape, std=1.0, layer=0, request=0):
    """float32 draws ~ N(0, std^2)."""
    g = rng(workload, tensor, layer, request)
    out = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


INDEXER_STD = 0.125          # N(0, 1/64): variance 1/64


@dataclass
class Workload:
    """Shapes and parameters of one synthetic workload."""
    wid: int
    name: str
    kind: str                 # 'csa_prefill' | 'hca_prefill' | 'csa_decode' | 'mixed_decode'
    heads: int
    dim: int
    m: int = 4
    w: int = 8
    k: int = 0
    window: int = 128
    idx_heads: int = 4
    idx_dim: int = 64
    seq: int = 0              # prefill: query tokens
    pos0: int = 0             # prefill: position of the first query token
    cached: int = 0           # prefill: entries already in the cache
    batch: int = 0            # decode: requests
    ctx: int = 0              # decode: context length L (query at t = L)
    kv_fmt: str = "f32"       # 'f32' | 'bf16' | 'fp8_mixed'
    act_fmt: str = "f32"      # raw rows / queries: 'f32' | 'bf16'
    idx_fmt: str = "f32"      # indexer operands: 'f32' | 'bf16' | 'mxfp4'
    score_fmt: str = "f32"    # 'f32' | 'bf16'
    out_fmt: str = "f32"
    layers: list = field(default_factory=list)   # mixed decode: [('csa', m, k) | ('hca', m, 0)]


WORKLOADS = {
    1: Workload(1, "csa_prefill_f32_s4096", "csa_prefill", heads=16, dim=128, m=4, w=8,
                k=64, seq=4096, kv_fmt="f32", act_fmt="f32", idx_fmt="f32",
                score_fmt="f32", out_fmt="f32"),
    2: Workload(2, "hca_prefill_bf16_s65536", "hca_prefill", heads=64, dim=128, m=128,
                w=256, seq=65536, kv_fmt="bf16", act_fmt="bf16", out_fmt="bf16"),
    3: Workload(3, "csa_decode_b32_ctx131072", "csa_decode", heads=64, dim=512, m=4, k=512,
                batch=32, ctx=131072, kv_fmt="fp8_mixed", act_fmt="bf16", idx_fmt="bf16",
                score_fmt="bf16", out_fmt="bf16"),
    4: Workload(4, "csa_chunk_prefill_s8192_at_1M", "csa_prefill", heads=128, dim=512, m=4,
                w=8, k=1024, seq=8192, pos0=2 ** 20, cached=262144, kv_fmt="fp8_mixed",
                act_fmt="bf16", idx_fmt="mxfp4", score_fmt="bf16", out_fmt="bf16"),
    5: Workload(5, "mixed_decode_4layer_b64_4K_1M", "mixed_decode", heads=64, dim=512,
                batch=64, kv_fmt="fp8_mixed", act_fmt="bf16", idx_fmt="mxfp4",
                score_fmt="bf16", out_fmt="bf16",
                layers=[("csa", 4, 1024), ("hca", 128, 0), ("csa", 4, 1024), ("hca", 128, 0)]),
}


def mixed_decode_lengths(wid=5, batch=64):
    """Per-request context lengths, log-uniform over [4096, 4096*256)."""
    u = rng(wid, LEN).random(batch)
    return np.floor(4096.0 * 256.0 ** u).astype(np.int64)


# ------------------------------------------------------------------ prefill

def prefill_inputs(wl, seq=None, pos0=None, cached=None, layer=0):
    """Inputs of a prefill workload (optionally at a reduced size).

    Returns a dict of float32 arrays:
      raw   [n_raw, D]  raw KV rows, positions raw_pos0 .. (history + chunk)
      z     [n_raw]     compression logits of those rows
      bias  [w]         slot position biases
      q     [seq, H, D] attention queries
      qi    [seq, H_I, d_I] indexer queries (CSA)
      ki    [n_entries, d_I] indexer keys of every entry (CSA)
      cache [cached, D] values of the entries already compressed (chunked prefill)
    plus integer metadata."""
    seq = wl.seq if seq is None else seq
    pos0 = wl.pos0 if pos0 is None else pos0
    cached = wl.cached if cached is None else cached
    hist = min(pos0, max(wl.window, wl.w - wl.m))   # raw rows before the chunk
    n_raw = hist + seq
    d, h = wl.dim, wl.heads
    out = {
        "raw": normal(wl.wid, X, (n_raw, d), layer=layer),
        "z": normal(wl.wid, Z, (n_raw,), layer=layer),
        "bias": normal(wl.wid, BIAS, (wl.w,), layer=layer),
        "q": normal(wl.wid, Q, (seq, h, d), layer=layer),
        "raw_pos0": pos0 - hist, "pos0": pos0, "seq": seq,
    }
    n_entries = (pos0 + seq) // wl.m
    out["n_entries"] = n_entries
    out["first_new_entry"] = pos0 // wl.m
    if wl.kind == "csa_prefill":
        out["qi"] = normal(wl.wid, QI, (seq, wl.idx_heads, wl.idx_dim), INDEXER_STD, layer)
        out["ki"] = normal(wl.wid, KI, (n_entries, wl.idx_dim), INDEXER_STD, layer)
    if pos0 > 0:
        assert cached == pos0 // wl.m
        out["cache"] = normal(wl.wid, CACHE, (cached, d), layer=layer)
    return out


# ------------------------------------------------------------------ decode

def decode_request(wl, r, ctx, m, csa, layer=0):
    """Inputs of request r of a decode workload at context ctx (query at t = ctx).

    cache [n_c, D] entry values (n_c = floor((ctx+1)/m)), swa [W, D] raw rows of
    positions ctx-W+1 .. ctx, q [H, D]; CSA layers add qi [H_I, d_I] and
    ki [n_c, d_I]."""
    n_c = (ctx + 1) // m
    d = wl.dim
    n_swa = min(wl.window, ctx + 1)
    out = {
        "cache": normal(wl.wid, CACHE, (n_c, d), layer=layer, request=r),
        "swa": normal(wl.wid, SWA, (n_swa, d), layer=layer, request=r),
        "q": normal(wl.wid, Q, (wl.heads, d), layer=layer, request=r),
        "t": ctx, "n_c": n_c, "swa_pos0": ctx - n_swa + 1,
    }
    if csa:
        out["qi"] = normal(wl.wid, QI, (wl.idx_heads, wl.idx_dim), INDEXER_STD, layer, r)
        out["ki"] = normal(wl.wid, KI, (n_c, wl.idx_dim), INDEXER_STD, layer, r)
    return out


def decode_contexts(wl, batch=None):
    batch = wl.batch if batch is None else batch
    if wl.kind == "mixed_decode":
        return mixed_decode_lengths(wl.wid, batch)
    return np.full(batch, wl.ctx, dtype=np.int64)
