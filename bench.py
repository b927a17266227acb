#!/usr/bin/env python3
"""Throughput of the CSA/HCA compressed-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N]

A step is one pass of a layer's whole path over one batch of synthetic
inputs already resident in HBM:
  1  CSA prefill, fp32, 4096 tokens:   compress -> indexer -> top-k -> attention
  2  HCA prefill, bf16, 65536 tokens:  compress -> dense attention
  3  CSA decode, 32 x 128K context:    indexer -> top-k -> attention -> merge
  4  CSA chunked prefill, 8192 tokens at 1M context (default): compress ->
                                       MXFP4 indexer + top-k -> attention
  5  4-layer C/H/C/H decode, 64 requests, 4K-1M contexts
Prints one JSON line: throughput, the roofline (for a CSA prefill the
indexer and the attention together: the sum over both of their algorithmic
flops over the peak of their own dtype, divided by their measured time), and
the CPU oracle timed on a bounded sample of the same workload on the host's
cores.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from long_context_compressed_kv_amd import ops  # noqa: E402
from long_context_compressed_kv_amd.ops import BF16, F32, FP8_MIXED, KV, MXFP4  # noqa: E402
from long_context_compressed_kv_amd.pipeline import DecodeLayer, PrefillLayer  # noqa: E402

PEAK = {"hbm": 8000.0, "bf16": 2500.0, "f32": 157.3, "fp4": 10100.0}   # GB/s, TFLOP/s
FMT = {"f32": F32, "bf16": BF16, "fp8_mixed": FP8_MIXED, "mxfp4": MXFP4}
ENTRY_BYTES = {"fp8_mixed": 580, "bf16": 1024, "f32": 2048}
IDX_KEY_BYTES = {"mxfp4": 34, "bf16": 128, "f32": 256}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def src_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_compressed_kv_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ inputs on the GPU


class Gen:
    """Seeded synthetic draws made directly on the device (plumbing)."""

    def __init__(self, seed):
        self.g = torch.Generator(device="cuda")
        self.g.manual_seed(seed)

    def normal(self, shape, std=1.0):
        t = torch.randn(shape, generator=self.g, device="cuda", dtype=torch.float32)
        return t.mul_(std) if std != 1.0 else t

    def kv(self, rows, dim, fmt, std=1.0, chunk=1 << 20):
        """rows x dim draws stored in `fmt` (quantised by the library)."""
        if fmt == "f32":
            return KV(F32, dim, self.normal((rows, dim), std))
        if fmt == "bf16":
            return KV(BF16, dim, self.normal((rows, dim), std).to(torch.bfloat16))
        out = KV.empty(FMT[fmt], rows, dim)
        for r0 in range(0, rows, chunk):
            n = min(chunk, rows - r0)
            ops.quantize(KV(F32, dim, self.normal((n, dim), std)), out.narrow(r0, n))
        return out


# ------------------------------------------------------------------ workloads


def attn_pairs_prefill(pos0, T, m, n_ent, window, k=None):
    """Sum over queries of (attended entries + window tokens)."""
    t = np.arange(pos0, pos0 + T, dtype=np.int64)
    nv = np.minimum((t + 1) // m, n_ent)
    ent = np.minimum(nv, k) if k is not None else nv
    win = np.minimum(window, t + 1)
    return int(ent.sum() + win.sum()), int(nv.sum())


class Prefill:
    def __init__(self, wid, copies=1, fp8_q=False):
        self.wl = wl = synth.WORKLOADS[wid]
        gen = Gen(1000 + wid)
        D, H, T = wl.dim, wl.heads, wl.seq
        csa = wl.kind == "csa_prefill"
        hist = min(wl.pos0, max(wl.window, wl.w - wl.m))
        raw_pos0 = wl.pos0 - hist
        n_ent = (wl.pos0 + T) // wl.m
        cache = gen.kv(n_ent, D, wl.kv_fmt)          # rows before pos0/m act as the cached prefix
        raw = gen.kv(hist + T, D, wl.act_fmt)
        z, bias = gen.normal((hist + T,)), gen.normal((wl.w,))
        # (fp8 queries: stored like KV entries, the variant's NoPE logits on
        # the fp8 matrix cores)
        q = gen.kv(T * H, D, "fp8_mixed" if fp8_q else wl.act_fmt)
        qi = gen.kv(T * 4, 64, wl.idx_fmt, synth.INDEXER_STD) if csa else None
        ki = gen.kv(n_ent, 64, wl.idx_fmt, synth.INDEXER_STD) if csa else None
        self.layer = PrefillLayer(csa=csa, H=H, m=wl.m, w=wl.w, k=wl.k, window=wl.window,
                                  raw=raw, z=z, bias=bias, raw_pos0=raw_pos0, pos0=wl.pos0, T=T,
                                  cache=cache, n_cached=wl.pos0 // wl.m, q=q, qi=qi, ki=ki,
                                  score_fmt=FMT[wl.score_fmt], out_fmt=FMT[wl.out_fmt])
        self.tokens = T
        self.csa = csa
        pairs, nv_sum = attn_pairs_prefill(wl.pos0, T, wl.m, n_ent, wl.window,
                                           wl.k if csa else None)
        self.attn_flops = 4.0 * D * H * pairs
        self.idx_flops = 2.0 * 4 * 64 * nv_sum if csa else 0.0
        cdt = "f32" if wl.act_fmt == "f32" else "bf16"
        idt = {"mxfp4": "fp4", "bf16": "bf16", "f32": "f32"}[wl.idx_fmt]
        attn = {"name": "attention", "work": self.attn_flops, "peak": PEAK[cdt], "dtype": cdt,
                "per_unit": f"4*D*H = {4 * D * H} flop per (query, key) pair; {pairs} pairs "
                            f"per launch",
                "sha": src_sha("attn.hip", "attn512.hip", "attn_common.h", "common.h")}
        idx = {"name": "indexer_topk", "work": self.idx_flops, "peak": PEAK[idt], "dtype": idt,
               "per_unit": f"2*4*64 = 512 flop per (query, visible entry) pair; {nv_sum} pairs "
                           f"per launch",
               "sha": src_sha("itk.hip", "indexer_core.h", "select_core.h", "common.h")}
        # the roofline covers the indexer (with its top-k) and the attention of a
        # CSA layer, the attention alone for HCA
        self.parts = [idx, attn] if csa else [attn]
        self.dominant = {"name": "+".join(p["name"] for p in self.parts), "bound": "mfma",
                         "unit": "TFLOP/s"}

    def step(self, ev=None):
        """ev: None, or three events recorded before the selection, between
        selection and attention, and after the attention."""
        L = self.layer
        L.compress()
        idx = None
        if ev is not None:
            ev[0].record()
        if self.csa:
            _, idx = L.select()
        if ev is not None:
            ev[1].record()
        L.attend(idx)
        if ev is not None:
            ev[2].record()


class Decode:
    """One decode step over one or more layers; `copies` input sets rotated so
    successive steps do not find their data in the last-level cache."""

    def __init__(self, wid, copies=3, paged=False, fp8_q=False):
        self.wl = wl = synth.WORKLOADS[wid]
        gen = Gen(2000 + wid)
        perm_gen = torch.Generator().manual_seed(3000 + wid)
        ctxs = [int(c) for c in synth.decode_contexts(wl)]
        B, D, H = len(ctxs), wl.dim, wl.heads
        specs = wl.layers if wl.kind == "mixed_decode" else [("csa", wl.m, wl.k)]
        self.copies = []
        self.bytes_idx = 0.0
        self.bytes_step = 0.0
        for c in range(copies):
            layers = []
            for kind, m, k in specs:
                csa = kind == "csa"
                n_ent = [(t + 1) // m for t in ctxs]
                swa_len = [min(wl.window, t + 1) for t in ctxs]
                rows, table, P = sum(n_ent), None, 0
                if paged:
                    # blocks of 128 raw tokens (128 / m entries), handed out in a
                    # shuffled order
                    P = 128 // m
                    nb = [(n + P - 1) // P for n in n_ent]
                    ids = torch.randperm(sum(nb), generator=perm_gen).to(torch.int32)
                    table = torch.full((B, max(nb)), -1, dtype=torch.int32)
                    s0 = 0
                    for r, n in enumerate(nb):
                        table[r, :n] = ids[s0:s0 + n]
                        s0 += n
                    table, rows = table.cuda(), sum(nb) * P
                cache = gen.kv(rows, D, wl.kv_fmt)
                swa = gen.kv(sum(swa_len), D, "bf16")
                q = gen.kv(B * H, D, "fp8_mixed" if fp8_q else "bf16")
                qi = gen.kv(B * 4, 64, wl.idx_fmt, synth.INDEXER_STD) if csa else None
                ki = gen.kv(rows, 64, wl.idx_fmt, synth.INDEXER_STD) if csa else None
                layers.append(DecodeLayer(csa=csa, H=H, m=m, k=k, window=wl.window, ctx=ctxs,
                                          n_entries=n_ent, swa_len=swa_len, cache=cache,
                                          swa=swa, q=q, qi=qi, ki=ki,
                                          score_fmt=FMT[wl.score_fmt], out_fmt=FMT[wl.out_fmt],
                                          kv_block_table=table, kv_block_rows=P))
                if c == 0:
                    nsum = sum(n_ent)
                    kb = IDX_KEY_BYTES[wl.idx_fmt]
                    if csa:
                        # indexer keys and queries read, selected indices written
                        self.bytes_idx += nsum * kb + B * 4 * kb + B * k * 4
                        sel = sum(min(k, n) for n in n_ent)
                    else:
                        sel = nsum
                    # index keys + entries read + window rows + q in + out
                    self.bytes_step += (nsum * kb if csa else 0) + \
                        sel * ENTRY_BYTES[wl.kv_fmt] + sum(swa_len) * D * 2 + 2 * B * H * D * 2
            self.copies.append(layers)
        self.tokens = B
        self.has_csa = any(s[0] == "csa" for s in specs)
        self.dominant = {"name": "indexer_topk", "bound": "hbm", "unit": "GB/s",
                         "work": self.bytes_idx, "peak": PEAK["hbm"],
                         "per_unit": f"{IDX_KEY_BYTES[wl.idx_fmt]} B key per (request, visible "
                                     f"entry), plus 4 B per selected index",
                         "sha": src_sha("itk.hip", "indexer_core.h", "select_core.h",
                                        "common.h")}
        self.graphs = None

    def step_copy(self, c):
        for L in self.copies[c]:
            L.run()

    def dominant_copy(self, c):
        for L in self.copies[c]:
            if L.csa:
                L.select()

    def capture(self):
        """One graph per input copy for the whole step, and one per copy for
        the dominant kernel alone."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        self.g_step, self.g_dom = [], []
        with torch.cuda.stream(s):
            for c in range(len(self.copies)):
                self.step_copy(c)          # allocate buffers outside capture
            torch.cuda.synchronize()
            for c in range(len(self.copies)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    self.step_copy(c)
                self.g_step.append(g)
                g2 = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g2, stream=s):
                    self.dominant_copy(c)
                self.g_dom.append(g2)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()


# ------------------------------------------------------------------ CPU baseline


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_CPU = {}       # inputs shared with the forked workers


def _cpu_prefill_worker(args):
    """Queries i0, i0 + stride, ... of the prefill sample until the deadline;
    returns how many were done."""
    from threadpoolctl import threadpool_limits
    from oracle import codecs
    from oracle import csa as ref
    i0, stride, deadline = args
    c = _CPU
    wl, inp, vals, newv, e0, n_ent = c["wl"], c["inp"], c["vals"], c["newv"], c["e0"], c["n_ent"]
    rawv, ki = c["rawv"], c.get("ki")
    done = 0
    with threadpool_limits(limits=1):
        for i in range(i0, inp["seq"], stride):
            if time.time() > deadline:
                break
            t = inp["pos0"] + i
            q = vals[wl.act_fmt](inp["q"][i])
            if wl.kind == "hca_prefill":
                ref.hca_query(t, q, newv, wl.m, rawv, inp["raw_pos0"], wl.window)
            elif e0 == 0:
                ref.csa_query(t, q, newv, vals[wl.idx_fmt](inp["qi"][i]), ki, wl.k, wl.m, rawv,
                              inp["raw_pos0"], wl.window, score_fmt=wl.score_fmt)
            else:
                # selection first, then only the selected cached rows are decoded
                nv = min((t + 1) // wl.m, n_ent)
                keys = ref.score_keys(ref.indexer_scores(vals[wl.idx_fmt](inp["qi"][i]),
                                                         ki[:nv]), wl.score_fmt)
                idx = ref.topk_indices(keys, wl.k)
                sel = idx[idx >= 0]
                old = sel[sel < e0]
                ent = np.concatenate([
                    ref.load_entries(ref.store_entries(inp["cache"][old], wl.kv_fmt), wl.kv_fmt),
                    newv[sel[sel >= e0] - e0]])
                pos = ref.window_positions(t, wl.window)
                ref.attend(q, np.concatenate([ent, rawv[pos - inp["raw_pos0"]]]),
                           1.0 / math.sqrt(wl.dim))
            done += 1
    return done


def _cpu_decode_worker(args):
    """Requests r0, r0 + stride, ...: each request's inputs are drawn (not
    timed), then the oracle runs it through every layer `runs` times (each
    timed); stops once the worker's compute time of one run passes the budget
    or its wall time passes the cap.  Returns (requests done, [compute seconds
    of run j])."""
    from threadpoolctl import threadpool_limits
    from oracle import codecs
    from oracle import csa as ref
    r0, stride, budget, cap, runs = args
    wl, ctxs, specs = _CPU["wl"], _CPU["ctxs"], _CPU["specs"]
    start = time.time()
    done, secs = 0, [0.0] * runs
    with threadpool_limits(limits=1):
        for r in range(r0, len(ctxs), stride):
            if secs[0] > budget or time.time() - start > cap:
                break
            layers = [synth.decode_request(wl, r, int(ctxs[r]), m, kind == "csa", layer=li)
                      for li, (kind, m, k) in enumerate(specs)]
            for j in range(runs):
                t0 = time.perf_counter()
                for (kind, m, k), d in zip(specs, layers):
                    cv = codecs.dequantize_kv_mixed(*codecs.quantize_kv_mixed(d["cache"]))
                    q = codecs.bf16_round(d["q"]).astype(np.float64)
                    sw = codecs.bf16_round(d["swa"]).astype(np.float64)
                    if kind == "csa":
                        qf = (lambda a: codecs.dequantize_mxfp4(*codecs.quantize_mxfp4(a))) \
                            if wl.idx_fmt == "mxfp4" else \
                            (lambda a: codecs.bf16_round(a).astype(np.float64))
                        ref.csa_query(d["t"], q, cv, qf(d["qi"]), qf(d["ki"]), k, m, sw,
                                      d["swa_pos0"], wl.window, score_fmt=wl.score_fmt)
                    else:
                        ref.hca_query(d["t"], q, cv, m, sw, d["swa_pos0"], wl.window)
                secs[j] += time.perf_counter() - t0
            done += 1
    return done, secs


def cpu_baseline(wid, budget_s=8.0, runs=3, max_workers=16):
    """The oracle as it stands on a bounded sample of the workload, on the
    host's cores: one forked worker per core (at most max_workers, the CPU
    share of one GPU), each with a single BLAS thread, takes an interleaved
    share of the sample's queries (prefill) or requests (decode) until a
    deadline of budget_s seconds.  Three such runs; the median rate is
    reported.  Input draws and the compression of the chunk's new entries are
    done once, before the timed runs, and are not counted."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import codecs
    from oracle import csa as ref
    wl = synth.WORKLOADS[wid]
    ncpu = os.cpu_count() or 1
    workers = max(1, min(ncpu, max_workers))
    t0 = time.perf_counter()
    prefill = wl.kind in ("csa_prefill", "hca_prefill")
    _CPU.clear()
    _CPU["wl"] = wl
    if prefill:
        # the whole chunk's queries; as many as the deadline allows are the sample
        seq = wl.seq
        inp = synth.prefill_inputs(wl, seq=seq)
        vals = {"f32": lambda a: a.astype(np.float64),
                "bf16": lambda a: codecs.bf16_round(a).astype(np.float64),
                "mxfp4": lambda a: codecs.dequantize_mxfp4(*codecs.quantize_mxfp4(a))}
        rawv = vals[wl.act_fmt](inp["raw"])
        e0, n_ent = inp["first_new_entry"], inp["n_entries"]
        with threadpool_limits(limits=workers):
            new = ref.compress_entries(rawv, inp["z"], inp["raw_pos0"], inp["bias"], wl.m,
                                       wl.w, e0, n_ent)
            newv = ref.load_entries(ref.store_entries(new, wl.kv_fmt), wl.kv_fmt)
        _CPU.update(inp=inp, vals=vals, rawv=rawv, e0=e0, n_ent=n_ent, newv=newv)
        if wl.kind == "csa_prefill":
            _CPU["ki"] = vals[wl.idx_fmt](inp["ki"])
        fn, total = _cpu_prefill_worker, inp["seq"]
        what = "query tokens (all heads)"
    else:
        _CPU["ctxs"] = synth.decode_contexts(wl)
        _CPU["specs"] = wl.layers if wl.kind == "mixed_decode" else [("csa", wl.m, wl.k)]
        fn, total = _cpu_decode_worker, len(_CPU["ctxs"])
        what = f"requests through all {len(_CPU['specs'])} layers (the cache " \
               f"quantisation included, the input draws not)"
    t_prep = time.perf_counter() - t0
    rates, dones = [], []
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        if prefill:
            for _ in range(runs):
                start = time.time()
                counts = pool.map(fn, [(i, workers, start + budget_s) for i in range(workers)])
                el = time.time() - start
                rates.append(sum(counts) / el)
                dones.append(sum(counts))
        else:
            # every request run `runs` times back to back after its draws; run j's
            # rate is the requests done over the longest worker's compute time
            res = pool.map(fn, [(i, workers, budget_s, 4 * budget_s, runs)
                                for i in range(workers)])
            n = sum(d for d, _ in res)
            for j in range(runs):
                rates.append(n / max(max(sec[j] for _, sec in res), 1e-9))
                dones.append(n)
    _CPU.clear()
    med = sorted(rates)[len(rates) // 2]
    blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")}
            for i in threadpool_info()]
    sample = f"up to {dones} of the first {total} {what}, in {runs} runs of about " \
             f"{budget_s:.0f} s on {workers} worker processes (one BLAS thread each)"
    if prefill and wl.pos0 > 0:
        sample += f"; the chunk's first {total} of {wl.seq} tokens"
    return {"value": round(med, 3), "unit": "tokens/s" if prefill else "requests/s",
            "cores": workers, "kind": "oracle", "sample": sample,
            "runs": [round(r, 3) for r in rates], "host_cpus": ncpu, "cpu_model": _cpu_model(),
            "blas_threads_per_worker": 1, "blas_libraries": blas,
            "prep_seconds": round(t_prep, 1)}


# ------------------------------------------------------------------ main


def traffic_for(dom, wid):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on this kernel source and workload; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(str(wid))
    except (ValueError, OSError):
        return None
    if isinstance(rec, dict) and dom["name"] in rec:
        rec = rec[dom["name"]]
    if not rec or rec.get("sha") != dom["sha"]:
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------- score precision study


def score_study():
    """How much the indexer's reduced precision changes the top-k set, and how
    much faster selection over bf16 scores is than over fp32 scores.

    Decode-shaped synthetic rows (every entry visible, one query per request):
    the reference set is the top-k of fp32 scores of fp32 operands; the
    others round the operands to bf16 or MXFP4 and/or the scores to bf16.
    Recall = |set & reference| / k per row, averaged.  Times are HIP-event
    means over repeated launches of the unfused selection (over a stored score
    matrix) and of the fused indexer + top-k."""
    m = 4
    cases = [("decode_b32_ctx131072_k512", 32, 32768, 512),
             ("decode_b16_ctx1M_k1024", 16, 262144, 1024)]
    gen = Gen(20262)
    out = []

    def timed(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for name, n_q, n_ent, k in cases:
        batch = ops.Batch.make([1] * n_q, [n_ent * m - 1] * n_q, kv_counts=[n_ent] * n_q)
        qi32 = KV(F32, 64, gen.normal((n_q * 4, 64), 0.125))
        ki32 = KV(F32, 64, gen.normal((n_q * n_ent, 64), 0.125))
        qib = KV(BF16, 64, qi32.data.to(torch.bfloat16))
        kib = KV(BF16, 64, ki32.data.to(torch.bfloat16))
        qi4, ki4 = KV.empty(MXFP4, n_q * 4, 64), KV.empty(MXFP4, n_q * n_ent, 64)
        ops.quantize(qi32, qi4)
        ops.quantize(ki32, ki4)
        sets = {
            "f32_operands_f32_scores": (qi32, ki32, F32),
            "f32_operands_bf16_scores": (qi32, ki32, BF16),
            "bf16_operands_f32_scores": (qib, kib, F32),
            "bf16_operands_bf16_scores": (qib, kib, BF16),
            "mxfp4_operands_bf16_scores": (qi4, ki4, BF16),
        }
        idx = {key: ops.indexer_topk(q, 4, kk, batch, m, sf, k).cpu().numpy()
               for key, (q, kk, sf) in sets.items()}
        ref = idx["f32_operands_f32_scores"]
        recall = {}
        for key, got in idx.items():
            if key == "f32_operands_f32_scores":
                continue
            r = [len(np.intersect1d(got[i], ref[i])) / k for i in range(n_q)]
            recall[key] = round(float(np.mean(r)), 5)
        s32 = torch.empty(n_q, n_ent, device="cuda", dtype=torch.float32)
        s16 = torch.empty(n_q, n_ent, device="cuda", dtype=torch.bfloat16)
        ops.indexer_score(qib, 4, kib, batch, m, s32, F32)
        ops.indexer_score(qib, 4, kib, batch, m, s16, BF16)
        sel32 = timed(lambda: ops.topk_select(s32, F32, batch, m, k))
        sel16 = timed(lambda: ops.topk_select(s16, BF16, batch, m, k))
        fus32 = timed(lambda: ops.indexer_topk(qib, 4, kib, batch, m, F32, k))
        fus16 = timed(lambda: ops.indexer_topk(qib, 4, kib, batch, m, BF16, k))
        log(f"{name}: recall {recall}; select f32 {sel32:.4f} ms, bf16 {sel16:.4f} ms; "
            f"fused f32 {fus32:.4f} ms, bf16 {fus16:.4f} ms")
        out.append({"workload": name, "requests": n_q, "entries": n_ent, "k": k,
                    "recall_vs_f32": recall,
                    "select_ms": {"f32_scores": round(sel32, 5), "bf16_scores": round(sel16, 5),
                                  "speedup": round(sel32 / sel16, 3)},
                    "fused_indexer_topk_ms": {"f32_scores": round(fus32, 5),
                                              "bf16_scores": round(fus16, 5),
                                              "speedup": round(fus32 / fus16, 3)}})
    print(json.dumps({"study": "indexer score precision (bf16 / MXFP4 vs fp32)",
                      "data": "synthetic, N(0, 1/64) queries and keys", "cases": out}), flush=True)


# ------------------------------------------------- projections around the path

# Sizes of the projections (the pages give none): model width 7168, a
# low-rank query side of rank 1536 into every head's 512-dim entry space, the
# KV row (512) and the indexer's key (64) from the token, the indexer's
# queries (4 x 64) from the query rank, and the grouped output projection:
# 8 groups of heads, 1024 values each, then back to the model width.
PROJ = {"d_model": 7168, "q_rank": 1536, "groups": 8, "d_group": 1024}


def proj_bench(reps=10):
    """csa_linear and csa_grouped_out_proj at the chunked prefill's shapes
    (8192 tokens, 128 heads) and the 4-layer decode's (64 requests, 64
    heads); flop = 2 M N K per product.  torch.matmul (hipBLASLt) on the same
    bf16 operands is timed beside each plain product for reference."""
    gen = Gen(20264)
    dm, rq, G, dg = PROJ["d_model"], PROJ["q_rank"], PROJ["groups"], PROJ["d_group"]

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    cases = []
    for wl, M, H in (("csa_chunk_prefill_s8192_at_1M", 8192, 128), ("mixed_decode_4layer_b64_4K_1M", 64, 64)):
        D = 512
        prods = [("q_down", M, rq, dm), ("q_up", M, H * D, rq), ("kv", M, D, dm),
                 ("indexer_q", M, 4 * 64, rq), ("indexer_k", M, 64, dm)]
        tot_ms = tot_fl = 0.0
        for name, m_, n_, k_ in prods:
            x = gen.normal((m_, k_)).to(torch.bfloat16)
            w = (0.02 * gen.normal((n_, k_))).to(torch.bfloat16)
            y = torch.empty(m_, n_, dtype=torch.bfloat16, device="cuda")
            ms = timed(lambda: ops.linear(x, w, y))
            ref = timed(lambda: torch.matmul(x, w.t()))
            fl = 2.0 * m_ * n_ * k_
            tot_ms += ms
            tot_fl += fl
            cases.append({"workload": wl, "product": name, "M": m_, "N": n_, "K": k_, "us": round(ms * 1e3, 2),
                          "tflops": round(fl / ms / 1e9, 1), "mfma_frac": round(fl / ms / 1e9 / PEAK["bf16"], 4),
                          "weight_gbs": round(n_ * k_ * 2 / ms / 1e6, 1), "torch_matmul_us": round(ref * 1e3, 2)})
            log(f"proj {wl} {name} {m_}x{n_}x{k_}: {ms * 1e3:.1f} us, {fl / ms / 1e9:.1f} TFLOP/s "
                f"(torch.matmul {ref * 1e3:.1f} us)")
            del x, w, y
        o = gen.normal((M, H, D)).to(torch.bfloat16)
        wg = (0.02 * gen.normal((G, dg, (H // G) * D))).to(torch.bfloat16)
        wo = (0.02 * gen.normal((dm, G * dg))).to(torch.bfloat16)
        y = torch.empty(M, dm, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(ops.grouped_out_proj_workspace_size(M, G, dg), dtype=torch.uint8, device="cuda")
        ms = timed(lambda: ops.grouped_out_proj(o, H, wg, wo, y, ws))
        fl = 2.0 * M * (H * D * dg + G * dg * dm)
        tot_ms += ms
        tot_fl += fl
        cases.append({"workload": wl, "product": "grouped_out", "M": M, "heads": H, "us": round(ms * 1e3, 2),
                      "tflops": round(fl / ms / 1e9, 1), "mfma_frac": round(fl / ms / 1e9 / PEAK["bf16"], 4)})
        log(f"proj {wl} grouped output: {ms * 1e3:.1f} us, {fl / ms / 1e9:.1f} TFLOP/s")
        cases.append({"workload": wl, "product": "all", "us": round(tot_ms * 1e3, 2),
                      "tflops": round(tot_fl / tot_ms / 1e9, 1)})
    print(json.dumps({"measure": "projections around the path (csa_linear, csa_grouped_out_proj)",
                      "sizes": PROJ, "data": "synthetic, random weights", "cases": cases}), flush=True)


# ------------------------------------------------- decode-time compression


def append_bench(reps=200):
    """One csa_kv_compress_append call per decode step and layer: 64 requests
    at spread positions append a 512-dim bf16 token; entries go to a mixed
    cache, the raw row to a 128-row window ring.  Algorithmic bytes per
    request and call: the token (1024 B) and its logit / position / offset,
    the two open entries read and written ((512 + 4) * 4 B each way), the
    window row (1024 B), plus one 580-byte entry every m calls."""
    n_req, D, C = 64, 512, 128
    gen = Gen(20263)
    out = []
    for name, m, w in (("csa_m4_w8", 4, 8), ("hca_m128_w256", 128, 256)):
        pos0 = torch.randint(4 * w, 1 << 16, (n_req,), generator=gen.g, device="cuda")
        x = KV(BF16, D, gen.normal((reps + 2 * w, n_req, D)).to(torch.bfloat16).reshape(-1, D))
        z = gen.normal((reps + 2 * w, n_req))
        b = gen.normal((w,))
        n_ent = (pos0.max().item() + reps + 2 * w) // m + 1
        cache = KV.empty(FP8_MIXED, n_req * n_ent, D)
        e_off = torch.arange(n_req, dtype=torch.int64, device="cuda") * n_ent
        win = KV(BF16, D, torch.zeros(n_req * C, D, dtype=torch.bfloat16, device="cuda"))
        w_off = torch.arange(n_req, dtype=torch.int64, device="cuda") * C
        state = torch.zeros(ops.kv_append_state_size(n_req, D) // 4, device="cuda")
        pos = torch.stack([pos0 + i for i in range(reps + 2 * w)])
        # the first 2w calls open every request's entries (warm-up, untimed)
        call = lambda i: ops.kv_compress_append(x.narrow(i * n_req, n_req), z[i], b, m, w, pos[i],
                                                state, e_off, cache, win, w_off, C)
        for i in range(2 * w):
            call(i)
        torch.cuda.synchronize()
        # the timed calls as one captured graph, as a decode step would run them
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(2 * w, 2 * w + reps):
                    call(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        per_req = 1024 + 4 + 8 + 8 + 2 * 2 * (D + 4) * 4 + 1024 + 580.0 / m
        gbs = n_req * per_req / (us * 1e-6) / 1e9
        log(f"append {name}: {us:.2f} us per call, {gbs:.1f} GB/s algorithmic")
        out.append({"workload": f"decode_append_b{n_req}_{name}_d512_mixed", "us_per_call": round(us, 3),
                    "bytes_per_call": int(n_req * per_req), "achieved_gbs": round(gbs, 2),
                    "hbm_frac": round(gbs / PEAK["hbm"], 5)})
    print(json.dumps({"measure": "decode-time compression (csa_kv_compress_append)",
                      "data": "synthetic", "cases": out}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (three "
                         "times): the reference for scaling HBM byte counters")
    ap.add_argument("--score-study", action="store_true",
                    help="instead of the benchmark: top-k recall and selection time with "
                         "bf16 / MXFP4 indexer precision against fp32")
    ap.add_argument("--fp8-q", action="store_true",
                    help="workloads with 512-dim mixed entries: queries stored like KV entries "
                         "(fp8 NoPE dims), the attention's NoPE logits on the fp8 matrix cores")
    ap.add_argument("--proj", action="store_true",
                    help="instead of the benchmark: time the projections around the path")
    ap.add_argument("--kv-append", action="store_true",
                    help="instead of the benchmark: time decode-time compression per call")
    ap.add_argument("--paged", action="store_true",
                    help="decode workloads: compressed entries and indexer keys in a paged "
                         "cache (blocks of 128 raw tokens in a shuffled order)")
    args = ap.parse_args()
    if args.proj:
        torch.cuda.init()
        proj_bench()
        return
    if args.kv_append:
        torch.cuda.init()
        append_bench()
        return
    if args.score_study:
        torch.cuda.init()
        score_study()
        return
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("this benchmark runs on one GPU only: the path has no multi-GPU part "
              "(requests shard across GPUs with no communication)", file=sys.stderr)
        sys.exit(2)
    wid = args.config
    wl = synth.WORKLOADS[wid]
    decode = wl.kind in ("csa_decode", "mixed_decode")
    if args.paged and not decode:
        print("--paged applies to the decode workloads", file=sys.stderr)
        sys.exit(2)
    torch.cuda.init()
    t0 = time.time()
    if args.fp8_q and (wl.dim != 512 or wl.kv_fmt != "fp8_mixed"):
        print("--fp8-q applies to the workloads with 512-dim mixed entries", file=sys.stderr)
        sys.exit(2)
    w = Decode(wid, paged=args.paged, fp8_q=args.fp8_q) if decode else Prefill(wid, fp8_q=args.fp8_q)
    torch.cuda.synchronize()
    log(f"workload {wl.name}: inputs ready in {time.time() - t0:.1f}s")

    dom = w.dominant
    if decode:
        w.capture()
        nc = len(w.copies)
        for i in range(args.warmup):
            w.g_step[i % nc].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            w.g_step[i % nc].replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        # dominant kernel alone, same rotation
        reps = max(args.steps, 30)
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record()
        for i in range(reps):
            w.g_dom[i % nc].replay()
        d1.record()
        torch.cuda.synchronize()
        n_launch = sum(1 for L in w.copies[0] if L.csa)
        dom_ms = d0.elapsed_time(d1) / reps / n_launch
        work = dom["work"] / n_launch
    else:
        for _ in range(args.warmup):
            w.step()
        torch.cuda.synchronize()
        # events on the stream the library launches on (torch's current one)
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
               for _ in range(args.steps)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            w.step(evs[i])
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        sel_ms = sum(a.elapsed_time(b) for a, b, _ in evs) / args.steps
        att_ms = sum(b.elapsed_time(c) for _, b, c in evs) / args.steps
        part_ms = {"indexer_topk": sel_ms, "attention": att_ms}
        dom_ms = sum(part_ms[p["name"]] for p in w.parts)
    log(f"step {ms:.4f} ms, dominant kernel ({dom['name']}) {dom_ms:.4f} ms per launch")

    value = w.tokens / (ms * 1e-3)
    if decode:
        achieved = work / (dom_ms * 1e-3) / 1e9
        roof = {"bound": dom["bound"], "achieved": round(achieved, 2), "peak": dom["peak"],
                "unit": dom["unit"], "frac": round(achieved / dom["peak"], 4),
                "traffic": traffic_for(dom, wid), "kernel": dom["name"],
                "work_per_launch": dom["per_unit"], "launch_ms": round(dom_ms, 5)}
    else:
        # sum over the parts of (work / own peak) = ideal time; frac = ideal / measured;
        # achieved and peak are the total work over the measured and the ideal time
        ideal_s = sum(p["work"] / (p["peak"] * 1e12) for p in w.parts)
        work = sum(p["work"] for p in w.parts)
        t_s = dom_ms * 1e-3
        kernels = []
        traffic = 0
        for p in w.parts:
            pm = part_ms[p["name"]]
            tb = traffic_for(p, wid)
            traffic = None if traffic is None or tb is None else traffic + tb
            kernels.append({"name": p["name"], "dtype": p["dtype"], "ms": round(pm, 5),
                            "achieved": round(p["work"] / (pm * 1e-3) / 1e12, 2),
                            "peak": p["peak"], "frac": round(p["work"] / (p["peak"] * 1e12) /
                                                             (pm * 1e-3), 4),
                            "work_per_launch": p["per_unit"], "traffic": tb})
        roof = {"bound": "mfma", "achieved": round(work / t_s / 1e12, 2),
                "peak": round(work / ideal_s / 1e12, 2), "unit": "TFLOP/s",
                "frac": round(ideal_s / t_s, 4), "traffic": traffic,
                "kernel": dom["name"], "launch_ms": round(dom_ms, 5),
                "peak_is": "the work-weighted mix of the parts' dtype peaks "
                           "(sum of work / sum of work over own peak)",
                "kernels": kernels}
    cpu = None
    if not args.no_cpu_baseline and not args.fp8_q:   # (the oracle leg times the bf16-query path)
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(wid)
    metric = "CSA/HCA layer tokens/s (prefill + decode) at 128K-1M ctx; % HBM/MFMA peak"
    line = {
        "metric": metric, "value": round(value, 2),
        "unit": "tokens/s" if not decode else "decode tokens/s (requests x steps)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {"f32": "f32"}.get(wl.act_fmt, "bf16"),
        "data": "synthetic", "roofline": roof, "cpu_baseline": cpu,
        "config": {"workload": wl.name, "tokens_per_step": w.tokens, "heads": wl.heads,
                   "dim": wl.dim, "parallelism": "single GPU"},
    }
    if decode:
        line["config"]["step_bytes_algorithmic"] = int(w.bytes_step)
        line["config"]["step_hbm_frac"] = round(w.bytes_step / (ms * 1e-3) / 8e12, 4)
        line["config"]["graph_replay"] = True
        if args.paged:
            line["config"]["kv_layout"] = "paged: blocks of 128 raw tokens, shuffled"
    if args.fp8_q:
        line["config"]["queries"] = "fp8: stored like KV entries, NoPE logits on the fp8 matrix cores"
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
