"""End-to-end parity at the five workload sizes, through the same layer
pipeline the benchmark times.  The oracle evaluates sampled queries (prefill)
or requests (decode) one by one from the same seeded float32 draws.

Checks per workload:
  - top-k: equal index sets, except entries whose exact score lies within
    the fp32 accumulation bound of the point where its rounding decides its
    side of the oracle's k-th key (or whose key ties with it), in few rows;
  - attention, stage-wise: the GPU attention re-run on the oracle's index sets
    matches the oracle within 1e-4 (fp32 compute) or 2e-2 (bf16 compute);
  - attention, end to end: rows whose index sets agree match within the same
    bound.
"""
import math
import sys
import time

import numpy as np
import pytest
import torch

import synth
from long_context_compressed_kv_amd import ops
from long_context_compressed_kv_amd.ops import BF16, F32, KV, Batch
from long_context_compressed_kv_amd.pipeline import DecodeLayer, PrefillLayer
from oracle import codecs
from oracle import csa as ref

from gpu_inputs import FMT, bf16_ulp, dev_f32, dev_kv, ref_vals, to_np

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def log(*a):
    print("[configs]", *a, flush=True)
    sys.stdout.flush()


# fp32 accumulation bound of one score: four 64-term dot products summed
# (each product exact), relative to the sum of the products' magnitudes
ACC_BOUND = 70 * 2.0 ** -24


def topk_ok(got, want, keys, score_fmt, s, qiv, kiv):
    """The GPU's index set equals the oracle's, or every entry in which they
    differ is explained by the fp32 accumulation order: its exact (fp64)
    score s lies within the accumulation bound of the point where the score's
    rounding decides its side of the k-th key tau (for bf16 keys the midpoints
    between tau and its bf16 neighbours; for fp32 keys tau itself), or its key
    equals tau (then the lowest-index rule among tied entries moves with the
    others).  qiv [4, 64], kiv [n, 64]: the oracle's operand values."""
    got = set(int(x) for x in got if x >= 0)
    want_s = set(int(x) for x in want if x >= 0)
    if got == want_s:
        return True
    if len(got) != len(want_s):
        return False
    tau = float(np.sort(keys)[::-1][len(want_s) - 1])
    aq = np.abs(np.asarray(qiv, np.float64)).sum(axis=0)
    if score_fmt == "bf16":
        one = lambda a: float(np.asarray(a, np.float64).reshape(-1)[0])
        up = one(codecs.bf16_round(np.array([np.nextafter(np.float32(tau), np.float32(np.inf)) +
                                             np.float32(one(bf16_ulp(tau)) / 2)], np.float32)))
        below = np.nextafter(np.float32(tau), np.float32(-np.inf)) if tau != 0 else 0.0
        points = [(tau + up) / 2, tau - one(bf16_ulp(below)) / 2]
    else:
        points = [tau]
    for j in got ^ want_s:
        if float(keys[j]) == tau:
            continue
        eps = ACC_BOUND * float(np.abs(np.asarray(kiv[j], np.float64)) @ aq) + abs(tau) * 2.0 ** -23
        if not any(abs(float(s[j]) - p) <= eps for p in points):
            return False
    return True


def max_mismatched_rows(n_rows):
    """Rows whose index set may differ from the oracle's (each difference also
    explained entry by entry by topk_ok)."""
    return max(2, math.ceil(0.1 * n_rows))


# ------------------------------------------------------------------ prefill


def _prefill_device(wl, inp):
    """Device tensors of a prefill workload built from the float32 draws."""
    D = wl.dim
    raw = dev_kv(inp["raw"], wl.act_fmt)
    n_ent = inp["n_entries"]
    cache = KV.empty(FMT[wl.kv_fmt], n_ent, D)
    if inp.get("cache") is not None:          # entries compressed before the chunk
        n_old = inp["cache"].shape[0]
        old = dev_kv(inp["cache"], "f32")
        if wl.kv_fmt == "f32":
            cache.data[:n_old].copy_(old.data)
        else:
            ops.quantize(old, cache.narrow(0, n_old))
        del old
    q = dev_kv(inp["q"].reshape(-1, D), wl.act_fmt)
    qi = ki = None
    if wl.kind == "csa_prefill":
        qi = dev_kv(inp["qi"].reshape(-1, wl.idx_dim), wl.idx_fmt)
        ki = dev_kv(inp["ki"], wl.idx_fmt)
    layer = PrefillLayer(csa=wl.kind == "csa_prefill", H=wl.heads, m=wl.m, w=wl.w, k=wl.k,
                         window=wl.window, raw=raw, z=dev_f32(inp["z"]),
                         bias=dev_f32(inp["bias"]), raw_pos0=inp["raw_pos0"], pos0=inp["pos0"],
                         T=inp["seq"], cache=cache, n_cached=inp["first_new_entry"], q=q, qi=qi,
                         ki=ki, score_fmt=FMT[wl.score_fmt], out_fmt=FMT[wl.out_fmt])
    return layer


def run_prefill(wid, seq=None, n_sample=48):
    wl = synth.WORKLOADS[wid]
    t0 = time.time()
    inp = synth.prefill_inputs(wl, seq=seq)
    log(f"workload {wid}: inputs drawn in {time.time() - t0:.1f}s")
    layer = _prefill_device(wl, inp)
    res = layer.run()
    torch.cuda.synchronize()
    log(f"workload {wid}: GPU pass done")
    T, H, D = inp["seq"], wl.heads, wl.dim
    rng = np.random.default_rng(wid)
    sample = np.unique(np.concatenate([np.arange(min(T, 8)), [T - 1],
                                       rng.choice(T, min(T, n_sample), replace=False)]))
    e0, n_ent = inp["first_new_entry"], inp["n_entries"]
    rawv = ref_vals(inp["raw"], wl.act_fmt)
    new = ref.compress_entries(rawv, inp["z"], inp["raw_pos0"], inp["bias"], wl.m, wl.w, e0, n_ent)
    newv = ref.load_entries(ref.store_entries(new, wl.kv_fmt), wl.kv_fmt)

    def entry_rows(rows):
        rows = np.asarray(rows, np.int64)
        out = np.empty((len(rows), D))
        old = rows < e0
        if old.any():
            out[old] = ref_vals(inp["cache"][rows[old]], wl.kv_fmt)
        out[~old] = newv[rows[~old] - e0]
        return out

    qv = ref_vals(inp["q"][sample], wl.act_fmt)
    sc = 1.0 / math.sqrt(D)
    csa = wl.kind == "csa_prefill"
    out_g = to_np(res["out"]).reshape(T, H, D)
    tol = TOL["bf16"] if wl.act_fmt == "bf16" else TOL["f32"]
    n_mismatch = 0
    worst_e2e = 0.0
    oracle_idx = {}
    if csa:
        qiv = ref_vals(inp["qi"][sample], wl.idx_fmt)
        kiv = ref_vals(inp["ki"], wl.idx_fmt)
        idx_g = res["idx"].cpu().numpy()
    for si, i in enumerate(sample):
        t = inp["pos0"] + int(i)
        nv = min((t + 1) // wl.m, n_ent)
        if csa:
            s = ref.indexer_scores(qiv[si], kiv[:nv])
            keys = ref.score_keys(s, wl.score_fmt)
            want = ref.topk_indices(keys, wl.k)
            oracle_idx[int(i)] = want
            assert topk_ok(idx_g[i], want, keys, wl.score_fmt, s, qiv[si], kiv[:nv]), \
                f"top-k of query {i}"
            sel = want[want >= 0]
            same = set(idx_g[i][idx_g[i] >= 0].tolist()) == set(sel.tolist())
            n_mismatch += 0 if same else 1
            ke = entry_rows(sel)
        else:
            same = True
            ke = entry_rows(np.arange(nv))
        pos = ref.window_positions(t, wl.window)
        keys_all = np.concatenate([ke, rawv[pos - inp["raw_pos0"]]])
        o, _ = ref.attend(qv[si], keys_all, sc)
        if same:
            worst_e2e = max(worst_e2e, float(np.max(np.abs(out_g[i] - o))))
    log(f"workload {wid}: end-to-end max err {worst_e2e:.3g}, top-k set mismatches "
        f"{n_mismatch}/{len(sample)}")
    assert worst_e2e <= tol
    assert n_mismatch <= max_mismatched_rows(len(sample))
    if csa:
        # stage-wise: GPU attention over the oracle's selections, sampled queries only
        idx_o = np.stack([oracle_idx[int(i)] for i in sample]).astype(np.int32)
        qs = KV(layer.q.fmt, D, layer.q.data.view(T, H, D)[torch.from_numpy(sample).cuda()]
                .reshape(-1, D).contiguous())
        errs = []
        for si, i in enumerate(sample):
            b1 = Batch.make([1], [inp["pos0"] + int(i)], kv_counts=[n_ent],
                            raw_counts=[layer.raw.rows], raw_pos=[inp["raw_pos0"]])
            o1 = torch.empty(H, D, device="cuda", dtype=torch.float32)
            ops.sparse_mqa_attn(qs.narrow(si * H, H), H, layer.cache,
                                torch.from_numpy(idx_o[si:si + 1]).cuda(), wl.k, layer.raw,
                                wl.window, b1, wl.m, o1, F32)
            t = inp["pos0"] + int(i)
            sel = idx_o[si][idx_o[si] >= 0]
            pos = ref.window_positions(t, wl.window)
            o, _ = ref.attend(qv[si], np.concatenate([entry_rows(sel), rawv[pos - inp["raw_pos0"]]]), sc)
            errs.append(float(np.max(np.abs(to_np(o1) - o))))
        log(f"workload {wid}: stage-wise attention max err {max(errs):.3g}")
        assert max(errs) <= tol


def test_workload1_csa_prefill_f32():
    run_prefill(1, n_sample=256)


def test_workload2_hca_prefill_bf16():
    run_prefill(2, n_sample=96)


def test_workload4_csa_chunk_prefill_at_1m():
    run_prefill(4, n_sample=12)


def test_workload4_small_chunk():
    run_prefill(4, seq=300, n_sample=40)


# ------------------------------------------------------------------ decode


def run_decode(wid, batch=None, layers=None, sample_req=None):
    wl = synth.WORKLOADS[wid]
    ctxs = [int(c) for c in synth.decode_contexts(wl, batch)]
    B = len(ctxs)
    specs = wl.layers if wl.kind == "mixed_decode" else [("csa", wl.m, wl.k)]
    layers = range(len(specs)) if layers is None else layers
    sample_req = list(range(B)) if sample_req is None else sample_req
    D, H = wl.dim, wl.heads
    sc = 1.0 / math.sqrt(D)
    for li in layers:
        kind, m, k = specs[li]
        csa = kind == "csa"
        n_ent = [(c + 1) // m for c in ctxs]
        swa_len = [min(wl.window, c + 1) for c in ctxs]
        t0 = time.time()
        cache = KV.empty(FMT[wl.kv_fmt], sum(n_ent), D)
        swa = torch.empty(sum(swa_len), D, dtype=torch.bfloat16, device="cuda")
        q = torch.empty(B * H, D, dtype=torch.bfloat16, device="cuda")
        qi = KV.empty(FMT[wl.idx_fmt], B * 4, 64) if wl.idx_fmt == "mxfp4" else None
        ki = KV.empty(FMT[wl.idx_fmt], sum(n_ent), 64) if wl.idx_fmt == "mxfp4" else None
        qi_b = torch.empty(B * 4, 64, dtype=torch.bfloat16, device="cuda")
        ki_b = torch.empty(sum(n_ent), 64, dtype=torch.bfloat16, device="cuda") \
            if wl.idx_fmt == "bf16" else None
        reqs = {}
        off = soff = 0
        for r in range(B):
            d = synth.decode_request(wl, r, ctxs[r], m, csa, layer=li)
            n = n_ent[r]
            src = KV(F32, D, dev_f32(d["cache"]))
            ops.quantize(src, cache.narrow(off, n))
            swa[soff: soff + swa_len[r]] = dev_f32(d["swa"]).to(torch.bfloat16)
            q[r * H:(r + 1) * H] = dev_f32(d["q"]).to(torch.bfloat16)
            if csa:
                if wl.idx_fmt == "mxfp4":
                    ops.quantize(KV(F32, 64, dev_f32(d["qi"])), qi.narrow(4 * r, 4))
                    ops.quantize(KV(F32, 64, dev_f32(d["ki"])), ki.narrow(off, n))
                else:
                    qi_b[4 * r: 4 * r + 4] = dev_f32(d["qi"]).to(torch.bfloat16)
                    ki_b[off: off + n] = dev_f32(d["ki"]).to(torch.bfloat16)
            if r in sample_req:
                reqs[r] = (d, off)
            off += n
            soff += swa_len[r]
        torch.cuda.synchronize()
        log(f"workload {wid} layer {li} ({kind}): inputs on device in {time.time() - t0:.1f}s")
        if csa and wl.idx_fmt == "bf16":
            qi, ki = KV(BF16, 64, qi_b), KV(BF16, 64, ki_b)
        layer = DecodeLayer(csa=csa, H=H, m=m, k=k, window=wl.window, ctx=ctxs, n_entries=n_ent,
                            swa_len=swa_len, cache=cache, swa=KV(BF16, D, swa), q=KV(BF16, D, q),
                            qi=qi if csa else None, ki=ki if csa else None,
                            score_fmt=FMT[wl.score_fmt], out_fmt=FMT[wl.out_fmt])
        res = layer.run()
        torch.cuda.synchronize()
        out_g = to_np(res["out"]).reshape(B, H, D)
        idx_g = res["idx"].cpu().numpy() if csa else None
        worst, worst_sw, mism = 0.0, 0.0, 0
        for r, (d, koff) in reqs.items():
            qv = ref_vals(d["q"], "bf16")
            swv = ref_vals(d["swa"], "bf16")
            if csa:
                qiv, kiv = ref_vals(d["qi"], wl.idx_fmt), ref_vals(d["ki"], wl.idx_fmt)
                s = ref.indexer_scores(qiv, kiv)
                keys = ref.score_keys(s, wl.score_fmt)
                want = ref.topk_indices(keys, k)
                assert topk_ok(idx_g[r], want, keys, wl.score_fmt, s, qiv, kiv), \
                    f"top-k of request {r}"
                sel = want[want >= 0]
                same = set(idx_g[r][idx_g[r] >= 0].tolist()) == set(sel.tolist())
                mism += 0 if same else 1
                ev = ref_vals(d["cache"][sel], wl.kv_fmt)
                # stage-wise: GPU attention of this request on the oracle's selection
                b1 = Batch.make([1], [ctxs[r]], kv_counts=[n_ent[r]], raw_counts=[swa_len[r]],
                                raw_pos=[ctxs[r] - swa_len[r] + 1])
                o1 = torch.empty(H, D, device="cuda")
                ops.sparse_mqa_attn(layer.q.narrow(r * H, H), H, cache.narrow(koff, n_ent[r]),
                                    torch.from_numpy(want[None].astype(np.int32)).cuda(), k,
                                    layer.swa.narrow(sum(swa_len[:r]), swa_len[r]), wl.window,
                                    b1, m, o1, F32)
                o, _ = ref.attend(qv, np.concatenate([ev, swv]), sc)
                worst_sw = max(worst_sw, float(np.max(np.abs(to_np(o1) - o))))
            else:
                same = True
                o, _ = ref.attend(qv, np.concatenate([ref_vals(d["cache"], wl.kv_fmt), swv]), sc)
            if same:
                worst = max(worst, float(np.max(np.abs(out_g[r] - o))))
        log(f"workload {wid} layer {li}: end-to-end max err {worst:.3g}, stage-wise "
            f"{worst_sw:.3g}, top-k set mismatches {mism}/{len(reqs)}")
        assert worst <= TOL["bf16"] and worst_sw <= TOL["bf16"]
        assert mism <= max_mismatched_rows(len(reqs))
        del layer, cache, swa, q, qi, ki, res
        torch.cuda.empty_cache()


def test_workload3_csa_decode():
    run_decode(3, sample_req=[0, 1, 2, 17, 31])


def test_workload5_mixed_decode():
    L = synth.mixed_decode_lengths()
    order = np.argsort(L)
    run_decode(5, sample_req=[int(order[0]), int(order[1]), int(order[32]), int(order[-1])])


def test_workload5_small_batch():
    run_decode(5, batch=6)
