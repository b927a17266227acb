"""A request's decode result does not depend on the rest of the batch (page
wmrh.cn/news/726125, "V4 改进二": the same token gives the same output
wherever it sits in a batch), on the path the decode workloads run: attention
split over keys (the pipeline's split_keys) and merged, after the fused
indexer + top-k.

The 64 requests of the 4-layer decode workload (contexts log-uniform from 4K
to 1M) run as one batch in order, as the same batch permuted, and alone; the
selection and the output of every request must be the same bits each time.
Inputs are drawn on the device per request (a seeded generator per request),
so a request's inputs are identical in every batch."""
import numpy as np
import pytest
import torch

import synth
from long_context_compressed_kv_amd import ops
from long_context_compressed_kv_amd.ops import BF16, F32, FP8_MIXED, KV, MXFP4
from long_context_compressed_kv_amd.pipeline import DecodeLayer

pytestmark = pytest.mark.gpu

H, D, W = 64, 512, 128


def _request_inputs(r, ctx, m, csa):
    g = torch.Generator(device="cuda")
    g.manual_seed(7000 + 131 * r + m)
    n_c = (ctx + 1) // m
    rn = lambda *s: torch.randn(*s, generator=g, device="cuda", dtype=torch.float32)
    cache = KV.empty(FP8_MIXED, n_c, D)
    ops.quantize(KV(F32, D, rn(n_c, D)), cache)
    out = {"n_c": n_c, "cache": cache, "swa": rn(min(W, ctx + 1), D).to(torch.bfloat16),
           "q": rn(H, D).to(torch.bfloat16)}
    if csa:
        qi, ki = KV.empty(MXFP4, 4, 64), KV.empty(MXFP4, n_c, 64)
        ops.quantize(KV(F32, 64, rn(4, 64) * 0.125), qi)
        ops.quantize(KV(F32, 64, rn(n_c, 64) * 0.125), ki)
        out.update(qi=qi, ki=ki)
    return out


def _cat(kvs):
    """Concatenate device KV tensors of one format along rows."""
    cat = lambda name: None if getattr(kvs[0], name) is None else \
        torch.cat([getattr(x, name) for x in kvs])
    return KV(kvs[0].fmt, kvs[0].dim, cat("data"), cat("scale"), cat("rope"))


def _run(reqs, ctxs, order, m, k, csa):
    sel = [reqs[r] for r in order]
    layer = DecodeLayer(csa=csa, H=H, m=m, k=k, window=W, ctx=[int(ctxs[r]) for r in order],
                        n_entries=[x["n_c"] for x in sel],
                        swa_len=[x["swa"].shape[0] for x in sel],
                        cache=_cat([x["cache"] for x in sel]),
                        swa=KV(BF16, D, torch.cat([x["swa"] for x in sel])),
                        q=KV(BF16, D, torch.cat([x["q"] for x in sel])),
                        qi=_cat([x["qi"] for x in sel]) if csa else None,
                        ki=_cat([x["ki"] for x in sel]) if csa else None,
                        score_fmt=BF16, out_fmt=BF16)
    res = layer.run()
    torch.cuda.synchronize()
    out = res["out"].view(len(order), H, D).clone()
    idx = res["idx"].clone() if csa else None
    return out, idx


@pytest.mark.parametrize("kind,m,k", [("csa", 4, 1024), ("hca", 128, 0)])
def test_decode_result_independent_of_batch(kind, m, k):
    csa = kind == "csa"
    ctxs = synth.decode_contexts(synth.WORKLOADS[5])
    B = len(ctxs)
    reqs = [_request_inputs(r, int(ctxs[r]), m, csa) for r in range(B)]
    print(f"[invariance] {kind}: {B} requests, contexts {int(ctxs.min())}..{int(ctxs.max())}",
          flush=True)
    base_out, base_idx = _run(reqs, ctxs, list(range(B)), m, k, csa)
    perm = list(np.random.default_rng(5).permutation(B))
    p_out, p_idx = _run(reqs, ctxs, perm, m, k, csa)
    for j, r in enumerate(perm):
        assert torch.equal(p_out[j], base_out[r]), f"request {r} differs when permuted"
        if csa:
            assert torch.equal(p_idx[j], base_idx[r]), f"selection of request {r} differs"
    # alone: the longest request, the shortest and one in between
    for r in (int(np.argmax(ctxs)), int(np.argmin(ctxs)), 17):
        a_out, a_idx = _run(reqs, ctxs, [r], m, k, csa)
        assert torch.equal(a_out[0], base_out[r]), f"request {r} differs alone"
        if csa:
            assert torch.equal(a_idx[0], base_idx[r])
    # and a batch of two, the request second
    two_out, _ = _run(reqs, ctxs, [3, 40], m, k, csa)
    assert torch.equal(two_out[1], base_out[40])
