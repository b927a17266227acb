"""csa_indexer_topk_noalloc (the fused indexer + top-k for callers that cannot
allocate) gives the same indices, bit for bit, as csa_indexer_topk with a
caller workspace: two calls in a row on the same GPU, the second smaller (the
static scratch keeps the first call's contents), in both of the fused
selection's modes (one query per request; a single request's query groups)."""
import ctypes

import numpy as np
import pytest
import torch

from long_context_compressed_kv_amd import _lib, ops
from long_context_compressed_kv_amd.ops import BF16, Batch

from gpu_inputs import dev_kv

pytestmark = pytest.mark.gpu


def _call_noalloc(qd, kd, batch, m, score_fmt, k):
    """Through the C ABI directly."""
    lib = _lib.load()
    idx = torch.full((batch.n_q, k), -7, dtype=torch.int32, device="cuda")
    qc, kc, bc = qd.c(), kd.c(), batch.c()
    st = lib.csa_indexer_topk_noalloc(ctypes.byref(qc), 4, None, ctypes.byref(kc),
                                      ctypes.byref(bc), m, 1, score_fmt, k,
                                      ctypes.c_void_p(idx.data_ptr()),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.csa_last_error()
    return idx


def _case(rng, ctx, fmt, k, m=4):
    n_req = len(ctx)
    kv = [(c + 1) // m for c in ctx]
    qi = (rng.standard_normal((n_req * 4, 64)) * 0.125).astype(np.float32)
    ki = (rng.standard_normal((sum(kv), 64)) * 0.125).astype(np.float32)
    return dev_kv(qi, fmt), dev_kv(ki, fmt), Batch.make([1] * n_req, ctx, kv_counts=kv)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4"])
def test_noalloc_equals_workspace_decode(fmt):
    rng = np.random.default_rng(91)
    m, k = 4, 1024
    big = _case(rng, [int(c) for c in rng.integers(2000, 400000, 48)], fmt, k)
    small = _case(rng, [int(c) for c in rng.integers(100, 30000, 9)], fmt, k)
    got = []
    for qd, kd, b in (big, small):
        got.append(_call_noalloc(qd, kd, b, m, BF16, k))
    torch.cuda.synchronize()
    for (qd, kd, b), g in zip((big, small), got):
        want = ops.indexer_topk(qd, 4, kd, b, m, BF16, k)
        torch.cuda.synchronize()
        assert torch.equal(g, want)


def test_noalloc_equals_workspace_prefill():
    rng = np.random.default_rng(92)
    m, k = 4, 256
    cases = []
    for T, pos0 in ((256, 60000), (96, 9000)):
        n_keys = (pos0 + T) // m
        qi = (rng.standard_normal((T * 4, 64)) * 0.125).astype(np.float32)
        ki = (rng.standard_normal((n_keys, 64)) * 0.125).astype(np.float32)
        cases.append((dev_kv(qi, "mxfp4"), dev_kv(ki, "mxfp4"),
                      Batch.make([T], [pos0], kv_counts=[n_keys])))
    got = [_call_noalloc(qd, kd, b, m, BF16, k) for qd, kd, b in cases]
    torch.cuda.synchronize()
    for (qd, kd, b), g in zip(cases, got):
        want = ops.indexer_topk(qd, 4, kd, b, m, BF16, k)
        torch.cuda.synchronize()
        assert torch.equal(g, want)


def test_noalloc_refuses_beyond_its_scratch():
    rng = np.random.default_rng(93)
    k = 4096
    n_q = ops.indexer_topk_noalloc_max_bytes() // ops.indexer_topk_workspace_size(1, k) + 1
    qd, kd, b = _case(rng, [5000] * int(n_q), "bf16", k)
    with pytest.raises(_lib.CsaError):
        ops.indexer_topk_noalloc(qd, 4, kd, b, 4, BF16, k,
                                 torch.empty(b.n_q, k, dtype=torch.int32, device="cuda"))
