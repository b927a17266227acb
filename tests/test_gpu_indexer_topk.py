"""csa_indexer_topk (scores and selection fused, CSA step 2): the same indices,
bit for bit, as csa_indexer_score followed by csa_topk_select, including rows
shorter than k, rows the candidate list takes whole, sampled rows, ties, and
rows redone exactly; and the oracle's selection on the oracle's scores."""
import numpy as np
import pytest
import torch

from long_context_compressed_kv_amd import ops
from long_context_compressed_kv_amd.ops import BF16, F32, Batch
from oracle import csa as ref

from gpu_inputs import bf16_ulp, dev_f32, dev_kv, ref_vals

pytestmark = pytest.mark.gpu

SFMT = {"f32": F32, "bf16": BF16}


def _inputs(rng, n_q, n_keys, fmt, qi_scale=0.125, ki_levels=None):
    qi = (rng.standard_normal((n_q, 4, 64)) * qi_scale).astype(np.float32)
    if ki_levels is None:
        ki = (rng.standard_normal((n_keys, 64)) * 0.125).astype(np.float32)
    else:
        # few distinct key rows: many exactly equal scores
        base = (rng.standard_normal((ki_levels, 64)) * 0.125).astype(np.float32)
        ki = base[rng.integers(0, ki_levels, n_keys)]
    return qi, ki


def _both(qi, ki, fmt, batch, m, k, score_fmt, head_w=None, relu=True):
    """(fused, unfused) index tensors for the same inputs."""
    qd, kd = dev_kv(qi.reshape(-1, 64), fmt), dev_kv(ki, fmt)
    w = dev_f32(head_w) if head_w is not None else None
    fused = ops.indexer_topk(qd, 4, kd, batch, m, SFMT[score_fmt], k, head_w=w, relu=relu)
    dt = torch.float32 if score_fmt == "f32" else torch.bfloat16
    scores = torch.empty(batch.n_q, max(batch.max_kv, 1), device="cuda", dtype=dt)
    ops.indexer_score(qd, 4, kd, batch, m, scores, SFMT[score_fmt], head_w=w, relu=relu)
    unfused = ops.topk_select(scores, SFMT[score_fmt], batch, m, k)
    torch.cuda.synchronize()
    return fused.cpu().numpy(), unfused.cpu().numpy()


# decode: one query per request; contexts chosen so that rows fall shorter
# than k, inside the candidate list (n <= 4096), and above it (sampled)
DECODE_CTX = [20003, 40000, 803, 255, 100, 70001, 16387, 4]


@pytest.mark.parametrize("fmt,score_fmt", [("bf16", "bf16"), ("mxfp4", "bf16"), ("f32", "f32"),
                                           ("bf16", "f32"), ("mxfp4", "f32")])
def test_fused_equals_unfused_decode(fmt, score_fmt):
    rng = np.random.default_rng(61)
    m, k = 4, 64
    kv_counts = [(c + 1) // m for c in DECODE_CTX]
    qi, ki = _inputs(rng, len(DECODE_CTX), sum(kv_counts), fmt)
    batch = Batch.make([1] * len(DECODE_CTX), DECODE_CTX, kv_counts=kv_counts)
    f, u = _both(qi, ki, fmt, batch, m, k, score_fmt)
    assert np.array_equal(f, u)


@pytest.mark.parametrize("fmt,score_fmt,k,T,pos0,relu,weights", [
    ("mxfp4", "bf16", 64, 45, 16360, True, False),    # groups straddle the 4096-entry list
    ("bf16", "bf16", 512, 67, 30000, True, True),     # every row sampled
    ("f32", "f32", 100, 29, 20000, False, True),      # no ReLU: negative scores too
    ("mxfp4", "f32", 8, 70, 0, True, False),          # from position 0: short rows
    ("bf16", "bf16", 64, 600, 20000, True, False),    # many rows: the narrow select
])
def test_fused_equals_unfused_prefill(fmt, score_fmt, k, T, pos0, relu, weights):
    rng = np.random.default_rng(62 + k)
    m = 4
    n_keys = (pos0 + T) // m + 5
    qi, ki = _inputs(rng, T, n_keys, fmt)
    w = rng.uniform(0.2, 2.0, (T, 4)).astype(np.float32) if weights else None
    batch = Batch.make([T], [pos0], kv_counts=[n_keys])
    f, u = _both(qi, ki, fmt, batch, m, k, score_fmt, head_w=w, relu=relu)
    assert np.array_equal(f, u)


def test_fused_all_ties_redo_and_short():
    """All scores equal (zero queries): the k lowest indices everywhere.  Rows
    above 4096 entries overflow the candidate list and are redone exactly;
    shorter ones resolve the ties in the select step."""
    rng = np.random.default_rng(63)
    m, k = 4, 100
    ctx = [40000, 8000, 1000, 300, 50]
    kv_counts = [(c + 1) // m for c in ctx]
    qi, ki = _inputs(rng, len(ctx), sum(kv_counts), "bf16", qi_scale=0.0)
    batch = Batch.make([1] * len(ctx), ctx, kv_counts=kv_counts)
    f, u = _both(qi, ki, "bf16", batch, m, k, "bf16")
    assert np.array_equal(f, u)
    for r, n in enumerate(kv_counts):
        want = np.full(k, -1, np.int32)
        want[:min(k, n)] = np.arange(min(k, n))
        assert np.array_equal(f[r], want)


@pytest.mark.parametrize("score_fmt", ["bf16", "f32"])
def test_fused_many_ties_at_threshold(score_fmt):
    """Keys drawn from 16 rows: each query's scores take 16 values, so the
    k-th score is shared by hundreds of entries."""
    rng = np.random.default_rng(64)
    m, k = 4, 512
    ctx = [60000, 12000, 3000]
    kv_counts = [(c + 1) // m for c in ctx]
    qi, ki = _inputs(rng, len(ctx), sum(kv_counts), "bf16", ki_levels=16)
    batch = Batch.make([1] * len(ctx), ctx, kv_counts=kv_counts)
    f, u = _both(qi, ki, "bf16", batch, m, k, score_fmt)
    assert np.array_equal(f, u)


def test_fused_long_rows_k1024():
    """A chunk of queries near position 2^20 (about 262k entries each),
    MXFP4 operands, k = 1024, as in the chunked prefill."""
    rng = np.random.default_rng(65)
    m, k, T, pos0 = 4, 1024, 96, 1 << 20
    n_keys = (pos0 + T) // m
    qi, ki = _inputs(rng, T, n_keys, "mxfp4")
    batch = Batch.make([T], [pos0], kv_counts=[n_keys])
    f, u = _both(qi, ki, "mxfp4", batch, m, k, "bf16")
    assert np.array_equal(f, u)


@pytest.mark.parametrize("score_fmt", ["bf16", "f32"])
def test_fused_prefill_groups_many_ties(score_fmt):
    """Query groups (prefill) over keys drawn from 8 rows: each query's scores
    take 8 values, so thousands of entries tie at the threshold and pass;
    the waves' staging areas fill and the rows are redone exactly."""
    rng = np.random.default_rng(71)
    m, k, T, pos0 = 4, 256, 40, 200000
    n_keys = (pos0 + T) // m
    qi, ki = _inputs(rng, T, n_keys, "bf16", ki_levels=8)
    batch = Batch.make([T], [pos0], kv_counts=[n_keys])
    f, u = _both(qi, ki, "bf16", batch, m, k, score_fmt)
    assert np.array_equal(f, u)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4"])
def test_fused_prefill_groups_crowded_wave(fmt):
    """Query groups (prefill) whose best entries form one run of 1100 keys:
    for every query nearly all entries of the waves covering the run pass,
    more than a staging area holds, so every row takes the exact redo."""
    rng = np.random.default_rng(72)
    m, k, T, pos0 = 4, 512, 72, 131072
    n_keys = (pos0 + T) // m
    qi, ki = _inputs(rng, T, n_keys, fmt)
    ki[5000:6100] *= 4.0
    batch = Batch.make([T], [pos0], kv_counts=[n_keys])
    f, u = _both(qi, ki, fmt, batch, m, k, "bf16")
    assert np.array_equal(f, u)


def test_fused_matches_oracle():
    """Against the oracle's top-k of its own scores: equal except where a key
    lies within one rounding step of the k-th key."""
    rng = np.random.default_rng(66)
    m, k = 4, 48
    ctx = [30000, 9000, 2000, 150]
    kv_counts = [(c + 1) // m for c in ctx]
    qi, ki = _inputs(rng, len(ctx), sum(kv_counts), "mxfp4")
    batch = Batch.make([1] * len(ctx), ctx, kv_counts=kv_counts)
    idx = ops.indexer_topk(dev_kv(qi.reshape(-1, 64), "mxfp4"), 4, dev_kv(ki, "mxfp4"), batch, m,
                           BF16, k)
    torch.cuda.synchronize()
    qv, kv = ref_vals(qi, "mxfp4"), ref_vals(ki, "mxfp4")
    off = np.concatenate([[0], np.cumsum(kv_counts)])
    for r in range(len(ctx)):
        s = ref.indexer_scores(qv[r], kv[off[r]: off[r + 1]])
        keys = ref.score_keys(s, "bf16")
        want = ref.topk_indices(keys, k)
        got = idx[r].cpu().numpy()
        if not np.array_equal(got, want):
            tau = np.sort(keys)[::-1][min(k, len(keys)) - 1]
            for j in set(got.tolist()) ^ set(want.tolist()):
                assert j >= 0 and abs(keys[j] - tau) <= bf16_ulp(tau)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4"])
def test_fused_clustered_best_entries(fmt):
    """A row whose best entries all lie in one filter workgroup's chunk: that
    workgroup's own threshold sits above the row's k-th score, so the select
    finds its k-th candidate below the row's largest threshold and redoes the
    row exactly.  The other row clusters its best entries across a chunk
    boundary."""
    rng = np.random.default_rng(67)
    m, k = 4, 512
    ctx = [131071, 40003]
    kv_counts = [(c + 1) // m for c in ctx]
    qi, ki = _inputs(rng, len(ctx), sum(kv_counts), fmt)
    ki[:1024] *= 4.0                                            # row 0: its first chunk
    ki[kv_counts[0] + 7000: kv_counts[0] + 8100] *= 4.0         # row 1: straddles chunks
    batch = Batch.make([1] * len(ctx), ctx, kv_counts=kv_counts)
    f, u = _both(qi, ki, fmt, batch, m, k, "bf16")
    assert np.array_equal(f, u)


@pytest.mark.parametrize("fmt,score_fmt", [("bf16", "bf16"), ("mxfp4", "f32")])
def test_fused_largest_k(fmt, score_fmt):
    """k = 4096, the largest the call takes: decode rows shorter than k, inside
    the candidate list (cap = 6k) and far beyond it, and a prefill group of
    queries straddling the list size; the same indices as score + select."""
    rng = np.random.default_rng(66)
    m, k = 4, 4096
    ctx = [9000, 60000, 400000, 100]
    n_ent = [(c + 1) // m for c in ctx]
    qi, ki = _inputs(rng, len(ctx), sum(n_ent), fmt)
    f, u = _both(qi, ki, fmt, Batch.make([1] * len(ctx), ctx, kv_counts=n_ent), m, k, score_fmt)
    assert np.array_equal(f, u)
    T, pos0 = 24, 98000
    qi, ki = _inputs(rng, T, (pos0 + T) // m, fmt)
    f, u = _both(qi, ki, fmt, Batch.make([T], [pos0], kv_counts=[(pos0 + T) // m]), m, k, score_fmt)
    assert np.array_equal(f, u)


@pytest.mark.parametrize("fmt,score_fmt,T,pos0", [("f32", "f32", 4096, 0), ("bf16", "bf16", 600, 3400),
                                                  ("mxfp4", "bf16", 300, 0),
                                                  ("mxfp4", "bf16", 1024, 3000)])
def test_fused_short_rows_many_queries(fmt, score_fmt, T, pos0):
    """Prefill rows of at most 1024 entries (every entry a candidate), as in
    the fp32 CSA prefill at 4K: the same indices as score + select."""
    rng = np.random.default_rng(67 + T)
    m, k = 4, 64
    n_keys = (pos0 + T) // m
    qi, ki = _inputs(rng, T, n_keys, fmt)
    f, u = _both(qi, ki, fmt, Batch.make([T], [pos0], kv_counts=[n_keys]), m, k, score_fmt)
    assert np.array_equal(f, u)


@pytest.mark.parametrize("fmt,score_fmt", [("bf16", "bf16"), ("mxfp4", "bf16"), ("f32", "f32")])
def test_fused_many_short_single_query_requests(fmt, score_fmt):
    """600 decode requests (one query each) of at most 1024 visible entries,
    more rows than the device holds select workgroups at once: the streamed
    filter's per-workgroup regions and the select over them give the same
    indices as score + select."""
    rng = np.random.default_rng(71)
    m, k, n_req = 4, 64, 600
    ctx = [int(c) for c in rng.integers(3, 4096, n_req)]
    kv_counts = [(c + 1) // m for c in ctx]
    qi, ki = _inputs(rng, n_req, sum(kv_counts), fmt)
    batch = Batch.make([1] * n_req, ctx, kv_counts=kv_counts)
    f, u = _both(qi, ki, fmt, batch, m, k, score_fmt)
    assert np.array_equal(f, u)
