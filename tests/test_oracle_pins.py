"""Pins of the oracle's method steps against closed forms, library special
cases (torch's fp64 scaled_dot_product_attention, NumPy means and dot
products), brute force on tiny inputs, and invariants the method implies."""
import math

import numpy as np
import pytest
import torch

from oracle import codecs
from oracle import csa as ref


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa(q, k, mask_add=None, scale=None):
    """torch's fp64 attention: q [H, D] against keys k [n, D] (value = key);
    mask_add [n] additive logit bias (or -inf)."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, :, None, :]      # [1,H,1,D]
    kt = torch.from_numpy(np.asarray(k, np.float64))[None, None].expand(1, q.shape[0], -1, -1)
    am = None
    if mask_add is not None:
        am = torch.from_numpy(np.asarray(mask_add, np.float64))[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, attn_mask=am, scale=scale)
    return o[0, :, 0, :].numpy()


# ============================================================== compression

@pytest.mark.parametrize("m,w", [(4, 8), (128, 256), (4, 4), (3, 7)])
def test_uniform_logits_give_mean_pooling(m, w):
    rng = _rng(10)
    n = 6 * m + 5
    x = rng.standard_normal((n, 16))
    z = np.full(n, 0.37)
    b = np.full(w, -1.3)
    n_e = n // m
    c = ref.compress_entries(x, z, 0, b, m, w, 0, n_e)
    for i in range(n_e):
        lo, hi = max(0, (i + 1) * m - w), (i + 1) * m
        assert np.allclose(c[i], np.mean(x[lo:hi], axis=0), rtol=0, atol=1e-13)


def test_logit_and_bias_shift_invariance():
    rng = _rng(11)
    m, w, n = 4, 8, 64
    x, z, b = rng.standard_normal((n, 8)), rng.standard_normal(n), rng.standard_normal(w)
    c0 = ref.compress_entries(x, z, 0, b, m, w, 0, n // m)
    c1 = ref.compress_entries(x, z + 5.5, 0, b - 2.25, m, w, 0, n // m)
    assert np.allclose(c0, c1, atol=1e-13)


def test_dominant_logit_sets_overlap():
    """A huge logit on token p makes exactly the entries whose window holds p
    equal x[p]: with w = 2m these are blocks floor(p/m) and floor(p/m)+1."""
    rng = _rng(12)
    m, w, n = 4, 8, 64
    x, z, b = rng.standard_normal((n, 8)), rng.standard_normal(n), rng.standard_normal(w)
    p = 29
    z2 = z.copy()
    z2[p] = 200.0
    c0 = ref.compress_entries(x, z, 0, b, m, w, 0, n // m)
    c2 = ref.compress_entries(x, z2, 0, b, m, w, 0, n // m)
    hit = {p // m, p // m + 1}
    for i in range(n // m):
        if i in hit:
            assert np.allclose(c2[i], x[p], atol=1e-12)
        else:
            assert np.array_equal(c2[i], c0[i])


@pytest.mark.parametrize("j", [0, 1, 3])
def test_one_hot_bias_selects_slot(j):
    rng = _rng(13)
    m = w = 4
    n = 40
    x, z = rng.standard_normal((n, 8)), rng.standard_normal(n)
    b = np.full(w, -np.inf)
    b[j] = 0.0
    c = ref.compress_entries(x, z, 0, b, m, w, 0, n // m)
    assert np.array_equal(c, x[j::m][: n // m])


def test_identity_compression_m1():
    rng = _rng(14)
    x, z = rng.standard_normal((20, 8)), rng.standard_normal(20)
    c = ref.compress_entries(x, z, 0, np.zeros(1), 1, 1, 0, 20)
    assert np.array_equal(c, x)


@pytest.mark.parametrize("m,w", [(4, 8), (128, 256)])
def test_chunked_compression_equals_one_shot(m, w):
    rng = _rng(15)
    n, split = 8 * m, 3 * m
    x, z, b = rng.standard_normal((n, 8)), rng.standard_normal(n), rng.standard_normal(w)
    full = ref.compress_entries(x, z, 0, b, m, w, 0, n // m)
    hist = w - m                                     # history rows the chunk needs
    first = split // m
    part = ref.compress_entries(x[split - hist:], z[split - hist:], split - hist, b, m, w,
                                first, n // m)
    assert np.allclose(part, full[first:], atol=0, rtol=0)


# per-channel compression logits (the variant reading of the learned weight)

def test_channel_compression_reduces_to_scalar():
    """A logit and a bias shared by every channel give the scalar compression."""
    rng = _rng(16)
    for m, w in ((4, 8), (128, 256), (3, 5)):
        n, D = 5 * m + 3, 6
        x, z, b = rng.standard_normal((n, D)), rng.standard_normal(n), rng.standard_normal(w)
        c = ref.compress_entries_channel(x, np.repeat(z[:, None], D, 1), 0,
                                         np.repeat(b[:, None], D, 1), m, w, 0, n // m)
        assert np.allclose(c, ref.compress_entries(x, z, 0, b, m, w, 0, n // m), rtol=0, atol=1e-13)


def test_channel_compression_is_one_scalar_compression_per_channel():
    """Channel d of every entry is the scalar compression of the one-channel
    sequence x[:, d] with logits z[:, d] and biases b[:, d]."""
    rng = _rng(17)
    m, w, n, D = 4, 8, 70, 5
    x, z, b = rng.standard_normal((n, D)), rng.standard_normal((n, D)) * 2, rng.standard_normal((w, D))
    c = ref.compress_entries_channel(x, z, 0, b, m, w, 0, n // m)
    for d in range(D):
        cd = ref.compress_entries(x[:, d:d + 1], z[:, d], 0, b[:, d], m, w, 0, n // m)
        assert np.allclose(c[:, d], cd[:, 0], rtol=0, atol=1e-13)
    # and a shift of one channel's logits moves nothing
    z2 = z.copy()
    z2[:, 2] += 7.5
    assert np.allclose(ref.compress_entries_channel(x, z2, 0, b, m, w, 0, n // m), c, rtol=0, atol=1e-13)


def test_channel_compression_worked_example():
    """m = 2, w = 3, two channels, by hand: entry 1 covers positions 1, 2, 3
    (slots 0, 1, 2); entry 0 only positions 0, 1 (slot 0 would be -1)."""
    x = np.array([[1.0, 10.0], [2.0, 20.0], [3.0, 30.0], [4.0, 40.0]])
    z = np.array([[0.0, 1.0], [1.0, 0.0], [0.0, 0.0], [2.0, -1.0]])
    b = np.array([[0.0, 0.0], [0.0, 1.0], [-1.0, 0.0]])
    c = ref.compress_entries_channel(x, z, 0, b, 2, 3, 0, 2)
    e = math.exp
    # entry 0, slots 1, 2 = positions 0, 1
    w0 = [e(0 + 0), e(1 - 1)], [e(1 + 1), e(0 + 0)]
    ch0 = (w0[0][0] * 1 + w0[0][1] * 2) / sum(w0[0])
    ch1 = (w0[1][0] * 10 + w0[1][1] * 20) / sum(w0[1])
    assert np.allclose(c[0], [ch0, ch1], rtol=0, atol=1e-14)
    # entry 1, slots 0, 1, 2 = positions 1, 2, 3
    l0 = [1 + 0, 0 + 0, 2 - 1]
    l1 = [0 + 0, 0 + 1, -1 + 0]
    ch0 = sum(e(v) * xv for v, xv in zip(l0, [2, 3, 4])) / sum(e(v) for v in l0)
    ch1 = sum(e(v) * xv for v, xv in zip(l1, [20, 30, 40])) / sum(e(v) for v in l1)
    assert np.allclose(c[1], [ch0, ch1], rtol=0, atol=1e-13)


def test_visibility_and_lcm_block():
    """n_c(t) = floor((t+1)/m): entry i is usable once (i+1)m - 1 <= t.  One
    block of lcm(4, 128) = 128 raw tokens holds 32 CSA and 1 HCA entries."""
    assert math.lcm(4, 128) == 128
    t = np.arange(0, 4096)
    for m in (4, 128):
        nc = ref.n_visible(t, m)
        for i in (0, 1, 7, 30):
            first_t = (i + 1) * m - 1
            assert nc[first_t] == i + 1 and (first_t == 0 or nc[first_t - 1] == i)
    blk = np.arange(0, 4096 + 1, 128)
    assert np.all(np.diff(ref.n_visible(blk - 1, 4)) == 32)
    assert np.all(np.diff(ref.n_visible(blk - 1, 128)) == 1)
    # the configs' cache sizes
    assert ref.n_visible(131072, 4) == 32768
    assert ref.n_visible(2 ** 20 - 1, 4) == 262144
    assert ref.n_visible(2 ** 20 + 8191, 4) == 264192


# ============================================================== indexer

def test_indexer_linear_closed_form():
    rng = _rng(20)
    qi, ki = rng.standard_normal((4, 64)), rng.standard_normal((300, 64))
    s = ref.indexer_scores(qi, ki, relu=False)
    assert np.allclose(s, ki @ qi.sum(axis=0), atol=1e-12)


def test_indexer_relu_identity_on_positive_dots():
    rng = _rng(21)
    qi, ki = np.abs(rng.standard_normal((4, 64))), np.abs(rng.standard_normal((300, 64)))
    w = np.array([0.5, 1.0, 2.0, 3.0])
    s = ref.indexer_scores(qi, ki, head_w=w)
    assert np.allclose(s, ki @ (w[:, None] * qi).sum(axis=0), atol=1e-11)


def test_indexer_relu_placement_abs():
    """With q1 = -q0 and the other heads zero, sum_h ReLU(q_h . k) = |q0 . k|."""
    rng = _rng(22)
    q0 = rng.standard_normal(64)
    qi = np.stack([q0, -q0, np.zeros(64), np.zeros(64)])
    ki = rng.standard_normal((500, 64))
    assert np.allclose(ref.indexer_scores(qi, ki), np.abs(ki @ q0), atol=1e-12)
    # a negative dot product contributes nothing
    assert np.all(ref.indexer_scores(qi[:1], ki) >= 0)


def test_score_keys_bf16():
    s = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 0.1, -2.5])
    k = ref.score_keys(s, "bf16")
    ref_k = torch.from_numpy(s.astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(k, ref_k)


# ============================================================== top-k

def _topk_brute(keys, k):
    """Entry j is kept iff fewer than k entries beat it, where i beats j when
    keys[i] > keys[j], or keys[i] == keys[j] and i < j."""
    n = len(keys)
    kept = [j for j in range(n)
            if sum(1 for i in range(n)
                   if keys[i] > keys[j] or (keys[i] == keys[j] and i < j)) < k]
    return kept + [-1] * (k - len(kept))


@pytest.mark.parametrize("seed", range(12))
def test_topk_matches_brute_force(seed):
    rng = _rng(100 + seed)
    n = int(rng.integers(1, 60))
    k = int(rng.integers(1, 40))
    keys = rng.integers(-3, 4, n).astype(np.float32)       # many ties
    if seed % 3 == 0:
        keys = rng.standard_normal(n).astype(np.float32)
    assert list(ref.topk_indices(keys, k)) == _topk_brute(list(keys), k)


def test_topk_pads_short_rows():
    out = ref.topk_indices(np.array([0.5, 2.0, 1.0], np.float32), 5)
    assert list(out) == [0, 1, 2, -1, -1]


# ============================================================== attention

def test_attend_matches_torch_sdpa():
    rng = _rng(30)
    q, keys = rng.standard_normal((16, 128)), rng.standard_normal((77, 128))
    o, lse = ref.attend(q, keys, 1 / math.sqrt(128))
    assert np.allclose(o, _sdpa(q, keys), atol=1e-12)
    logits = q @ keys.T / math.sqrt(128)
    assert np.allclose(lse, np.log(np.exp(logits).sum(axis=1)), atol=1e-12)


def test_merge_equals_joint_softmax():
    rng = _rng(31)
    q, keys = rng.standard_normal((8, 64)), rng.standard_normal((50, 64))
    sc = 0.125
    o, lse = ref.attend(q, keys, sc)
    for split in (1, 17, 49):
        perm = rng.permutation(50)
        a, bb = keys[perm[:split]], keys[perm[split:]]
        oa, la = ref.attend(q, a, sc)
        ob, lb = ref.attend(q, bb, sc)
        om, lm = ref.merge(oa, la, ob, lb)
        om2, lm2 = ref.merge(ob, lb, oa, la)
        assert np.allclose(om, o, atol=1e-12) and np.allclose(lm, lse, atol=1e-12)
        assert np.allclose(om2, om, atol=1e-14) and np.allclose(lm2, lm, atol=1e-14)


def _csa_layer(x, z, b, qi_all, ki_src, q_all, m, w, k, window, ts, score_fmt="f32"):
    n = x.shape[0]
    entries = ref.compress_entries(x, z, 0, b, m, w, 0, n // m)
    ki = ki_src[: n // m]
    return [ref.csa_query(t, q_all[t], entries, qi_all[t], ki, k, m, x, 0, window,
                          score_fmt=score_fmt) for t in ts]


def test_m1_full_topk_no_window_is_dense_causal_mqa():
    rng = _rng(32)
    n, h, d = 40, 4, 32
    x, z = rng.standard_normal((n, d)), rng.standard_normal(n)
    q = rng.standard_normal((n, h, d))
    qi, ki = rng.standard_normal((n, 4, 16)), rng.standard_normal((n, 16))
    outs = _csa_layer(x, z, np.zeros(1), qi, ki, q, 1, 1, n, 0, range(n))
    for t, r in enumerate(outs):
        mask = np.where(np.arange(n) <= t, 0.0, -np.inf)
        assert np.allclose(r["o"], _sdpa(q[t], x, mask), atol=1e-12)


def test_m1_full_topk_with_window_doubles_recent_keys():
    """With m = 1 every raw token is also an entry, so a window of W adds the
    last W tokens a second time: the same as dense causal attention with
    +ln 2 added to those tokens' logits."""
    rng = _rng(33)
    n, h, d, win = 50, 2, 16, 8
    x, z = rng.standard_normal((n, d)), rng.standard_normal(n)
    q = rng.standard_normal((n, h, d))
    qi, ki = rng.standard_normal((n, 4, 16)), rng.standard_normal((n, 16))
    outs = _csa_layer(x, z, np.zeros(1), qi, ki, q, 1, 1, n, win, range(n))
    for t, r in enumerate(outs):
        pos = np.arange(n)
        mask = np.where(pos <= t, 0.0, -np.inf) + np.where((pos <= t) & (pos > t - win), math.log(2), 0)
        assert np.allclose(r["o"], _sdpa(q[t], x, mask), atol=1e-12)


def test_hca_before_first_entry_is_pure_window():
    rng = _rng(34)
    m, w, n, d = 128, 256, 300, 16
    x, z, b = rng.standard_normal((n, d)), rng.standard_normal(n), rng.standard_normal(w)
    q = rng.standard_normal((n, 4, d))
    entries = ref.compress_entries(x, z, 0, b, m, w, 0, n // m)
    for t in (0, 5, 126):
        r = ref.hca_query(t, q[t], entries, m, x, 0, window=128)
        assert np.allclose(r["o"], _sdpa(q[t], x[: t + 1]), atol=1e-12)
    # window covering the whole prefix and no entries -> dense causal over raw
    r = ref.hca_query(126, q[126], entries[:0], m, x, 0, window=1000)
    assert np.allclose(r["o"], _sdpa(q[126], x[:127]), atol=1e-12)


def test_hca_dense_attention_matches_sdpa():
    rng = _rng(35)
    m, w, n, d = 8, 16, 200, 16
    x, z, b = rng.standard_normal((n, d)), rng.standard_normal(n), rng.standard_normal(w)
    q = rng.standard_normal((n, 4, d))
    entries = ref.compress_entries(x, z, 0, b, m, w, 0, n // m)
    t = 150
    r = ref.hca_query(t, q[t], entries, m, x, 0, window=32)
    keys = np.concatenate([entries[: (t + 1) // m], x[t - 31: t + 1]])
    assert np.allclose(r["o"], _sdpa(q[t], keys), atol=1e-12)


def test_causality_full_csa_layer():
    rng = _rng(36)
    m, w, n, d, k = 4, 8, 96, 16, 6
    x, z, b = rng.standard_normal((n, d)), rng.standard_normal(n), rng.standard_normal(w)
    q = rng.standard_normal((n, 4, d))
    qi, ki = rng.standard_normal((n, 4, 8)), rng.standard_normal((n, 8))
    t = 61
    base = _csa_layer(x, z, b, qi, ki, q, m, w, k, 16, [t])[0]
    x2, z2, ki2 = x.copy(), z.copy(), ki.copy()
    x2[t + 1:] += 3.0
    z2[t + 1:] -= 2.0
    ki2[(t + 1) // m:] *= -1
    pert = _csa_layer(x2, z2, b, qi, ki2, q, m, w, k, 16, [t])[0]
    assert np.array_equal(base["idx"], pert["idx"])
    assert np.allclose(base["o"], pert["o"], atol=0)


def test_entry_permutation_permutes_selection():
    rng = _rng(37)
    n_e, d, k = 64, 32, 10
    entries = rng.standard_normal((n_e, d))
    ki = rng.standard_normal((n_e, 16))
    qi, q = rng.standard_normal((4, 16)), rng.standard_normal((8, d))
    raw = rng.standard_normal((600, d))
    t = 4 * n_e - 1                            # all entries visible (m = 4)
    r0 = ref.csa_query(t, q, entries, qi, ki, k, 4, raw, 0, window=16)
    perm = rng.permutation(n_e)
    r1 = ref.csa_query(t, q, entries[perm], qi, ki[perm], k, 4, raw, 0, window=16)
    inv = np.argsort(perm)
    assert sorted(perm[r1["idx"]]) == sorted(r0["idx"])
    assert sorted(inv[r0["idx"]]) == sorted(r1["idx"])
    assert np.allclose(r0["o"], r1["o"], atol=1e-12)


def test_mixed_cache_store_load_is_exact_view():
    rng = _rng(38)
    c = rng.standard_normal((5, 512))
    st = ref.store_entries(c, "fp8_mixed")
    v = ref.load_entries(st, "fp8_mixed")
    assert np.array_equal(v, codecs.dequantize_kv_mixed(*codecs.quantize_kv_mixed(c.astype(np.float32))))
    assert np.array_equal(ref.load_entries(ref.store_entries(c, "bf16"), "bf16"),
                          codecs.bf16_round(c).astype(np.float64))


def test_fp8_query_keeps_representable_rows():
    """A row whose non-RoPE blocks are e4m3 values times 2^e with each block's
    maximum exactly 448 * 2^e, and whose RoPE dims are bf16 values, is stored
    without change (the smallest power-of-two scale is 2^e)."""
    rng = np.random.default_rng(31)
    grid = np.array([0.0, 0.015625, 0.5, 1.0, 1.125, 1.5, 3.25, 13.0, 96.0, 240.0, 448.0])
    q = np.zeros((3, 512))
    for r in range(3):
        for b, (lo, hi) in enumerate([(0, 128), (128, 256), (256, 384), (384, 448)]):
            e = int(rng.integers(-8, 4))
            v = rng.choice(grid, hi - lo) * rng.choice([-1.0, 1.0], hi - lo)
            v[int(rng.integers(0, hi - lo))] = 448.0
            q[r, lo:hi] = v * 2.0 ** e
        q[r, 448:] = codecs.bf16_round(rng.standard_normal(64))
    assert np.array_equal(ref.fp8_query(q), q)


def test_fp8_query_error_bound_and_rope_in_bf16():
    """Each non-RoPE value moves by at most half an e4m3 step at its block's
    scale (2^-4 of the block's power-of-two scale times 2^floor(log2|x/s|),
    at most 16 * 2^-4 s at the top binade), the RoPE dims are their bf16
    rounding, and the attention over fp8 queries stays within the logit
    perturbation the rounding allows."""
    rng = np.random.default_rng(32)
    q = rng.standard_normal((4, 512)) * 3
    v = ref.fp8_query(q)
    q32 = q.astype(np.float32).astype(np.float64)
    for lo, hi in [(0, 128), (128, 256), (256, 384), (384, 448)]:
        blk = q32[:, lo:hi]
        s = 2.0 ** np.ceil(np.log2(np.max(np.abs(blk), axis=1, keepdims=True) / 448.0))
        step = 2.0 ** np.floor(np.log2(np.maximum(np.abs(blk) / s, 2.0 ** -6))) * 2.0 ** -3
        assert np.all(np.abs(v[:, lo:hi] - blk) <= step / 2 * s + 1e-300)
    assert np.array_equal(v[:, 448:], codecs.bf16_round(q[:, 448:]).astype(np.float64))
    keys = rng.standard_normal((40, 512))
    sc = 1 / math.sqrt(512)
    o_a, _ = ref.attend(v[:1], keys, sc)
    o_b, _ = ref.attend(q32[:1], keys, sc)
    dl = np.max(np.abs(keys @ (v[0] - q32[0]))) * sc
    assert np.max(np.abs(o_a - o_b)) <= 2 * dl * np.max(np.abs(keys)) + 1e-12
