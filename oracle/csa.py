"""Plain CPU oracle of the CSA / HCA compressed-attention layer.

TEST INFRASTRUCTURE. Nothing in the product path may import this module; only
the tests, the smoke check and the CPU-baseline leg of the benchmark use it.
It shares no code with the HIP library: it is NumPy in float64, one query at a
time, with no blocking or fusion beyond what each definition states.

The method (page "DeepSeek V4 深度解析", section 2 "核心技術創新", the three
CSA steps and the HCA paragraph; page "wmrh.cn/news/726125", "V4 改进一"):

1. compression: every m raw tokens' KV become one entry, a softmax-weighted
   sum with one learned weight per raw token plus a position bias; adjacent
   compressed blocks overlap a little;
2. a low-rank lightning indexer scores each query against the entries and the
   query keeps the top-k of them (k = 512 Flash, 1024 Pro);
3. a sliding-window branch keeps the latest 128 uncompressed tokens, attended
   together with the selected entries, as shared-KV multi-query attention.
HCA compresses at m' = 128, selects nothing, and attends densely, with the same
window branch.

Readings where the pages are silent (each is a named constant or argument):

* window and stride: entry i covers raw positions (i+1)m - w .. (i+1)m - 1
  (w = 2m: its own block and the previous one); slots before position 0 are
  left out of the softmax, not zero-padded;
* weights: softmax over the valid slots s of z[p] + b[s], one scalar logit
  per raw token and one bias per window slot (compress_entries_channel is the
  variant with a logit and a bias per channel, one softmax per channel);
* visibility: entry i is usable by the query at t once its block is complete,
  (i+1)m - 1 <= t, so n_c(t) = floor((t+1)/m) entries are visible;
* indexer: one shared d_I-dim key per entry; S = sum_h w_h ReLU(q_h . k)
  (w = 1 unless given; relu=False gives the linear form);
* top-k: order by (score desc, index asc) over the visible entries, keep
  min(k, n_c) of them, return them in ascending index order padded with -1;
* window: positions max(0, t-W+1) .. t, the query's own token included;
* attention: one softmax over the union of the selected (or, for HCA, all
  visible) entries and the window tokens; key = value = the same vector
  (shared-KV MQA); logits scaled by 1/sqrt(D);
* merge of two partial results over disjoint key sets by log-sum-exp.
"""
import math

import numpy as np

from . import codecs

SWA_WINDOW = 128


# ----------------------------------------------------------------------------
# Step 1: compression (page "DeepSeek V4 深度解析", CSA step 1; HCA paragraph)
# ----------------------------------------------------------------------------


def n_visible(t, m):
    """Number of compressed entries complete at query position t."""
    return (np.asarray(t, dtype=np.int64) + 1) // m


def compress_entries(x, z, x_pos0, b, m, w, i_begin, i_end):
    """Compressed entries i_begin .. i_end-1 in float64.

    x  : raw KV rows [n, D] for absolute positions x_pos0 .. x_pos0+n-1
    z  : per-token compression logits [n]
    b  : per-slot position biases [w]
    Entry i: slots s in [0, w) map to p = (i+1)m - w + s; slots with p < 0 are
    invalid and dropped; the weights are softmax_s(z[p] + b[s]) over the
    valid slots and the entry is sum_s weight_s * x[p].
    """
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert b.shape == (w,) and w >= m >= 1
    out = np.empty((i_end - i_begin, x.shape[1]), dtype=np.float64)
    for i in range(i_begin, i_end):
        p = (i + 1) * m - w + np.arange(w)
        valid = p >= 0
        p, s = p[valid], np.arange(w)[valid]
        assert p[0] >= x_pos0 and p[-1] < x_pos0 + x.shape[0], "raw rows missing"
        logit = z[p - x_pos0] + b[s]
        wgt = np.exp(logit - logit.max())
        wgt /= wgt.sum()
        out[i - i_begin] = wgt @ x[p - x_pos0]
    return out


def compress_entries_channel(x, z, x_pos0, b, m, w, i_begin, i_end):
    """Compressed entries with one compression logit per raw token and
    channel (page "DeepSeek V4 深度解析", section 2, CSA step 1, read with a
    learned weight per token and channel instead of one per token).

    x  : raw KV rows [n, D] for absolute positions x_pos0 .. x_pos0+n-1
    z  : compression logits [n, D]
    b  : position biases [w, D], one per window slot and channel
    Entry i covers the slots of compress_entries; for every channel d the
    weights are softmax_s(z[p][d] + b[s][d]) over the valid slots and the
    entry's channel d is sum_s weight_s,d * x[p][d].
    """
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert z.shape == x.shape and b.shape == (w, x.shape[1]) and w >= m >= 1
    out = np.empty((i_end - i_begin, x.shape[1]), dtype=np.float64)
    for i in range(i_begin, i_end):
        p = (i + 1) * m - w + np.arange(w)
        valid = p >= 0
        p, s = p[valid], np.arange(w)[valid]
        assert p[0] >= x_pos0 and p[-1] < x_pos0 + x.shape[0], "raw rows missing"
        logit = z[p - x_pos0] + b[s]                        # [slots, D]
        wgt = np.exp(logit - logit.max(axis=0))
        wgt /= wgt.sum(axis=0)
        out[i - i_begin] = (wgt * x[p - x_pos0]).sum(axis=0)
    return out


def store_entries(c, fmt):
    """Round float64 entries to the cache format.  Returns the stored form:
    'f32' -> fp32 array; 'bf16' -> bf16 bit patterns; 'fp8_mixed' ->
    (nope, scale, rope).  Rounding goes through fp32 first, the precision in
    which an fp32-accumulating implementation holds the entry."""
    c32 = np.asarray(c, dtype=np.float32)
    if fmt == "f32":
        return c32
    if fmt == "bf16":
        return codecs.bf16_bits(c32)
    if fmt == "fp8_mixed":
        return codecs.quantize_kv_mixed(c32)
    raise ValueError(fmt)


def load_entries(stored, fmt):
    """Stored cache rows -> float64 values (exact)."""
    if fmt == "f32":
        return np.asarray(stored, dtype=np.float64)
    if fmt == "bf16":
        return codecs.bf16_to_f32(stored).astype(np.float64)
    if fmt == "fp8_mixed":
        return codecs.dequantize_kv_mixed(*stored)
    raise ValueError(fmt)


# ----------------------------------------------------------------------------
# Step 2: lightning indexer and top-k (CSA step 2; BF16 indexer scores)
# ----------------------------------------------------------------------------


def indexer_scores(qi, ki, head_w=None, relu=True):
    """Scores of one query against entries.

    qi : [H_I, d_I] query heads of the indexer (float64 values)
    ki : [n, d_I]   one indexer key per entry
    returns float64 [n]: sum_h w_h * ReLU(qi[h] . ki[j])."""
    qi = np.asarray(qi, dtype=np.float64)
    ki = np.asarray(ki, dtype=np.float64)
    h_i = qi.shape[0]
    w = np.ones(h_i) if head_w is None else np.asarray(head_w, dtype=np.float64)
    dots = ki @ qi.T                                  # [n, H_I]
    if relu:
        dots = np.maximum(dots, 0.0)
    return dots @ w


def score_keys(s, score_fmt):
    """The comparison key of each score: the float64 score rounded to fp32,
    then, for 'bf16' scores, to bf16 (round to nearest-even)."""
    s32 = np.asarray(s, dtype=np.float32)
    if score_fmt == "f32":
        return s32
    if score_fmt == "bf16":
        return codecs.bf16_round(s32)
    raise ValueError(score_fmt)


def topk_indices(keys, k):
    """Indices of the min(k, n) largest keys, ties by lower index, returned in
    ascending index order and padded with -1 to length k."""
    keys = np.asarray(keys)
    n = keys.shape[0]
    order = np.lexsort((np.arange(n), -keys.astype(np.float64)))
    chosen = np.sort(order[: min(k, n)])
    out = np.full(k, -1, dtype=np.int64)
    out[: chosen.shape[0]] = chosen
    return out


# ----------------------------------------------------------------------------
# Step 3: shared-KV MQA over entries and the sliding window (CSA step 3; HCA)
# ----------------------------------------------------------------------------


def window_positions(t, window):
    """Raw positions of the sliding window of the query at t: max(0, t-W+1)..t."""
    return np.arange(max(t - window + 1, 0), t + 1, dtype=np.int64)


def _window_rows(t, window, raw, raw_pos0):
    pos = window_positions(t, window)
    if pos.size:
        assert pos[0] >= raw_pos0 and pos[-1] < raw_pos0 + len(raw), "window rows missing"
    return np.asarray(raw, np.float64)[pos - raw_pos0]


def fp8_query(q):
    """Query rows as the fp8-Q attention variant sees them (page "DeepSeek V4
    深度解析", section 2, the mixed-precision paragraph: RoPE dims BF16, the rest
    FP8; read here for the query side as well): each row is stored like a KV
    entry, its 448 non-RoPE dims as e4m3 codes with a power-of-two scale per
    128-dim block and its 64 RoPE dims in bf16, and the logits use the stored
    values exactly.  q [..., 512] -> float64 values of the same shape."""
    a = np.asarray(q, np.float32)
    rows = a.reshape(-1, a.shape[-1])
    return codecs.dequantize_kv_mixed(*codecs.quantize_kv_mixed(rows)).reshape(a.shape)


def attend(q, keys, scale):
    """Shared-KV multi-query attention of one query token.

    q    : [H, D] query heads
    keys : [n, D] the key vectors; each is also its own value
    returns (o [H, D], lse [H]) in float64; lse is the natural log-sum-exp
    of the scaled logits."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    logits = (q @ keys.T) * scale                     # [H, n]
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    denom = e.sum(axis=1, keepdims=True)
    o = (e / denom) @ keys
    lse = (mx + np.log(denom))[:, 0]
    return o, lse


def merge(o_a, lse_a, o_b, lse_b):
    """Combine two partial attentions over disjoint key sets."""
    o_a, o_b = np.asarray(o_a, np.float64), np.asarray(o_b, np.float64)
    lse_a, lse_b = np.asarray(lse_a, np.float64), np.asarray(lse_b, np.float64)
    mx = np.maximum(lse_a, lse_b)
    wa = np.exp(lse_a - mx)
    wb = np.exp(lse_b - mx)
    den = wa + wb
    o = (wa[..., None] * o_a + wb[..., None] * o_b) / den[..., None]
    return o, mx + np.log(den)


def default_scale(d):
    return 1.0 / math.sqrt(d)


# ----------------------------------------------------------------------------
# One query of a layer
# ----------------------------------------------------------------------------


def csa_query(t, q, entries, qi, ki, k, m, raw, raw_pos0, window=SWA_WINDOW,
              head_w=None, relu=True, score_fmt="f32", scale=None):
    """CSA output of the query token at absolute position t.

    entries : float64 [N, D] compressed entries of the sequence (entry j = row j)
    ki      : [N, d_I] indexer keys; qi : [H_I, d_I] indexer query of t
    raw     : raw KV rows for positions raw_pos0 .. (window source)
    Returns dict(o, lse, idx, keys) for the query."""
    n_c = min(int(n_visible(t, m)), entries.shape[0])
    s = indexer_scores(qi, ki[:n_c], head_w, relu)
    keys = score_keys(s, score_fmt)
    idx = topk_indices(keys, k)
    sel = idx[idx >= 0]
    kv = np.concatenate([entries[sel], _window_rows(t, window, raw, raw_pos0)])
    scale = default_scale(q.shape[1]) if scale is None else scale
    o, lse = attend(q, kv, scale)
    return {"o": o, "lse": lse, "idx": idx, "keys": keys}


def hca_query(t, q, entries, m, raw, raw_pos0, window=SWA_WINDOW, scale=None):
    """HCA output of the query token at t: all visible entries plus the window."""
    n_c = min(int(n_visible(t, m)), entries.shape[0])
    kv = np.concatenate([entries[:n_c], _window_rows(t, window, raw, raw_pos0)])
    scale = default_scale(q.shape[1]) if scale is None else scale
    o, lse = attend(q, kv, scale)
    return {"o": o, "lse": lse}
