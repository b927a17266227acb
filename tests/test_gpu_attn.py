"""csa_sparse_mqa_attn and csa_swa_merge against the oracle's attention.

The selected-entry lists come from the oracle (or from seeded draws), so the
comparison isolates the attention step."""
import math

import numpy as np
import pytest
import torch

from long_context_compressed_kv_amd import ops
from long_context_compressed_kv_amd.ops import BF16, F32, KV, Batch
from oracle import csa as ref

from gpu_inputs import dev_f32, dev_kv, ref_vals, to_np

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _prefill_case(rng, T, H, D, n_ent, m, k, window, q_fmt, kv_fmt, out_fmt, sparse,
                  pos0=0, raw_hist=0, amp=1.0, raw_fmt=None):
    raw_fmt = raw_fmt or q_fmt
    raw = (amp * rng.standard_normal((raw_hist + T, D))).astype(np.float32)
    ent = (amp * rng.standard_normal((n_ent, D))).astype(np.float32)
    q = (amp * rng.standard_normal((T, H, D))).astype(np.float32)
    raw_pos0 = pos0 - raw_hist
    qd, kvd, rd = dev_kv(q.reshape(-1, D), q_fmt), dev_kv(ent, kv_fmt), dev_kv(raw, raw_fmt)
    # (fp8 queries: the oracle's reading of the stored query, ref.fp8_query)
    qv = ref.fp8_query(q) if q_fmt == "fp8_mixed" else ref_vals(q, q_fmt)
    ev, rv = ref_vals(ent, kv_fmt), ref_vals(raw, raw_fmt)
    idx = None
    if sparse:
        idx = np.full((T, k), -1, np.int64)
        for i in range(T):
            t = pos0 + i
            nv = min((t + 1) // m, n_ent)
            cnt = min(k, nv) if i % 5 else max(0, min(k, nv) - 3)    # some short rows
            sel = np.sort(rng.choice(nv, cnt, replace=False)) if cnt else np.zeros(0, np.int64)
            idx[i, :cnt] = sel
    batch = Batch.make([T], [pos0], kv_counts=[n_ent], raw_counts=[raw_hist + T],
                       raw_pos=[raw_pos0])
    out = torch.empty(T * H, D, device="cuda",
                      dtype=torch.float32 if out_fmt == "f32" else torch.bfloat16)
    lse = torch.empty(T * H, device="cuda")
    idx_d = torch.from_numpy(idx.astype(np.int32)).cuda() if sparse else None
    ops.sparse_mqa_attn(qd, H, kvd, idx_d, k if sparse else 0, rd, window, batch, m, out,
                        F32 if out_fmt == "f32" else BF16, lse)
    torch.cuda.synchronize()
    g, gl = to_np(out).reshape(T, H, D), to_np(lse).reshape(T, H)
    sc = 1 / math.sqrt(D)
    err, lerr = 0.0, 0.0
    for i in range(T):
        t = pos0 + i
        nv = min((t + 1) // m, n_ent)
        keys_e = ev[idx[i][idx[i] >= 0]] if sparse else ev[:nv]
        pos = ref.window_positions(t, window)
        keys = np.concatenate([keys_e, rv[pos - raw_pos0]])
        o, l = ref.attend(qv[i], keys, sc)
        err = max(err, np.max(np.abs(g[i] - o)))
        lerr = max(lerr, np.max(np.abs(gl[i] - l)))
    return err, lerr


@pytest.mark.parametrize("T,H,D,n_ent,m,k,window,qf,kvf,of,sparse,pos0,hist", [
    (67, 16, 128, 16, 4, 8, 128, "f32", "f32", "f32", True, 0, 0),     # fp32 CSA, H=16
    (67, 16, 128, 16, 4, 8, 128, "f32", "f32", "f32", False, 0, 0),
    (29, 16, 128, 90, 4, 40, 128, "f32", "f32", "f32", True, 330, 128),
    (301, 64, 128, 18, 16, 0, 128, "bf16", "bf16", "bf16", False, 0, 0),  # HCA-like
    (45, 64, 128, 40, 4, 24, 32, "bf16", "bf16", "f32", True, 0, 0),
    (21, 64, 512, 130, 4, 100, 16, "bf16", "fp8_mixed", "bf16", True, 500, 16),
    (9, 128, 512, 277, 4, 200, 128, "bf16", "fp8_mixed", "bf16", True, 1100, 128),
    (40, 64, 512, 9, 4, 0, 16, "bf16", "fp8_mixed", "f32", False, 0, 0),
    (33, 32, 512, 20, 2, 12, 8, "bf16", "bf16", "bf16", True, 0, 0),
    (37, 128, 512, 600, 4, 0, 64, "bf16", "bf16", "f32", False, 2000, 64),
    (19, 128, 512, 700, 4, 300, 128, "bf16", "bf16", "bf16", True, 2400, 128),
])
def test_attn_prefill(T, H, D, n_ent, m, k, window, qf, kvf, of, sparse, pos0, hist):
    rng = np.random.default_rng(T * 7 + H + D)
    err, lerr = _prefill_case(rng, T, H, D, n_ent, m, k, window, qf, kvf, of, sparse,
                              pos0=pos0, raw_hist=hist)
    # bf16 compute (bf16 operands and probabilities, fp32 accumulation) is held
    # to the bf16 bound whatever the output format; fp32 compute to 1e-4
    tol = TOL["bf16"] if qf == "bf16" else TOL["f32"]
    assert err <= tol, err
    assert lerr <= (1e-4 if qf == "f32" else 2e-2), lerr


@pytest.mark.parametrize("T,H,D,n_ent,m,k,window,qf,kvf,sparse,pos0,hist", [
    (67, 16, 128, 16, 4, 8, 128, "f32", "f32", True, 0, 0),
    (301, 64, 128, 18, 16, 0, 128, "bf16", "bf16", False, 0, 0),
    (45, 64, 128, 40, 4, 24, 32, "bf16", "bf16", True, 0, 0),
    (21, 64, 512, 130, 4, 100, 16, "bf16", "fp8_mixed", True, 500, 16),
    (9, 128, 512, 277, 4, 200, 128, "bf16", "fp8_mixed", True, 1100, 128),
    (23, 128, 512, 400, 4, 0, 32, "bf16", "fp8_mixed", False, 1500, 32),
])
def test_attn_large_logits(T, H, D, n_ent, m, k, window, qf, kvf, sparse, pos0, hist):
    """Inputs scaled by 6: logits spread over hundreds of units, so a running
    maximum that missed part of a row would overflow the exponentials.  Errors
    are measured relative to the scale of the values (x6) and logits (x36)."""
    amp = 6.0
    rng = np.random.default_rng(T * 11 + H + D)
    err, lerr = _prefill_case(rng, T, H, D, n_ent, m, k, window, qf, kvf, "f32", sparse,
                              pos0=pos0, raw_hist=hist, amp=amp)
    tol = TOL["bf16"] if qf == "bf16" else TOL["f32"]
    assert np.isfinite(err) and err <= tol * amp, err
    assert np.isfinite(lerr) and lerr <= (1e-4 if qf == "f32" else 2e-2) * amp * amp, lerr


@pytest.mark.parametrize("k,window", [(2, 8), (40, 16), (70, 16), (100, 28), (150, 10)])
def test_attn_128_heads_few_tiles(k, window):
    """128 heads over 512 dims with 1 .. 5 key tiles of 32 (the pipelined
    path's start-up and drain), the last tile ragged."""
    rng = np.random.default_rng(k + window)
    err, lerr = _prefill_case(rng, 6, 128, 512, 300, 4, k, window, "bf16", "fp8_mixed", "bf16",
                              True, pos0=1000, raw_hist=window)
    assert err <= 2e-2 and lerr <= 2e-2, (err, lerr)


def test_attn_chunk_with_history():
    """Queries at positions 1000.. with 128 history rows in the raw buffer."""
    rng = np.random.default_rng(3)
    err, lerr = _prefill_case(rng, 40, 128, 512, 260, 4, 64, 128, "bf16", "fp8_mixed", "bf16",
                              True, pos0=1000, raw_hist=128)
    assert err <= 2e-2 and lerr <= 2e-2


@pytest.mark.parametrize("H,sparse,k,window,n_ent,T", [
    (128, True, 100, 128, 400, 20), (64, True, 40, 16, 300, 9), (128, False, 0, 128, 200, 12),
    (64, False, 0, 28, 90, 7), (128, True, 2, 8, 300, 6)])
def test_attn_fp8_queries_prefill(H, sparse, k, window, n_ent, T):
    """fp8 queries (stored like KV entries): the NoPE logits of entry tiles on
    the fp8 matrix cores, tiles holding window rows in bf16; against the
    oracle's attention of the stored query values (ref.fp8_query) over the
    same keys.  Tiles of entries only, of entries and window rows, of window
    rows only; selected and dense entries; 64 and 128 heads."""
    rng = np.random.default_rng(H + k + window + n_ent)
    print(f"[attn] fp8 queries prefill H={H} sparse={sparse} k={k} window={window}", flush=True)
    err, lerr = _prefill_case(rng, T, H, 512, n_ent, 4, k, window, "fp8_mixed", "fp8_mixed", "bf16",
                              sparse, pos0=1600, raw_hist=window, raw_fmt="bf16")
    assert err <= 2e-2 and lerr <= 2e-2, (err, lerr)


@pytest.mark.parametrize("H,sparse,split_keys", [(64, True, 288), (64, False, 96), (128, True, 128)])
def test_attn_fp8_queries_decode_split(H, sparse, split_keys):
    """fp8 queries at decode, split over keys and merged: ragged contexts,
    rows shorter than k, against the oracle."""
    rng = np.random.default_rng(H + split_keys)
    D, m, k, window = 512, 4, 200, 128
    ctxs = [3000, 50, 999, 12000, 400]
    B = len(ctxs)
    n_ent = [(c + 1) // m for c in ctxs]
    swa_len = [min(window, c + 1) for c in ctxs]
    ents = [rng.standard_normal((n, D)).astype(np.float32) for n in n_ent]
    swas = [rng.standard_normal((s, D)).astype(np.float32) for s in swa_len]
    q = rng.standard_normal((B, H, D)).astype(np.float32)
    idx = np.full((B, k), -1, np.int64)
    for r in range(B):
        cnt = min(k, n_ent[r]) - (5 if r == 2 else 0)
        idx[r, :cnt] = np.sort(rng.choice(n_ent[r], cnt, replace=False))
    batch = Batch.make([1] * B, ctxs, kv_counts=n_ent, raw_counts=swa_len,
                       raw_pos=[c - s + 1 for c, s in zip(ctxs, swa_len)])
    out = torch.empty(B * H, D, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(B * H, device="cuda")
    idx_d = torch.from_numpy(idx.astype(np.int32)).cuda() if sparse else None
    print(f"[attn] fp8 queries decode H={H} sparse={sparse} split={split_keys}", flush=True)
    ops.sparse_mqa_attn(dev_kv(q.reshape(-1, D), "fp8_mixed"), H, dev_kv(np.concatenate(ents), "fp8_mixed"),
                        idx_d, k if sparse else 0, dev_kv(np.concatenate(swas), "bf16"), window, batch, m,
                        out, BF16, lse, split_keys=split_keys)
    torch.cuda.synchronize()
    qv, sc = ref.fp8_query(q), 1 / math.sqrt(D)
    for r in range(B):
        ev, sv = ref_vals(ents[r], "fp8_mixed"), ref_vals(swas[r], "bf16")
        ke = ev[idx[r][idx[r] >= 0]] if sparse else ev
        o, l = ref.attend(qv[r], np.concatenate([ke, sv]), sc)
        sl = slice(r * H, (r + 1) * H)
        assert np.max(np.abs(to_np(out[sl]) - o)) <= 2e-2
        assert np.max(np.abs(to_np(lse[sl]) - l)) <= 2e-2


def _decode_case(rng, ctxs, H, D, m, k, window, kv_fmt, amp=1.0):
    B = len(ctxs)
    n_ent = [(c + 1) // m for c in ctxs]
    swa_len = [min(window, c + 1) for c in ctxs]
    ents = [(amp * rng.standard_normal((n, D))).astype(np.float32) for n in n_ent]
    swas = [(amp * rng.standard_normal((s, D))).astype(np.float32) for s in swa_len]
    q = (amp * rng.standard_normal((B, H, D))).astype(np.float32)
    idx = np.full((B, k), -1, np.int64)
    for r in range(B):
        cnt = min(k, n_ent[r])
        idx[r, :cnt] = np.sort(rng.choice(n_ent[r], cnt, replace=False))
    ent_all, swa_all = np.concatenate(ents), np.concatenate(swas)
    kvd, sd, qd = dev_kv(ent_all, kv_fmt), dev_kv(swa_all, "bf16"), dev_kv(q.reshape(-1, D), "bf16")
    batch = Batch.make([1] * B, ctxs, kv_counts=n_ent, raw_counts=swa_len,
                       raw_pos=[c - s + 1 for c, s in zip(ctxs, swa_len)])
    rows = B * H
    oc, lc = torch.empty(rows, D, device="cuda"), torch.empty(rows, device="cuda")
    ow, lw = torch.empty(rows, D, device="cuda"), torch.empty(rows, device="cuda")
    ou, lu = torch.empty(rows, D, device="cuda"), torch.empty(rows, device="cuda")
    idx_d = torch.from_numpy(idx.astype(np.int32)).cuda()
    ops.sparse_mqa_attn(qd, H, kvd, idx_d, k, None, 0, batch, m, oc, F32, lc)
    ops.sparse_mqa_attn(qd, H, None, None, 0, sd, window, batch, m, ow, F32, lw)
    ops.sparse_mqa_attn(qd, H, kvd, idx_d, k, sd, window, batch, m, ou, F32, lu)
    om, lm = torch.empty(rows, D, device="cuda"), torch.empty(rows, device="cuda")
    ops.swa_merge(oc, lc, ow, lw, om, F32, lm)
    torch.cuda.synchronize()
    sc = 1 / math.sqrt(D)
    qv = ref_vals(q, "bf16")
    errs = []
    for r in range(B):
        ev, sv = ref_vals(ents[r], kv_fmt), ref_vals(swas[r], "bf16")
        keys = np.concatenate([ev[idx[r][idx[r] >= 0]], sv[-min(window, ctxs[r] + 1):]])
        o, l = ref.attend(qv[r], keys, sc)
        sl = slice(r * H, (r + 1) * H)
        errs.append(max(np.max(np.abs(to_np(om[sl]) - o)), np.max(np.abs(to_np(ou[sl]) - o)),
                        np.max(np.abs(to_np(lm[sl]) - l))))
    return max(errs), (om, ou)


def test_attn_decode_split_merge_equals_union():
    rng = np.random.default_rng(4)
    err, (om, ou) = _decode_case(rng, [5000, 131, 40, 2047, 700], 64, 512, 4, 64, 128, "fp8_mixed")
    assert err <= 2e-2
    # split + merge and the one-kernel union round the probabilities to bf16
    # against different running maxima: both are within the bf16 bound
    assert torch.max(torch.abs(om - ou)).item() <= 2e-2


@pytest.mark.parametrize("split_keys,kv_fmt,sparse,amp", [
    (32, "fp8_mixed", True, 1.0), (64, "fp8_mixed", False, 1.0), (128, "bf16", True, 1.0),
    (1, "fp8_mixed", True, 1.0), (64, "fp8_mixed", True, 6.0)])
def test_attn_decode_split_k(split_keys, kv_fmt, sparse, amp):
    """Split-K over key chunks merged by log-sum-exp equals the oracle (amp = 6:
    logits spread over hundreds of units, errors relative to that scale)."""
    rng = np.random.default_rng(40 + split_keys + int(amp))
    H, D, m, k, window = 64, 512, 4, 100, 128
    ctxs = [3000, 50, 999, 400, 127, 20000]
    B = len(ctxs)
    n_ent = [(c + 1) // m for c in ctxs]
    swa_len = [min(window, c + 1) for c in ctxs]
    ents = [(amp * rng.standard_normal((n, D))).astype(np.float32) for n in n_ent]
    swas = [(amp * rng.standard_normal((s, D))).astype(np.float32) for s in swa_len]
    q = (amp * rng.standard_normal((B, H, D))).astype(np.float32)
    idx = np.full((B, k), -1, np.int64)
    for r in range(B):
        cnt = min(k, n_ent[r]) - (3 if r == 1 else 0)
        idx[r, :cnt] = np.sort(rng.choice(n_ent[r], cnt, replace=False))
    kvd = dev_kv(np.concatenate(ents), kv_fmt)
    sd, qd = dev_kv(np.concatenate(swas), "bf16"), dev_kv(q.reshape(-1, D), "bf16")
    batch = Batch.make([1] * B, ctxs, kv_counts=n_ent, raw_counts=swa_len,
                       raw_pos=[c - s + 1 for c, s in zip(ctxs, swa_len)])
    out = torch.empty(B * H, D, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(B * H, device="cuda")
    idx_d = torch.from_numpy(idx.astype(np.int32)).cuda() if sparse else None
    ops.sparse_mqa_attn(qd, H, kvd, idx_d, k if sparse else 0, sd, window, batch, m, out, BF16,
                        lse, split_keys=split_keys)
    torch.cuda.synchronize()
    qv, sc = ref_vals(q, "bf16"), 1 / math.sqrt(D)
    worst = 0.0
    for r in range(B):
        ev, sv = ref_vals(ents[r], kv_fmt), ref_vals(swas[r], "bf16")
        ke = ev[idx[r][idx[r] >= 0]] if sparse else ev
        o, l = ref.attend(qv[r], np.concatenate([ke, sv]), sc)
        sl = slice(r * H, (r + 1) * H)
        worst = max(worst, np.max(np.abs(to_np(out[sl]) - o)) / amp,
                    np.max(np.abs(to_np(lse[sl]) - l)) / (amp * amp))
    assert np.isfinite(worst) and worst <= 2e-2, worst


@pytest.mark.parametrize("H,sparse,split_keys", [(32, True, 128), (96, False, 160), (32, False, 1)])
def test_attn_decode_split_other_head_counts(H, sparse, split_keys):
    """D = 512 split over keys with head counts the 16-heads-per-wave kernel
    does not take (32, 96: the general kernel with its plan of work items),
    ragged contexts, against the oracle."""
    rng = np.random.default_rng(H + split_keys + int(sparse))
    D, m, k, window = 512, 4, 120, 128
    ctxs = [2500, 40, 900, 6000]
    B = len(ctxs)
    n_ent = [(c + 1) // m for c in ctxs]
    swa_len = [min(window, c + 1) for c in ctxs]
    ents = [rng.standard_normal((n, D)).astype(np.float32) for n in n_ent]
    swas = [rng.standard_normal((s, D)).astype(np.float32) for s in swa_len]
    q = rng.standard_normal((B, H, D)).astype(np.float32)
    idx = np.full((B, k), -1, np.int64)
    for r in range(B):
        cnt = min(k, n_ent[r])
        idx[r, :cnt] = np.sort(rng.choice(n_ent[r], cnt, replace=False))
    batch = Batch.make([1] * B, ctxs, kv_counts=n_ent, raw_counts=swa_len,
                       raw_pos=[c - s + 1 for c, s in zip(ctxs, swa_len)])
    out = torch.empty(B * H, D, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(B * H, device="cuda")
    idx_d = torch.from_numpy(idx.astype(np.int32)).cuda() if sparse else None
    print(f"[attn] split, {H} heads, sparse={sparse}, split_keys={split_keys}", flush=True)
    ops.sparse_mqa_attn(dev_kv(q.reshape(-1, D), "bf16"), H, dev_kv(np.concatenate(ents), "fp8_mixed"),
                        idx_d, k if sparse else 0, dev_kv(np.concatenate(swas), "bf16"), window, batch, m,
                        out, BF16, lse, split_keys=split_keys)
    torch.cuda.synchronize()
    qv, sc = ref_vals(q, "bf16"), 1 / math.sqrt(D)
    for r in range(B):
        ev, sv = ref_vals(ents[r], "fp8_mixed"), ref_vals(swas[r], "bf16")
        ke = ev[idx[r][idx[r] >= 0]] if sparse else ev
        o, l = ref.attend(qv[r], np.concatenate([ke, sv]), sc)
        sl = slice(r * H, (r + 1) * H)
        assert np.max(np.abs(to_np(out[sl]) - o)) <= 2e-2
        assert np.max(np.abs(to_np(lse[sl]) - l)) <= 2e-2


@pytest.mark.parametrize("q_fmt", ["bf16", "fp8_mixed"])
def test_attn_split_request_without_keys(q_fmt):
    """Split-K at D = 512: a request with no keys at all (no entries, no
    window rows) between two that have many: its rows are o = 0 and
    lse = -inf, the others match the oracle (dense keys, parts of several
    lengths, the short request's missing parts skipped); bf16 and fp8
    queries."""
    rng = np.random.default_rng(77)
    H, D, m, window = 64, 512, 4, 128
    ctxs = [9000, 2, 700]
    n_ent = [2250, 0, 175]
    swa_len = [128, 0, 128]
    ents = [rng.standard_normal((n, D)).astype(np.float32) for n in n_ent if n]
    swas = [rng.standard_normal((s, D)).astype(np.float32) for s in swa_len if s]
    q = rng.standard_normal((3, H, D)).astype(np.float32)
    batch = Batch.make([1] * 3, ctxs, kv_counts=n_ent, raw_counts=swa_len,
                       raw_pos=[c - s + 1 for c, s in zip(ctxs, swa_len)])
    out = torch.full((3 * H, D), 5.0, device="cuda")
    lse = torch.zeros(3 * H, device="cuda")
    print(f"[attn] split over keys, request without keys, {q_fmt} queries", flush=True)
    ops.sparse_mqa_attn(dev_kv(q.reshape(-1, D), q_fmt), H, dev_kv(np.concatenate(ents), "fp8_mixed"),
                        None, 0, dev_kv(np.concatenate(swas), "bf16"), window, batch, m, out, F32,
                        lse, split_keys=96)
    torch.cuda.synchronize()
    qv = ref.fp8_query(q) if q_fmt == "fp8_mixed" else ref_vals(q, "bf16")
    sc = 1 / math.sqrt(D)
    assert torch.all(out[H:2 * H] == 0)
    assert torch.all(torch.isneginf(lse[H:2 * H]))
    for r, (e, s) in ((0, (ents[0], swas[0])), (2, (ents[1], swas[1]))):
        o, l = ref.attend(qv[r], np.concatenate([ref_vals(e, "fp8_mixed"), ref_vals(s, "bf16")]), sc)
        sl = slice(r * H, (r + 1) * H)
        assert np.max(np.abs(to_np(out[sl]) - o)) <= 2e-2
        assert np.max(np.abs(to_np(lse[sl]) - l)) <= 2e-2


def test_attn_window_only_and_empty_rows():
    """No entries and window 0 for some rows: o = 0, lse = -inf."""
    H, D = 32, 128
    q = dev_kv(np.random.default_rng(1).standard_normal((2 * H, D)).astype(np.float32), "bf16")
    batch = Batch.make([2], [0], kv_counts=[0], raw_counts=[2], raw_pos=[0])
    out = torch.full((2 * H, D), 7.0, device="cuda")
    lse = torch.zeros(2 * H, device="cuda")
    kv = dev_kv(np.zeros((1, D), np.float32), "bf16")
    ops.sparse_mqa_attn(q, H, kv, None, 0, None, 0, batch, 4, out, F32, lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isinf(lse)) and torch.all(lse < 0)


def test_swa_merge_random_and_infinite():
    rng = np.random.default_rng(9)
    rows, D = 1000, 512
    oa, ob = rng.standard_normal((rows, D)), rng.standard_normal((rows, D))
    la, lb = rng.standard_normal(rows) * 5, rng.standard_normal(rows) * 5
    la[:10] = -np.inf
    lb[5:15] = -np.inf
    out = torch.empty(rows, D, device="cuda")
    lo = torch.empty(rows, device="cuda")
    ops.swa_merge(dev_f32(oa), dev_f32(la), dev_f32(ob), dev_f32(lb), out, F32, lo)
    outb = torch.empty(rows, D, device="cuda", dtype=torch.bfloat16)
    ops.swa_merge(dev_f32(oa), dev_f32(la), dev_f32(ob), dev_f32(lb), outb, BF16)
    torch.cuda.synchronize()
    fa, fb = oa.astype(np.float32).astype(np.float64), ob.astype(np.float32).astype(np.float64)
    la32, lb32 = la.astype(np.float32).astype(np.float64), lb.astype(np.float32).astype(np.float64)
    with np.errstate(invalid="ignore"):
        o, l = ref.merge(fa, la32, fb, lb32)
    both = np.isinf(la32) & np.isinf(lb32)
    o[both] = 0.0
    g, gl = to_np(out), to_np(lo)
    assert np.max(np.abs(g - o)) <= 1e-5
    assert np.all(np.isneginf(gl[both]))
    assert np.max(np.abs(gl[~both] - l[~both])) <= 1e-5
    assert np.max(np.abs(to_np(outb) - o)) <= 2e-2


def test_attn_deterministic_and_batch_invariant():
    """A request's output is bitwise the same alone and inside a batch."""
    rng = np.random.default_rng(10)
    H, D, m, k = 64, 512, 4, 32
    ctxs = [900, 300, 1500]
    n_ent = [(c + 1) // m for c in ctxs]
    ents = [rng.standard_normal((n, D)).astype(np.float32) for n in n_ent]
    q = rng.standard_normal((3, H, D)).astype(np.float32)
    idx = np.stack([np.sort(rng.choice(n, k, replace=False)) for n in n_ent]).astype(np.int32)

    def run(order):
        e = np.concatenate([ents[r] for r in order])
        kvd = dev_kv(e, "fp8_mixed")
        qd = dev_kv(q[order].reshape(-1, D), "bf16")
        b = Batch.make([1] * len(order), [ctxs[r] for r in order],
                       kv_counts=[n_ent[r] for r in order])
        out = torch.empty(len(order) * H, D, device="cuda")
        ops.sparse_mqa_attn(qd, H, kvd, torch.from_numpy(idx[order]).cuda(), k, None, 0, b, m,
                            out, F32)
        torch.cuda.synchronize()
        return out.view(len(order), H, D)

    a = run([0, 1, 2])
    b = run([2, 0, 1])
    c = run([1])
    assert torch.equal(a[0], b[1]) and torch.equal(a[2], b[0]) and torch.equal(a[1], c[0])
    assert torch.equal(a, run([0, 1, 2]))


def test_attn_decode_largest_selection_and_heads():
    """The largest sizes the call takes at decode: k = 4096 selected entries,
    128 heads (two head groups when split over keys), D = 512 mixed entries
    with the 128-token window; one union call, split-K, against the oracle."""
    rng = np.random.default_rng(12)
    H, D, m, k, window = 128, 512, 4, 4096, 128
    ctxs = [40000, 20000, 9000]
    n_ent = [(c + 1) // m for c in ctxs]
    ents = [rng.standard_normal((n, D)).astype(np.float32) for n in n_ent]
    swas = [rng.standard_normal((window, D)).astype(np.float32) for _ in ctxs]
    q = rng.standard_normal((len(ctxs), H, D)).astype(np.float32)
    idx = np.full((len(ctxs), k), -1, np.int32)
    for r, n in enumerate(n_ent):
        c = min(k, n) - 7 * r                      # one full row, two shorter ones
        idx[r, :c] = np.sort(rng.choice(n, c, replace=False))
    batch = Batch.make([1] * len(ctxs), ctxs, kv_counts=n_ent, raw_counts=[window] * len(ctxs),
                       raw_pos=[c - window + 1 for c in ctxs])
    out = torch.empty(len(ctxs) * H, D, device="cuda")
    lse = torch.empty(len(ctxs) * H, device="cuda")
    ops.sparse_mqa_attn(dev_kv(q.reshape(-1, D), "bf16"), H, dev_kv(np.concatenate(ents), "fp8_mixed"),
                        torch.from_numpy(idx).cuda(), k, dev_kv(np.concatenate(swas), "bf16"), window,
                        batch, m, out, F32, lse, split_keys=128)
    torch.cuda.synchronize()
    qv, sc = ref_vals(q, "bf16"), 1 / math.sqrt(D)
    for r in range(len(ctxs)):
        keys = np.concatenate([ref_vals(ents[r], "fp8_mixed")[idx[r][idx[r] >= 0]],
                               ref_vals(swas[r], "bf16")])
        o, l = ref.attend(qv[r], keys, sc)
        sl = slice(r * H, (r + 1) * H)
        assert np.max(np.abs(to_np(out[sl]) - o)) <= 2e-2
        assert np.max(np.abs(to_np(lse[sl]) - l)) <= 2e-2
