"""D = 128 prefill attention over thousands of token groups (more groups than
the device holds workgroups at once), checked on sampled query tokens against
the oracle: groups with one key tile and with many, requests that see no key
at all between requests that do, selected entries, and window rows kept as a
ring."""
import dataclasses
import math

import numpy as np
import pytest
import torch

from long_context_compressed_kv_amd import ops
from long_context_compressed_kv_amd.ops import BF16, F32, Batch
from oracle import csa as ref

from gpu_inputs import dev_kv, ref_vals, to_np

pytestmark = pytest.mark.gpu


def _requests(rng, reqs, H, D, m, window, sparse, k):
    """reqs: (tokens, first position, entries, raw history rows, has raw rows)
    per request.  Returns host arrays and the device call's inputs."""
    q = rng.standard_normal((sum(r[0] for r in reqs), H, D)).astype(np.float32)
    ents, raws, idx_rows, meta = [], [], [], []
    for T, pos0, n_ent, hist, has_raw in reqs:
        ents.append(rng.standard_normal((n_ent, D)).astype(np.float32))
        n_raw = hist + T if has_raw else 0
        raws.append(rng.standard_normal((n_raw, D)).astype(np.float32))
        for i in range(T):
            t = pos0 + i
            nv = min((t + 1) // m, n_ent)
            row = np.full(max(k, 1), -1, np.int64)
            if sparse and nv:
                cnt = min(k, nv) if i % 3 else max(0, min(k, nv) - 5)   # some short rows
                row[:cnt] = np.sort(rng.choice(nv, cnt, replace=False))
            idx_rows.append(row)
        meta.append((T, pos0, n_ent, pos0 - hist, n_raw))
    return q, ents, raws, np.stack(idx_rows), meta


def _oracle_token(qv, ev, rv, meta_r, i, idx_row, m, window, sparse):
    T, pos0, n_ent, raw_pos0, n_raw = meta_r
    t = pos0 + i
    nv = min((t + 1) // m, n_ent)
    keys_e = ev[idx_row[idx_row >= 0]] if sparse else ev[:nv]
    pos = ref.window_positions(t, window) if n_raw else np.zeros(0, np.int64)
    keys = np.concatenate([keys_e, rv[pos - raw_pos0]]) if len(pos) else keys_e
    if len(keys) == 0:
        return np.zeros(qv.shape), np.full(qv.shape[0], -np.inf)
    return ref.attend(qv, keys, 1 / math.sqrt(qv.shape[1]))


def _run(seed, reqs, H, m, window, sparse=False, k=0, n_sample=160, out_fmt="bf16"):
    D = 128
    rng = np.random.default_rng(seed)
    q, ents, raws, idx, meta = _requests(rng, reqs, H, D, m, window, sparse, k)
    n_q = q.shape[0]
    e_all = np.concatenate(ents) if sum(len(e) for e in ents) else np.zeros((1, D), np.float32)
    r_all = np.concatenate(raws) if sum(len(r) for r in raws) else np.zeros((1, D), np.float32)
    batch = Batch.make([r[0] for r in reqs], [r[1] for r in reqs], kv_counts=[r[2] for r in reqs],
                       raw_counts=[mr[4] for mr in meta], raw_pos=[mr[3] for mr in meta])
    out = torch.empty(n_q * H, D, device="cuda",
                      dtype=torch.bfloat16 if out_fmt == "bf16" else torch.float32)
    lse = torch.empty(n_q * H, device="cuda")
    idx_d = torch.from_numpy(idx[:, :k].astype(np.int32)).cuda() if sparse else None
    ops.sparse_mqa_attn(dev_kv(q.reshape(-1, D), "bf16"), H, dev_kv(e_all, "bf16"), idx_d,
                        k if sparse else 0, dev_kv(r_all, "bf16"), window, batch, m, out,
                        BF16 if out_fmt == "bf16" else F32, lse)
    torch.cuda.synchronize()
    g, gl = to_np(out).reshape(n_q, H, D), to_np(lse).reshape(n_q, H)
    assert np.all(np.isfinite(g))

    # sampled tokens: the first and last of every request, and a seeded draw
    starts = np.cumsum([0] + [r[0] for r in reqs])
    pick = set(rng.choice(n_q, min(n_q, n_sample), replace=False).tolist())
    for r in range(len(reqs)):
        if reqs[r][0]:
            pick.update([int(starts[r]), int(starts[r + 1] - 1)])
    qv = ref_vals(q, "bf16")
    e_off = np.cumsum([0] + [len(e) for e in ents])
    r_off = np.cumsum([0] + [len(x) for x in raws])
    ev_all, rv_all = ref_vals(e_all, "bf16"), ref_vals(r_all, "bf16")
    worst = 0.0
    for qi in sorted(pick):
        r = int(np.searchsorted(starts, qi, side="right") - 1)
        i = qi - int(starts[r])
        o, l = _oracle_token(qv[qi], ev_all[e_off[r]:e_off[r + 1]], rv_all[r_off[r]:r_off[r + 1]],
                             meta[r], i, idx[qi, :k], m, window, sparse)
        if np.all(np.isinf(l)):
            assert np.all(g[qi] == 0) and np.all(np.isneginf(gl[qi])), qi
            continue
        worst = max(worst, np.max(np.abs(g[qi] - o)), np.max(np.abs(gl[qi] - l)))
    assert worst <= 2e-2, worst
    return out, lse


def test_dense_single_request_many_groups():
    """HCA-like: 64 heads, two tokens per group, 3000 groups; the tile count
    per group grows from 2 to 12 along the sequence."""
    _run(21, [(6000, 100, 6100 // 16, 100, True)], 64, 16, 128)


def test_multi_request_with_keyless_requests():
    """128 heads (one token per group); ragged requests, among them requests
    with neither entries nor raw rows (zero output, lse = -inf) placed
    between requests with keys."""
    rng = np.random.default_rng(5)
    reqs = []
    for r in range(40):
        T = int(rng.integers(1, 90))
        pos0 = int(rng.integers(0, 3000))
        if r % 7 == 3:
            reqs.append((T, pos0, 0, 0, False))
        else:
            reqs.append((T, pos0, (pos0 + T) // 4, min(pos0, 130), True))
    _run(22, reqs, 128, 4, 128, n_sample=200, out_fmt="f32")


def test_sparse_many_groups():
    """Selected entries (k = 64 per token, some rows short) with the window,
    2000 groups of two tokens."""
    _run(23, [(4000, 3000, 7000 // 4, 128, True)], 64, 4, 128, sparse=True, k=64)


def test_ring_window_many_requests_equals_in_order():
    """1500 single-token requests: window rows kept as rings of 160 rows give
    bitwise the output of the same rows stored in order."""
    rng = np.random.default_rng(24)
    H, D, m, window, C = 128, 128, 4, 128, 160
    ts = rng.integers(0, 5000, 1500)
    n_ent = [(int(t) + 1) // m for t in ts]
    ent = rng.standard_normal((sum(n_ent), D)).astype(np.float32)
    q = rng.standard_normal((len(ts), H, D)).astype(np.float32)
    lin, ring, p0s = [], np.zeros((len(ts) * C, D), np.float32), []
    for r, t in enumerate(ts):
        p0 = max(0, int(t) - C + 1)
        rows = rng.standard_normal((int(t) - p0 + 1, D)).astype(np.float32)
        lin.append(rows)
        p0s.append(p0)
        for i, p in enumerate(range(p0, int(t) + 1)):
            ring[r * C + p % C] = rows[i]
    qd, kvd = dev_kv(q.reshape(-1, D), "bf16"), dev_kv(ent, "bf16")
    b_lin = Batch.make([1] * len(ts), ts.tolist(), kv_counts=n_ent, raw_counts=[len(x) for x in lin],
                       raw_pos=p0s)
    b_ring = dataclasses.replace(Batch.make([1] * len(ts), ts.tolist(), kv_counts=n_ent,
                                            raw_counts=[C] * len(ts), raw_pos=[0] * len(ts)),
                                 window_ring=True)
    outs = []
    for raw_d, bt in ((dev_kv(np.concatenate(lin), "bf16"), b_lin), (dev_kv(ring, "bf16"), b_ring)):
        out = torch.empty(len(ts) * H, D, device="cuda", dtype=torch.bfloat16)
        lse = torch.empty(len(ts) * H, device="cuda")
        ops.sparse_mqa_attn(qd, H, kvd, None, 0, raw_d, window, bt, m, out, BF16, lse)
        outs.append((out, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    # and the in-order result against the oracle on a few requests
    g = to_np(outs[0][0]).reshape(len(ts), H, D)
    qv, ev = ref_vals(q, "bf16"), ref_vals(ent, "bf16")
    e_off = np.cumsum([0] + n_ent)
    for r in [0, 1, 700, 1499]:
        t = int(ts[r])
        keys = np.concatenate([ev[e_off[r]:e_off[r + 1]],
                               ref_vals(lin[r], "bf16")[ref.window_positions(t, window) - p0s[r]]])
        o, _ = ref.attend(qv[r], keys, 1 / math.sqrt(D))
        assert np.max(np.abs(g[r] - o)) <= 2e-2
