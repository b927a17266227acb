"""csa_kv_compress_append (decode-time compression through a per-request
state) against the oracle's compression of the whole sequence, and attention
over a ring of window rows against the same rows stored in order and against
the oracle (page "DeepSeek V4 深度解析", section 4, KV-cache management: the
raw tokens of the window kept in a state cache)."""
import dataclasses

import numpy as np
import pytest
import torch

from long_context_compressed_kv_amd import ops
from long_context_compressed_kv_amd.ops import BF16, F32, KV, Batch
from oracle import csa as ref

from gpu_inputs import FMT, bf16_ulp, check_attention, check_mixed, dev_f32, dev_kv, ref_vals, to_np

pytestmark = pytest.mark.gpu


def _append_all(xs, zs, b, m, w, in_fmt, out_fmt, ring=0):
    """Appends request r's tokens 0 .. len-1 one call per position (requests
    already finished pass position -1).  The state starts as NaN: every open
    entry must be reset at its first slot."""
    n_req, D = len(xs), xs[0].shape[1]
    lens = [len(x) for x in xs]
    n_ent = [L // m for L in lens]
    T = max(lens)
    steps = np.zeros((T, n_req, D), np.float32)
    zsteps = np.zeros((T, n_req), np.float32)
    pos = np.full((T, n_req), -1, np.int64)
    for r, (x, z) in enumerate(zip(xs, zs)):
        steps[: len(x), r] = x
        zsteps[: len(x), r] = z
        pos[: len(x), r] = np.arange(len(x))
    x_dev = dev_kv(steps.reshape(-1, D), in_fmt)
    z_dev, p_dev = dev_f32(zsteps), torch.from_numpy(pos).cuda()
    off = np.concatenate([[0], np.cumsum(n_ent)]).astype(np.int64)
    cache = KV.empty(FMT[out_fmt], max(int(off[-1]), 1), D)
    state = torch.full((ops.kv_append_state_size(n_req, D) // 4,), float("nan"), device="cuda")
    e_off = torch.from_numpy(off[:-1].copy()).cuda()
    win = win_off = None
    if ring:
        win = KV(BF16 if in_fmt == "bf16" else F32, D,
                 torch.zeros(n_req * ring, D, device="cuda",
                             dtype=torch.bfloat16 if in_fmt == "bf16" else torch.float32))
        win_off = torch.arange(n_req, dtype=torch.int64, device="cuda") * ring
    bd = dev_f32(b)
    for t in range(T):
        ops.kv_compress_append(x_dev.narrow(t * n_req, n_req), z_dev[t], bd, m, w, p_dev[t], state,
                               e_off, cache, win, win_off, ring)
    torch.cuda.synchronize()
    return cache, off, n_ent, win


@pytest.mark.parametrize("in_fmt,out_fmt,m,w,D,lens", [
    ("bf16", "bf16", 4, 8, 128, [37, 64, 5, 0]),          # CSA ratio, ragged, an empty request
    ("f32", "f32", 4, 8, 64, [33, 8, 1]),
    ("f32", "f32", 3, 5, 256, [40, 17]),                  # odd ratio and window
    ("f32", "bf16", 4, 4, 128, [29]),                     # no overlap
    ("bf16", "bf16", 128, 256, 128, [600, 300, 129]),     # the HCA ratio and window
])
def test_append_equals_compression(in_fmt, out_fmt, m, w, D, lens):
    rng = np.random.default_rng(sum(lens) + D + m)
    xs = [rng.standard_normal((L, D)).astype(np.float32) for L in lens]
    zs = [rng.standard_normal(L).astype(np.float32) for L in lens]
    b = rng.standard_normal(w).astype(np.float32)
    cache, off, n_ent, _ = _append_all(xs, zs, b, m, w, in_fmt, out_fmt)
    g = to_np(cache.data).astype(np.float64)
    for r, (x, z) in enumerate(zip(xs, zs)):
        if n_ent[r] == 0:
            continue
        c = ref.compress_entries(ref_vals(x, in_fmt), z.astype(np.float64), 0, b, m, w, 0, n_ent[r])
        gr = g[off[r]: off[r + 1]]
        if out_fmt == "f32":
            assert np.max(np.abs(gr - c)) <= 1e-5
        else:
            assert np.all(np.abs(gr - c) <= bf16_ulp(c) * 1.0001)


def test_append_mixed_format_csa():
    """512-dim entries in the mixed format (e4m3 + e8m0 scales + bf16 RoPE),
    the decode cache of the CSA layers."""
    rng = np.random.default_rng(71)
    m, w, D, lens = 4, 8, 512, [41, 16, 3, 24]
    xs = [rng.standard_normal((L, D)).astype(np.float32) for L in lens]
    zs = [rng.standard_normal(L).astype(np.float32) for L in lens]
    b = rng.standard_normal(w).astype(np.float32)
    cache, off, n_ent, _ = _append_all(xs, zs, b, m, w, "bf16", "fp8_mixed")
    for r, (x, z) in enumerate(zip(xs, zs)):
        if n_ent[r] == 0:
            continue
        xv = ref_vals(x, "bf16")
        c = ref.compress_entries(xv, z.astype(np.float64), 0, b, m, w, 0, n_ent[r])
        cabs = ref.compress_entries(np.abs(xv), z.astype(np.float64), 0, b, m, w, 0, n_ent[r])
        part = cache.narrow(int(off[r]), n_ent[r])
        # the online softmax rounds a few more times than the one-pass sum
        nd = check_mixed(part, c, cabs, rel=2.0 ** -18)
        assert nd <= n_ent[r] * 448 * 2e-3


def test_append_writes_the_window_ring():
    rng = np.random.default_rng(72)
    m, w, D, C = 4, 8, 128, 128
    lens = [300, 90]
    xs = [rng.standard_normal((L, D)).astype(np.float32) for L in lens]
    zs = [rng.standard_normal(L).astype(np.float32) for L in lens]
    b = rng.standard_normal(w).astype(np.float32)
    _, _, _, win = _append_all(xs, zs, b, m, w, "bf16", "bf16", ring=C)
    ring = win.data.float().cpu().numpy()
    for r, x in enumerate(xs):
        xb = ref_vals(x, "bf16")
        for p in range(max(0, len(x) - C), len(x)):
            assert np.array_equal(ring[r * C + p % C], xb[p])


def _ring_case(rng, ts, H, D, kv_fmt, sparse, k, window, C, split):
    """Decode batch: request r at position ts[r]; the same window rows stored
    in order (rows for positions max(0, t-C+1) .. t) and as a ring of C rows."""
    m = 4
    n_req = len(ts)
    n_ent = [(t + 1) // m for t in ts]
    ent = rng.standard_normal((sum(n_ent), D)).astype(np.float32)
    q = rng.standard_normal((n_req, H, D)).astype(np.float32)
    lin_rows, ring_rows, lin_pos = [], np.zeros((n_req * C, D), np.float32), []
    for r, t in enumerate(ts):
        p0 = max(0, t - C + 1)
        rows = rng.standard_normal((t - p0 + 1, D)).astype(np.float32)
        lin_rows.append(rows)
        lin_pos.append(p0)
        for i, p in enumerate(range(p0, t + 1)):
            ring_rows[r * C + p % C] = rows[i]
    qd, kvd = dev_kv(q.reshape(-1, D), "bf16"), dev_kv(ent, kv_fmt)
    lin_d = dev_kv(np.concatenate(lin_rows), "bf16")
    ring_d = dev_kv(ring_rows, "bf16")
    idx_d = None
    if sparse:
        idx = np.full((n_req, k), -1, np.int32)
        for r, n in enumerate(n_ent):
            c = min(k, n)
            idx[r, :c] = np.sort(rng.choice(n, c, replace=False))
        idx_d = torch.from_numpy(idx).cuda()
    b_lin = Batch.make([1] * n_req, ts, kv_counts=n_ent, raw_counts=[len(x) for x in lin_rows],
                       raw_pos=lin_pos)
    b_ring = dataclasses.replace(Batch.make([1] * n_req, ts, kv_counts=n_ent, raw_counts=[C] * n_req,
                                            raw_pos=[0] * n_req), window_ring=True)
    outs = []
    for raw_d, bt in ((lin_d, b_lin), (ring_d, b_ring)):
        out = torch.empty(n_req * H, D, device="cuda", dtype=torch.bfloat16)
        lse = torch.empty(n_req * H, device="cuda")
        ops.sparse_mqa_attn(qd, H, kvd, idx_d, k if sparse else 0, raw_d, window, bt, m, out, BF16,
                            lse, split_keys=split)
        outs.append((out, lse))
    torch.cuda.synchronize()
    # the ring result against the oracle: each request's keys (selected or
    # visible entries) and its window rows in position order
    qv = ref_vals(q, "bf16")
    ev = ref_vals(ent, kv_fmt)
    off = np.concatenate([[0], np.cumsum(n_ent)])
    ent_rows, win_rows = [], []
    for r, t in enumerate(ts):
        mine = ev[off[r]: off[r + 1]]
        ent_rows.append(mine[idx[r][idx[r] >= 0]] if sparse else mine)
        win_rows.append(ref_vals(lin_rows[r], "bf16")[ref.window_positions(t, window) - lin_pos[r]])
    check_attention(outs[1][0], outs[1][1], qv, H, ent_rows, win_rows)
    return outs


@pytest.mark.parametrize("D,kv_fmt,sparse,k,split", [
    (128, "bf16", False, 0, 0),          # HCA-like dense, one workgroup per query
    (512, "fp8_mixed", True, 64, 128),   # CSA decode, split-K over selected keys
    (512, "fp8_mixed", False, 0, 128),   # dense decode, planned split-K
])
def test_attention_over_ring_equals_in_order(D, kv_fmt, sparse, k, split):
    rng = np.random.default_rng(73 + D)
    ts = [1000, 50, 4097, 127]
    (o_lin, l_lin), (o_ring, l_ring) = _ring_case(rng, ts, 64, D, kv_fmt, sparse, k, 128, 160, split)
    assert torch.equal(o_lin, o_ring)
    assert torch.equal(l_lin, l_ring)
