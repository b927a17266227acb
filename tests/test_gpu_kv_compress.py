"""csa_kv_compress against the oracle's compression (CSA step 1 / HCA)."""
import numpy as np
import pytest
import torch

import synth
from long_context_compressed_kv_amd import ops
from long_context_compressed_kv_amd.ops import KV
from oracle import csa as ref

from gpu_inputs import FMT, bf16_ulp, check_mixed, dev_f32, dev_kv, ref_vals, to_np

pytestmark = pytest.mark.gpu


def _run(x_np, z, bias, m, w, x_pos0, e0, n, in_fmt, out_fmt):
    x = dev_kv(x_np, in_fmt)
    out = KV.empty(FMT[out_fmt], n, x_np.shape[1])
    ops.kv_compress(x, dev_f32(z), x_pos0, dev_f32(bias), m, w, e0, n, out)
    torch.cuda.synchronize()
    return out


def _oracle(x_np, z, bias, m, w, x_pos0, e0, n, in_fmt):
    xv = ref_vals(x_np, in_fmt)
    return ref.compress_entries(xv, z.astype(np.float64), x_pos0, bias, m, w, e0, e0 + n)


@pytest.mark.parametrize("in_fmt,out_fmt,m,w,D,T", [
    ("f32", "f32", 4, 8, 128, 4096),        # the fp32 CSA prefill shape
    ("bf16", "bf16", 128, 256, 128, 65536),  # the bf16 HCA prefill shape
    ("f32", "f32", 4, 8, 16, 37),            # ragged tail, small dim
    ("bf16", "f32", 3, 7, 64, 100),          # odd ratio and window
    ("f32", "bf16", 4, 4, 256, 64),          # no overlap
])
def test_compress_dense_formats(in_fmt, out_fmt, m, w, D, T):
    rng = np.random.default_rng(T + D)
    x = rng.standard_normal((T, D)).astype(np.float32)
    z = rng.standard_normal(T).astype(np.float32)
    b = rng.standard_normal(w).astype(np.float32)
    n = T // m
    out = _run(x, z, b, m, w, 0, 0, n, in_fmt, out_fmt)
    c = _oracle(x, z, b, m, w, 0, 0, n, in_fmt)
    g = to_np(out.data).astype(np.float64)
    if out_fmt == "f32":
        assert np.max(np.abs(g - c)) <= 1e-5
    else:
        assert np.all(np.abs(g - c) <= bf16_ulp(c) * 1.0001)


def test_compress_chunk_mixed_at_1m():
    """The chunked-prefill shape: 8192 new bf16 tokens at position 2^20, four
    history rows, 2048 new entries in the mixed format."""
    wl = synth.WORKLOADS[4]
    inp = synth.prefill_inputs(wl, seq=8192)
    raw, z, b = inp["raw"], inp["z"], inp["bias"]
    e0, n = inp["first_new_entry"], inp["n_entries"] - inp["first_new_entry"]
    assert n == 2048
    out = _run(raw, z, b, 4, 8, inp["raw_pos0"], e0, n, "bf16", "fp8_mixed")
    c = _oracle(raw, z, b, 4, 8, inp["raw_pos0"], e0, n, "bf16")
    cabs = _oracle(np.abs(raw), z, b, 4, 8, inp["raw_pos0"], e0, n, "bf16")
    nd = check_mixed(out, c, cabs)
    assert nd <= 2048 * 448 * 1e-3


def test_compress_first_entries_partial_window():
    rng = np.random.default_rng(5)
    m, w, T, D = 128, 256, 300, 128
    x = rng.standard_normal((T, D)).astype(np.float32)
    z = np.full(T, 0.3, np.float32)
    b = np.zeros(w, np.float32)
    out = _run(x, z, b, m, w, 0, 0, 2, "f32", "f32")
    g = to_np(out.data)
    assert np.allclose(g[0], x[:128].mean(0), atol=2e-6)       # only positions 0..127
    assert np.allclose(g[1], x[:256].mean(0), atol=2e-6)


def test_compress_chunked_equals_one_shot_bitwise():
    rng = np.random.default_rng(6)
    m, w, T, D = 4, 8, 400, 512
    x = rng.standard_normal((T, D)).astype(np.float32)
    z = rng.standard_normal(T).astype(np.float32)
    b = rng.standard_normal(w).astype(np.float32)
    full = _run(x, z, b, m, w, 0, 0, T // m, "bf16", "fp8_mixed")
    split = 160
    part = _run(x[split - 4:], z[split - 4:], b, m, w, split - 4, split // m, (T - split) // m,
                "bf16", "fp8_mixed")
    assert torch.equal(full.data[split // m:], part.data)
    assert torch.equal(full.scale[split // m:], part.scale)
    assert torch.equal(full.rope[split // m:], part.rope)


def test_compress_deterministic():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1024, 128)).astype(np.float32)
    z = rng.standard_normal(1024).astype(np.float32)
    b = rng.standard_normal(256).astype(np.float32)
    a = _run(x, z, b, 128, 256, 0, 0, 8, "bf16", "bf16")
    c = _run(x, z, b, 128, 256, 0, 0, 8, "bf16", "bf16")
    assert torch.equal(a.data, c.data)


# ------------------------------------------------- per-channel logits variant

@pytest.mark.parametrize("in_fmt,out_fmt,m,w,D,T,x_pos0,e0", [
    ("f32", "f32", 4, 8, 128, 2048, 0, 0),         # CSA ratio, four entries a workgroup
    ("bf16", "bf16", 128, 256, 128, 8192, 0, 0),   # HCA ratio and window
    ("f32", "f32", 4, 8, 16, 37, 0, 0),            # 32 entries a workgroup, ragged tail
    ("bf16", "f32", 3, 7, 64, 100, 0, 0),          # odd ratio and window
    ("f32", "bf16", 4, 8, 256, 300, 96, 26),       # a chunk: history rows, later first entry
])
def test_compress_channel_against_oracle(in_fmt, out_fmt, m, w, D, T, x_pos0, e0):
    rng = np.random.default_rng(T + D + m)
    x = rng.standard_normal((T, D)).astype(np.float32)
    z = (rng.standard_normal((T, D)) * 2).astype(np.float32)
    b = rng.standard_normal((w, D)).astype(np.float32)
    n = (x_pos0 + T) // m - e0
    out = KV.empty(FMT[out_fmt], n, D)
    ops.kv_compress_channel(dev_kv(x, in_fmt), dev_f32(z), x_pos0, dev_f32(b), m, w, e0, n, out)
    torch.cuda.synchronize()
    c = ref.compress_entries_channel(ref_vals(x, in_fmt), z, x_pos0, b, m, w, e0, e0 + n)
    g = to_np(out.data).astype(np.float64)
    if out_fmt == "f32":
        assert np.max(np.abs(g - c)) <= 1e-5
    else:
        assert np.all(np.abs(g - c) <= bf16_ulp(c) * 1.0001)


def test_compress_channel_mixed_format():
    """512-dim entries stored in the mixed format (e4m3 + e8m0 + bf16 RoPE)."""
    rng = np.random.default_rng(77)
    m, w, T, D = 4, 8, 600, 512
    x = rng.standard_normal((T, D)).astype(np.float32)
    z = rng.standard_normal((T, D)).astype(np.float32)
    b = rng.standard_normal((w, D)).astype(np.float32)
    n = T // m
    out = KV.empty(FMT["fp8_mixed"], n, D)
    ops.kv_compress_channel(dev_kv(x, "bf16"), dev_f32(z), 0, dev_f32(b), m, w, 0, n, out)
    torch.cuda.synchronize()
    xv = ref_vals(x, "bf16")
    c = ref.compress_entries_channel(xv, z, 0, b, m, w, 0, n)
    cabs = ref.compress_entries_channel(np.abs(xv), z, 0, b, m, w, 0, n)
    nd = check_mixed(out, c, cabs)
    assert nd <= n * 448 * 2e-3


def test_indexer_keys_compressed_with_the_same_weights():
    """The reading where an entry's indexer key is the compression of the raw
    tokens' indexer keys with the entry's own softmax weights: the same call
    on the 64-dim key rows with the same logits and biases, checked against
    the oracle's compression of those rows, and the result used as indexer
    keys gives the oracle's top-k."""
    rng = np.random.default_rng(78)
    m, w, T, D, DI = 4, 8, 2048, 512, 64
    x = rng.standard_normal((T, D)).astype(np.float32)
    xi = (rng.standard_normal((T, DI)) * 0.125).astype(np.float32)
    z = rng.standard_normal(T).astype(np.float32)
    b = rng.standard_normal(w).astype(np.float32)
    n = T // m
    kv = KV.empty(FMT["bf16"], n, D)
    ki = KV.empty(FMT["f32"], n, DI)
    zd, bd = dev_f32(z), dev_f32(b)
    ops.kv_compress(dev_kv(x, "bf16"), zd, 0, bd, m, w, 0, n, kv)
    ops.kv_compress(dev_kv(xi, "f32"), zd, 0, bd, m, w, 0, n, ki)
    torch.cuda.synchronize()
    ki_ref = ref.compress_entries(xi, z, 0, b, m, w, 0, n)
    assert np.max(np.abs(to_np(ki.data) - ki_ref)) <= 1e-6
    # the compressed keys drive the selection of a query at the last position
    qi = (rng.standard_normal((1, 4, DI)) * 0.125).astype(np.float32)
    batch = ops.Batch.make([1], [T - 1], kv_counts=[n])
    k = 32
    idx = ops.indexer_topk(dev_kv(qi.reshape(-1, DI), "f32"), 4, ki, batch, m, ops.F32, k)
    torch.cuda.synchronize()
    s = ref.indexer_scores(qi[0].astype(np.float64), to_np(ki.data).astype(np.float64), np.ones(4))
    want = set(ref.topk_indices(ref.score_keys(s, "f32"), k).tolist())
    got = set(idx.cpu().numpy()[0].tolist())
    # the selections agree except, at most, between entries tied at the k-th
    # score within the fp32 accumulation's rounding
    kth = np.sort(s)[-k]
    assert all(abs(s[j] - kth) <= 1e-5 * abs(kth) + 1e-7 for j in got ^ want)


# ------------------------------------------------------------ ragged batch

def _batch_case(rng, chunks, m, w, D, in_fmt, out_fmt, paged=0):
    """chunks: [(q_pos, T)]; each request's raw rows start at the first slot
    of its first new entry (or at 0).  Returns (device out, per-request oracle
    entries, first entry index, cache rows of each entry, owned-row mask)."""
    from gpu_inputs import dev_kv as _dev
    raws, zs, rpos, kv_counts = [], [], [], []
    for pos, T in chunks:
        p0 = max(0, (pos // m + 1) * m - w)      # the first new entry's first slot
        raws.append(rng.standard_normal((pos + T - p0, D)).astype(np.float32))
        zs.append(rng.standard_normal(pos + T - p0).astype(np.float32))
        rpos.append(p0)
        kv_counts.append((pos + T) // m + 3)        # the cache holds every entry up to the chunk
    b = rng.standard_normal(w).astype(np.float32)
    batch = ops.Batch.make([T for _, T in chunks], [p for p, _ in chunks], kv_counts=kv_counts,
                           raw_counts=[len(x) for x in raws], raw_pos=rpos)
    n_rows = sum(kv_counts)
    rows_of = []
    if paged:
        nb = [(c + paged - 1) // paged for c in kv_counts]
        ids = rng.permutation(sum(nb) + 3)
        table = np.full((len(chunks), max(nb)), -1, np.int32)
        k = 0
        for r, n in enumerate(nb):
            table[r, :n] = ids[k:k + n]
            k += n
        n_rows = (sum(nb) + 3) * paged
        import dataclasses
        batch = dataclasses.replace(batch, kv_block_table=torch.from_numpy(table).cuda(), kv_block_rows=paged)
        rows_of = lambda r, i: int(table[r, i // paged]) * paged + i % paged
    else:
        off = np.concatenate([[0], np.cumsum(kv_counts)])
        rows_of = lambda r, i: int(off[r]) + i
    sentinel = (rng.standard_normal((n_rows, D)) * 40).astype(np.float32)
    out = _dev(sentinel, out_fmt if out_fmt != "f32" else "f32")
    before = [t.clone() for t in (out.data, out.scale, out.rope) if t is not None]
    ops.kv_compress_batch(_dev(np.concatenate(raws), in_fmt), dev_f32(np.concatenate(zs)), dev_f32(b), m, w,
                          batch, out)
    torch.cuda.synchronize()
    want, places = [], []
    for r, (pos, T) in enumerate(chunks):
        e0, e1 = pos // m, (pos + T) // m
        c = ref.compress_entries(ref_vals(raws[r], in_fmt), zs[r].astype(np.float64), rpos[r], b, m, w, e0, e1)
        ca = ref.compress_entries(np.abs(ref_vals(raws[r], in_fmt)), zs[r].astype(np.float64), rpos[r], b, m, w,
                                  e0, e1)
        want.append((c, ca))
        places.append([rows_of(r, i) for i in range(e0, e1)])
    owned = np.zeros(n_rows, bool)
    for pl in places:
        owned[pl] = True
    return out, want, places, owned, before


@pytest.mark.parametrize("out_fmt,in_fmt,m,w,D,paged", [
    ("f32", "f32", 4, 8, 128, 0),
    ("bf16", "bf16", 128, 256, 128, 0),
    ("fp8_mixed", "bf16", 4, 8, 512, 0),
    ("bf16", "f32", 4, 8, 256, 32),      # a paged cache
])
def test_compress_batch_against_oracle(out_fmt, in_fmt, m, w, D, paged):
    """One launch for a ragged batch of prefill chunks: every request's new
    entries match the oracle's compression of its own rows; a chunk that
    completes no entry, an empty chunk and a chunk at position 0 are in the
    batch; rows that no new entry owns keep their contents."""
    rng = np.random.default_rng(D + m + paged)
    if m == 4:
        chunks = [(0, 300), (1001, 2), (5000, 777), (64, 0), (90, 45), (1 << 20, 129)]
    else:
        chunks = [(0, 1000), (70000, 300), (130, 10), (4096, 2048)]
    out, want, places, owned, before = _batch_case(rng, chunks, m, w, D, in_fmt, out_fmt, paged)
    for (c, ca), pl in zip(want, places):
        if not pl:
            continue
        if out_fmt == "fp8_mixed":
            view = KV(out.fmt, out.dim, out.data[pl], out.scale[pl], out.rope[pl])
            assert check_mixed(view, c, ca) <= len(pl) * 448 * 1e-3
        else:
            g = to_np(out.data[pl]).astype(np.float64)
            if out_fmt == "f32":
                assert np.max(np.abs(g - c)) <= 1e-5
            else:
                assert np.all(np.abs(g - c) <= bf16_ulp(c) * 1.0001)
    free = torch.from_numpy(~owned).cuda()
    for a, b0 in zip([t for t in (out.data, out.scale, out.rope) if t is not None], before):
        assert torch.equal(a[free], b0[free])


def test_compress_batch_equals_per_request_calls():
    """The batch call gives bit for bit what one csa_kv_compress call per
    request gives (the same arithmetic per entry), whatever the order of the
    requests in the batch."""
    rng = np.random.default_rng(11)
    m, w, D = 4, 8, 512
    chunks = [(2000, 513), (0, 64), (777, 1000), (10, 1)]
    raws, zs, rpos = [], [], []
    for pos, T in chunks:
        p0 = max(0, (pos // m + 1) * m - w)      # the first new entry's first slot
        raws.append(rng.standard_normal((pos + T - p0, D)).astype(np.float32))
        zs.append(rng.standard_normal(pos + T - p0).astype(np.float32))
        rpos.append(p0)
    b = dev_f32(rng.standard_normal(w).astype(np.float32))
    singles = []
    for r, (pos, T) in enumerate(chunks):
        e0, n = pos // m, (pos + T) // m - pos // m
        one = KV.empty(FMT["fp8_mixed"], max(n, 1), D)
        if n:
            ops.kv_compress(dev_kv(raws[r], "bf16"), dev_f32(zs[r]), rpos[r], b, m, w, e0, n, one)
        singles.append((one, n))
    for order in ([0, 1, 2, 3], [3, 2, 0, 1]):
        kv_counts = [(chunks[r][0] + chunks[r][1]) // m for r in order]
        batch = ops.Batch.make([chunks[r][1] for r in order], [chunks[r][0] for r in order], kv_counts=kv_counts,
                               raw_counts=[len(raws[r]) for r in order], raw_pos=[rpos[r] for r in order])
        out = KV.empty(FMT["fp8_mixed"], sum(kv_counts), D)
        ops.kv_compress_batch(dev_kv(np.concatenate([raws[r] for r in order]), "bf16"),
                              dev_f32(np.concatenate([zs[r] for r in order])), b, m, w, batch, out)
        torch.cuda.synchronize()
        off = np.concatenate([[0], np.cumsum(kv_counts)])
        for j, r in enumerate(order):
            one, n = singles[r]
            e0 = chunks[r][0] // m
            rows = slice(int(off[j]) + e0, int(off[j]) + e0 + n)
            assert torch.equal(out.data[rows], one.data[:n]), r
            assert torch.equal(out.scale[rows], one.scale[:n]) and torch.equal(out.rope[rows], one.rope[:n])
