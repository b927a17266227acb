"""The projections around the path (csa_linear, csa_grouped_out_proj) against
the oracle (oracle/proj.py) on the same bf16 operands.

Tolerances follow from the arithmetic: the GPU accumulates in fp32, so a
result differs from the exact sum by at most K u sum_k |x_k w_k| (u = 2^-24);
a bf16 output adds half an ulp (2^-8 of the value at most); the grouped
projection's bf16 group results can round to neighbouring values where the
fp32 sum and the exact sum straddle a rounding midpoint (one ulp of the
group result, carried through the final projection's weights).

Shapes: small ragged cases spanning several 128 x 128 tiles and a partial
one, strided and batched views, and the full-size projections of the
chunked prefill at 1M (8192 tokens, 128 heads) and of the 64-request decode
(64 heads), checked on sampled rows and columns computed one by one."""
import numpy as np
import pytest
import torch

from long_context_compressed_kv_amd import ops
from oracle import codecs, proj

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _bf(rng, shape, scale=1.0):
    """Seeded float32 draws -> (device bf16 tensor, the exact bf16 values)."""
    a = (scale * rng.standard_normal(shape)).astype(np.float32)
    v = codecs.bf16_round(a.reshape(-1, shape[-1])).astype(np.float64).reshape(shape)
    return torch.from_numpy(a).cuda().to(torch.bfloat16), v


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def _acc_bound(xv, wv):
    return xv.shape[-1] * U * (np.abs(xv) @ np.abs(wv).T)


def _check(got, ref, tol, bf16_out):
    if bf16_out:
        tol = tol + np.abs(ref) * 2.0 ** -8
    err = np.abs(got - ref)
    assert np.all(err <= tol + 1e-30), float(np.max(err - tol))


@pytest.mark.parametrize("M,N,K,out", [
    (1, 1, 64, "f32"), (37, 300, 128, "f32"), (256, 256, 1024, "f32"), (200, 130, 448, "bf16"),
    (129, 257, 192, "bf16"), (5, 1000, 64, "f32"), (300, 64, 4096, "f32")])
def test_linear_against_oracle(M, N, K, out):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    x, xv = _bf(rng, (M, K))
    w, wv = _bf(rng, (N, K), 0.05)
    y = torch.full((M, N), float("nan"), device="cuda",
                   dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    print(f"[proj] linear M={M} N={N} K={K} {out}", flush=True)
    ops.linear(x, w, y)
    torch.cuda.synchronize()
    _check(_host(y), proj.linear(xv, wv), _acc_bound(xv, wv), out == "bf16")


def test_linear_batched_and_strided():
    """A batch of three in one launch; x a column window of a wider matrix
    (row stride above K); every output row written, nothing beyond."""
    rng = np.random.default_rng(11)
    B, M, N, K = 3, 70, 150, 320
    xb, xbv = _bf(rng, (B, M, K + 96))
    x, xv = xb[:, :, 32:32 + K], xbv[:, :, 32:32 + K]
    w, wv = _bf(rng, (B, N, K), 0.05)
    y = torch.full((B, M, N + 8), 7.0, device="cuda")
    print("[proj] batched, strided", flush=True)
    ops.linear(x, w, y[:, :, :N])
    torch.cuda.synchronize()
    g = _host(y)
    for b in range(B):
        _check(g[b, :, :N], proj.linear(xv[b], wv[b]), _acc_bound(xv[b], wv[b]), False)
    assert np.all(g[:, :, N:] == 7.0)


def _grouped_ref_and_tol(ov, wgv, wov, bf16_out):
    """The oracle's grouped projection (bf16 group results) and its bound."""
    n, H, D = ov.shape
    G, d_g, kg = wgv.shape
    hpg = H // G
    ref = proj.grouped_out_proj(ov, wgv, wov, mid_round=codecs.bf16_round)
    # group results: exact, rounded, and how far the GPU's may sit from them
    mids, bnds = [], []
    for g in range(G):
        xg = ov[:, g * hpg:(g + 1) * hpg, :].reshape(n, kg)
        mids.append(proj.linear(xg, wgv[g]))
        bnds.append(_acc_bound(xg, wgv[g]))
    mid = np.concatenate(mids, axis=1)
    midr = codecs.bf16_round(mid).astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(midr), 2.0 ** -126))) - 7)
    mid_err = ulp + np.concatenate(bnds, axis=1)
    tol = mid_err @ np.abs(wov).T + _acc_bound(midr + mid_err, wov)
    return ref, tol


@pytest.mark.parametrize("n,H,D,G,d_g,d_model,out", [
    (40, 64, 512, 8, 256, 384, "f32"), (3, 16, 128, 4, 64, 200, "bf16"), (130, 8, 64, 1, 128, 64, "f32")])
def test_grouped_out_proj_against_oracle(n, H, D, G, d_g, d_model, out):
    rng = np.random.default_rng(n + H + G)
    o, ov = _bf(rng, (n, H, D))
    wg, wgv = _bf(rng, (G, d_g, (H // G) * D), 0.03)
    wo, wov = _bf(rng, (d_model, G * d_g), 0.03)
    y = torch.empty(n, d_model, device="cuda", dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    print(f"[proj] grouped n={n} H={H} D={D} G={G} d_g={d_g} d_model={d_model}", flush=True)
    ops.grouped_out_proj(o, H, wg, wo, y)
    torch.cuda.synchronize()
    ref, tol = _grouped_ref_and_tol(ov, wgv, wov, out == "bf16")
    _check(_host(y), ref, tol, out == "bf16")


def test_full_size_prefill_projections_sampled():
    """The chunked prefill at 1M: 8192 tokens of width 7168 through the
    query's low-rank pair (7168 -> 1536 -> 128 heads x 512) and the grouped
    output projection (8 groups of 16 heads, 1024 each, -> 7168); sampled rows
    (and columns of the 65536-wide query) against the oracle."""
    rng = np.random.default_rng(21)
    T, dm, rq, H, D, G, d_g = 8192, 7168, 1536, 128, 512, 8, 1024
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    rn = lambda *s, sc=1.0: (sc * torch.randn(*s, generator=g, device="cuda")).to(torch.bfloat16)
    x = rn(T, dm)
    w_dq = rn(rq, dm, sc=0.02)
    w_uq = rn(H * D, rq, sc=0.03)
    cq = torch.empty(T, rq, device="cuda", dtype=torch.bfloat16)
    q = torch.empty(T, H * D, device="cuda", dtype=torch.bfloat16)
    print("[proj] full-size query projections", flush=True)
    ops.linear(x, w_dq, cq)
    ops.linear(cq, w_uq, q)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(T, 3, replace=False))
    cols = np.sort(rng.choice(H * D, 512, replace=False))
    xv, wdv, cqv = _host(x[rows]), _host(w_dq), _host(cq[rows])
    _check(cqv, proj.linear(xv, wdv), _acc_bound(xv, wdv), True)
    wuv = _host(w_uq[cols])
    _check(_host(q[rows][:, cols]), proj.linear(cqv, wuv), _acc_bound(cqv, wuv), True)
    del x, w_dq, w_uq, cq, q
    o = rn(T, H, D)
    wg = rn(G, d_g, (H // G) * D, sc=0.01)
    wo = rn(dm, G * d_g, sc=0.01)
    y = torch.empty(T, dm, device="cuda", dtype=torch.bfloat16)
    print("[proj] full-size grouped output projection", flush=True)
    ops.grouped_out_proj(o, H, wg, wo, y)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(T, 2, replace=False))
    ref, tol = _grouped_ref_and_tol(_host(o[rows]), _host(wg), _host(wo), True)
    _check(_host(y[rows]), ref, tol, True)
