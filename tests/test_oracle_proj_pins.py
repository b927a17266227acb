"""Pins of the projection oracle (oracle/proj.py) against closed forms and
structural identities that do not reuse its own computation."""
import numpy as np
import pytest

from oracle import proj


def test_linear_one_hot_rows_pick_weight_columns():
    """x = e_k gives y = W[:, k] exactly (the column of the stored [out, in]
    weight): a transposed operand or a wrong axis fails."""
    rng = np.random.default_rng(1)
    N, K = 7, 5
    w = rng.standard_normal((N, K))
    y = proj.linear(np.eye(K), w)
    assert y.shape == (K, N)
    for k in range(K):
        assert np.array_equal(y[k], w[:, k])


def test_linear_transposition_identity():
    """(x W^T)^T = W x^T: swapping the operands transposes the result."""
    rng = np.random.default_rng(2)
    x, w = rng.standard_normal((6, 9)), rng.standard_normal((4, 9))
    assert np.allclose(proj.linear(x, w), proj.linear(w, x).T, rtol=0, atol=1e-12)


def test_linear_worked_example():
    """[1 2; 3 4] times the weight rows [1 0], [1 1], [0 -2]."""
    y = proj.linear([[1, 2], [3, 4]], [[1, 0], [1, 1], [0, -2]])
    assert np.array_equal(y, [[1, 3, -4], [3, 7, -8]])


def _case(rng, n=5, H=8, D=6, G=4, d_g=3, d_model=7):
    o = rng.standard_normal((n, H, D))
    wg = rng.standard_normal((G, d_g, (H // G) * D))
    wo = rng.standard_normal((d_model, G * d_g))
    return o, wg, wo


def test_grouped_equals_block_diagonal_projection():
    """The grouped projection equals one projection of all heads through the
    block-diagonal weight whose block g is group g's weight, then w_out."""
    rng = np.random.default_rng(3)
    o, wg, wo = _case(rng)
    n, H, D = o.shape
    G, d_g, kg = wg.shape
    big = np.zeros((G * d_g, H * D))
    for g in range(G):
        big[g * d_g:(g + 1) * d_g, g * kg:(g + 1) * kg] = wg[g]
    ref = proj.linear(proj.linear(o.reshape(n, H * D), big), wo)
    assert np.allclose(proj.grouped_out_proj(o, wg, wo), ref, rtol=0, atol=1e-10)


def test_grouped_one_group_is_two_projections():
    rng = np.random.default_rng(4)
    o, wg, wo = _case(rng, G=1, d_g=5)
    n, H, D = o.shape
    ref = proj.linear(proj.linear(o.reshape(n, H * D), wg[0]), wo)
    assert np.allclose(proj.grouped_out_proj(o, wg, wo), ref, rtol=0, atol=1e-10)


@pytest.mark.parametrize("h,d", [(0, 0), (3, 5), (5, 2), (7, 4)])
def test_grouped_one_hot_head_value(h, d):
    """A single nonzero output (head h, dim d) reaches the model width only
    through its group g = h // (H/G), at column (h - g H/G) D + d of that
    group's weight: out = w_out[:, g d_g:(g+1) d_g] @ w_group[g][:, col]."""
    rng = np.random.default_rng(5)
    o, wg, wo = _case(rng)
    n, H, D = o.shape
    G, d_g, _ = wg.shape
    o = np.zeros((1, H, D))
    o[0, h, d] = 1.0
    g = h // (H // G)
    col = (h - g * (H // G)) * D + d
    expect = wo[:, g * d_g:(g + 1) * d_g] @ wg[g][:, col]
    assert np.allclose(proj.grouped_out_proj(o, wg, wo)[0], expect, rtol=0, atol=1e-12)


def test_grouped_mid_rounding_applies_between_the_projections():
    rng = np.random.default_rng(6)
    o, wg, wo = _case(rng)
    r = lambda v: np.round(v)
    n, H, D = o.shape
    G, d_g, kg = wg.shape
    mid = np.concatenate([proj.linear(o[:, g * (H // G):(g + 1) * (H // G)].reshape(n, kg), wg[g])
                          for g in range(G)], axis=1)
    assert np.allclose(proj.grouped_out_proj(o, wg, wo, mid_round=r), proj.linear(np.round(mid), wo),
                       rtol=0, atol=1e-10)
