"""Plain CPU oracle of the projections around the compressed-attention path.

TEST INFRASTRUCTURE. Nothing in the product path may import this module; only
the tests, the smoke check and the CPU-baseline leg of the benchmark use it.
It shares no code with the HIP library: NumPy in float64.

What the pages say (no sizes, no formulas):
* page "DeepSeek V4 深度解析", section 2, HCA paragraph: CSA and HCA both use a
  grouped output projection to cut compute;
* page "wmrh.cn/news/726125", "V4 改进一": the output side is projected in
  groups; the MLA passage before it: the query side is low-rank compressed as
  well, and the key/value up-projections are absorbed into the query and the
  output projection, so attention works on the compressed vectors directly.

Readings:
* a projection is y = x W^T with W stored [out, in]; operands bf16, products
  summed exactly (float64 here), the result rounded to the output format;
* the grouped output projection splits the H heads' outputs into G groups of
  H/G consecutive heads; group g maps its heads' outputs, concatenated in head
  order ((H/G) D values), to d_g values with a weight of its own; the G
  results, concatenated in group order and rounded to bf16 (an activation),
  go through one final projection to the model width.
"""
import numpy as np


def linear(x, w):
    """y = x W^T: x [..., K], w [N, K] -> [..., N] (float64)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    return x @ w.T


def grouped_out_proj(o, w_group, w_out, mid_round=None):
    """Grouped output projection of attention outputs o [n, H, D].

    w_group [G, d_g, (H/G) D]: group g's weight over heads g H/G ..
    (g+1) H/G - 1; w_out [d_model, G d_g]. mid_round (a rounding to the
    activation format) is applied to the concatenated group results.
    Returns [n, d_model] float64."""
    o = np.asarray(o, np.float64)
    n, H, D = o.shape
    G, d_g, kg = w_group.shape
    hpg = H // G
    assert hpg * G == H and kg == hpg * D, "groups must split the heads evenly"
    mid = np.empty((n, G * d_g))
    for g in range(G):
        xg = o[:, g * hpg:(g + 1) * hpg, :].reshape(n, hpg * D)
        mid[:, g * d_g:(g + 1) * d_g] = linear(xg, w_group[g])
    if mid_round is not None:
        mid = mid_round(mid)
    return linear(mid, w_out)
