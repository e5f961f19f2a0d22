"""Grouped output projection of the attention outputs, in fp64 (the oracle).

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Source: "DeepSeek-V4: Towards Highly Efficient Million-Token Context
Intelligence", section 3.3: because c * n_h (the width of all heads' outputs
side by side) is large, the output projection is grouped -- each group of
heads is first projected down to an intermediate width d_g, the groups'
results are concatenated and projected back to the model width d.

Readings (the page gives no more):

* the n_h heads split into g groups of n_h / g consecutive heads; group q owns
  the columns [q W, (q+1) W) of the concatenated head outputs, W = n_h c / g;
* each group has its own down-projection W1[q] of shape d_g x W; the up
  projection W2 is d x (g d_g) over the concatenated group results;
* the intermediate result is stored in the activation format (bf16) between the
  two products, as a bf16 model stores every activation.

Weights are given output-major ([out][in], the input axis contiguous), so both
products read their operands along the contraction axis.
"""
from __future__ import annotations

import numpy as np

from .codecs import f64_to_bf16_value


def grouped_output_projection(o, W1, W2, *, groups: int, y_dtype: str = "bf16"):
    """o: [T, n_h c]; W1: [g, d_g, n_h c / g]; W2: [d, g d_g].  Returns (y, out):
    y[t, q d_g + e] = sum_i o[t, q W + i] W1[q, e, i] (rounded to y_dtype) and
    out[t, :] = y[t, :] @ W2^T (fp64, the caller rounds to its format)."""
    o = np.asarray(o, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    T, HC = o.shape
    g, d_g, Wq = W1.shape
    if g != groups or g * Wq != HC:
        raise ValueError("W1 must be [groups, d_g, n_h c / groups]")
    y = np.empty((T, g * d_g))
    for q in range(g):
        y[:, q * d_g:(q + 1) * d_g] = o[:, q * Wq:(q + 1) * Wq] @ W1[q].T
    if y_dtype == "bf16":
        y = f64_to_bf16_value(y)
    return y, y @ W2.T
