"""Seeded random weights for the attention router's two MLPs.

The trained router weights of the pages are not available, so the router is
exercised with seeded random weights of the right shapes: Task MLP
d -> hidden -> d and Router MLP 2d -> hidden -> 2, weights stored [in][out],
drawn N(0, 1/fan_in), biases N(0, 0.1^2).  Only input preparation lives here;
the forward pass itself is in the oracle and in the HIP library.
"""

import numpy as np

SHAPES = ("w1", "b1", "w2", "b2", "w3", "b3", "w4", "b4")


def make_router_weights(d, hidden, seed):
    """Dict of float32 arrays w1 [d,H], b1 [H], w2 [H,d], b2 [d], w3 [2d,H],
    b3 [H], w4 [H,2], b4 [2]."""
    rng = np.random.Generator(np.random.PCG64(seed))

    def lin(fan_in, fan_out):
        w = rng.standard_normal((fan_in, fan_out)) / np.sqrt(fan_in)
        b = 0.1 * rng.standard_normal(fan_out)
        return w.astype(np.float32), b.astype(np.float32)

    w1, b1 = lin(d, hidden)
    w2, b2 = lin(hidden, d)
    w3, b3 = lin(2 * d, hidden)
    w4, b4 = lin(hidden, 2)
    return dict(w1=w1, b1=b1, w2=w2, b2=b2, w3=w3, b3=b3, w4=w4, b4=b4)
