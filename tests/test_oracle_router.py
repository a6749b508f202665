"""Pins of the fp64 router oracle (boundary pooling, the two MLPs, arg max)."""

import json
import os

import numpy as np
import pytest

from oracle import router as ORT
from synth.router_weights import make_router_weights

HERE = os.path.dirname(__file__)
FACTS = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))["router_config"]
WORKED = json.load(open(os.path.join(HERE, "golden", "router_worked_example.json")))


def _sq_sum(n):
    # sum_{t=0}^{n-1} t^2
    return n * (n - 1) * (2 * n - 1) // 6


@pytest.mark.parametrize("L", [0, 1, 57, 100, 150, 199, 200, 201, 1000, 65536])
def test_boundary_set(L):
    pos = ORT.boundary_positions(L, FACTS["pool_head_tokens"], FACTS["pool_tail_tokens"])
    assert len(np.unique(pos)) == len(pos) == min(L, 200)
    if L >= 200:
        assert pos[:100].tolist() == list(range(100)) and pos[100:].tolist() == list(range(L - 100, L))
    else:
        assert pos.tolist() == list(range(L))


@pytest.mark.parametrize("L", [1, 150, 200, 333, 4096])
def test_pool_quadratic_closed_form(L):
    # k = t^2 on every channel: the boundary mean is
    # (S(100) + S(L) - S(L - 100)) / 200 for L >= 200 and S(L) / L below,
    # where S(n) = sum_{t<n} t^2.  A pool over all tokens, or one that counts
    # the overlap of the two ends twice, misses it.
    k = (np.arange(L, dtype=np.float64) ** 2)[:, None, None] * np.ones((1, 2, 4))
    got = ORT.boundary_pool(k, [0, L])[0]
    if L >= 200:
        want = (_sq_sum(100) + _sq_sum(L) - _sq_sum(L - 100)) / 200
    else:
        want = _sq_sum(L) / L
    assert np.allclose(got, want, rtol=1e-14)


def test_pool_per_sequence_offsets_and_empty():
    # Global ramp k = T index: each sequence pools its own tokens; the mean of
    # a ramp over a set symmetric about its midpoint is the midpoint.
    seqlens = [300, 0, 64, 1000]
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    T = int(cu[-1])
    k = np.arange(T, dtype=np.float64)[:, None, None] * np.ones((1, 3, 2))
    got = ORT.boundary_pool(k, cu)
    for b, L in enumerate(seqlens):
        want = 0.0 if L == 0 else cu[b] + (L - 1) / 2
        assert np.allclose(got[b], want)


def test_parameter_count_matches_the_pages():
    d = FACTS["head_dim"]
    n = ORT.param_count(d, FACTS["hidden_multiple_of_head_dim"] * d)
    assert n == 264322
    assert abs(n / 1e6 - FACTS["params_per_layer_millions"]) / FACTS["params_per_layer_millions"] < 0.03


def test_worked_example():
    w = {n: np.array(WORKED[n], dtype=np.float64) for n in ("w1", "b1", "w2", "b2", "w3", "b3", "w4", "b4")}
    z = ORT.router_logits(np.array(WORKED["x"], dtype=np.float64), w)
    assert z.tolist() == WORKED["logits"]
    assert int(ORT.decide(z, 0, 1)) == WORKED["decision"]


def test_decision_mapping_and_ties():
    z = np.array([[0.0, 1.0], [1.0, 0.0], [0.5, 0.5], [-np.inf, 0.0]])
    assert ORT.decide(z, ORT.MODE_FA, ORT.MODE_SSA).tolist() == [1, 0, 0, 1]
    assert ORT.decide(z, ORT.MODE_XA, ORT.MODE_SSA).tolist() == [1, 2, 2, 1]
    assert ORT.decide(z, ORT.MODE_FA, ORT.MODE_XA).tolist() == [2, 0, 0, 2]


def test_route_shapes_and_determinism():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((900, 8, 128))
    w = make_router_weights(128, 512, seed=7)
    m1, z1 = ORT.route(k, [0, 500, 900], w, retrieval_mode=0, sparse_mode=1)
    m2, z2 = ORT.route(k, [0, 500, 900], w, retrieval_mode=0, sparse_mode=1)
    assert m1.shape == (2, 8) and z1.shape == (2, 8, 2)
    assert np.array_equal(m1, m2) and np.array_equal(z1, z2)
    assert set(np.unique(m1)) <= {0, 1}
