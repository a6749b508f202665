"""Pins of the fp64 XA oracle (antidiagonal scoring and top-mass selection).

The pages fix no number for XA, so the pins are closed forms (q = 0), a
brute-force enumeration of the antidiagonal entries, row normalization, and a
subset brute force of the selector.
"""

import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import xa as OX


def _closed_form_zero_q(I, r):
    """P[I, J] for q = 0 as exact fractions: p[a, b'] = 1/(a+1) for b' <= a."""
    off = sum(Fraction(1, a + 1) for a in range(I * r, I * r + r))
    diag = sum(Fraction(a - I * r + 1, a + 1) for a in range(I * r, I * r + r)) / r
    return off, diag


def test_zero_query_closed_form_worked_values():
    B, S, d = 128, 8, 8
    r = B // S
    L = 32 * B
    k = np.random.default_rng(0).standard_normal((L, d))
    P = OX.block_mass(np.zeros((L, d)), k, S, B, 0.1, rows=[0, 3, 17, 31])
    for I in (0, 3, 17, 31):
        off, diag = _closed_form_zero_q(I, r)
        np.testing.assert_allclose(P[I, :I], float(off), rtol=0, atol=1e-14)
        assert abs(P[I, I] - float(diag)) < 1e-14
    # Worked values at B = 128, S = 8.
    np.testing.assert_allclose(P[3, :4], [0.285094, 0.285094, 0.285094, 0.144719], atol=5e-7)
    assert abs(P[31, 0] - 0.031717) < 5e-7 and abs(P[31, 31] - 0.016766) < 5e-7


def _exact_select(weights, I, tau):
    """Exact-rational reference of the selector on integer weights."""
    W = sum(weights)
    order = sorted(range(I + 1), key=lambda J: (-weights[J], J))
    acc = 0
    chosen = set()
    for J in order:
        acc += weights[J]
        chosen.add(J)
        if Fraction(acc, W) >= tau:
            break
    return chosen | {0, I}


def test_zero_query_selection_excludes_29_30():
    # q = 0, I = 31: 31 equal off-diagonal masses (0.031717) and a smaller
    # diagonal (0.016766).  tau = 0.9 needs 29 of the equal blocks; ties go to
    # the lower J; the sink and diagonal are added: {0..28, 31}.
    B, S, d = 128, 8, 4
    L = 32 * B
    k = np.random.default_rng(1).standard_normal((L, d))
    P = OX.block_mass(np.zeros((L, d)), k, S, B, 0.3, rows=[31])
    m = OX.select_row(P[31], 31, 9, 10)
    assert set(np.nonzero(m)[0]) == set(range(29)) | {31}
    off, diag = _closed_form_zero_q(31, B // S)
    w = [int(np.floor(float(off) * 2**24 + 0.5))] * 31 + [int(np.floor(float(diag) * 2**24 + 0.5))]
    assert _exact_select(w, 31, Fraction(9, 10)) == set(range(29)) | {31}


def _brute_block_mass(q, k, S, B, c):
    """Explicit loops over every (i, j) with (i mod S) + (j mod S) = S - 1."""
    L = q.shape[0]
    n = L // S
    s = np.zeros((n, n))
    for i in range(L):
        for j in range(L):
            if (i % S) + (j % S) == S - 1:
                s[i // S, j // S] += c * float(np.dot(q[i], k[j]))
    p = np.zeros((n, n))
    for a in range(n):
        row = s[a, : a + 1]
        e = np.exp(row - row.max())
        p[a, : a + 1] = e / e.sum()
    r = B // S
    nb = L // B
    P = np.zeros((nb, nb))
    for a in range(n):
        for b in range(a + 1):
            P[a // r, b // r] += p[a, b] / r
    return P


@pytest.mark.parametrize("L,B,S,d", [(64, 16, 4, 5), (48, 8, 2, 3), (32, 32, 8, 4)])
def test_antidiagonal_bruteforce(L, B, S, d):
    rng = np.random.default_rng(L + B + S)
    q, k = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    P = OX.block_mass(q, k, S, B, 0.7, chunk_rows=5)
    ref = _brute_block_mass(q, k, S, B, 0.7)
    nb = L // B
    for I in range(nb):
        np.testing.assert_allclose(P[I, : I + 1], ref[I, : I + 1], atol=1e-13)


def test_row_normalization():
    rng = np.random.default_rng(7)
    L, B, S, d = 512, 64, 8, 16
    q, k = rng.standard_normal((L, d)) * 2, rng.standard_normal((L, d))
    P = OX.block_mass(q, k, S, B, 0.25)
    for I in range(L // B):
        assert abs(P[I, : I + 1].sum() - 1.0) < 1e-12
        assert np.all(P[I, : I + 1] >= 0)


def test_selector_subset_bruteforce():
    rng = np.random.default_rng(11)
    cases = 0
    for trial in range(400):
        I = int(rng.integers(0, 12))
        raw = rng.random(I + 1) ** rng.choice([1, 4, 12])
        if trial % 5 == 0:          # plant exact ties
            raw[rng.integers(0, I + 1, size=3)] = raw[0]
        P = raw / raw.sum()
        tn, td = [(9, 10), (1, 2), (99, 100), (1, 1), (1, 3)][trial % 5]
        mask = OX.select_row(P, I, tn, td)
        w = OX.quantize(P)
        W = int(w.sum())
        reach = lambda sub: sum(int(w[j]) for j in sub) * td >= tn * W
        kmin = min(len(sub) for n in range(1, I + 2)
                   for sub in itertools.combinations(range(I + 1), n) if reach(sub))
        sel = set(_exact_select([int(x) for x in w], I, Fraction(tn, td))) - set()
        # Property form: a minimum-cardinality set that reaches tau, whose
        # members all precede every non-member in (w desc, J asc) order,
        # united with the sink and diagonal blocks.
        order = sorted(range(I + 1), key=lambda J: (-int(w[J]), J))
        top = set(order[:kmin])
        assert reach(top)
        assert set(np.nonzero(mask)[0]) == top | {0, I} == sel
        cases += 1
    assert cases == 400


def test_tau_one_keeps_every_block():
    rng = np.random.default_rng(3)
    for I in range(0, 40, 7):
        P = rng.random(I + 1) ** 8
        P /= P.sum()
        assert OX.select_row(P, I, 1, 1).all()


def test_quantization_rounds_half_up():
    half = (5 + 0.5) / 2**24
    assert OX.quantize([half])[0] == 6
    assert OX.quantize([0.0])[0] == 1            # floor at 1
    assert OX.quantize([1.0])[0] == 2**24


def test_r1_normalization_is_nearly_one_hot():
    # The literal "softmax over raw block sums" reading concentrates all mass
    # in one block for unit-variance inputs, which is why R2 is the default.
    rng = np.random.default_rng(5)
    L, B, S, d = 1024, 128, 8, 128
    q, k = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    P1 = OX.block_mass(q, k, S, B, d ** -0.5, normalization="R1", rows=[7])
    P2 = OX.block_mass(q, k, S, B, d ** -0.5, rows=[7])
    assert P1[7, :8].max() > 0.99
    assert P2[7, :8].max() < 0.5


def test_group_query_is_the_mean_of_the_scores():
    # The group mask is scored with the mean query: its reduced scores are the
    # mean of the heads' reduced scores (brute force), not their sum, and a
    # group of identical heads selects exactly the per-head mask.
    rng = np.random.default_rng(9)
    L, d, S, B, G = 64, 8, 4, 16, 4
    qg = rng.standard_normal((G, L, d))
    kg = rng.standard_normal((L, d))
    qm = OX.group_query(qg)
    n = L // S
    for a in range(n):
        for bq in range(a + 1):
            per_head = [sum(qg[h, a * S + t] @ kg[bq * S + S - 1 - t] for t in range(S)) for h in range(G)]
            pooled = sum(qm[a * S + t] @ kg[bq * S + S - 1 - t] for t in range(S))
            assert np.isclose(pooled, np.mean(per_head), rtol=1e-12, atol=1e-12)
    same = np.repeat(qg[:1], G, axis=0)
    m1, P1 = OX.head_mask(qg[0], kg, S, B, 0.3, 9, 10)
    mg, Pg = OX.head_mask(OX.group_query(same), kg, S, B, 0.3, 9, 10)
    assert np.array_equal(m1, mg) and np.allclose(P1, Pg, rtol=1e-13, equal_nan=True)
    assert np.array_equal(OX.group_query(qg[:1]), qg[0])
