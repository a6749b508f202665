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


# ---- attended-pair count ------------------------------------------------

def _brute_pairs(mask, L, B):
    """(i, j) pairs counted one by one from the XA key-set definition:
    j <= i, both inside the sequence, and block pair (i // B, j // B) selected."""
    n = 0
    for i in range(L):
        for j in range(i + 1):
            if mask[i // B, j // B]:
                n += 1
    return n


@pytest.mark.parametrize("L,B", [(64, 8), (61, 8), (96, 16), (100, 16), (17, 16), (1, 4)])
def test_kept_pairs_brute_force(L, B):
    rng = np.random.default_rng(L * 31 + B)
    nb = -(-L // B)
    for trial in range(6):
        m = np.tril(rng.random((nb, nb)) < (0.2 + 0.15 * trial))
        if trial % 2:
            m[np.arange(nb), np.arange(nb)] = True
            m[:, 0] = True
        assert OX.kept_pairs(m, L, B) == _brute_pairs(m, L, B)


def test_kept_pairs_hand_counts():
    B = 16
    # Every causal block of 5 full blocks: the causal triangle of 80 tokens.
    assert OX.kept_pairs(np.tril(np.ones((5, 5), dtype=bool)), 80, B) == 80 * 81 // 2
    # Diagonal blocks only: B (B + 1) / 2 each, not B * B.
    assert OX.kept_pairs(np.eye(5, dtype=bool), 80, B) == 5 * (16 * 17 // 2)
    # Sink block of row 3 plus its diagonal: 16 * 16 + 136.
    m = np.zeros((5, 5), dtype=bool)
    m[3, 0] = m[3, 3] = True
    assert OX.kept_pairs(m, 80, B) == 256 + 136
    # A last block cut to 5 tokens: its diagonal block holds 5 * 6 / 2 pairs
    # and its sink block 5 * 16.
    m = np.zeros((5, 5), dtype=bool)
    m[4, 0] = m[4, 4] = True
    assert OX.kept_pairs(m, 69, B) == 15 + 80


# ---- boundary-tie diagnostics -------------------------------------------

def _row(sorted_masses, n_rest=6):
    """Block row I = len + n_rest - 1 whose largest masses are `sorted_masses`
    (in that order, at J = 1, 2, ...) and whose remaining mass is spread
    evenly over the other n_rest blocks (J = 0 and the tail)."""
    head = list(sorted_masses)
    rest = (1.0 - sum(head)) / n_rest
    assert 0 < rest < head[-1]
    P = np.array([rest] + head + [rest] * (n_rest - 1))
    return P, len(P) - 1


def test_tie_info_cumulative_mass_at_tau():
    # tau = 0.9.  The prefix 0.5 + 0.40005 reaches 0.90005: the cut's
    # cumulative mass is 5e-5 above tau, a boundary tie.
    P, I = _row([0.5, 0.40005])
    t = OX.tie_info(P, I, 9, 10)
    assert t["k"] == 1 and t["cum_tie"] and not t["gap_tie"]
    assert abs(t["c_k"] - 0.90005) < 1e-12
    # The prefix before the cut ends 5e-5 below tau.
    P, I = _row([0.5, 0.39995, 0.05])
    t = OX.tie_info(P, I, 9, 10)
    assert t["k"] == 2 and t["cum_tie"] and abs(t["c_prev"] - 0.89995) < 1e-12


def test_tie_info_threshold_is_1e4():
    # 9e-5 above tau is a tie, 1.1e-4 above is not.
    P, I = _row([0.5, 0.40009])
    assert OX.tie_info(P, I, 9, 10)["cum_tie"]
    P, I = _row([0.5, 0.40011])
    t = OX.tie_info(P, I, 9, 10)
    assert not t["cum_tie"] and not t["gap_tie"]


def test_tie_info_near_equal_masses_at_the_cut():
    # 0.5 + 0.35 + 0.07 = 0.92 passes tau at k = 2; the first dropped mass is
    # 1e-6 relative below the last kept one: its order is within rounding.
    P, I = _row([0.5, 0.35, 0.07, 0.07 * (1 - 1e-6)])
    t = OX.tie_info(P, I, 9, 10)
    assert t["k"] == 2 and t["gap_tie"] and not t["cum_tie"]
    # 5e-6 apart (7e-5 relative): a real order, not a tie.
    P, I = _row([0.5, 0.35, 0.07, 0.07 - 5e-6])
    t = OX.tie_info(P, I, 9, 10)
    assert t["k"] == 2 and not t["gap_tie"] and not t["cum_tie"]


def test_tie_info_cut_agrees_with_selector():
    # The cut position k is the selector's: k + 1 blocks of the sorted order
    # are the top-mass prefix.
    rng = np.random.default_rng(21)
    for trial in range(200):
        I = int(rng.integers(1, 40))
        P = rng.random(I + 1) ** 6
        P /= P.sum()
        t = OX.tie_info(P, I, 9, 10)
        m = OX.select_row(P, I, 9, 10)
        order = np.lexsort((np.arange(I + 1), -OX.quantize(P)))
        top = set(order[: t["k"] + 1].tolist())
        assert set(np.nonzero(m)[0].tolist()) == top | {0, I}
        assert t["c_k"] >= 0.9 - 1e-12 > t["c_prev"] - 1e-12 or t["cum_tie"]


# ---- block-sum masses (reading R1) --------------------------------------

def _brute_block_mass_r1(q, k, S, B, c):
    """R1 from explicit loops: the raw block sum adds c <q_i, k_j> over every
    antidiagonal entry ((i mod S) + (j mod S) = S - 1) of block (I, J) whose
    reduced key is not after its reduced query (j // S <= i // S); each block
    row is then softmaxed over J <= I."""
    L = q.shape[0]
    nb = L // B
    raw = np.zeros((nb, nb))
    for i in range(L):
        for j in range(L):
            if (i % S) + (j % S) == S - 1 and j // S <= i // S:
                raw[i // B, j // B] += c * float(np.dot(q[i], k[j]))
    P = np.zeros((nb, nb))
    for I in range(nb):
        e = np.exp(raw[I, : I + 1] - raw[I, : I + 1].max())
        P[I, : I + 1] = e / e.sum()
    return P


@pytest.mark.parametrize("L,B,S,d", [(64, 16, 4, 5), (48, 8, 2, 3), (96, 32, 8, 4)])
def test_r1_block_mass_bruteforce(L, B, S, d):
    rng = np.random.default_rng(L + 7 * B + S)
    q, k = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    P = OX.block_mass(q, k, S, B, 0.35, normalization="R1")
    ref = _brute_block_mass_r1(q, k, S, B, 0.35)
    for I in range(L // B):
        np.testing.assert_allclose(P[I, : I + 1], ref[I, : I + 1], rtol=0, atol=1e-13)


def test_r1_zero_query_is_uniform():
    # q = 0: every raw block sum is 0, so each block row is uniform, 1 / (I + 1)
    # (R2 instead gives the diagonal block about half the weight of the others).
    L, B, S, d = 512, 64, 8, 6
    k = np.random.default_rng(4).standard_normal((L, d))
    P = OX.block_mass(np.zeros((L, d)), k, S, B, 0.5, normalization="R1")
    for I in range(L // B):
        np.testing.assert_allclose(P[I, : I + 1], 1.0 / (I + 1), rtol=0, atol=1e-15)


# ---- sequences that are not a whole number of blocks --------------------

@pytest.mark.parametrize("L", [77, 130, 5])
def test_partial_last_block_is_fa(L):
    # XA needs a whole number of blocks to score; such a sequence keeps every
    # causal block (the tau = 1 selection), so its XA attention is FA.
    from oracle import attention as OA
    B, S, d = 16, 4, 6
    rng = np.random.default_rng(L)
    q, k, v = (rng.standard_normal((L, d)) for _ in range(3))
    M, P = OX.head_mask(q, k, S, B, 0.4, 9, 10)
    nb = -(-L // B)
    assert P is None and M.shape == (nb, nb)
    assert np.array_equal(M, np.tril(np.ones((nb, nb), dtype=bool)))
    ox, lx = OA.head_attention(q, k, v, OA.MODE_XA, 0.4, block=B, xa_mask=M, chunk=32)
    of, lf = OA.head_attention(q, k, v, OA.MODE_FA, 0.4, chunk=32)
    np.testing.assert_array_equal(ox, of)
    np.testing.assert_array_equal(lx, lf)
    # Its pair count is the causal triangle of L tokens.
    assert OX.kept_pairs(M, L, B) == L * (L + 1) // 2


def test_tie_info_weight_rounding_at_the_cut():
    # A flat row whose last kept block scales to 4998.3 (weight 4998) and
    # whose first dropped block scales to 4997.4996 (weight 4997, 0.0004 below
    # the rounding boundary): fp32 masses can round that block up to 4998,
    # where the J-ascending order puts it first.  The masses differ by
    # 1.7e-4 relative, so the gap rule does not see it; the rounding rule does.
    S = float(1 << 24)

    def row(x_drop):
        # Head masses sum to tau - 1.5e-4, so the prefix crosses tau on the
        # 4998.3 block; 400 light blocks (weight ~4176) follow the cut.
        head = [0.4, 0.3, 0.9 - 1.5e-4 - 0.7]
        n_tail = 400
        rest = (1.0 - sum(head) - 4998.3 / S - x_drop / S) / (n_tail + 1)
        P = np.array([rest] + head + [4998.3 / S, x_drop / S] + [rest] * n_tail)
        return P, len(P) - 1
    P, I = row(4997.4996)
    t = OX.tie_info(P, I, 9, 10)
    order = np.lexsort((np.arange(I + 1), -OX.quantize(P)))
    assert order[t["k"]] == 4 and order[t["k"] + 1] == 5          # the two blocks sit at the cut
    assert t["round_tie"] and not t["gap_tie"] and not t["cum_tie"]
    P, I = row(4997.3)                                             # far from the boundary
    t = OX.tie_info(P, I, 9, 10)
    assert not t["round_tie"] and not t["gap_tie"] and not t["cum_tie"]
    # A block near a rounding boundary far from the cut weight is no tie.
    P, I = row(4997.3)
    P[7] = 1234.4999 / S
    P[0] -= (P.sum() - 1.0)
    t = OX.tie_info(P, I, 9, 10)
    assert not t["round_tie"]


def test_tie_info_heavy_block_at_a_rounding_boundary_is_no_tie():
    # A peaked row: the last kept block scales to exactly n + 1/2, but the
    # first dropped block is far below it, so no rounding step can cross the
    # cut (the masses' relative precision matters only through the gap rule).
    S = float(1 << 24)
    heavy = 5_035_000.5 / S                    # 0.3001..., weight 5,035,001
    P = np.array([0.01, 0.6, heavy] + [(1.0 - 0.61 - heavy) / 30] * 30)
    I = len(P) - 1
    t = OX.tie_info(P, I, 9, 10)
    order = np.lexsort((np.arange(I + 1), -OX.quantize(P)))
    assert order[t["k"]] == 2 and not t["cum_tie"] and not t["gap_tie"]   # 0.6 + 0.3001 passes tau
    assert not t["round_tie"]
