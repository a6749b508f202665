"""Pins of the fp64 attention oracle against what the pages and mathematics fix.

None of these checks re-types the oracle's formula: each compares it with an
independent route (torch's textbook attention, brute-force enumeration of the
allowed key sets, identities that the definitions imply).
"""

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import xa as OX
from synth import make_inputs, get_config, bf16_bits_to_f64, MODE_FA, MODE_SSA, MODE_XA


def _rand(L, d, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal((L, d)), r.standard_normal((L, d)), r.standard_normal((L, d))


def _brute_allowed(mode, L, sink, window, B=None, blockmask=None):
    """A(i) enumerated with plain loops, straight from the prose definitions."""
    sets = []
    for i in range(L):
        s = []
        for j in range(L):
            if j > i:
                continue
            if mode == MODE_FA:
                s.append(j)
            elif mode == MODE_SSA:
                if j < sink or i - j < window:
                    s.append(j)
            else:
                if blockmask[i // B][j // B]:
                    s.append(j)
        sets.append(s)
    return sets


def test_fa_matches_textbook_sdpa():
    # P1: full causal attention is a textbook routine.
    L, d = 203, 24
    q, k, v = _rand(L, d, 0)
    c = 1 / np.sqrt(d)
    o, lse = OA.head_attention(q, k, v, MODE_FA, c, chunk=64)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=c)
    np.testing.assert_allclose(o, ref[0, 0].numpy(), rtol=0, atol=1e-12)
    s = (tq[0, 0] @ tk[0, 0].T) * c
    s = s.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=1).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,sink,window", [(97, 5, 17), (256, 64, 64), (300, 0, 1), (130, 200, 3)])
def test_ssa_zero_query_closed_form(L, sink, window):
    # P5: with q = 0 every allowed score is equal, so o_i is the plain mean of
    # v over A(i) and lse_i = ln |A(i)|; this pins the SSA key set exactly.
    d = 8
    _, k, v = _rand(L, d, 1)
    q = np.zeros((L, d))
    o, lse = OA.head_attention(q, k, v, MODE_SSA, 0.3, sink=sink, window=window, chunk=41)
    sets = _brute_allowed(MODE_SSA, L, sink, window)
    for i in range(L):
        A = sets[i]
        np.testing.assert_allclose(o[i], v[A].mean(axis=0), atol=1e-12)
        assert abs(lse[i] - np.log(len(A))) < 1e-12


def test_xa_zero_query_closed_form():
    L, d, B = 96, 8, 16
    _, k, v = _rand(L, d, 2)
    r = np.random.default_rng(3)
    nb = L // B
    bm = np.tril(r.random((nb, nb)) < 0.5)
    bm[:, 0] = True
    bm[np.arange(nb), np.arange(nb)] = True
    o, lse = OA.head_attention(np.zeros((L, d)), k, v, MODE_XA, 1.0, block=B, xa_mask=bm, chunk=40)
    sets = _brute_allowed(MODE_XA, L, 0, 0, B, bm)
    for i in range(L):
        np.testing.assert_allclose(o[i], v[sets[i]].mean(axis=0), atol=1e-12)
        assert abs(lse[i] - np.log(len(sets[i]))) < 1e-12


def test_ssa_window_at_least_length_equals_fa():
    # P2: SSA with window >= L (or sink >= L) keeps every causal key.
    L, d = 150, 16
    q, k, v = _rand(L, d, 4)
    fa = OA.head_attention(q, k, v, MODE_FA, 0.25)
    for sink, window in [(0, L), (3, L + 7), (L, 1)]:
        ssa = OA.head_attention(q, k, v, MODE_SSA, 0.25, sink=sink, window=window)
        np.testing.assert_array_equal(ssa[0], fa[0])
        np.testing.assert_array_equal(ssa[1], fa[1])
    # ...and a real window is not FA.
    ssa = OA.head_attention(q, k, v, MODE_SSA, 0.25, sink=4, window=20)
    assert np.abs(ssa[0] - fa[0]).max() > 1e-3


def test_xa_tau_one_equals_fa():
    # P3: with tau = 1 every causal block is selected, so XA equals FA.
    L, d, B, S = 128, 16, 32, 4
    q, k, v = _rand(L, d, 5)
    P = OX.block_mass(q, k, S, B, 0.25)
    M = OX.select(P, 1, 1)
    assert M.sum() == (L // B) * (L // B + 1) // 2
    xa = OA.head_attention(q, k, v, MODE_XA, 0.25, block=B, xa_mask=M)
    fa = OA.head_attention(q, k, v, MODE_FA, 0.25)
    np.testing.assert_array_equal(xa[0], fa[0])
    np.testing.assert_array_equal(xa[1], fa[1])


def test_head_concatenation_eq3():
    # P4: the hybrid layer output is the head-wise concatenation (Eq. 3) of
    # single-mode runs.
    cfg = get_config("tiny-1k").with_(seqlens=(200, 64), num_q_heads=4, num_kv_heads=2,
                                      head_dim=16, block=16, ssa_sink=8, ssa_window=40,
                                      modes=((MODE_FA, MODE_SSA), (MODE_XA, MODE_FA)))
    inp = make_inputs(cfg)
    q, k, v = (bf16_bits_to_f64(inp[n]) for n in ("q", "k", "v"))
    cu, modes = inp["cu_seqlens"], inp["modes"]
    # XA heads (b=1, h in {0,1}) use a fixed hand-built block pattern.
    bm = np.tril(np.ones((4, 4), dtype=bool))
    bm[3, 1] = False
    xm = {(1, 0): bm, (1, 1): bm}
    kw = dict(scale=0.25, block=16, sink=8, window=40)
    O, LSE = OA.prefill(q, k, v, cu, modes, xa_masks=xm, **kw)
    for mode in (MODE_FA, MODE_SSA, MODE_XA):
        single = np.full_like(modes, mode)
        bm0 = np.tril(np.ones((13, 13), dtype=bool))
        bm0[7, 2:5] = False
        xms = {(b, h): (bm0 if b == 0 else bm) for b in range(2) for h in range(4)}
        Os, Ls = OA.prefill(q, k, v, cu, single, xa_masks=xms, **kw)
        for b in range(2):
            t0, t1 = cu[b], cu[b + 1]
            for h in range(4):
                if modes[b, h // 2] == mode:
                    np.testing.assert_array_equal(O[t0:t1, h], Os[t0:t1, h])
                    np.testing.assert_array_equal(LSE[h, t0:t1], Ls[h, t0:t1])


def test_prefill_rows_match_full():
    cfg = get_config("tiny-1k").with_(seqlens=(130, 64), head_dim=16, block=16, ssa_sink=5, ssa_window=33)
    inp = make_inputs(cfg)
    q, k, v = (bf16_bits_to_f64(inp[n]) for n in ("q", "k", "v"))
    cu, modes = inp["cu_seqlens"], inp["modes"]
    kw = dict(scale=0.25, block=16, sink=5, window=33)
    O, LSE = OA.prefill(q, k, v, cu, modes, **kw)
    rows = [(0, 0, 0), (0, 3, 129), (1, 1, 7), (1, 2, 63), (0, 2, 50)]
    o, l = OA.prefill_rows(q, k, v, cu, modes, rows, **kw)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(o[n], O[cu[b] + i, h], atol=1e-13)
        assert abs(l[n] - LSE[h, cu[b] + i]) < 1e-13


@pytest.mark.parametrize("mode", [MODE_FA, MODE_SSA, MODE_XA])
def test_row_range_is_the_same_rows(mode):
    # Restricting the computed query rows changes nothing in them beyond the
    # rounding order of the chunked products (the rows of one long head can
    # then be split over threads).
    L, d, B = 300, 8, 16
    q, k, v = _rand(L, d, 9)
    nb = -(-L // B)
    bm = np.tril(np.random.default_rng(4).random((nb, nb)) < 0.6)
    bm[np.arange(nb), np.arange(nb)] = True
    kw = dict(sink=7, window=40, block=B, xa_mask=bm, chunk=64)
    o, lse = OA.head_attention(q, k, v, mode, 0.3, **kw)
    for r0, r1 in ((0, 300), (17, 131), (299, 300), (64, 128)):
        o2, l2 = OA.head_attention(q, k, v, mode, 0.3, row_range=(r0, r1), **kw)
        np.testing.assert_allclose(o2, o[r0:r1], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l2, lse[r0:r1], rtol=0, atol=1e-13)
