"""Pins of the fp64 decode-step oracle."""

import numpy as np
import pytest
import torch

from oracle import decode as OD
from oracle.attention import MODE_FA, MODE_SSA, MODE_XA


def _batch(seqlens, hq, hkv, d, seed):
    rng = np.random.default_rng(seed)
    T = int(sum(seqlens))
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    q = rng.standard_normal((len(seqlens), hq, d))
    k = rng.standard_normal((T, hkv, d))
    v = rng.standard_normal((T, hkv, d))
    return cu, q, k, v


def _gathered_keys(mode, L, sink, window):
    # Written out from the definition, independently of the oracle: the
    # decoded query i = L - 1 keeps j <= i with (SSA) j < sink or i - j < window.
    i = L - 1
    if mode == MODE_SSA:
        return [j for j in range(L) if j < sink or i - j < window]
    return list(range(L))


@pytest.mark.parametrize("sink,window", [(4, 16), (0, 1), (64, 300), (10, 10 ** 6)])
def test_decode_matches_sdpa_on_gathered_keys(sink, window):
    seqlens = [1, 37, 200, 513]
    hq, hkv, d = 4, 2, 16
    cu, q, k, v = _batch(seqlens, hq, hkv, d, seed=sink + window)
    modes = np.array([[MODE_FA, MODE_SSA], [MODE_SSA, MODE_XA], [MODE_XA, MODE_FA],
                      [MODE_SSA, MODE_SSA]], dtype=np.uint8)
    scale = 0.3
    O, LSE = OD.decode(q, k, v, cu, modes, scale=scale, sink=sink, window=window)
    for b, L in enumerate(seqlens):
        for h in range(hq):
            g = h // (hq // hkv)
            keys = np.array(_gathered_keys(int(modes[b, g]), L, sink, window)) + cu[b]
            qt = torch.from_numpy(q[b, h][None, None, None, :])
            kt = torch.from_numpy(k[keys, g][None, None])
            vt = torch.from_numpy(v[keys, g][None, None])
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
            assert np.allclose(O[b, h], ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-12)
            s = scale * (k[keys, g] @ q[b, h])
            assert np.isclose(LSE[b, h], np.log(np.exp(s - s.max()).sum()) + s.max(), rtol=1e-13)


@pytest.mark.parametrize("L,sink,window", [(1, 4, 8), (9, 4, 8), (12, 4, 8), (13, 4, 8),
                                           (500, 128, 64), (500, 0, 1), (40, 100, 5)])
def test_zero_query_closed_form(L, sink, window):
    # q = 0: every kept key scores 0, so o = mean of the kept v and
    # lse = ln |A|, with |A| in closed form.
    hkv, d = 1, 8
    cu = np.array([0, L])
    rng = np.random.default_rng(L)
    v = rng.standard_normal((L, hkv, d))
    k = rng.standard_normal((L, hkv, d))
    q = np.zeros((1, 2, d))
    for mode in (MODE_FA, MODE_SSA, MODE_XA):
        O, LSE = OD.decode(q, k, v, cu, np.array([[mode]]), scale=1.0, sink=sink, window=window)
        n = OD.kept_keys(MODE_FA if mode == MODE_XA else mode, L, sink, window)
        assert n == len(_gathered_keys(mode, L, sink, window))
        keep = _gathered_keys(mode, L, sink, window)
        assert np.allclose(O[0, 0], v[keep, 0].mean(axis=0), rtol=1e-13, atol=1e-14)
        assert np.isclose(LSE[0, 1], np.log(n), rtol=1e-14)


def test_ssa_with_long_window_is_fa_and_xa_is_fa():
    seqlens = [300, 77]
    cu, q, k, v = _batch(seqlens, 4, 2, 8, seed=3)
    fa = OD.decode(q, k, v, cu, np.zeros((2, 2), np.uint8), scale=0.5, sink=3, window=7)
    ssa = OD.decode(q, k, v, cu, np.ones((2, 2), np.uint8), scale=0.5, sink=3, window=300)
    xa = OD.decode(q, k, v, cu, np.full((2, 2), 2, np.uint8), scale=0.5, sink=3, window=7)
    assert np.array_equal(fa[0], ssa[0]) and np.array_equal(fa[1], ssa[1])
    assert np.array_equal(fa[0], xa[0]) and np.array_equal(fa[1], xa[1])


def test_empty_sequence():
    cu, q, k, v = _batch([0, 5, 0], 2, 1, 4, seed=1)
    O, LSE = OD.decode(q, k, v, cu, np.zeros((3, 1), np.uint8), scale=1.0, sink=1, window=2)
    assert np.all(O[0] == 0) and np.all(O[2] == 0)
    assert np.all(np.isneginf(LSE[0])) and np.all(np.isneginf(LSE[2]))
    assert np.all(np.isfinite(LSE[1]))
