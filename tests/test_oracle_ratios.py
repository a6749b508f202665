"""Pins of the fp64 sparsity-ratio oracle (Eqs. 4-5)."""

import json
import os

import numpy as np
import pytest

from oracle import ratios as OR
from synth import MODE_FA, MODE_SSA, MODE_XA

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def _brute_ssa_pairs(L, sink, window):
    return sum(1 for i in range(L) for j in range(i + 1) if j < sink or i - j < window)


def _closed_form_ssa_pairs(L, s, W):
    # Valid for s <= W and L >= W + s - 1.
    return W * (W + 1) // 2 + (L - W) * (W + s) - s * (s - 1) // 2


@pytest.mark.parametrize("L,s,W", [(1024, 64, 256), (300, 7, 40), (100, 0, 10), (64, 16, 16), (97, 5, 90)])
def test_ssa_pairs_brute_and_closed_form(L, s, W):
    got = OR.ssa_kept_pairs(L, s, W)
    assert got == _brute_ssa_pairs(L, s, W)
    if s <= W and L >= W + s - 1:
        assert got == _closed_form_ssa_pairs(L, s, W)


def test_ssa_pairs_edge_cases():
    assert OR.ssa_kept_pairs(0, 4, 4) == 0
    assert OR.ssa_kept_pairs(50, 0, 1) == 50                 # self only
    assert OR.ssa_kept_pairs(50, 100, 1) == 50 * 51 // 2     # sink covers all
    assert OR.ssa_kept_pairs(50, 0, 50) == 50 * 51 // 2      # window covers all


def test_page_fact_keep_ten_percent_is_rho_point_nine():
    fact = GOLDEN["rho_keep_10_percent"]
    L, Hq = 1000, 4
    causal = L * (L + 1) // 2
    modes = np.array([[MODE_XA, MODE_FA]], dtype=np.uint8)
    xa_pairs = np.zeros((1, Hq), dtype=np.int64)
    xa_pairs[0, :2] = int(fact["kept_fraction"] * causal + 0.5)   # 10 % of each XA q-head
    res = OR.sparsity_ratios([L], modes, Hq, sink=0, window=1, sparse_mode=MODE_XA, xa_pairs=xa_pairs)
    assert abs(res["rho"][0, 0] - fact["rho"]) < 1e-12
    assert res["rho"][0, 1] == 0.0                                # FA head: rho = 0
    assert abs(res["esr"][0] - fact["rho"] / 2) < 1e-12


def test_page_fact_msr_steps_of_one_over_LH():
    fact = GOLDEN["msr_step"]
    H = fact["kv_heads"]
    prev = None
    for n_sparse in range(H + 1):
        modes = np.array([[MODE_SSA] * n_sparse + [MODE_FA] * (H - n_sparse)], dtype=np.uint8)
        res = OR.sparsity_ratios([512], modes, 4 * H, sink=16, window=64, sparse_mode=MODE_SSA)
        if prev is not None:
            assert abs(res["msr"][0] - prev - fact["step"]) < 1e-15
        prev = res["msr"][0]
    assert prev == 1.0


def test_workload_ratio_values():
    # Closed forms for the FA-SSA workloads (derived from the SSA pair count).
    def rho(L, s, W):
        return 1 - _closed_form_ssa_pairs(L, s, W) / (L * (L + 1) / 2)
    r1 = OR.sparsity_ratios([1024], np.array([[MODE_FA, MODE_SSA]]), 4, sink=64, window=256, sparse_mode=MODE_SSA)
    assert abs(r1["rho"][0, 1] - rho(1024, 64, 256)) < 1e-12
    assert abs(r1["rho"][0, 1] - 0.472866) < 1e-6
    assert r1["msr"][0] == 0.5 and abs(r1["esr"][0] - 0.236433) < 1e-6
    m2 = np.array([[0, 1, 1, 0, 1, 1, 0, 1]], dtype=np.uint8)
    r2 = OR.sparsity_ratios([16384], m2, 32, sink=128, window=2048, sparse_mode=MODE_SSA)
    assert abs(r2["rho"][0, 1] - 0.752021) < 1e-6
    assert r2["msr"][0] == 0.625 and abs(r2["esr"][0] - 0.470013) < 1e-6
    r64 = OR.sparsity_ratios([65536], m2, 32, sink=128, window=2048, sparse_mode=MODE_SSA)
    assert abs(r64["rho"][0, 1] - 0.934697) < 1e-6 and abs(r64["esr"][0] - 0.584185) < 1e-6
    # Pair-weighted batch ESR: 1/(1 - esr_pairs) is the FLOP ratio vs all-FA.
    assert abs(r64["esr_pairs"] - r64["esr"][0]) < 1e-12           # one sequence


def test_batch_means_and_pair_weighting():
    modes = np.array([[MODE_FA, MODE_SSA], [MODE_SSA, MODE_SSA]], dtype=np.uint8)
    res = OR.sparsity_ratios([100, 300], modes, 2, sink=4, window=10, sparse_mode=MODE_SSA)
    assert res["msr"][2] == pytest.approx((0.5 + 1.0) / 2)
    assert res["esr"][2] == pytest.approx(res["esr"][:2].mean())
    kept = 1 * 100 * 101 // 2 + 1 * OR.ssa_kept_pairs(100, 4, 10) + 2 * OR.ssa_kept_pairs(300, 4, 10)
    causal = 2 * 100 * 101 // 2 + 2 * 300 * 301 // 2
    assert res["esr_pairs"] == pytest.approx(1 - kept / causal, abs=1e-15)
