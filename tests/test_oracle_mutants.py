"""The pins catch plausible oracle mistakes.

Each case plants one mistake in the oracle (on the CPU, via monkeypatch) and
checks that at least one pin then fails.  This is evidence that the pins are
sensitive, not only that the current oracle passes them.
"""

import numpy as np
import pytest

from oracle import attention as OA
from oracle import ratios as OR
from oracle import xa as OX
import test_oracle_attention as TA
import test_oracle_ratios as TR
import test_oracle_xa as TX


def _window_inclusive(mode, i_idx, j_idx, L, sink, window, block=None, xa_mask=None):
    i = np.asarray(i_idx)[:, None]
    j = np.asarray(j_idx)[None, :]
    ok = (j <= i) & (j < L) & (i < L)
    if mode == OA.MODE_SSA:
        return ok & ((j < sink) | (i - j <= window))     # planted: <= instead of <
    return _orig_allowed(mode, i_idx, j_idx, L, sink, window, block, xa_mask)


_orig_allowed = OA.allowed_matrix


def test_mutant_window_off_by_one(monkeypatch):
    monkeypatch.setattr(OA, "allowed_matrix", _window_inclusive)
    with pytest.raises(AssertionError):
        TA.test_ssa_zero_query_closed_form(97, 5, 17)


def test_mutant_dropped_scale(monkeypatch):
    orig = OA.head_attention

    def no_scale(qh, kh, vh, mode, scale, *a, **kw):
        return orig(qh, kh, vh, mode, 1.0, *a, **kw)      # planted: scale dropped
    monkeypatch.setattr(OA, "head_attention", no_scale)
    with pytest.raises(AssertionError):
        TA.test_fa_matches_textbook_sdpa()


def test_mutant_main_diagonal_instead_of_antidiagonal(monkeypatch):
    def reduced_no_reverse(qh, kg, S):
        L, d = qh.shape
        n = L // S
        return qh.reshape(n, S * d), kg.reshape(n, S * d)   # planted: k not reversed
    monkeypatch.setattr(OX, "_reduced", reduced_no_reverse)
    with pytest.raises(AssertionError):
        TX.test_antidiagonal_bruteforce(64, 16, 4, 5)


def test_mutant_tie_break_descending(monkeypatch):
    orig = OX.select_row

    def desc_ties(P_row, I, tn, td):
        # planted: equal weights ordered by J descending
        w = OX.quantize(P_row[: I + 1])
        J = np.arange(I + 1)
        order = np.lexsort((-J, -w))
        cs = np.cumsum(w[order])
        k = int(np.argmax(cs * td >= tn * int(cs[-1])))
        m = np.zeros(I + 1, dtype=bool)
        m[order[: k + 1]] = True
        m[0] = m[I] = True
        return m
    monkeypatch.setattr(OX, "select_row", desc_ties)
    with pytest.raises(AssertionError):
        TX.test_zero_query_selection_excludes_29_30()
    monkeypatch.setattr(OX, "select_row", orig)


def test_mutant_pooling_without_one_over_r(monkeypatch):
    orig = OX.block_mass

    def no_r(qh, kg, S, B, scale, *a, **kw):
        return orig(qh, kg, S, B, scale, *a, **kw) * (B // S)   # planted: missing 1/r
    monkeypatch.setattr(OX, "block_mass", no_r)
    with pytest.raises(AssertionError):
        TX.test_row_normalization()


def test_mutant_ssa_pairs_sink_double_counted(monkeypatch):
    def double(L, sink, window):
        i = np.arange(L, dtype=np.int64)
        lo = np.maximum(i - window + 1, 0)
        return int((np.minimum(i + 1, sink) + (i - lo + 1)).sum())   # planted: overlap counted twice
    monkeypatch.setattr(OR, "ssa_kept_pairs", double)
    with pytest.raises(AssertionError):
        TR.test_ssa_pairs_brute_and_closed_form(300, 7, 40)


# ---- router -------------------------------------------------------------

import test_oracle_router as TRT
from oracle import router as ORT


def test_mutant_router_pools_every_token(monkeypatch):
    monkeypatch.setattr(ORT, "boundary_positions", lambda L, head=100, tail=100: np.arange(int(L)))
    with pytest.raises(AssertionError):
        TRT.test_pool_quadratic_closed_form(333)


def test_mutant_router_counts_overlap_twice(monkeypatch):
    def twice(L, head=100, tail=100):
        L = int(L)
        return np.concatenate([np.arange(min(head, L)), np.arange(max(L - tail, 0), L)])
    monkeypatch.setattr(ORT, "boundary_positions", twice)
    with pytest.raises(AssertionError):
        TRT.test_pool_quadratic_closed_form(150)


def test_mutant_router_concat_swapped(monkeypatch):
    def swapped(pooled, w):
        f = {n: np.asarray(a, dtype=np.float64) for n, a in w.items()}
        x = np.asarray(pooled, dtype=np.float64)
        z_task = ORT.relu(x @ f["w1"] + f["b1"]) @ f["w2"] + f["b2"]
        h = ORT.relu(np.concatenate([z_task, x], axis=-1) @ f["w3"] + f["b3"])   # planted
        return h @ f["w4"] + f["b4"]
    monkeypatch.setattr(ORT, "router_logits", swapped)
    with pytest.raises(AssertionError):
        TRT.test_worked_example()


def test_mutant_router_transposed_w3(monkeypatch):
    orig = ORT.router_logits

    def transposed(pooled, w):
        w = dict(w)
        w["w3"] = np.asarray(w["w3"]).T                                         # planted
        return orig(pooled, w)
    monkeypatch.setattr(ORT, "router_logits", transposed)
    with pytest.raises(AssertionError):
        TRT.test_worked_example()


def test_mutant_router_no_relu(monkeypatch):
    monkeypatch.setattr(ORT, "relu", lambda x: x)                               # planted
    with pytest.raises(AssertionError):
        TRT.test_worked_example()


def test_mutant_router_ties_to_sparse(monkeypatch):
    def ties_sparse(logits, retrieval_mode, sparse_mode):
        z = np.asarray(logits)
        r = (z[..., 1] >= z[..., 0]).astype(np.int64)                          # planted
        return np.where(r == 1, sparse_mode, retrieval_mode).astype(np.uint8)
    monkeypatch.setattr(ORT, "decide", ties_sparse)
    with pytest.raises(AssertionError):
        TRT.test_decision_mapping_and_ties()


# ---- decode -------------------------------------------------------------

import test_oracle_decode as TD
from oracle import decode as OD


def test_mutant_decode_xa_as_ssa(monkeypatch):
    src = OD.decode

    def decode_xa_as_ssa(q_new, k, v, cu, modes, **kw):
        m = np.where(np.asarray(modes) == OD.MODE_XA, OD.MODE_SSA, modes)       # planted
        return src(q_new, k, v, cu, m, **kw)
    monkeypatch.setattr(OD, "decode", decode_xa_as_ssa)
    with pytest.raises(AssertionError):
        TD.test_decode_matches_sdpa_on_gathered_keys(4, 16)


def test_mutant_decode_query_one_back(monkeypatch):
    orig = OD.row_attention

    def one_back(q_i, k_seq, v_seq, i, mode, scale, **kw):
        return orig(q_i, k_seq, v_seq, max(i - 1, 0), mode, scale, **kw)          # planted
    monkeypatch.setattr(OD, "row_attention", one_back)
    with pytest.raises(AssertionError):
        TD.test_zero_query_closed_form(13, 4, 8)


def test_mutant_group_scores_summed(monkeypatch):
    monkeypatch.setattr(OX, "group_query", lambda q: np.asarray(q, dtype=np.float64).sum(axis=0))  # planted
    with pytest.raises(AssertionError):
        TX.test_group_query_is_the_mean_of_the_scores()


# ---- XA pair count, tie diagnostics, block-sum masses, partial blocks ----

def test_mutant_kept_pairs_diagonal_full_square(monkeypatch):
    def square(mask, L, B):
        nb = mask.shape[0]
        return sum(B * B for I in range(nb) for J in np.nonzero(mask[I, : I + 1])[0])  # planted
    monkeypatch.setattr(OX, "kept_pairs", square)
    with pytest.raises(AssertionError):
        TX.test_kept_pairs_hand_counts()


def test_mutant_kept_pairs_ignores_sequence_end(monkeypatch):
    def full_blocks(mask, L, B):
        nb = mask.shape[0]
        return sum(B * B if J < I else B * (B + 1) // 2                                 # planted
                   for I in range(nb) for J in np.nonzero(mask[I, : I + 1])[0])
    monkeypatch.setattr(OX, "kept_pairs", full_blocks)
    with pytest.raises(AssertionError):
        TX.test_kept_pairs_brute_force(61, 8)


def test_mutant_tie_rule_too_broad(monkeypatch):
    orig = OX.tie_info
    monkeypatch.setattr(OX, "tie_info", lambda P, I, tn, td, cum_eps=1e-4, gap_rel=1e-5:
                        orig(P, I, tn, td, cum_eps=1e-2, gap_rel=gap_rel))               # planted
    with pytest.raises(AssertionError):
        TX.test_tie_info_threshold_is_1e4()


def test_mutant_tie_gap_absolute(monkeypatch):
    orig = OX.tie_info

    def absolute_gap(P_row, I, tn, td, cum_eps=1e-4, gap_rel=1e-5):
        t = orig(P_row, I, tn, td, cum_eps=cum_eps, gap_rel=gap_rel)
        w = OX.quantize(P_row[: I + 1])
        order = np.lexsort((np.arange(I + 1), -w))
        p = np.asarray(P_row[: I + 1])[order]
        k = t["k"]
        t["gap_tie"] = bool(k + 1 < len(p) and p[k] - p[k + 1] < 1e-4)              # planted
        return t
    monkeypatch.setattr(OX, "tie_info", absolute_gap)
    with pytest.raises(AssertionError):
        TX.test_tie_info_near_equal_masses_at_the_cut()


def test_mutant_tie_cut_one_late(monkeypatch):
    orig = OX.tie_info

    def late(P_row, I, tn, td, cum_eps=1e-4, gap_rel=1e-5):
        t = orig(P_row, I, tn, td, cum_eps=cum_eps, gap_rel=gap_rel)
        t["k"] = min(t["k"] + 1, I)                                                    # planted
        return t
    monkeypatch.setattr(OX, "tie_info", late)
    with pytest.raises(AssertionError):
        TX.test_tie_info_cut_agrees_with_selector()


def _r1_variant(strict=False, scaled=True):
    orig = OX.block_mass

    def bm(qh, kg, S, B, scale, normalization="R2", chunk_rows=1024, rows=None):
        if normalization != "R1":
            return orig(qh, kg, S, B, scale, normalization, chunk_rows, rows)
        L, d = qh.shape
        nb, r = L // B, B // S
        Qr, Kr = OX._reduced(qh, kg, S)
        P = np.full((nb, nb), np.nan)
        for I in range(nb):
            a = np.arange(I * r, (I + 1) * r)
            s = (scale if scaled else 1.0) * (Qr[a] @ Kr[: (I + 1) * r].T)
            bq = np.arange((I + 1) * r)
            keep = bq[None, :] < a[:, None] if strict else bq[None, :] <= a[:, None]
            raw = np.where(keep, s, 0.0).reshape(r, I + 1, r).sum(axis=(0, 2))
            e = np.exp(raw - raw.max())
            P[I, : I + 1] = e / e.sum()
        return P
    return bm


def test_mutant_r1_drops_diagonal_reduced_entry(monkeypatch):
    monkeypatch.setattr(OX, "block_mass", _r1_variant(strict=True))                    # planted
    with pytest.raises(AssertionError):
        TX.test_r1_block_mass_bruteforce(64, 16, 4, 5)


def test_mutant_r1_drops_scale(monkeypatch):
    monkeypatch.setattr(OX, "block_mass", _r1_variant(scaled=False))                   # planted
    with pytest.raises(AssertionError):
        TX.test_r1_block_mass_bruteforce(48, 8, 2, 3)


def test_mutant_partial_block_diagonal_only(monkeypatch):
    orig = OX.head_mask

    def diag_only(qh, kg, S, B, scale, tn, td, rows=None, normalization="R2"):
        L = qh.shape[0]
        if L % B:
            nb = -(-L // B)
            return np.eye(nb, dtype=bool), None                                         # planted
        return orig(qh, kg, S, B, scale, tn, td, rows=rows, normalization=normalization)
    monkeypatch.setattr(OX, "head_mask", diag_only)
    with pytest.raises(AssertionError):
        TX.test_partial_last_block_is_fa(77)


def test_mutant_tie_without_weight_rounding(monkeypatch):
    orig = OX.tie_info

    def no_round(P_row, I, tn, td, cum_eps=1e-4, gap_rel=1e-5):
        t = orig(P_row, I, tn, td, cum_eps=cum_eps, gap_rel=gap_rel)
        t["round_tie"] = False                                                          # planted
        return t
    monkeypatch.setattr(OX, "tie_info", no_round)
    with pytest.raises(AssertionError):
        TX.test_tie_info_weight_rounding_at_the_cut()


def test_mutant_tie_rounding_any_weight(monkeypatch):
    orig = OX.tie_info

    def any_weight(P_row, I, tn, td, cum_eps=1e-4, gap_rel=1e-5):
        t = orig(P_row, I, tn, td, cum_eps=cum_eps, gap_rel=gap_rel)
        x = np.asarray(P_row[: I + 1]) * float(1 << 24)
        t["round_tie"] = t["round_tie"] or bool((np.abs(x - np.floor(x) - 0.5) < 1e-5 * x).any())  # planted
        return t
    monkeypatch.setattr(OX, "tie_info", any_weight)
    with pytest.raises(AssertionError):
        TX.test_tie_info_weight_rounding_at_the_cut()


def test_mutant_tie_rounding_near_cut_weight(monkeypatch):
    orig = OX.tie_info

    def near_cut_weight(P_row, I, tn, td, cum_eps=1e-4, gap_rel=1e-5):
        t = orig(P_row, I, tn, td, cum_eps=cum_eps, gap_rel=gap_rel)
        w = OX.quantize(P_row[: I + 1])
        order = np.lexsort((np.arange(I + 1), -w))
        x = np.asarray(P_row[: I + 1]) * float(1 << 24)
        near = np.abs(x - np.floor(x) - 0.5) < 1e-5 * x
        wk = w[order[t["k"]]]
        t["round_tie"] = t["round_tie"] or bool((near & (np.abs(w - wk) <= 1)).any())     # planted
        return t
    monkeypatch.setattr(OX, "tie_info", near_cut_weight)
    with pytest.raises(AssertionError):
        TX.test_tie_info_heavy_block_at_a_rounding_boundary_is_no_tie()
