"""fp64 reference: XA antidiagonal block scoring and top-mass block selection.

TEST INFRASTRUCTURE ONLY (see the package header).

The pages name XA only as training-free block-sparse attention that scores
blocks by antidiagonals and keeps blocks up to a cumulative threshold
(glossary of both paper-reading notes; Table 8 of the notes gives
stride / threshold 16 / 0.9 and block 64; the workloads here use block 128,
stride 8, threshold 0.9).  The scoring and the selector are therefore
algorithms written from that description, step by step:

Scoring (reading "R2": softmax per reduced query row, then pool into blocks)
  1. r = B / S reduced rows per block; reduced query a in [0, L/S), reduced
     key b' <= a (causal at the reduced level; the diagonal entry is kept whole).
  2. s^[a, b'] = c * sum_{t<S} <q_{aS+t}, k_{b'S+S-1-t}>: the stride-S
     antidiagonal of each S x S sub-tile of Q K^T, i.e. the entries with
     (i + j) mod S == S - 1.
  3. p[a, .] = softmax over b' in [0, a] of s^[a, .].
  4. P[I, J] = (1/r) sum_{a in block I} sum_{b' in block J, b' <= a} p[a, b'],
     so every block row of P sums to one.
  Reading "R1" (raw antidiagonal sums per block, softmaxed over each block row)
  is kept behind normalization="R1" for comparison only.

Selection (integer-exact)
  1. w_J = max(1, floor(P[I, J] * 2^24 + 1/2)) as integers, W = sum_J w_J.
  2. Order blocks by (w_J descending, J ascending).
  3. Keep the shortest prefix whose integer mass satisfies
     (sum_prefix w) * tau_den >= tau_num * W.
  4. Always keep the sink block J = 0 and the diagonal block J = I (union).
  With tau = 1 every causal block is kept, so XA equals FA.

Parity status: the scoring normalization (R2), the reduced-level causal rule,
the scale c on every product, the union rule for forced blocks and the
tie-break are readings, not fixed by the pages (as is the optional
one-mask-per-KV-head variant, group_query); they are pinned only by
self-consistency (q = 0 closed form, brute-force antidiagonal enumeration,
row normalization, subset brute force of the selector) -- parity unpinned by
the pages themselves.  The R1 masses are pinned by explicit enumeration of the
block sums; kept_pairs by a token-by-token count; tie_info by hand-built rows
on both sides of its thresholds; the partial-block rule of head_mask by its
identity with FA.
"""

import numpy as np

QUANT_BITS = 24


def _reduced(qh, kg, S):
    L, d = qh.shape
    n = L // S
    Qr = qh.reshape(n, S * d)
    Kr = kg.reshape(n, S, d)[:, ::-1, :].reshape(n, S * d)
    return Qr, Kr


def block_mass(qh, kg, S, B, scale, normalization="R2", chunk_rows=1024, rows=None):
    """P [nb, nb] (lower triangle) for one (sequence, q-head); L % B == 0.

    `rows` optionally restricts the computation to the listed block rows I
    (others are left NaN), so single rows of the largest workloads are cheap.
    """
    L, d = qh.shape
    if L % B or B % S:
        raise ValueError("XA needs L % B == 0 and S | B")
    nb = L // B
    r = B // S
    Qr, Kr = _reduced(qh, kg, S)
    P = np.full((nb, nb), np.nan)
    block_rows = range(nb) if rows is None else sorted(set(int(x) for x in rows))
    if normalization == "R1":
        for I in block_rows:
            a = np.arange(I * r, (I + 1) * r)
            s = scale * (Qr[a] @ Kr[: (I + 1) * r].T)
            bq = np.arange((I + 1) * r)
            s = np.where(bq[None, :] <= a[:, None], s, 0.0)
            raw = s.reshape(r, I + 1, r).sum(axis=(0, 2))
            e = np.exp(raw - raw.max())
            P[I, : I + 1] = e / e.sum()
        return P
    # R2: group consecutive requested block rows into chunks of reduced rows.
    block_rows = list(block_rows)
    per = max(1, chunk_rows // r)
    for c0 in range(0, len(block_rows), per):
        Is = block_rows[c0:c0 + per]
        a = np.concatenate([np.arange(I * r, (I + 1) * r) for I in Is])
        amax = int(a.max()) + 1
        s = scale * (Qr[a] @ Kr[:amax].T)                      # [rows, amax]
        bq = np.arange(amax)
        allowed = bq[None, :] <= a[:, None]
        s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.where(allowed, np.exp(s - m), 0.0)
        p = e / e.sum(axis=1, keepdims=True)
        for n, I in enumerate(Is):
            pr = p[n * r:(n + 1) * r, : (I + 1) * r]
            P[I, : I + 1] = pr.reshape(r, I + 1, r).sum(axis=(0, 2)) / r
    return P


def quantize(P_row):
    """Integer weights w_J = max(1, floor(P * 2^24 + 1/2)) (exact in float64)."""
    x = np.floor(np.asarray(P_row, dtype=np.float64) * float(1 << QUANT_BITS) + 0.5)
    return np.maximum(1, x).astype(np.int64)


def select_row(P_row, I, tau_num, tau_den):
    """Boolean mask over J in [0, I] for block row I; P_row has >= I+1 entries."""
    w = quantize(P_row[: I + 1])
    J = np.arange(I + 1)
    order = np.lexsort((J, -w))                 # w descending, then J ascending
    cs = np.cumsum(w[order])
    W = int(cs[-1])
    need = cs * int(tau_den) >= int(tau_num) * W
    k = int(np.argmax(need))                    # first prefix index reaching tau
    mask = np.zeros(I + 1, dtype=bool)
    mask[order[: k + 1]] = True
    mask[0] = True
    mask[I] = True
    return mask


def select(P, tau_num, tau_den, rows=None):
    """Block mask [nb, nb] (bool) from P; rows optionally restricts block rows."""
    nb = P.shape[0]
    M = np.zeros((nb, nb), dtype=bool)
    for I in (range(nb) if rows is None else rows):
        M[I, : I + 1] = select_row(P[I], I, tau_num, tau_den)
    return M


def tie_info(P_row, I, tau_num, tau_den, cum_eps=1e-4, gap_rel=1e-5):
    """Boundary-tie diagnostics of block row I under the fp64 masses.

    Sorted as the selector sorts, with the cut after position k:
      cum_tie    |C_{k-1} - tau| < cum_eps or |C_k - tau| < cum_eps
                 (the pages' threshold boundary; counted and reported);
      gap_tie    the last kept and first dropped masses differ by less than
                 gap_rel * P_(k) (the order at the cut is within rounding);
      round_tie  a kept block whose weight is at most 1 above the first
                 dropped block's, or a dropped block whose weight is at most 1
                 below the last kept block's, has P * 2^24 within
                 gap_rel * P * 2^24 of a rounding boundary (n + 1/2): one
                 rounding step of its weight can move it across the cut, so
                 the order at the cut is within rounding too.
    """
    tau = tau_num / tau_den
    w = quantize(P_row[: I + 1])
    J = np.arange(I + 1)
    order = np.lexsort((J, -w))
    p = np.asarray(P_row[: I + 1], dtype=np.float64)[order]
    cs_w = np.cumsum(w[order])
    k = int(np.argmax(cs_w * int(tau_den) >= int(tau_num) * int(cs_w[-1])))
    C = np.cumsum(p)
    c_prev = C[k - 1] if k > 0 else 0.0
    cum_tie = abs(c_prev - tau) < cum_eps or abs(C[k] - tau) < cum_eps
    gap_tie = (k + 1 < len(p)) and (p[k] - p[k + 1] < gap_rel * p[k])
    round_tie = False
    if k + 1 < len(p):
        x = np.asarray(P_row[: I + 1], dtype=np.float64) * float(1 << QUANT_BITS)
        near_half = np.abs(x - np.floor(x) - 0.5) < gap_rel * np.maximum(x, 1.0)
        wk, wn = int(w[order[k]]), int(w[order[k + 1]])
        kept = np.zeros(I + 1, dtype=bool)
        kept[order[: k + 1]] = True
        can_cross = np.where(kept, w <= wn + 1, w >= wk - 1)
        round_tie = bool((near_half & can_cross).any())
    return dict(k=k, cum_tie=bool(cum_tie), gap_tie=bool(gap_tie), round_tie=round_tie,
                c_prev=float(c_prev), c_k=float(C[k]))


def kept_pairs(mask, L, B):
    """Attended (i, j) pairs of one XA (sequence, q-head) of length L.

    For every selected block pair (I, J) with J <= I: the pairs with query i in
    block I and key j in block J, both inside the sequence, and j <= i (the
    causal rule inside the diagonal block).  A full block below the diagonal
    gives B * B pairs, a full diagonal block B (B + 1) / 2, and a block cut by
    the sequence end fewer.
    """
    nb = mask.shape[0]
    total = 0
    for I in range(nb):
        i = np.arange(I * B, min((I + 1) * B, L), dtype=np.int64)
        for J in np.nonzero(mask[I, : I + 1])[0]:
            j0, j1 = int(J) * B, min((int(J) + 1) * B, L)
            total += int(np.clip(np.minimum(i, j1 - 1) - j0 + 1, 0, None).sum())
    return total


def group_query(q_group):
    """Reading S9-group: one XA mask per KV head.  The antidiagonal scores are
    linear in the query, so the mean of the group's per-head scores s^_h is
    the score of the group-mean query; P, the weights and the selection then
    follow the per-head steps unchanged.  q_group [G, L, d] -> [L, d]."""
    return np.asarray(q_group, dtype=np.float64).mean(axis=0)


def head_mask(qh, kg, S, B, scale, tau_num, tau_den, rows=None, normalization="R2"):
    """XA block mask of one (sequence, q-head) and its block masses.

    A sequence whose length is not a whole number of blocks has no complete
    last block row to score, so it gets every causal block: the selection that
    tau = 1 makes, under which XA is FA.  P is None for it.  `rows` restricts
    scoring and selection to those block rows.
    """
    L = qh.shape[0]
    nb = -(-L // B)
    if L % B:
        return np.tril(np.ones((nb, nb), dtype=bool)), None
    P = block_mass(qh, kg, S, B, scale, normalization=normalization, rows=rows)
    return select(P, tau_num, tau_den, rows=rows), P
