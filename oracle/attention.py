"""fp64 reference: masked causal softmax attention for FA, SSA and XA heads.

TEST INFRASTRUCTURE ONLY (see the package header).

What it computes (the plain definition, not an algorithm):
  Paper Reading . Elastic Attention: Test-time Adaptive Sparsity Ratios
  (English notes), "02 . Background": Eq. (1) full attention
  O_r = Softmax(Q K^T) V, Eq. (2) sparse attention over a key subset
  O_s = Softmax(Q K~^T) V~, Eq. (3) head-wise concatenation of the layer output.
  The same equations appear in the Chinese notes (section on retrieval and
  sparse heads).  The glossary of both notes defines SSA as attention sink plus
  sliding window and XA as block-sparse attention with antidiagonal scoring.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * scale c = 1/sqrt(d) and a causal mask j <= i (decoder prefill);
  * SSA keeps key j for query i iff j < sink or i - j < window (token level,
    the union counted once); with window >= L this is exactly FA;
  * XA keeps key j for query i iff the block pair (i // B, j // B) is selected
    in the head's block mask and j <= i;
  * lse_i = m_i + ln(l_i), natural log.

Each query row is an exact two-pass softmax over its allowed key set A(i):
  m_i = max_{j in A(i)} s_ij,  l_i = sum exp(s_ij - m_i),
  o_i = sum exp(s_ij - m_i) v_j / l_i,  s_ij = c <q_i, k_j>.
Query chunks and a restriction to keys that can possibly be allowed are the
only blocking; the token mask is always applied explicitly.

Parity pins (tests/test_oracle_attention.py): textbook causal attention
(torch scaled_dot_product_attention in float64), SSA with window >= L equals
FA, XA with an all-causal mask equals FA, head concatenation, and the q = 0
closed form o_i = mean_{j in A(i)} v_j, lse_i = ln |A(i)|.
"""

import numpy as np

MODE_FA = 0
MODE_SSA = 1
MODE_XA = 2


def allowed_matrix(mode, i_idx, j_idx, L, sink, window, block=None, xa_mask=None):
    """Boolean matrix A[i, j]: may query i (local index) attend key j.

    i_idx, j_idx are 1-D arrays of local token indices.  xa_mask is the
    head's boolean block mask [nQB, nQB] (only for XA).
    """
    i = np.asarray(i_idx)[:, None]
    j = np.asarray(j_idx)[None, :]
    ok = (j <= i) & (j < L) & (i < L)
    if mode == MODE_FA:
        return ok
    if mode == MODE_SSA:
        return ok & ((j < sink) | (i - j < window))
    if mode == MODE_XA:
        if xa_mask is None:
            raise ValueError("XA head needs a block mask")
        return ok & xa_mask[(i // block), (j // block)]
    raise ValueError(f"bad mode {mode}")


def _candidate_keys(mode, i0, i1, sink, window):
    """Key indices that can be allowed for queries in [i0, i1) (superset)."""
    if mode == MODE_SSA:
        lo = max(0, i0 - window + 1)
        head = np.arange(0, min(sink, lo), dtype=np.int64)
        return np.concatenate([head, np.arange(lo, i1, dtype=np.int64)])
    return np.arange(0, i1, dtype=np.int64)


def _softmax_rows(s, allowed, vj):
    """Exact two-pass softmax of masked scores; returns (o, lse)."""
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1)
    e = np.where(allowed, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    o = (e @ vj) / l[:, None]
    return o, m + np.log(l)


def head_attention(qh, kh, vh, mode, scale, sink=0, window=1, block=None,
                   xa_mask=None, chunk=512, row_range=None):
    """One (sequence, query head): qh [L,d], kh/vh [L,d] float64 -> o [L,d], lse [L].

    row_range = (r0, r1) computes only query rows r0 <= i < r1 (returned as
    o [r1 - r0, d], lse [r1 - r0]), so that the rows of one long head can be
    split over host threads; each row is the same sum, up to the rounding
    order of the matrix products over a differently cut chunk.
    """
    L, d = qh.shape
    r0, r1 = (0, L) if row_range is None else (int(row_range[0]), int(row_range[1]))
    o = np.empty((r1 - r0, d), dtype=np.float64)
    lse = np.empty(r1 - r0, dtype=np.float64)
    for i0 in range(r0, r1, chunk):
        i1 = min(r1, i0 + chunk)
        ii = np.arange(i0, i1)
        jj = _candidate_keys(mode, i0, i1, sink, window)
        allowed = allowed_matrix(mode, ii, jj, L, sink, window, block, xa_mask)
        s = scale * (qh[i0:i1] @ kh[jj].T)
        o[i0 - r0:i1 - r0], lse[i0 - r0:i1 - r0] = _softmax_rows(s, allowed, vh[jj])
    return o, lse


def prefill(q, k, v, cu_seqlens, modes, *, scale, block, sink, window,
            xa_masks=None, heads=None):
    """Whole layer.  q [T,Hq,d], k/v [T,Hkv,d] float64; modes [num_seqs,Hkv].

    xa_masks: dict {(b, h): bool [nQB_b, nQB_b]} for every XA (sequence, q-head).
    Returns O [T,Hq,d] and LSE [Hq,T] (float64).  `heads` restricts the q-heads
    computed (others stay NaN).
    """
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    O = np.full((T, Hq, d), np.nan)
    LSE = np.full((Hq, T), np.nan)
    heads = range(Hq) if heads is None else heads
    for b in range(len(cu_seqlens) - 1):
        t0, t1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        if t1 == t0:
            continue
        for h in heads:
            g = h // G
            mode = int(modes[b, g])
            xm = xa_masks[(b, h)] if mode == MODE_XA else None
            o, lse = head_attention(q[t0:t1, h], k[t0:t1, g], v[t0:t1, g], mode, scale,
                                    sink, window, block, xm)
            O[t0:t1, h] = o
            LSE[h, t0:t1] = lse
    return O, LSE


def row_attention(q_i, k_seq, v_seq, i, mode, scale, *, sink=0, window=1, block=None,
                  xa_mask=None):
    """One query row: q_i [d], k_seq / v_seq [L, d] of the row's sequence and
    KV head (float64), i the local query index.  Returns (o_i [d], lse_i)."""
    L = k_seq.shape[0]
    jj = _candidate_keys(mode, i, i + 1, sink, window)
    allowed = allowed_matrix(mode, np.array([i]), jj, L, sink, window, block, xa_mask)
    s = scale * (k_seq[jj] @ q_i)[None, :]
    o, lse = _softmax_rows(s, allowed, v_seq[jj])
    return o[0], lse[0]


def prefill_rows(q, k, v, cu_seqlens, modes, rows, *, scale, block, sink, window,
                 xa_masks=None):
    """Selected query rows only: rows is a list of (b, h, i) with i local.

    Returns o [n,d] and lse [n]; the cost is O(L d) per row, so rows of the
    largest workloads can be checked one by one.
    """
    Hq = q.shape[1]
    G = Hq // k.shape[1]
    out_o = np.empty((len(rows), q.shape[2]))
    out_l = np.empty(len(rows))
    for n, (b, h, i) in enumerate(rows):
        t0, t1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        g = h // G
        mode = int(modes[b, g])
        xm = xa_masks[(b, h)] if mode == MODE_XA else None
        out_o[n], out_l[n] = row_attention(q[t0 + i, h], k[t0:t1, g], v[t0:t1, g], i, mode, scale,
                                           sink=sink, window=window, block=block, xa_mask=xm)
    return out_o, out_l
