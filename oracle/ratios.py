"""fp64 reference: model and effective sparsity ratios.

TEST INFRASTRUCTURE ONLY (see the package header).

Definitions (Chinese paper-reading notes, section on the two sparsity ratios,
Eq. (4) and Eq. (5); the English notes, "02 . Background", describe the same
pair in words):
  Omega_MSR = (1/(L H)) sum_{l,h} [pi(l,h) = SA]    -- share of sparse heads
  Omega_ESR = (1/(L H)) sum_{l,h} rho(l,h)          -- mean pruning rate
with rho = 0 for a full-attention head, and, by the worked example on the
Chinese page, keeping 10 % of tokens gives rho = 0.9.  One layer here, so the
sums run over the KV heads of the layer (the router assigns modes per KV
head), per sequence, and the batch value is the mean over sequences.

Readings: rho of a (sequence, KV head) is one minus the attended (i, j) pairs
of its q-heads over their causal pairs G * L (L + 1) / 2, and the SA slot is
the mode that fills the "sparse" half of the {retrieval}-{sparse} mode-set
name (FA-SSA, FA-XA: SSA resp. XA; XA-SSA: SSA).  The pair-weighted
Omega_ESR of the batch, 1 - sum kept / sum causal, is reported as well.

Parity pins: the page's worked value (10 % kept -> 0.9), the 1/(L H) step of
Omega_MSR, and the SSA kept-pair closed form checked against brute force.
"""

import numpy as np

from .attention import MODE_FA, MODE_SSA, MODE_XA


def ssa_kept_pairs(L, sink, window):
    """sum_i |A(i)| for an SSA head, counted per query from the definition:
    A(i) = {j <= i : j < sink} union {j <= i : i - j < window}."""
    i = np.arange(L, dtype=np.int64)
    n_sink = np.minimum(i + 1, sink)
    lo = np.maximum(i - window + 1, 0)
    n_win_outside_sink = np.maximum(0, i - np.maximum(lo, sink) + 1)
    return int((n_sink + n_win_outside_sink).sum())


def sparsity_ratios(seqlens, modes, num_q_heads, *, sink, window, sparse_mode,
                    xa_pairs=None):
    """Returns dict(msr [nseq+1], esr [nseq+1], rho [nseq, Hkv], esr_pairs).

    xa_pairs[b, h]: attended pairs of XA q-head h of sequence b (required when
    any head is XA).  The last entry of msr / esr is the batch mean.
    """
    modes = np.asarray(modes)
    nseq, Hkv = modes.shape
    G = num_q_heads // Hkv
    rho = np.zeros((nseq, Hkv))
    msr = np.zeros(nseq + 1)
    esr = np.zeros(nseq + 1)
    kept_tot = 0
    causal_tot = 0
    for b in range(nseq):
        L = int(seqlens[b])
        causal = L * (L + 1) // 2
        for g in range(Hkv):
            m = int(modes[b, g])
            if m == MODE_FA:
                kept = G * causal
            elif m == MODE_SSA:
                kept = G * ssa_kept_pairs(L, sink, window)
            elif m == MODE_XA:
                kept = int(sum(int(xa_pairs[b, h]) for h in range(g * G, (g + 1) * G)))
            else:
                raise ValueError(m)
            kept_tot += kept
            causal_tot += G * causal
            rho[b, g] = 0.0 if causal == 0 else 1.0 - kept / (G * causal)
        msr[b] = float(np.mean(modes[b] == sparse_mode))
        esr[b] = float(np.mean(rho[b]))
    if nseq:
        msr[nseq] = float(np.mean(msr[:nseq]))
        esr[nseq] = float(np.mean(esr[:nseq]))
    esr_pairs = 0.0 if causal_tot == 0 else 1.0 - kept_tot / causal_tot
    return dict(msr=msr, esr=esr, rho=rho, esr_pairs=esr_pairs)
