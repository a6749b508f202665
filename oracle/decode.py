"""fp64 reference: one decode step of hybrid-head attention.

TEST INFRASTRUCTURE ONLY (see the package header).

What it computes: for every sequence, the attention of its newest token over
the keys that its head's mode keeps.  That is the last row of the prefill
definition (attention.py, Eqs. 1-3) for the sequence that already holds the
new token.  The pages fix that routing is decided once per request, at the
prefill stage, and reused for every generated token ([EN] 08 Commentary,
the authors' stated limits, item 3; [ZH] 10 Commentary, item 3), and that
SSA heads attend the attention sink plus a sliding window (glossaries of
[EN] and [ZH]).

Readings (each listed in the design notes):
  DX1 the key/value cache already holds the current token: a sequence of
      cached length L >= 1 decodes query index i = L - 1 over keys j <= i;
  DX2 XA heads attend every cached key in decode.  Antidiagonal block
      selection scores blocks of query rows against blocks of keys, which a
      single decoded query does not have, so the plainest reading is that an
      XA head behaves as FA once prefill is over;
  DX3 a sequence with no cached token has no query: o = 0 and lse = -inf.

Parity pins (tests/test_oracle_decode.py): torch scaled_dot_product_attention
in float64 on the explicitly gathered key set (FA, SSA, XA); the q = 0 closed
form o = mean of the kept v, lse = ln |A| with |A| counted in closed form; SSA
with window >= L equals FA; empty sequences.
"""

import numpy as np

from .attention import MODE_FA, MODE_SSA, MODE_XA, row_attention


def decode(q_new, k, v, cu_seqlens, modes, *, scale, sink, window):
    """q_new [num_seqs, Hq, d]; k, v [T, Hkv, d] (the cache, current token
    included); modes [num_seqs, Hkv].  All float64.  Returns
    O [num_seqs, Hq, d] and LSE [num_seqs, Hq]."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    nseq, Hq, d = q_new.shape
    G = Hq // k.shape[1]
    O = np.zeros((nseq, Hq, d), dtype=np.float64)
    LSE = np.full((nseq, Hq), -np.inf, dtype=np.float64)
    for b in range(nseq):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        if t1 == t0:
            continue                                   # DX3
        i = t1 - t0 - 1                                # DX1
        for h in range(Hq):
            g = h // G
            mode = int(modes[b, g])
            mode = MODE_FA if mode == MODE_XA else mode  # DX2
            O[b, h], LSE[b, h] = row_attention(q_new[b, h], k[t0:t1, g], v[t0:t1, g], i, mode,
                                               scale, sink=sink, window=window)
    return O, LSE


def kept_keys(mode, L, sink, window):
    """|A| of the decoded query of a sequence of cached length L (closed form)."""
    if L <= 0:
        return 0
    if mode == MODE_SSA:
        head = min(sink, L)
        return head + max(0, L - max(head, L - window))
    return L
