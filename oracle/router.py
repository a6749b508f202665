"""fp64 reference: the Attention Router's forward pass (inference).

TEST INFRASTRUCTURE ONLY (see the package header).

What the pages fix ([EN] 03 Method, Figure 3 (b)(c) and the paragraph on the
configuration drawn from Appendix C.1; [ZH] 04 Method; [HY] Method summary):
  * input: the key states x_K of the layer, one d'-vector per token and KV
    head, i.e. the same k tensor the attention reads;
  * pooling along the sequence over the first 100 and the last 100 tokens
    only, giving one task representation x'_K per KV head;
  * a Task MLP and a Router MLP, hidden size 4 d' by default ([EN] 06
    Analysis, Table 4 ablates 2 d', 4 d', 8 d');
  * the pooled representation feeds both MLPs; the Router MLP emits two
    logits per head, z in R^{H x 2};
  * at inference the decision is the arg max of z: r = 0 is FA (the
    retrieval mode), r = 1 is SA (the sparse mode) ([ZH] 04 Method).  The
    Gumbel noise and the straight-through estimator are training-only.
  * about 0.27 M parameters per layer at d' = 128.

Readings where the pages are open (each one listed in the design notes):
  R1 pooling is the mean over the boundary set {0..h-1} U {L-t..L-1} of a
     sequence of length L (h = t = 100), each token counted once; a sequence
     shorter than h + t therefore pools over all its tokens, and an empty one
     pools to the zero vector;
  R2 Task MLP: d' -> H_m -> d' (bias, ReLU between); Router MLP takes the
     concatenation [x'_K, Task MLP output] (2 d') -> H_m -> 2 (bias, ReLU
     between).  With d' = 128 and H_m = 4 d' this has 264,322 parameters,
     within 2 % of the pages' 0.27 M per layer; feeding the Router MLP the
     Task MLP output alone would give 198,786, 26 % short of it;
  R3 the MLP weights are shared by the KV heads of the layer (one router per
     layer, applied to each head's own pooled keys);
  R4 arg max with ties to index 0 (FA).

Parity: the pooling is pinned by closed forms (ramp and constant inputs, the
short-sequence union), the MLP by a hand-computed worked example under
tests/golden, the architecture reading by the pages' parameter count, and the
tie rule directly.  The trained weights are not available: the weights are
seeded random, so which head gets which mode is not a claim about the pages.
"""

import numpy as np

MODE_FA, MODE_SSA, MODE_XA = 0, 1, 2


def boundary_positions(L, head=100, tail=100):
    """Local token indices pooled for a sequence of length L (reading R1)."""
    L = int(L)
    idx = set(range(min(head, L))) | set(range(max(L - tail, 0), L))
    return np.array(sorted(idx), dtype=np.int64)


def boundary_pool(k_f64, cu_seqlens, head=100, tail=100):
    """x'_K[b, g, :] = mean of k over the boundary tokens of sequence b.

    k_f64: [T, Hkv, d] float64; cu_seqlens: [num_seqs + 1].
    Returns [num_seqs, Hkv, d] float64 (zeros for an empty sequence)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    nseq = len(cu) - 1
    _, hkv, d = k_f64.shape
    out = np.zeros((nseq, hkv, d), dtype=np.float64)
    for b in range(nseq):
        pos = boundary_positions(cu[b + 1] - cu[b], head, tail)
        if pos.size:
            out[b] = k_f64[cu[b] + pos].mean(axis=0)
    return out


def param_count(d, hidden):
    """Parameters of Task MLP (d -> hidden -> d) plus Router MLP
    (2d -> hidden -> 2), biases included (reading R2)."""
    task = d * hidden + hidden + hidden * d + d
    router = 2 * d * hidden + hidden + hidden * 2 + 2
    return task + router


def relu(x):
    return np.maximum(x, 0.0)


def router_logits(pooled, w):
    """z = RouterMLP([x', TaskMLP(x')]) for every (sequence, head) row.

    pooled: [..., d] float64.  w: dict of arrays w1 [d, H], b1 [H], w2 [H, d],
    b2 [d], w3 [2d, H], b3 [H], w4 [H, 2], b4 [2] (any float dtype; widened to
    float64).  Returns [..., 2] float64."""
    f = {n: np.asarray(a, dtype=np.float64) for n, a in w.items()}
    x = np.asarray(pooled, dtype=np.float64)
    z_task = relu(x @ f["w1"] + f["b1"]) @ f["w2"] + f["b2"]
    h = relu(np.concatenate([x, z_task], axis=-1) @ f["w3"] + f["b3"])
    return h @ f["w4"] + f["b4"]


def decide(logits, retrieval_mode, sparse_mode):
    """Hard routing: arg max over the two logits, ties to FA (reading R4);
    r = 0 maps to the retrieval mode and r = 1 to the sparse mode."""
    z = np.asarray(logits)
    r = (z[..., 1] > z[..., 0]).astype(np.int64)
    return np.where(r == 1, sparse_mode, retrieval_mode).astype(np.uint8)


def route(k_f64, cu_seqlens, w, *, retrieval_mode, sparse_mode, head=100, tail=100):
    """Modes [num_seqs, Hkv] (uint8) and logits [num_seqs, Hkv, 2]."""
    z = router_logits(boundary_pool(k_f64, cu_seqlens, head, tail), w)
    return decide(z, retrieval_mode, sparse_mode), z
