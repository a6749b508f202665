"""Seeded synthetic generator for hybrid-head prefill inputs.

Stand-in for the long-context evaluation data the pages use (RULER, which is
not available here): Gaussian q, k, v with a shared "needle" direction planted
into 1 % of key positions, so that about half of all queries concentrate their
attention on a few keys, as retrieval-style prompts do.

Draw order from one numpy Generator(PCG64(seed)) is fixed:
  1. ragged lengths (if drawn), 2. per-sequence modes (if drawn),
  3. q, k, v (standard normal fp32, in token chunks), 4. the needle direction,
  5. needle positions per (sequence, KV head), sequence-major.
Everything is rounded to bfloat16 (round to nearest even) at the end.

Outputs are bf16 bit patterns (uint16); `bf16_bits_to_f64` widens them exactly.
"""

import numpy as np

from .configs import Config, MODE_FA, MODE_SSA, MODE_XA

_CHUNK_TOKENS = 8192


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)


def _normal_bf16(rng, tokens: int, heads: int, d: int) -> np.ndarray:
    out = np.empty((tokens, heads, d), dtype=np.uint16)
    for t0 in range(0, tokens, _CHUNK_TOKENS):
        t1 = min(tokens, t0 + _CHUNK_TOKENS)
        out[t0:t1] = f32_to_bf16_bits(rng.standard_normal((t1 - t0, heads, d), dtype=np.float32))
    return out


def _draw_modes(rng, cfg: Config, num_seqs: int) -> np.ndarray:
    hkv = cfg.num_kv_heads
    modes = np.full((num_seqs, hkv), MODE_SSA, dtype=np.uint8)
    for b in range(num_seqs):
        omega = cfg.omega_choices[int(rng.integers(0, len(cfg.omega_choices)))]
        n_sparse = int(np.floor(hkv * omega + 0.5))
        perm = rng.permutation(hkv)
        retrieval = sorted(int(x) for x in perm[: hkv - n_sparse])
        for idx, g in enumerate(retrieval):
            modes[b, g] = MODE_FA if idx % 2 == 0 else MODE_XA
    return modes


def make_inputs(cfg: Config, with_values: bool = True):
    """Build the seeded inputs of one workload.

    Returns a dict with q [T,Hq,d], k and v [T,Hkv,d] (uint16 bf16 bits),
    cu_seqlens int32 [num_seqs+1], seqlens, modes uint8 [num_seqs,Hkv] and cfg.
    With with_values=False only the lengths and modes are drawn.
    """
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    if cfg.seqlens is not None:
        seqlens = np.asarray(cfg.seqlens, dtype=np.int64)
    else:
        lo, hi = cfg.ragged_blocks
        seqlens = cfg.block * rng.integers(lo, hi + 1, size=cfg.ragged_count).astype(np.int64)
    num_seqs = len(seqlens)
    cu = np.zeros(num_seqs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    if cfg.modes is not None:
        m = np.asarray(cfg.modes, dtype=np.uint8)
        if m.shape[0] == 1 and num_seqs > 1:
            m = np.repeat(m, num_seqs, axis=0)
        modes = np.ascontiguousarray(m)
    else:
        modes = _draw_modes(rng, cfg, num_seqs)
    assert modes.shape == (num_seqs, cfg.num_kv_heads)
    out = dict(cfg=cfg, seqlens=seqlens, cu_seqlens=cu, modes=modes)
    if not with_values:
        return out

    T = int(cu[-1])
    d = cfg.head_dim
    q = _normal_bf16(rng, T, cfg.num_q_heads, d)
    kf = np.empty((T, cfg.num_kv_heads, d), dtype=np.float32)
    for t0 in range(0, T, _CHUNK_TOKENS):
        t1 = min(T, t0 + _CHUNK_TOKENS)
        kf[t0:t1] = rng.standard_normal((t1 - t0, cfg.num_kv_heads, d), dtype=np.float32)
    v = _normal_bf16(rng, T, cfg.num_kv_heads, d)

    u = rng.standard_normal(d)
    u *= np.sqrt(d) / np.linalg.norm(u)
    needle = (cfg.needle_gain * u).astype(np.float32)
    for b in range(num_seqs):
        L = int(seqlens[b])
        base = int(cu[b])
        n = int(np.floor(cfg.needle_fraction * L + 0.5))
        for g in range(cfg.num_kv_heads):
            if n == 0:
                continue
            if cfg.needle_layout == "uniform":
                pos = rng.choice(L, size=n, replace=False)
            elif cfg.needle_layout == "clustered":
                nblk_all = max(1, L // 128)
                nblk = min(nblk_all, max(1, (cfg.needle_blocks_per_64k * L) // 65536))
                blocks = rng.choice(nblk_all, size=nblk, replace=False)
                cand = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)
                cand = cand[cand < L]
                pos = rng.choice(cand, size=min(n, cand.size), replace=False)
            else:
                raise ValueError(cfg.needle_layout)
            kf[base + pos, g, :] += needle
    k = f32_to_bf16_bits(kf)
    del kf
    out.update(q=q, k=k, v=v)
    return out
