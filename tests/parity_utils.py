"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and compute the matching oracle values on the host."""

import numpy as np

from oracle import attention as OA
from oracle import xa as OX
from synth import bf16_bits_to_f64, MODE_XA

O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_REL = 1e-3


def run_gpu(inp, block_mass=True, stream=None):
    import torch
    from hybrid_sparse_full_amd.layer import HybridPrefill, bf16_tensor, desc_for
    cfg = inp["cfg"]
    dev = torch.device("cuda:0")
    desc = desc_for(cfg, inp["seqlens"])
    layer = HybridPrefill(desc, inp["cu_seqlens"], inp["modes"], device=dev, block_mass=block_mass)
    q = bf16_tensor(inp["q"], dev)
    k = bf16_tensor(inp["k"], dev)
    v = bf16_tensor(inp["v"], dev)
    layer(q, k, v, stream)
    torch.cuda.synchronize()
    out = dict(layer=layer, q=q, k=k, v=v,
               o=layer.o.float().cpu().numpy().astype(np.float64),
               lse=layer.lse.cpu().numpy().astype(np.float64))
    if layer.has_xa:
        out["mask"] = layer.mask.cpu().numpy().view(np.uint32)
        out["row_count"] = layer.row_count.cpu().numpy()
        out["xa_pairs"] = layer.xa_pairs.cpu().numpy().reshape(len(inp["seqlens"]), -1)
        if layer.block_mass is not None:
            out["block_mass"] = layer.block_mass.cpu().numpy()
    return out


def qb_prefix(seqlens, B):
    nqb = [-(-int(L) // B) for L in seqlens]
    return np.concatenate([[0], np.cumsum(nqb)]).astype(np.int64)


def gpu_mask_row(gout, inp, b, h, I):
    """Decoded GPU mask row (bool over J in [0, I])."""
    cfg = inp["cfg"]
    P = qb_prefix(inp["seqlens"], cfg.block)
    row = (P[b] + I) * cfg.num_q_heads + h
    words = gout["mask"][row]
    bits = np.unpackbits(words.view(np.uint8), bitorder="little")
    return bits[: I + 1].astype(bool)


def gpu_block_mass_row(gout, inp, b, h, I):
    cfg = inp["cfg"]
    P = qb_prefix(inp["seqlens"], cfg.block)
    row = (P[b] + I) * cfg.num_q_heads + h
    return gout["block_mass"][row][: I + 1].astype(np.float64)


def widen_head(inp, name, b, head):
    cu = inp["cu_seqlens"]
    return bf16_bits_to_f64(inp[name][cu[b]:cu[b + 1], head])


def oracle_xa(inp, pairs=None, rows=None):
    """Oracle XA masks and masses for every XA (b, h) (or the listed ones).

    rows: optional {(b, h): [I, ...]} restricting the block rows computed."""
    cfg = inp["cfg"]
    G = cfg.gqa
    res = {}
    for b in range(len(inp["seqlens"])):
        for h in range(cfg.num_q_heads):
            if inp["modes"][b, h // G] != MODE_XA:
                continue
            if pairs is not None and (b, h) not in pairs:
                continue
            if getattr(cfg, "xa_group", 0):
                # One mask per KV head: scored with the group-mean query.
                qh = OX.group_query([widen_head(inp, "q", b, hg)
                                     for hg in range((h // G) * G, (h // G + 1) * G)])
            else:
                qh = widen_head(inp, "q", b, h)
            kg = widen_head(inp, "k", b, h // G)
            r = None if rows is None else rows.get((b, h))
            res[(b, h)] = OX.head_mask(qh, kg, cfg.xa_stride, cfg.block, cfg.softmax_scale,
                                       cfg.tau_num, cfg.tau_den, rows=r,
                                       normalization="R1" if getattr(cfg, "xa_norm", 0) else "R2")
    return res


def check_masks(gout, inp, oxa, rows=None):
    """Bit-exact mask check outside boundary-tie rows.

    Returns dict(rows, ties_reported, mismatched, mismatched_ties, p_max_abs).
    Also re-runs the oracle's selector on the GPU's own fp32 masses: that must
    reproduce every GPU mask row exactly."""
    cfg = inp["cfg"]
    stats = dict(rows=0, ties_reported=0, order_ties=0, mismatched=0, mismatched_ties=0,
                 p_max_abs=0.0, tie_rows=[])
    for (b, h), (M, P) in oxa.items():
        nb = M.shape[0]
        Is = range(nb) if rows is None else rows[(b, h)]
        for I in Is:
            g = gpu_mask_row(gout, inp, b, h, I)
            o = M[I, : I + 1]
            stats["rows"] += 1
            if P is None:
                assert g.all(), (b, h, I)
                continue
            gp = gpu_block_mass_row(gout, inp, b, h, I)
            stats["p_max_abs"] = max(stats["p_max_abs"], float(np.abs(gp - P[I, : I + 1]).max()))
            rerun = OX.select_row(gp, I, cfg.tau_num, cfg.tau_den)
            assert np.array_equal(rerun, g), f"selector on GPU masses differs at {(b, h, I)}"
            t = OX.tie_info(P[I], I, cfg.tau_num, cfg.tau_den)
            tie = t["cum_tie"] or t["gap_tie"] or t["round_tie"]
            stats["ties_reported"] += int(t["cum_tie"])
            stats["order_ties"] += int(not t["cum_tie"] and (t["gap_tie"] or t["round_tie"]))
            if not np.array_equal(g, o):
                stats["mismatched"] += 1
                if tie:
                    stats["mismatched_ties"] += 1
                    stats["tie_rows"].append((b, h, I))
                else:
                    diff = np.nonzero(g != o)[0]
                    raise AssertionError(
                        f"mask mismatch outside ties at {(b, h, I)}: blocks {diff.tolist()[:16]} "
                        f"(gpu has {g[diff].astype(int).tolist()[:16]}); oracle P "
                        f"{P[I, diff][:16].tolist()}, gpu P {gp[diff][:16].tolist()}; cut {t}; "
                        f"gpu blocks {int(g.sum())}, oracle blocks {int(o.sum())}")
    return stats


def check_close(o_gpu, o_ref, lse_gpu, lse_ref, what=""):
    err = np.abs(o_gpu - o_ref)
    max_abs, mean_abs = float(err.max()), float(err.mean())
    lse_err = np.abs(lse_gpu - lse_ref) / np.maximum(1.0, np.abs(lse_ref))
    assert max_abs <= O_MAX_ABS, f"{what}: O max-abs {max_abs}"
    assert mean_abs <= O_MEAN_ABS, f"{what}: O mean-abs {mean_abs}"
    assert float(lse_err.max()) <= LSE_REL, f"{what}: LSE rel {float(lse_err.max())}"
    return dict(max_abs=max_abs, mean_abs=mean_abs, lse_rel=float(lse_err.max()))


def oracle_full(inp, masks, heads=None):
    cfg = inp["cfg"]
    q, k, v = (bf16_bits_to_f64(inp[n]) for n in ("q", "k", "v"))
    xm = {key: val[0] for key, val in masks.items()}
    return OA.prefill(q, k, v, inp["cu_seqlens"], inp["modes"], scale=cfg.softmax_scale,
                      block=cfg.block, sink=cfg.ssa_sink, window=cfg.ssa_window, xa_masks=xm,
                      heads=heads)


def oracle_rows(inp, rows, masks):
    """rows: list of (b, h, i); masks {(b, h): (M, P)} covering XA rows."""
    cfg = inp["cfg"]
    G = cfg.gqa
    o = np.empty((len(rows), cfg.head_dim))
    l = np.empty(len(rows))
    by_bg = {}
    for n, (b, h, i) in enumerate(rows):
        by_bg.setdefault((b, h // G), []).append(n)
    for (b, g), idx in by_bg.items():
        kg = widen_head(inp, "k", b, g)
        vg = widen_head(inp, "v", b, g)
        cu = inp["cu_seqlens"]
        for n in idx:
            _, h, i = rows[n]
            mode = int(inp["modes"][b, g])
            xm = masks[(b, h)][0] if mode == MODE_XA else None
            qi = bf16_bits_to_f64(inp["q"][cu[b] + i, h])
            o[n], l[n] = OA.row_attention(qi, kg, vg, i, mode, cfg.softmax_scale,
                                          sink=cfg.ssa_sink, window=cfg.ssa_window,
                                          block=cfg.block, xa_mask=xm)
    return o, l


def sample_rows(inp, n, seed):
    """n random (b, h, i) rows, always including first / last tokens."""
    rng = np.random.default_rng(seed)
    cfg = inp["cfg"]
    seqlens = inp["seqlens"]
    rows = []
    nonempty = [b for b in range(len(seqlens)) if seqlens[b] > 0]
    for b in nonempty:
        for h in (0, cfg.num_q_heads - 1):
            rows += [(b, h, 0), (b, h, int(seqlens[b]) - 1)]
    while len(rows) < n:
        b = int(rng.choice(nonempty))
        rows.append((b, int(rng.integers(cfg.num_q_heads)), int(rng.integers(seqlens[b]))))
    return rows


def gather_rows(gout, inp, rows):
    cu = inp["cu_seqlens"]
    o = np.stack([gout["o"][cu[b] + i, h] for (b, h, i) in rows])
    l = np.array([gout["lse"][h, cu[b] + i] for (b, h, i) in rows])
    return o, l


def host_threads():
    """Host threads for the oracle: the cores this process may use, at most 16."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_whole_heads(inp, heads, masks, rows_per_task=1024):
    """Every row of the listed (b, h): {(b, h): (o [L, d], lse [L])}.

    The oracle's head_attention runs on row ranges of each head in a thread
    pool (numpy releases the GIL in its products and elementwise loops), with
    single-threaded BLAS in each task."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    cfg = inp["cfg"]
    G = cfg.gqa
    cu = inp["cu_seqlens"]
    tasks = []
    widened = {}
    for (b, h) in heads:
        g = h // G
        L = int(cu[b + 1] - cu[b])
        key = (b, h)
        widened[key] = (widen_head(inp, "q", b, h), widen_head(inp, "k", b, g), widen_head(inp, "v", b, g),
                        int(inp["modes"][b, g]))
        for r0 in range(0, L, rows_per_task):
            tasks.append((key, r0, min(L, r0 + rows_per_task)))

    def run(t):
        key, r0, r1 = t
        qh, kh, vh, mode = widened[key]
        xm = masks[key][0] if mode == MODE_XA else None
        return OA.head_attention(qh, kh, vh, mode, cfg.softmax_scale, sink=cfg.ssa_sink,
                                 window=cfg.ssa_window, block=cfg.block, xa_mask=xm, chunk=256,
                                 row_range=(r0, r1))

    # Costly tasks (late rows see more keys) first.
    order = sorted(range(len(tasks)), key=lambda i: -tasks[i][2])
    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(max_workers=host_threads()) as ex:
            res = dict(zip(order, ex.map(run, [tasks[i] for i in order])))
    out = {}
    for (b, h) in heads:
        L = int(cu[b + 1] - cu[b])
        d = inp["q"].shape[2]
        out[(b, h)] = (np.empty((L, d)), np.empty(L))
    for i, (key, r0, r1) in enumerate(tasks):
        out[key][0][r0:r1], out[key][1][r0:r1] = res[i]
    return out


def oracle_xa_parallel(inp, pairs, rows=None):
    """oracle_xa for the listed (b, h), one head per thread."""
    from concurrent.futures import ThreadPoolExecutor
    pairs = sorted(pairs)
    with ThreadPoolExecutor(max_workers=min(host_threads(), max(1, len(pairs)))) as ex:
        parts = list(ex.map(lambda p: oracle_xa(inp, pairs={p}, rows=rows), pairs))
    res = {}
    for p in parts:
        res.update(p)
    return res
