"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small workloads are compared element by element; the 256K, ragged and variant
workloads here on sampled rows that the oracle computes one by one (the 16K and
64K workloads are compared whole in test_gpu_fullsize.py).  Tolerances: O max-abs
2e-2 and mean-abs 2e-3, LSE 1e-3 * max(1, |lse|); XA masks bit-exact outside
boundary-tie rows, and the oracle's selector re-run on the GPU's own fp32 block
masses reproduces every GPU mask row exactly.
"""

import numpy as np
import pytest

from synth import get_config, make_inputs, MODE_FA, MODE_SSA, MODE_XA
from synth.generate import bf16_bits_to_f32, f32_to_bf16_bits
import parity_utils as PU

pytestmark = pytest.mark.gpu


def _small(name="small", **kw):
    base = dict(name=name, seed=11, num_q_heads=8, num_kv_heads=2, head_dim=128, block=128,
                ssa_sink=64, ssa_window=200, xa_stride=8)
    base.update(kw)
    return get_config("tiny-1k").with_(**base)


def _full_check(inp, tag):
    gout = PU.run_gpu(inp)
    masks = PU.oracle_xa(inp)
    stats = {}
    if masks:
        stats = PU.check_masks(gout, inp, masks)
    O, LSE = PU.oracle_full(inp, masks)
    T = int(inp["cu_seqlens"][-1])
    res = PU.check_close(gout["o"].reshape(T, -1), O.reshape(T, -1), gout["lse"], LSE, tag)
    print(tag, res, {k: v for k, v in stats.items() if k != "tie_rows"}, flush=True)
    return gout, masks, stats


def test_tiny_1k_full():
    inp = make_inputs(get_config("tiny-1k"))
    _full_check(inp, "tiny-1k")


@pytest.mark.parametrize("D,B", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_small_mixed_ragged(D, B):
    # Ragged lengths (with an empty and a 1-token sequence), every mode, GQA 4.
    modes = ((MODE_FA, MODE_SSA), (MODE_XA, MODE_SSA), (MODE_SSA, MODE_XA), (MODE_XA, MODE_FA),
             (MODE_XA, MODE_XA))
    cfg = _small(seqlens=(3 * B, 200, 1, 0, 5 * B), modes=modes, head_dim=D, block=B,
                 xa_stride=B // 16)
    inp = make_inputs(cfg)
    _full_check(inp, f"small-mixed D{D} B{B}")


def test_xa_masks_many_rows():
    cfg = _small(name="xa-many", seqlens=(2048, 1024), num_q_heads=8, num_kv_heads=2,
                 modes=((MODE_XA, MODE_XA), (MODE_XA, MODE_SSA)), needle_layout="clustered",
                 needle_blocks_per_64k=512)
    inp = make_inputs(cfg)
    gout, masks, stats = _full_check(inp, "xa-many")
    assert stats["rows"] > 100
    # Attended pairs per XA q-head agree with the oracle's masks.
    for (b, h), (M, P) in masks.items():
        L = int(inp["seqlens"][b])
        from oracle import xa as OX
        if not stats["tie_rows"]:
            assert gout["xa_pairs"][b, h] == OX.kept_pairs(M, L, cfg.block)


@pytest.mark.parametrize("Hq,Hkv,D,B", [(4, 4, 128, 128), (4, 2, 128, 128), (6, 2, 128, 128),
                                         (6, 2, 64, 64), (3, 3, 64, 128)])
def test_gqa_group_sizes(Hq, Hkv, D, B):
    # Group sizes 1, 2 and 3: one head per attention workgroup when G is odd,
    # and 1 or 2 heads per XA scoring item.
    modes = ((MODE_XA,) + (MODE_SSA, MODE_FA) * Hkv)[:Hkv]
    modes2 = ((MODE_FA,) + (MODE_XA, MODE_SSA) * Hkv)[:Hkv]
    cfg = _small(name=f"gqa-{Hq}-{Hkv}", seqlens=(12 * B, 7 * B + 5, 5 * B), num_q_heads=Hq,
                 num_kv_heads=Hkv, head_dim=D, block=B, xa_stride=B // 16,
                 modes=(modes, modes2, modes))
    inp = make_inputs(cfg)
    _full_check(inp, f"gqa Hq{Hq} Hkv{Hkv} D{D} B{B}")


@pytest.mark.parametrize("B,S", [(64, 16), (128, 32)])
def test_xa_four_reduced_rows_per_block(B, S):
    # B / S = 4: each block of a 32-key MFMA tile lies in one half-wave.
    cfg = _small(name=f"xa-r4-B{B}", seqlens=(32 * B, 13 * B), num_q_heads=8, num_kv_heads=2,
                 block=B, xa_stride=S, modes=((MODE_XA, MODE_SSA), (MODE_XA, MODE_XA)),
                 needle_layout="clustered", needle_blocks_per_64k=512)
    inp = make_inputs(cfg)
    gout, masks, stats = _full_check(inp, f"xa-r4 B{B} S{S}")
    assert stats["rows"] > 40


@pytest.mark.parametrize("sink,window", [(0, 1), (0, 128), (5000, 64), (1, 2)])
def test_ssa_degenerate_sink_window(sink, window):
    # Window 1 keeps only the diagonal key; a sink longer than the sequence
    # makes SSA equal to FA; sink 0 leaves the window alone.
    cfg = _small(name=f"ssa-s{sink}-w{window}", seqlens=(1000, 128, 3),
                 modes=((MODE_SSA, MODE_FA),), ssa_sink=sink, ssa_window=window)
    inp = make_inputs(cfg)
    _full_check(inp, f"ssa sink {sink} window {window}")


def test_xa_tiny_tau():
    # tau = 1/1000: the top-mass prefix is a single block, so each mask row
    # is that block plus the forced sink and diagonal blocks.
    cfg = _small(name="xa-tiny-tau", seqlens=(2048, 640), modes=((MODE_XA, MODE_XA),),
                 tau_num=1, tau_den=1000, needle_layout="clustered", needle_blocks_per_64k=512)
    inp = make_inputs(cfg)
    gout, masks, stats = _full_check(inp, "xa tau 1/1000")
    nrows = int(PU.qb_prefix(inp["seqlens"], cfg.block)[-1]) * cfg.num_q_heads
    rc = gout["row_count"][:nrows]
    assert (rc >= 1).all() and (rc <= 3).all()


def _all_fa(inp):
    inp1 = dict(inp)
    inp1["modes"] = np.zeros_like(inp["modes"])
    return PU.run_gpu(inp1)


def test_ssa_window_ge_len_is_bitwise_fa():
    # SSA with window >= L keeps every causal key: the same heads of an all-FA
    # run must be bit-identical.
    cfg = _small(seqlens=(700, 256), modes=((MODE_SSA, MODE_FA),), ssa_window=10 ** 6)
    inp = make_inputs(cfg)
    g = PU.run_gpu(inp)
    f = _all_fa(inp)
    assert np.array_equal(g["o"], f["o"]) and np.array_equal(g["lse"], f["lse"])


def test_tau_one_is_bitwise_fa():
    cfg = _small(seqlens=(1024,), modes=((MODE_XA, MODE_FA),), tau_num=1, tau_den=1)
    inp = make_inputs(cfg)
    g = PU.run_gpu(inp)
    G = cfg.gqa
    assert g["row_count"].reshape(-1, cfg.num_q_heads)[:8, :G].sum() == 8 * 9 // 2 * G
    f = _all_fa(inp)
    assert np.array_equal(g["o"], f["o"]) and np.array_equal(g["lse"], f["lse"])


def test_eq3_concatenation_bitwise():
    # Each head of the hybrid layer equals the same head of a single-mode run.
    cfg = _small(seqlens=(512, 384), modes=((MODE_FA, MODE_SSA), (MODE_XA, MODE_FA)))
    inp = make_inputs(cfg)
    hyb = PU.run_gpu(inp)
    G = cfg.gqa
    for mode in (MODE_FA, MODE_SSA, MODE_XA):
        inp1 = dict(inp)
        inp1["modes"] = np.full_like(inp["modes"], mode)
        one = PU.run_gpu(inp1)
        cu = inp["cu_seqlens"]
        for b in range(2):
            for h in range(cfg.num_q_heads):
                if inp["modes"][b, h // G] == mode:
                    sl = slice(cu[b], cu[b + 1])
                    assert np.array_equal(hyb["o"][sl, h], one["o"][sl, h])
                    assert np.array_equal(hyb["lse"][h, sl], one["lse"][h, sl])


def test_xa_tile_list_is_the_union():
    # Each XA row lists the union of its two heads' mask rows once, in J
    # order, each entry flagged with the heads that attend it.
    from hybrid_sparse_full_amd import ea as E
    cfg = _small(name="xa-order", seqlens=(3072, 1280), modes=((MODE_XA, MODE_SSA), (MODE_XA, MODE_XA)),
                 needle_layout="clustered", needle_blocks_per_64k=512)
    inp = make_inputs(cfg)
    gout = PU.run_gpu(inp)
    layer = gout["layer"]
    ws = layer.ws_prefill.cpu().numpy()
    off = lambda name: E.ea_workspace_offset(layer.desc, E.EA_OP_PREFILL, name)
    def arr(name, dt):
        a = ws[off(name):]
        n = len(a) // np.dtype(dt).itemsize
        return a[: n * np.dtype(dt).itemsize].view(dt)
    tiles, row_off, row_cost = arr("tiles", np.uint32), arr("row_off", np.int64), arr("row_cost", np.int32)
    G, hpw, Hkv = cfg.gqa, 2, cfg.num_kv_heads
    P = PU.qb_prefix(inp["seqlens"], cfg.block)
    checked = 0
    for b in range(len(inp["seqlens"])):
        for I in range(int(P[b + 1] - P[b])):
            qbg = int(P[b]) + I
            for g in range(Hkv):
                if inp["modes"][b, g] != MODE_XA:
                    continue
                for kg in range(G // hpw):
                    row = (qbg * Hkv + g) * (G // hpw) + kg
                    ent = tiles[row_off[row]: row_off[row] + row_cost[row]]
                    J = (ent & 0x1FFFFFFF).astype(np.int64)
                    h0 = (ent >> 29) & 1
                    h1 = (ent >> 30) & 1
                    m0 = PU.gpu_mask_row(gout, inp, b, g * G + kg * hpw, I)
                    m1 = PU.gpu_mask_row(gout, inp, b, g * G + kg * hpw + 1, I)
                    assert J.tolist() == np.nonzero(m0 | m1)[0].tolist()
                    assert np.array_equal(h0.astype(bool), m0[J]) and np.array_equal(h1.astype(bool), m1[J])
                    checked += 1
    assert checked > 50


def test_plan_then_run_equals_prefill():
    # ea_hybrid_attn_plan + ea_hybrid_attn_run is the one-call prefill, and a
    # second run over the same plan gives the same result.
    import torch
    cfg = _small(seqlens=(768, 300), modes=((MODE_XA, MODE_SSA), (MODE_FA, MODE_XA)))
    inp = make_inputs(cfg)
    ref = PU.run_gpu(inp)
    layer = ref["layer"]
    layer.o.zero_()
    layer.lse.zero_()
    layer.plan(ref["k"], ref["v"])
    for _ in range(2):
        layer.run(ref["q"])
        torch.cuda.synchronize()
        o = layer.o.float().cpu().numpy().astype(np.float64)
        lse = layer.lse.cpu().numpy().astype(np.float64)
        assert np.array_equal(o, ref["o"]) and np.array_equal(lse, ref["lse"])


def test_rising_and_overflowing_scores():
    # Keys scaled up along each sequence make the row max rise tile after
    # tile, and a few spike keys aligned with a third of the queries score so
    # far above the running max that exp2 overflows against it: both cases
    # must leave the fast softmax path for the exact one and still match.
    cfg = _small(name="spikes", seqlens=(1024, 640), modes=((MODE_FA, MODE_SSA), (MODE_XA, MODE_FA)))
    inp = make_inputs(cfg)
    rng = np.random.Generator(np.random.PCG64(5))
    d = cfg.head_dim
    cu = inp["cu_seqlens"]
    T = int(cu[-1])
    kf = bf16_bits_to_f32(inp["k"]).copy()
    qf = bf16_bits_to_f32(inp["q"]).copy()
    for b in range(len(inp["seqlens"])):
        L = int(cu[b + 1] - cu[b])
        kf[cu[b]:cu[b + 1]] *= (1.0 + 3.0 * np.arange(L, dtype=np.float32) / L)[:, None, None]
    u = rng.standard_normal(d).astype(np.float32)
    u *= np.float32(np.sqrt(d) / np.linalg.norm(u))
    kf[rng.choice(T, size=12, replace=False)] = 12.0 * u
    qf[0::3] += 2.0 * u
    inp["k"] = f32_to_bf16_bits(kf)
    inp["q"] = f32_to_bf16_bits(qf)
    _full_check(inp, "rising and overflowing scores")


def test_deterministic():
    cfg = _small(seqlens=(640, 300), modes=((MODE_XA, MODE_SSA), (MODE_FA, MODE_XA)))
    inp = make_inputs(cfg)
    a = PU.run_gpu(inp)
    b = PU.run_gpu(inp)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])
    # Mask rows past the last existing q-block (the row count is a bound) are
    # written empty.
    nrows = int(PU.qb_prefix(inp["seqlens"], cfg.block)[-1]) * cfg.num_q_heads
    assert len(a["mask"]) > nrows
    assert (a["mask"][nrows:] == 0).all() and (a["row_count"][nrows:] == 0).all()
    assert np.array_equal(a["mask"], b["mask"])
    assert np.array_equal(a["xa_pairs"], b["xa_pairs"])


def _sampled_check(name, n_rows, seed, xa_rows_per_head=6):
    inp = make_inputs(get_config(name))
    cfg = inp["cfg"]
    gout = PU.run_gpu(inp)
    rows = PU.sample_rows(inp, n_rows, seed)
    # XA: score and select only the block rows that the sampled queries touch,
    # plus a few random block rows per XA head for the mask check.
    rng = np.random.default_rng(seed + 1)
    need = {}
    G = cfg.gqa
    for (b, h, i) in rows:
        if inp["modes"][b, h // G] == MODE_XA:
            need.setdefault((b, h), set()).add(i // cfg.block)
    for b in range(len(inp["seqlens"])):
        nb = int(inp["seqlens"][b]) // cfg.block
        for h in range(cfg.num_q_heads):
            if inp["modes"][b, h // G] == MODE_XA and nb:
                need.setdefault((b, h), set()).update(
                    int(x) for x in rng.integers(0, nb, size=xa_rows_per_head))
                need[(b, h)].add(nb - 1)
    need = {key: sorted(v) for key, v in need.items()}
    masks = PU.oracle_xa(inp, pairs=set(need), rows=need) if need else {}
    stats = PU.check_masks(gout, inp, masks, rows=need) if masks else {}
    # For rows whose mask is a boundary tie that the GPU resolved differently,
    # the GPU mask row (already checked to be the selector's answer on the GPU
    # masses) defines the key set.
    for (b, h, I) in stats.get("tie_rows", []):
        masks[(b, h)][0][I, : I + 1] = PU.gpu_mask_row(gout, inp, b, h, I)
    o_ref, l_ref = PU.oracle_rows(inp, rows, masks)
    o_gpu, l_gpu = PU.gather_rows(gout, inp, rows)
    res = PU.check_close(o_gpu, o_ref, l_gpu, l_ref, name)
    print(name, res, {k: v for k, v in stats.items() if k != "tie_rows"}, flush=True)


def test_xassa_64k_b64s16_sampled():
    _sampled_check("xassa-64k-b64s16", 192, 6)


def test_qwen8b_faxa_256k_sampled():
    _sampled_check("qwen8b-faxa-256k", 96, 4, xa_rows_per_head=2)


def test_qwen8b_xassa_256k_sampled():
    _sampled_check("qwen8b-xassa-256k", 96, 4, xa_rows_per_head=3)


@pytest.mark.parametrize("hq,hkv", [(8, 2), (8, 4), (4, 4)])
def test_xa_one_mask_per_kv_head(hq, hkv):
    # xa_group = 1: every q-head of an XA KV head gets the mask selected from
    # the group-mean antidiagonal scores; masks equal across the group, parity
    # with the oracle's group reading, and the attention on those masks.
    cfg = _small(name="xa-group", seqlens=(1024, 640, 384), num_q_heads=hq, num_kv_heads=hkv,
                 modes=tuple(tuple(MODE_XA if (b + g) % 3 != 2 else MODE_SSA for g in range(hkv))
                             for b in range(3)),
                 xa_group=1, needle_layout="clustered", needle_blocks_per_64k=512)
    inp = make_inputs(cfg)
    gout, masks, stats = _full_check(inp, f"xa group Hq {hq} Hkv {hkv}")
    G = cfg.gqa
    m = gout["mask"].reshape(-1, hq, gout["mask"].shape[-1])
    nrows = int(PU.qb_prefix(inp["seqlens"], cfg.block)[-1])
    for g in range(hkv):
        for u in range(1, G):
            assert np.array_equal(m[:nrows, g * G], m[:nrows, g * G + u])


def test_xassa_64k_group_sampled():
    _sampled_check("xassa-64k-group", 192, 7)


@pytest.mark.parametrize("group", [0, 1])
def test_xa_block_sum_masses(group):
    # xa_norm = 1 (reading R1): P is the softmax over each block row of the
    # raw block sums of s^; per q-head and per KV head.
    cfg = _small(name="xa-r1", seqlens=(1024, 640), num_q_heads=8, num_kv_heads=2,
                 modes=((MODE_XA, MODE_SSA), (MODE_XA, MODE_XA)), xa_norm=1, xa_group=group,
                 needle_layout="clustered", needle_blocks_per_64k=512)
    inp = make_inputs(cfg)
    gout, masks, stats = _full_check(inp, f"xa R1 group {group}")
    assert stats["rows"] > 0


def test_xassa_64k_r1_sampled():
    _sampled_check("xassa-64k-r1", 192, 5)


def test_every_output_row_written():
    # O and LSE are filled with NaN before the call: afterwards every token of
    # every q-head must hold a finite value (each query attends at least its
    # own key), in every mode, on a ragged batch with empty and one-token
    # sequences; the same for the serial dispatch and the decode step.
    import torch
    from hybrid_sparse_full_amd import ea as E
    from hybrid_sparse_full_amd.layer import HybridPrefill, HybridDecode, bf16_tensor, desc_for
    dev = torch.device("cuda:0")
    modes = ((MODE_FA, MODE_SSA), (MODE_XA, MODE_SSA), (MODE_SSA, MODE_XA), (MODE_XA, MODE_FA), (MODE_XA, MODE_XA))
    cfg = _small(name="written", seqlens=(3 * 128 + 5, 1, 0, 700, 5 * 128), modes=modes)
    inp = make_inputs(cfg)
    desc = desc_for(cfg, inp["seqlens"])
    layer = HybridPrefill(desc, inp["cu_seqlens"], inp["modes"], device=dev)
    q, k, v = (bf16_tensor(inp[n], dev) for n in ("q", "k", "v"))
    layer.o.fill_(float("nan"))
    layer.lse.fill_(float("nan"))
    layer(q, k, v)
    torch.cuda.synchronize()
    assert torch.isfinite(layer.o.float()).all() and torch.isfinite(layer.lse).all()
    # Serial dispatch (FA / SSA heads only).
    cfg2 = _small(name="written-serial", seqlens=(3 * 128 + 5, 1, 0, 700), modes=((MODE_SSA, MODE_FA),))
    inp2 = make_inputs(cfg2)
    d2 = desc_for(cfg2, inp2["seqlens"])
    q2, k2, v2 = (bf16_tensor(inp2[n], dev) for n in ("q", "k", "v"))
    o2 = torch.full((d2.total_tokens, d2.num_q_heads, d2.head_dim), float("nan"), dtype=torch.bfloat16, device=dev)
    l2 = torch.full((d2.num_q_heads, d2.total_tokens), float("nan"), dtype=torch.float32, device=dev)
    ws2 = torch.empty(E.ea_workspace_bytes(d2, E.EA_OP_PREFILL_SERIAL), dtype=torch.uint8, device=dev)
    cu2 = torch.from_numpy(inp2["cu_seqlens"].astype(np.int32)).to(dev)
    E.ea_hybrid_attn_prefill_serial(d2, q2, k2, v2, cu2, np.ascontiguousarray(inp2["modes"][0]), o2, l2, ws2)
    torch.cuda.synchronize()
    assert torch.isfinite(o2.float()).all() and torch.isfinite(l2).all()
    # Decode: empty sequences give o = 0 and lse = -inf; nothing stays NaN.
    dec = HybridDecode(desc, inp["cu_seqlens"], inp["modes"], device=dev)
    dec.o.fill_(float("nan"))
    dec.lse.fill_(float("nan"))
    qn = bf16_tensor(inp["q"][np.maximum(inp["cu_seqlens"][1:] - 1, 0)], dev)
    dec(qn, k, v)
    torch.cuda.synchronize()
    assert not torch.isnan(dec.o.float()).any() and not torch.isnan(dec.lse).any()
