"""Full-size GPU parity: whole tensors and whole heads at the workloads' real
shapes, in the launch configuration the benchmark times, against the fp64
oracle (computed on the host cores, head rows split over threads).

* 16K FA-SSA layer: every row of every q-head.
* 64K FA-SSA layer (the benchmark's workload): every row of every q-head.
* 64K XA-SSA layer: every mask row of all 8 XA q-heads (bit-exact outside
  boundary ties, ties counted and printed), then every row of every q-head.
* 256K FA-XA and XA-SSA: every mask row of two XA q-heads each, and every
  row of two q-heads of different modes.
* The ragged 8-sequence batch: every mask row, then every row of every q-head.
* The XA variants at 64K (Table 8's block 64 / stride 16, one mask per KV
  head, block-sum masses): every mask row of all 8 XA q-heads (of one q-head
  per XA KV head for the block-sum masses), then every row of one XA and one
  SSA q-head.
* One sequence of 2^20 tokens (q holds 2^32 elements): query rows at both
  ends and the middle of an FA and an SSA q-head, and a decode step over the
  same cache against the prefill's last row.
* Configurations no other test runs: B / S = 8 and 32 at both block sizes,
  a selector row of more than 2,048 blocks, and GQA groups of 8 q-heads.

Tolerances as everywhere: O max-abs 2e-2 and mean-abs 2e-3 (here also per
whole head), LSE 1e-3 * max(1, |lse|).
"""

import functools
import time

import numpy as np
import pytest

from synth import get_config, make_inputs, MODE_FA, MODE_SSA, MODE_XA
import parity_utils as PU

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def _inputs(name):
    return make_inputs(get_config(name))


@functools.lru_cache(maxsize=1)
def _gpu(name):
    return PU.run_gpu(_inputs(name), block_mass=True)


@functools.lru_cache(maxsize=1)
def _oracle_masks(name):
    inp = _inputs(name)
    cfg = inp["cfg"]
    G = cfg.gqa
    pairs = {(b, h) for b in range(len(inp["seqlens"])) for h in range(cfg.num_q_heads)
             if inp["modes"][b, h // G] == MODE_XA}
    return PU.oracle_xa_parallel(inp, pairs)


def _check_heads(name, heads, masks):
    """Every row of the listed (b, h) against the oracle; per head and overall."""
    inp = _inputs(name)
    gout = _gpu(name)
    cu = inp["cu_seqlens"]
    t0 = time.time()
    ref = PU.oracle_whole_heads(inp, heads, masks)
    worst = dict(max_abs=0.0, mean_abs=0.0, lse_rel=0.0)
    for (b, h), (o_ref, l_ref) in ref.items():
        sl = slice(int(cu[b]), int(cu[b + 1]))
        r = PU.check_close(gout["o"][sl, h], o_ref, gout["lse"][h, sl], l_ref, f"{name} b{b} h{h}")
        worst = {k: max(worst[k], r[k]) for k in worst}
    print(name, f"{len(heads)} whole heads", worst, f"oracle {time.time() - t0:.1f} s", flush=True)


def test_16k_whole_layer():
    inp = _inputs("llama8b-fassa-16k")
    _check_heads("llama8b-fassa-16k", [(0, h) for h in range(inp["cfg"].num_q_heads)], {})


@pytest.mark.parametrize("part", range(4))
def test_64k_fassa_whole_layer(part):
    _check_heads("llama8b-fassa-64k", [(0, h) for h in range(8 * part, 8 * part + 8)], {})


def test_xassa_64k_every_mask_row():
    name = "xassa-64k"
    inp = _inputs(name)
    gout = _gpu(name)
    t0 = time.time()
    masks = _oracle_masks(name)
    stats = PU.check_masks(gout, inp, masks)
    assert len(masks) == 8 and stats["rows"] == 8 * 512
    print(name, "every mask row of 8 XA q-heads:", {k: v for k, v in stats.items() if k != "tie_rows"},
          "tie rows", stats["tie_rows"], f"oracle {time.time() - t0:.1f} s", flush=True)


@pytest.mark.parametrize("part", range(4))
def test_xassa_64k_whole_layer(part):
    name = "xassa-64k"
    inp = _inputs(name)
    gout = _gpu(name)
    masks = dict(_oracle_masks(name))
    # A boundary-tie row that the GPU resolved the other way (already checked
    # to be the selector's answer on the GPU's own masses) attends the GPU's
    # blocks.
    stats = PU.check_masks(gout, inp, masks)
    for (b, h, I) in stats["tie_rows"]:
        M = masks[(b, h)][0].copy()
        M[I, : I + 1] = PU.gpu_mask_row(gout, inp, b, h, I)
        masks[(b, h)] = (M, masks[(b, h)][1])
    _check_heads(name, [(0, h) for h in range(8 * part, 8 * part + 8)], masks)


@pytest.mark.parametrize("name,heads,whole", [("qwen8b-faxa-256k", (4, 31), (0, 4)),
                                              ("qwen8b-xassa-256k", (0, 19), (0, 4))])
def test_256k_masks_and_whole_heads(name, heads, whole):
    # Every mask row of two XA q-heads, then every row of two q-heads of
    # different modes (FA-XA: FA head 0 and XA head 4; XA-SSA: XA head 0 and
    # SSA head 4).
    inp = _inputs(name)
    gout = _gpu(name)
    G = inp["cfg"].gqa
    assert all(inp["modes"][0, h // G] == MODE_XA for h in heads)
    t0 = time.time()
    masks = PU.oracle_xa_parallel(inp, {(0, h) for h in heads})
    stats = PU.check_masks(gout, inp, masks)
    assert stats["rows"] == 2 * 2048
    print(name, f"every mask row of q-heads {heads}:", {k: v for k, v in stats.items() if k != "tie_rows"},
          f"oracle {time.time() - t0:.1f} s", flush=True)
    wmasks = {k: v for k, v in masks.items() if k in {(0, h) for h in whole}}
    for (b, h, I) in stats["tie_rows"]:
        if (b, h) in wmasks:
            M = wmasks[(b, h)][0].copy()
            M[I, : I + 1] = PU.gpu_mask_row(gout, inp, b, h, I)
            wmasks[(b, h)] = (M, wmasks[(b, h)][1])
    modes = {int(inp["modes"][0, h // G]) for h in whole}
    assert len(modes) == 2 and MODE_XA in modes
    _check_heads(name, [(0, h) for h in whole], wmasks)


@pytest.mark.parametrize("name", ["xassa-64k-b64s16", "xassa-64k-group", "xassa-64k-r1"])
def test_xa_variants_every_mask_row_and_whole_heads(name):
    inp = _inputs(name)
    gout = _gpu(name)
    cfg = inp["cfg"]
    t0 = time.time()
    # The block-sum oracle sums every antidiagonal entry in explicit loops
    # (~12 s per head at 64K): one q-head per XA KV head there, all 8 else.
    heads = {(0, 0), (0, 16)} if cfg.xa_norm else None
    masks = dict(PU.oracle_xa_parallel(inp, heads) if heads else _oracle_masks(name))
    stats = PU.check_masks(gout, inp, masks)
    n = len(heads) if heads else 8
    assert len(masks) == n and stats["rows"] == n * (int(inp["seqlens"][0]) // cfg.block)
    print(name, f"every mask row of {n} XA q-heads:", {k: v for k, v in stats.items() if k != "tie_rows"},
          f"oracle {time.time() - t0:.1f} s", flush=True)
    for (b, h, I) in stats["tie_rows"]:
        M = masks[(b, h)][0].copy()
        M[I, : I + 1] = PU.gpu_mask_row(gout, inp, b, h, I)
        masks[(b, h)] = (M, masks[(b, h)][1])
    G = cfg.gqa
    assert inp["modes"][0, 0] == MODE_XA and inp["modes"][0, 4 // G] == MODE_SSA
    _check_heads(name, [(0, 0), (0, 4)], {k: v for k, v in masks.items() if k == (0, 0)})


def test_ragged_8x_whole_tensor():
    # Every row of every q-head of the 8 ragged sequences (per-sequence modes);
    # the XA masks first, every row, bit-exact outside boundary ties.
    name = "ragged-8x"
    inp = _inputs(name)
    gout = _gpu(name)
    cfg = inp["cfg"]
    masks = dict(_oracle_masks(name))
    stats = PU.check_masks(gout, inp, masks)
    nqb = PU.qb_prefix(inp["seqlens"], cfg.block)
    assert stats["rows"] == sum(int(nqb[b + 1] - nqb[b]) for (b, h) in masks)
    print(name, "every mask row of", len(masks), "XA (sequence, q-head) pairs:",
          {k: v for k, v in stats.items() if k != "tie_rows"}, flush=True)
    for (b, h, I) in stats["tie_rows"]:
        M = masks[(b, h)][0].copy()
        M[I, : I + 1] = PU.gpu_mask_row(gout, inp, b, h, I)
        masks[(b, h)] = (M, masks[(b, h)][1])
    for b in range(len(inp["seqlens"])):
        if int(inp["seqlens"][b]) == 0:
            continue
        _check_heads(name, [(b, h) for h in range(cfg.num_q_heads)],
                     {k: v for k, v in masks.items() if k[0] == b})


def _small(name, **kw):
    base = dict(name=name, seed=17, num_q_heads=8, num_kv_heads=2, head_dim=128, block=128,
                ssa_sink=64, ssa_window=300, xa_stride=8)
    base.update(kw)
    return get_config("tiny-1k").with_(**base)


def _full(inp, tag):
    gout = PU.run_gpu(inp)
    masks = PU.oracle_xa(inp)
    stats = PU.check_masks(gout, inp, masks) if masks else {}
    for (b, h, I) in stats.get("tie_rows", []):
        masks[(b, h)][0][I, : I + 1] = PU.gpu_mask_row(gout, inp, b, h, I)
    O, LSE = PU.oracle_full(inp, masks)
    T = int(inp["cu_seqlens"][-1])
    res = PU.check_close(gout["o"].reshape(T, -1), O.reshape(T, -1), gout["lse"], LSE, tag)
    print(tag, res, {k: v for k, v in stats.items() if k != "tie_rows"}, flush=True)
    return stats


@pytest.mark.parametrize("B,S", [(128, 16), (128, 4), (64, 8), (64, 2)])
def test_xa_8_and_32_reduced_rows_per_block(B, S):
    # B / S = 8 and 32: the scoring epilogue's register groups and the
    # selector's per-row log-sum-exp over R partial sums.
    cfg = _small(f"xa-r{B // S}-B{B}", block=B, xa_stride=S, seqlens=(2048, 13 * B, 1000),
                 modes=((MODE_XA, MODE_XA), (MODE_XA, MODE_SSA), (MODE_FA, MODE_XA)),
                 needle_layout="clustered", needle_blocks_per_64k=512)
    stats = _full(make_inputs(cfg), f"xa B{B} S{S}")
    assert stats["rows"] > 100


def test_selector_row_over_2048_blocks():
    # 131,200 tokens at block 64: rows I >= 2048 have more than 2,048 blocks,
    # so the selector's threshold search runs from LDS, not registers.
    L = 131200
    cfg = _small("xa-2050-blocks", num_q_heads=4, num_kv_heads=1, block=64, xa_stride=8, seqlens=(L,),
                 modes=((MODE_XA,),), needle_layout="clustered")
    inp = make_inputs(cfg)
    gout = PU.run_gpu(inp)
    nb = L // 64
    rows = {(0, h): [nb - 1, nb - 2, 2048, 2047, 1500, 3] for h in range(4)}
    masks = PU.oracle_xa_parallel(inp, set(rows), rows=rows)
    stats = PU.check_masks(gout, inp, masks, rows=rows)
    for (b, h, I) in stats["tie_rows"]:
        masks[(b, h)][0][I, : I + 1] = PU.gpu_mask_row(gout, inp, b, h, I)
    qrows = [(0, h, I * 64 + off) for h in range(4) for I in rows[(0, h)] for off in (0, 31, 63)]
    o_ref, l_ref = PU.oracle_rows(inp, qrows, masks)
    o_gpu, l_gpu = PU.gather_rows(gout, inp, qrows)
    res = PU.check_close(o_gpu, o_ref, l_gpu, l_ref, "selector rows over 2048 blocks")
    print("selector rows over 2048 blocks", res, {k: v for k, v in stats.items() if k != "tie_rows"},
          flush=True)


@pytest.mark.parametrize("D,B", [(128, 128), (64, 64)])
def test_gqa_group_of_8(D, B):
    # 64 q-heads over 8 KV heads: four attention workgroups and two XA
    # scoring items per KV head.
    modes = ((MODE_XA, MODE_SSA, MODE_FA, MODE_XA, MODE_SSA, MODE_SSA, MODE_FA, MODE_XA),
             (MODE_SSA, MODE_XA, MODE_XA, MODE_FA, MODE_SSA, MODE_XA, MODE_SSA, MODE_FA))
    cfg = _small(f"gqa8-D{D}-B{B}", num_q_heads=64, num_kv_heads=8, head_dim=D, block=B,
                 xa_stride=B // 16, seqlens=(8 * B, 5 * B + 11), modes=modes)
    _full(make_inputs(cfg), f"GQA 8 D{D} B{B}")


def test_one_million_token_sequence():
    # 2^20 tokens, Llama-3.1-8B shape, KV head 0 FA and the rest SSA: q and o
    # hold 2^32 elements, so element offsets past 2^32 are exercised.  Inputs
    # are drawn on the device; the oracle gets the rows it needs.
    import torch
    from hybrid_sparse_full_amd.layer import HybridDecode, HybridPrefill, make_desc
    from oracle import attention as OA
    dev = torch.device("cuda:0")
    L, Hq, Hkv, D, B, sink, window = 1 << 20, 32, 8, 128, 128, 128, 2048
    gen = torch.Generator(device=dev)
    gen.manual_seed(20)
    q = torch.randn((L, Hq, D), generator=gen, device=dev, dtype=torch.bfloat16)
    k = torch.randn((L, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
    v = torch.randn((L, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16)
    modes = np.array([[MODE_FA] + [MODE_SSA] * (Hkv - 1)], dtype=np.uint8)
    cu = np.array([0, L], dtype=np.int32)
    desc = make_desc(num_seqs=1, total_tokens=L, max_seqlen=L, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                     block=B, ssa_sink=sink, ssa_window=window)
    layer = HybridPrefill(desc, cu, modes, device=dev)
    t0 = time.time()
    layer(q, k, v)
    torch.cuda.synchronize()
    print(f"1M prefill {time.time() - t0:.2f} s", flush=True)
    scale = desc.softmax_scale
    qi = [0, 1, B - 1, B, L // 2 + 77, L - B - 1, L - B, L - 1]
    for h in (1, 9):  # FA (KV head 0) and SSA (KV head 2)
        g = h // (Hq // Hkv)
        kg = k[:, g].double().cpu().numpy()
        vg = v[:, g].double().cpu().numpy()
        o_ref, l_ref = [], []
        for i in qi:
            o_i, l_i = OA.row_attention(q[i, h].double().cpu().numpy(), kg, vg, i, int(modes[0, g]), scale,
                                        sink=sink, window=window, block=B)
            o_ref.append(o_i)
            l_ref.append(l_i)
        idx = torch.tensor(qi, device=dev)
        o = layer.o[idx, h].double().cpu().numpy()
        lse = layer.lse[h, idx].double().cpu().numpy()
        print(f"1M head {h}", PU.check_close(o, np.array(o_ref), lse, np.array(l_ref), f"1M head {h}"), flush=True)
        del kg, vg
    # One decode step whose query is the last token's: the prefill's last row.
    o_last = layer.o[L - 1].clone()
    lse_last = layer.lse[:, L - 1].clone()
    del layer
    dec = HybridDecode(desc, cu, modes, device=dev)
    dec(q[L - 1:L].contiguous(), k, v)
    torch.cuda.synchronize()
    d_o = dec.o[0].double().cpu().numpy()
    d_l = dec.lse[0].double().cpu().numpy()
    print("1M decode vs prefill last row",
          PU.check_close(d_o, o_last.double().cpu().numpy(), d_l, lse_last.double().cpu().numpy(), "1M decode"),
          flush=True)
