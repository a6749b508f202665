"""GPU parity of one decode step (ea_hybrid_attn_decode) against the fp64 oracle.

The cache is a packed varlen k / v whose last token of each sequence is the
one being decoded; its query is that token's row of the seeded q.  Tolerances
are the prefill's: O max-abs 2e-2 and mean-abs 2e-3, LSE 1e-3 * max(1, |lse|).
"""

import numpy as np
import pytest
import torch

from hybrid_sparse_full_amd.layer import HybridDecode, HybridPrefill, bf16_tensor, desc_for
from oracle import decode as OD
from synth import get_config, make_inputs, bf16_bits_to_f64, MODE_FA, MODE_SSA, MODE_XA
import parity_utils as PU

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _last_queries(inp):
    cu = inp["cu_seqlens"]
    idx = np.maximum(cu[1:] - 1, 0)
    q = inp["q"][idx].copy()
    q[cu[1:] == cu[:-1]] = 0
    return q


def _run(inp):
    cfg = inp["cfg"]
    d = desc_for(cfg, inp["seqlens"])
    dec = HybridDecode(d, inp["cu_seqlens"], inp["modes"], device=DEV)
    qn = _last_queries(inp)
    q = bf16_tensor(qn, DEV)
    k, v = bf16_tensor(inp["k"], DEV), bf16_tensor(inp["v"], DEV)
    dec(q, k, v)
    torch.cuda.synchronize()
    return qn, dec.o.float().cpu().numpy().astype(np.float64), dec.lse.cpu().numpy().astype(np.float64)


def _check(inp, tag):
    cfg = inp["cfg"]
    qn, o, lse = _run(inp)
    O, LSE = OD.decode(bf16_bits_to_f64(qn), bf16_bits_to_f64(inp["k"]), bf16_bits_to_f64(inp["v"]),
                       inp["cu_seqlens"], inp["modes"], scale=cfg.softmax_scale, sink=cfg.ssa_sink,
                       window=cfg.ssa_window)
    empty = np.asarray(inp["seqlens"]) == 0
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    keep = ~empty
    res = PU.check_close(o[keep].reshape(-1), O[keep].reshape(-1), lse[keep], LSE[keep], tag)
    print(tag, res, flush=True)
    return o, lse


def _small(**kw):
    base = dict(name="decode-small", seed=31, num_q_heads=8, num_kv_heads=2, head_dim=128, block=128,
                ssa_sink=64, ssa_window=300, xa_stride=8,
                seqlens=(1, 2, 63, 64, 65, 1000, 0, 1024, 1025, 2049, 3000))
    base.update(kw)
    n = len(base["seqlens"])
    hkv = base["num_kv_heads"]
    rng = np.random.default_rng(base["seed"])
    modes = rng.integers(0, 3, size=(n, hkv)).astype(np.uint8)
    base.setdefault("modes", tuple(tuple(int(x) for x in r) for r in modes))
    return get_config("tiny-1k").with_(**base)


@pytest.mark.parametrize("hq,hkv,D", [(8, 2, 128), (8, 2, 64), (8, 8, 128), (16, 8, 64), (32, 4, 128),
                                      (12, 1, 128), (64, 4, 64)])
def test_decode_small_batches(hq, hkv, D):
    inp = make_inputs(_small(num_q_heads=hq, num_kv_heads=hkv, head_dim=D))
    _check(inp, f"decode Hq {hq} Hkv {hkv} d {D}")


@pytest.mark.parametrize("sink,window", [(0, 1), (5, 7), (3000, 10), (64, 10 ** 6), (128, 2048)])
def test_decode_ssa_windows(sink, window):
    inp = make_inputs(_small(ssa_sink=sink, ssa_window=window,
                             modes=tuple((MODE_SSA, MODE_FA) for _ in range(11))))
    _check(inp, f"decode SSA sink {sink} window {window}")


def test_decode_matches_last_prefill_row():
    # Same kernels' inputs: the decode of each sequence's last token must agree
    # with that token's row of the prefill (FA and SSA heads; an XA head in
    # prefill attends its selected blocks, in decode every key).
    cfg = _small(seqlens=(777, 1024, 1), modes=((MODE_FA, MODE_SSA),) * 3)
    inp = make_inputs(cfg)
    qn, o, lse = _run(inp)
    g = PU.run_gpu(inp)
    last = inp["cu_seqlens"][1:] - 1
    po = g["o"][last]
    plse = g["lse"][:, last].T
    assert np.abs(po - o).max() <= 2e-2
    assert np.all(np.abs(plse - lse) <= 1e-3 * np.maximum(1, np.abs(lse)))


def test_decode_64k_batch():
    # Llama-3.1-8B-shaped decode over 64K-token caches, batch 4, FA-SSA.
    cfg = get_config("llama8b-fassa-64k")
    inp = make_inputs(cfg.with_(name="decode-64k-b4", seqlens=(65536, 65536, 40000, 30001),
                                modes=((0, 1, 1, 0, 1, 1, 0, 1), (1, 1, 1, 1, 1, 1, 1, 1),
                                       (0, 0, 0, 0, 0, 0, 0, 0), (2, 1, 1, 2, 1, 1, 2, 1))))
    _check(inp, "decode 64K batch 4")


@pytest.mark.parametrize("modes", ["random", "all-ssa", "all-fa"])
def test_decode_split_from_kept_keys(modes):
    # 64 KV heads over ~17K tokens: the descriptor allows splits of 256 to
    # 1,024 keys, and the device picks one from the kept keys of the step
    # (random modes land in between, all-SSA at the floor, all-FA at the top).
    seqlens = (9000, 5000, 0, 20, 3000, 1)
    kw = dict(num_q_heads=64, num_kv_heads=64, head_dim=128, seqlens=seqlens, seed=77)
    if modes == "all-ssa":
        kw["modes"] = tuple((MODE_SSA,) * 64 for _ in seqlens)
    elif modes == "all-fa":
        kw["modes"] = tuple((MODE_FA,) * 64 for _ in seqlens)
    inp = make_inputs(_small(**kw))
    _check(inp, f"decode split from kept keys, {modes}")


def test_decode_plan_scans_several_chunks():
    # 200 ragged sequences x 8 KV heads = 1,600 (sequence, KV head) units, so
    # the plan's scan of per-unit split counts crosses a 1,024-unit chunk; the
    # ~100K cached tokens make the device choose the split.
    rng = np.random.default_rng(5)
    seqlens = tuple(int(x) for x in rng.integers(0, 1000, size=200))
    modes = tuple(tuple(int(m) for m in r) for r in rng.integers(0, 3, size=(200, 8)))
    cfg = _small(name="decode-many", num_q_heads=32, num_kv_heads=8, head_dim=128, seqlens=seqlens,
                 modes=modes, ssa_sink=16, ssa_window=200, seed=9)
    assert sum(seqlens) * 8 > 256 * 2048
    _check(make_inputs(cfg), "decode 200 sequences")


@pytest.mark.parametrize("nseq", [8, 9])
def test_decode_plan_at_the_unit_limit(nseq):
    # 8 KV heads of one q-head group each: 8 sequences are 64 (sequence, KV
    # head) units, where every decode wave plans the step itself; 9 are 72,
    # where the plan kernel does.  ~6K tokens per sequence make the device
    # choose the split either way.
    rng = np.random.default_rng(40 + nseq)
    seqlens = tuple(int(x) for x in rng.integers(4000, 8000, size=nseq))
    modes = tuple(tuple(int(m) for m in r) for r in rng.integers(0, 3, size=(nseq, 8)))
    cfg = _small(name=f"decode-units-{nseq * 8}", num_q_heads=32, num_kv_heads=8, head_dim=128,
                 seqlens=seqlens, modes=modes, ssa_sink=100, ssa_window=1500, seed=11)
    assert sum(seqlens) * 8 > 2 * 64 * 2048
    _check(make_inputs(cfg), f"decode {nseq * 8} units")
