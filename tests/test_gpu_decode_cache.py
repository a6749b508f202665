"""Decode over the segmented cache (SSA heads keep only sink + window keys)
through the C ABI.

* After ea_decode_cache_fill, every kept key sits in the row its layout
  defines (FA / XA: row j; SSA: j < sink in row j, else sink + (j - sink) mod
  window), bit for bit.
* ea_hybrid_attn_decode_cached equals ea_hybrid_attn_decode over the packed
  cache bit for bit (same split plan and key order).
* Tokens appended one by one wrap the SSA rings many times; every step
  matches the fp64 decode oracle over the packed cache of that length.
"""

import numpy as np
import pytest
import torch

from hybrid_sparse_full_amd import ea as E
from hybrid_sparse_full_amd.layer import HybridDecode, SegmentedDecodeCache, bf16_tensor, desc_for
from oracle import decode as OD
from synth import get_config, make_inputs, bf16_bits_to_f64, MODE_FA, MODE_SSA, MODE_XA
import parity_utils as PU

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _cfg(seqlens, hq=8, hkv=2, D=128, sink=64, window=300, seed=31, modes=None):
    rng = np.random.default_rng(seed)
    if modes is None:
        modes = tuple(tuple(int(x) for x in r) for r in rng.integers(0, 3, size=(len(seqlens), hkv)))
    return get_config("tiny-1k").with_(name="decode-cache", seed=seed, num_q_heads=hq, num_kv_heads=hkv,
                                       head_dim=D, block=128, ssa_sink=sink, ssa_window=window,
                                       seqlens=tuple(seqlens), modes=modes)


def _kept(mode, L, sink, window):
    if mode != MODE_SSA:
        return list(range(L))
    head = min(sink, L)
    return list(range(head)) + list(range(max(head, L - window), L))


def _slot(mode, j, sink, window):
    return j if (mode != MODE_SSA or j < sink) else sink + (j - sink) % window


def _last_q(inp):
    cu = inp["cu_seqlens"]
    q = inp["q"][np.maximum(cu[1:] - 1, 0)].copy()
    q[cu[1:] == cu[:-1]] = 0
    return q


def _cached_and_packed(inp):
    cfg = inp["cfg"]
    desc = desc_for(cfg, inp["seqlens"])
    cu = torch.from_numpy(inp["cu_seqlens"].astype(np.int32)).to(DEV)
    k, v = bf16_tensor(inp["k"], DEV), bf16_tensor(inp["v"], DEV)
    cache = SegmentedDecodeCache(desc, inp["modes"], np.asarray(inp["seqlens"], dtype=np.int32), device=DEV)
    cache.fill(desc, k, v, cu)
    qn = _last_q(inp)
    q = bf16_tensor(qn, DEV)
    n, Hq, D = desc.num_seqs, desc.num_q_heads, desc.head_dim
    o = torch.full((n, Hq, D), 5.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((n, Hq), 5.0, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(1, E.ea_workspace_bytes(desc, E.EA_OP_DECODE)), dtype=torch.uint8, device=DEV)
    cache.decode(desc, q, cu, o, lse, ws)
    packed = HybridDecode(desc, inp["cu_seqlens"], inp["modes"], device=DEV)
    packed(q, k, v)
    torch.cuda.synchronize()
    return cache, qn, (o, lse), (packed.o, packed.lse)


@pytest.mark.parametrize("sink,window", [(64, 300), (3, 7), (0, 1), (500, 64), (64, 10 ** 6)])
def test_fill_puts_every_kept_key_in_its_row(sink, window):
    seqlens = (1, 2, 63, 1000, 0, 1025, 3000)
    inp = make_inputs(_cfg(seqlens, sink=sink, window=window))
    cache, _, _, _ = _cached_and_packed(inp)
    kc = cache.k.view(torch.int16).cpu().numpy()
    vc = cache.v.view(torch.int16).cpu().numpy()
    seg = cache.seg_host
    cu = inp["cu_seqlens"]
    Hkv = inp["cfg"].num_kv_heads
    checked = 0
    for b, L in enumerate(seqlens):
        for g in range(Hkv):
            mode = int(inp["modes"][b, g])
            u = b * Hkv + g
            rows = int(seg[u + 1] - seg[u])
            expect = L if mode != MODE_SSA else min(L, sink + window)
            assert rows == expect, (b, g, rows, expect)
            for j in _kept(mode, L, sink, window):
                r = int(seg[u]) + _slot(mode, j, sink, window)
                assert np.array_equal(kc[r], inp["k"][cu[b] + j, g].view(np.int16)), (b, g, j)
                assert np.array_equal(vc[r], inp["v"][cu[b] + j, g].view(np.int16)), (b, g, j)
                checked += 1
    assert checked > 1000


@pytest.mark.parametrize("hq,hkv,D,sink,window", [(8, 2, 128, 64, 300), (32, 8, 128, 128, 2048),
                                                  (8, 8, 64, 5, 7), (12, 1, 128, 3000, 10),
                                                  (64, 4, 64, 0, 1)])
def test_cached_decode_bitwise_equals_packed(hq, hkv, D, sink, window):
    seqlens = (1, 2, 63, 64, 65, 1000, 0, 1024, 1025, 2049, 3000)
    inp = make_inputs(_cfg(seqlens, hq=hq, hkv=hkv, D=D, sink=sink, window=window))
    _, _, (o, lse), (po, plse) = _cached_and_packed(inp)
    assert torch.equal(o.view(torch.int16), po.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), plse.view(torch.int32))


def test_rings_wrap_over_appended_tokens():
    # Start from cached prefixes, then append 40 tokens one at a time; with
    # sink 3 and window 7 every SSA ring wraps several times.  Each step is
    # compared with the oracle over the packed prefix of that length and with
    # the packed decode bit for bit.
    L0, steps, sink, window = (40, 3, 0, 100, 7), 40, 3, 7
    full = tuple(l + steps for l in L0)
    modes = ((MODE_SSA, MODE_FA), (MODE_SSA, MODE_SSA), (MODE_XA, MODE_SSA), (MODE_FA, MODE_SSA),
             (MODE_SSA, MODE_XA))
    inp = make_inputs(_cfg(full, hq=4, hkv=2, sink=sink, window=window, modes=modes, seed=8))
    cfg = inp["cfg"]
    cuf = inp["cu_seqlens"]
    n = len(full)

    def prefix(lens):
        idx = np.concatenate([np.arange(cuf[b], cuf[b] + lens[b]) for b in range(n)]).astype(np.int64)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        return idx, cu

    idx0, cu0 = prefix(L0)
    d0 = desc_for(cfg, np.asarray(L0))
    cache = SegmentedDecodeCache(d0, inp["modes"], np.asarray(full, dtype=np.int32), device=DEV)
    cache.fill(d0, bf16_tensor(inp["k"][idx0], DEV), bf16_tensor(inp["v"][idx0], DEV),
               torch.from_numpy(cu0).to(DEV))
    assert cache.rows < sum(full) * cfg.num_kv_heads
    for s in range(1, steps + 1):
        lens = np.asarray([l + s for l in L0])
        idx, cu = prefix(lens)
        d = desc_for(cfg, lens)
        cu_dev = torch.from_numpy(cu).to(DEV)
        newest = cuf[:-1] + lens - 1
        cache.append(d, bf16_tensor(inp["k"][newest], DEV), bf16_tensor(inp["v"][newest], DEV), cu_dev)
        qn = inp["q"][newest]
        q = bf16_tensor(qn, DEV)
        o = torch.empty((n, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((n, cfg.num_q_heads), dtype=torch.float32, device=DEV)
        ws = torch.empty(E.ea_workspace_bytes(d, E.EA_OP_DECODE), dtype=torch.uint8, device=DEV)
        cache.decode(d, q, cu_dev, o, lse, ws)
        kp, vp = inp["k"][idx], inp["v"][idx]
        packed = HybridDecode(d, cu, inp["modes"], device=DEV)
        packed(q, bf16_tensor(kp, DEV), bf16_tensor(vp, DEV))
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), packed.o.view(torch.int16)), s
        assert torch.equal(lse.view(torch.int32), packed.lse.view(torch.int32)), s
        O, LSE = OD.decode(bf16_bits_to_f64(qn), bf16_bits_to_f64(kp), bf16_bits_to_f64(vp), cu, inp["modes"],
                           scale=cfg.softmax_scale, sink=sink, window=window)
        res = PU.check_close(o.float().cpu().numpy().reshape(-1), O.reshape(-1),
                             lse.cpu().numpy().astype(np.float64), LSE, f"append step {s}")
    print("ring wrap, last step", res, flush=True)


def test_cached_64k_batch():
    # Llama-3.1-8B-shaped caches of 64K tokens, FA-SSA: the SSA heads keep
    # 128 + 2048 rows each instead of 65,536.
    cfg = get_config("llama8b-fassa-64k")
    row = (0, 1, 1, 0, 1, 1, 0, 1)
    inp = make_inputs(cfg.with_(name="decode-cache-64k", seqlens=(65536, 65536, 40000),
                                modes=(row, (1,) * 8, (2, 1, 1, 2, 1, 1, 2, 1))))
    cache, qn, (o, lse), (po, plse) = _cached_and_packed(inp)
    assert torch.equal(o.view(torch.int16), po.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), plse.view(torch.int32))
    ring = 128 + 2048
    assert cache.rows == 3 * 65536 + 5 * ring + 8 * ring + 3 * 40000 + 5 * ring
    O, LSE = OD.decode(bf16_bits_to_f64(qn), bf16_bits_to_f64(inp["k"]), bf16_bits_to_f64(inp["v"]),
                       inp["cu_seqlens"], inp["modes"], scale=cfg.softmax_scale, sink=cfg.ssa_sink,
                       window=cfg.ssa_window)
    res = PU.check_close(o.float().cpu().numpy().reshape(-1), O.reshape(-1),
                         lse.cpu().numpy().astype(np.float64), LSE, "cached decode 64K")
    print("cached decode 64K", res, flush=True)
