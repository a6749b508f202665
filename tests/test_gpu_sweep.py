"""Seeded sweep over combinations of the layer's parameters.

Each case draws head dim, block, reduced rows per block (B / S), KV heads and
GQA group size, one XA mask per q-head or per KV head, the XA normalisation,
tau, SSA sink and window (including 0 / 1 and longer than the sequences),
needle layout, ragged lengths around block edges (empty and one-token
sequences included) and random modes per (sequence, KV head).  Prefill with
XA selection must match the oracle (masks bit-exact outside boundary ties,
O and LSE within the tolerances), a decode step over the same cache must
match the decode oracle, and the segmented cache filled from it must decode
bit for bit the same.  Small enough that the oracle runs whole tensors.
"""

import numpy as np
import pytest
import torch

from hybrid_sparse_full_amd import ea as E
from hybrid_sparse_full_amd.layer import HybridDecode, SegmentedDecodeCache, bf16_tensor, desc_for
from oracle import decode as OD
from synth import get_config, make_inputs, bf16_bits_to_f64
import parity_utils as PU

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CASES = 64


def _draw(seed):
    rng = np.random.default_rng(9000 + seed)
    D = int(rng.choice([64, 128]))
    B = int(rng.choice([64, 128]))
    S = B // int(rng.choice([4, 8, 16, 32]))
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2])) if G == 8 else int(rng.choice([1, 2, 4]))
    xa_group = int(G <= 4 and rng.random() < 0.3)
    xa_norm = int(rng.random() < 0.25)
    tau = [(1, 2), (9, 10), (99, 100), (1, 1)][int(rng.integers(4))]
    sink = int(rng.choice([0, 1, 17, 64, 300]))
    window = int(rng.choice([1, 5, 100, 257, 5000]))
    nseq = int(rng.integers(1, 5))
    pool = [0, 1, B - 1, B, B + 1, 3 * B + 5, 8 * B, int(rng.integers(2, 3000))]
    seqlens = tuple(int(pool[int(i)]) for i in rng.integers(0, len(pool), size=nseq))
    if sum(seqlens) == 0:
        seqlens = seqlens[:-1] + (2 * B,)
    modes = tuple(tuple(int(m) for m in r) for r in rng.integers(0, 3, size=(nseq, hkv)))
    layout = "clustered" if rng.random() < 0.5 else "uniform"
    cfg = get_config("tiny-1k").with_(
        name=f"sweep-{seed}", seed=seed + 500, num_q_heads=hkv * G, num_kv_heads=hkv, head_dim=D, block=B,
        ssa_sink=sink, ssa_window=window, xa_stride=S, tau_num=tau[0], tau_den=tau[1], xa_group=xa_group,
        xa_norm=xa_norm, seqlens=seqlens, modes=modes, needle_layout=layout, needle_blocks_per_64k=2048)
    return cfg


@pytest.mark.parametrize("seed", range(CASES))
def test_parameter_sweep(seed):
    cfg = _draw(seed)
    inp = make_inputs(cfg)
    tag = (f"sweep {seed}: d {cfg.head_dim} B {cfg.block} S {cfg.xa_stride} Hq/Hkv {cfg.num_q_heads}/"
           f"{cfg.num_kv_heads} group {cfg.xa_group} norm {cfg.xa_norm} tau {cfg.tau_num}/{cfg.tau_den} "
           f"sink {cfg.ssa_sink} window {cfg.ssa_window} lens {cfg.seqlens}")
    print(tag, flush=True)
    d = desc_for(cfg, inp["seqlens"])
    assert E.ea_workspace_bytes(d, E.EA_OP_PREFILL) > 0, tag
    gout = PU.run_gpu(inp)
    masks = PU.oracle_xa(inp)
    stats = PU.check_masks(gout, inp, masks) if masks else {}
    for (b, h, I) in stats.get("tie_rows", []):
        masks[(b, h)][0][I, : I + 1] = PU.gpu_mask_row(gout, inp, b, h, I)
    O, LSE = PU.oracle_full(inp, masks)
    T = int(inp["cu_seqlens"][-1])
    res = PU.check_close(gout["o"].reshape(T, -1), O.reshape(T, -1), gout["lse"], LSE, tag)
    print("  prefill", res, {k: v for k, v in stats.items() if k != "tie_rows"}, flush=True)

    # Decode: the newest token of every sequence over the same cache.
    cu = inp["cu_seqlens"]
    qn = inp["q"][np.maximum(cu[1:] - 1, 0)].copy()
    qn[cu[1:] == cu[:-1]] = 0
    dec = HybridDecode(d, cu, inp["modes"], device=DEV)
    dec(bf16_tensor(qn, DEV), bf16_tensor(inp["k"], DEV), bf16_tensor(inp["v"], DEV))
    torch.cuda.synchronize()
    Od, Ld = OD.decode(bf16_bits_to_f64(qn), bf16_bits_to_f64(inp["k"]), bf16_bits_to_f64(inp["v"]), cu,
                       inp["modes"], scale=cfg.softmax_scale, sink=cfg.ssa_sink, window=cfg.ssa_window)
    o = dec.o.float().cpu().numpy().astype(np.float64)
    lse = dec.lse.cpu().numpy().astype(np.float64)
    keep = np.asarray(inp["seqlens"]) > 0
    assert np.all(o[~keep] == 0) and np.all(np.isneginf(lse[~keep])), tag
    print("  decode", PU.check_close(o[keep].reshape(-1), Od[keep].reshape(-1), lse[keep], Ld[keep], tag),
          flush=True)

    # The segmented cache (SSA heads keep sink + window keys), filled from the
    # same keys, decodes bit for bit like the packed cache.
    cache = SegmentedDecodeCache(d, inp["modes"], np.asarray(inp["seqlens"], dtype=np.int32), device=DEV)
    cu_dev = torch.from_numpy(np.ascontiguousarray(cu, dtype=np.int32)).to(DEV)
    cache.fill(d, bf16_tensor(inp["k"], DEV), bf16_tensor(inp["v"], DEV), cu_dev)
    oc, lc = torch.empty_like(dec.o), torch.empty_like(dec.lse)
    cache.decode(d, bf16_tensor(qn, DEV), cu_dev, oc, lc, torch.empty_like(dec.ws))
    torch.cuda.synchronize()
    assert torch.equal(oc.view(torch.int16), dec.o.view(torch.int16)), tag
    assert torch.equal(lc.view(torch.int32), dec.lse.view(torch.int32)), tag
