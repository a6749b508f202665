"""Malformed device data: cu_seqlens and modes that the host cannot check.

The library cannot read cu_seqlens or modes on the host without a
synchronisation, so the kernels sanitise them (include/ea.h): mode bytes
other than 0/1/2 run as FA, and sequence bounds are clamped.  Prefill,
selection and attention make the sequences disjoint and inside [0, T), with
at most max_seqlen tokens each:

    s_b = clamp(cu[b]), e_b = min(max(clamp(cu[b+1]), s_b), s_b + max_seqlen),
    start_b = max(s_b, max_{b' < b} e_b'),  len_b = max(0, e_b - start_b);

decode and the router clamp each sequence on its own (s_b, e_b as above),
so their sequences may overlap.  With cu_seqlens that decrease, overlap and
leave [0, T), and mode bytes 3, 7 and 255, every call must return EA_OK and
each sanitised sequence must match the oracle run on that sequence alone.
(Tokens that no sanitised sequence covers have no defined output.)
"""

import numpy as np
import pytest
import torch

from hybrid_sparse_full_amd import ea as E
from hybrid_sparse_full_amd.layer import HybridDecode, HybridPrefill, Router, bf16_tensor, make_desc
from oracle import decode as OD
from oracle import router as ORT
from synth import get_config, make_inputs, bf16_bits_to_f64, MODE_FA, MODE_SSA, MODE_XA
from synth.router_weights import make_router_weights
import parity_utils as PU

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
HQ, HKV, D, B = 8, 2, 128, 128
T, MAXL = 2560, 1024

# (cu_seqlens as given, the sanitised prefill sequences as (start, len) worked
# out by hand from the rule above)
CASES = {
    "backwards-and-past-T": ([0, 640, 256, 1920, 5000], [(0, 640), (640, 0), (640, 640), (1920, 640)]),
    "negative": ([-100, 384, 384, -5, 2560], [(0, 384), (384, 0), (384, 0), (384, 640)]),
}
MODES = np.array([[MODE_XA, 7], [MODE_SSA, 255], [MODE_FA, MODE_XA], [3, MODE_SSA]], dtype=np.uint8)


def _clamp(x):
    return min(max(int(x), 0), T)


def _prefill_rule(cu):
    out, prev = [], 0
    for b in range(len(cu) - 1):
        s = _clamp(cu[b])
        e = min(max(_clamp(cu[b + 1]), s), s + MAXL)
        start = max(s, prev)
        out.append((start, max(0, e - start)))
        prev = max(prev, e)
    return out


def _decode_rule(cu):
    out = []
    for b in range(len(cu) - 1):
        s = _clamp(cu[b])
        e = min(max(_clamp(cu[b + 1]), s), s + MAXL)
        out.append((s, e - s))
    return out


def _sane(modes):
    m = modes.copy()
    m[m > MODE_XA] = MODE_FA
    return m


def _base(seed):
    cfg = get_config("tiny-1k").with_(name=f"malformed-{seed}", seed=seed, num_q_heads=HQ, num_kv_heads=HKV,
                                      head_dim=D, block=B, ssa_sink=64, ssa_window=200, xa_stride=8,
                                      seqlens=(T,), modes=((MODE_FA,) * HKV,))
    return cfg, make_inputs(cfg)


def _desc(nseq):
    return make_desc(num_seqs=nseq, total_tokens=T, max_seqlen=MAXL, num_q_heads=HQ, num_kv_heads=HKV,
                     head_dim=D, block=B, ssa_sink=64, ssa_window=200, xa_stride=8)


@pytest.mark.parametrize("name", sorted(CASES))
def test_malformed_batch_prefill(name):
    cu, expect = CASES[name]
    assert _prefill_rule(cu) == expect
    cfg, base = _base(71)
    nseq = len(cu) - 1
    layer = HybridPrefill(_desc(nseq), np.array(cu, dtype=np.int32), MODES, device=DEV, block_mass=True)
    q, k, v = (bf16_tensor(base[n], DEV) for n in ("q", "k", "v"))
    layer(q, k, v)
    torch.cuda.synchronize()

    # The oracle on the sanitised batch: its sequences packed one after another.
    lens = [n for _, n in expect]
    idx = np.concatenate([np.arange(s, s + n) for s, n in expect]).astype(np.int64)
    inp = dict(cfg=cfg.with_(seqlens=tuple(lens)), seqlens=np.array(lens), modes=_sane(MODES),
               cu_seqlens=np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
               q=base["q"][idx], k=base["k"][idx], v=base["v"][idx])
    masks = PU.oracle_xa(inp)
    assert masks, "the case has XA heads on non-empty sequences"
    gout = dict(mask=layer.mask.cpu().numpy().view(np.uint32), block_mass=layer.block_mass.cpu().numpy())
    stats = PU.check_masks(gout, inp, masks)
    assert stats["mismatched"] == stats["mismatched_ties"], stats
    O, LSE = PU.oracle_full(inp, masks)
    # Only the covered tokens: the others hold whatever the buffer held.
    o = layer.o.float().cpu().numpy()[idx].astype(np.float64).reshape(len(idx), -1)
    lse = layer.lse.cpu().numpy()[:, idx].astype(np.float64)
    res = PU.check_close(o, O.reshape(len(idx), -1), lse, LSE, f"malformed prefill {name}")
    print(name, res, {k_: v_ for k_, v_ in stats.items() if k_ != "tie_rows"}, flush=True)


@pytest.mark.parametrize("name", sorted(CASES))
def test_malformed_batch_decode_and_router(name):
    cu, _ = CASES[name]
    seqs = _decode_rule(cu)
    cfg, base = _base(72)
    nseq = len(cu) - 1
    d = _desc(nseq)
    k, v = bf16_tensor(base["k"], DEV), bf16_tensor(base["v"], DEV)
    qn = base["q"][:nseq].copy()
    dec = HybridDecode(d, np.array(cu, dtype=np.int32), MODES, device=DEV)
    dec(bf16_tensor(qn, DEV), k, v)

    w = make_router_weights(D, 4 * D, seed=9)
    router = Router(w, DEV)
    modes_out = torch.full((nseq * HKV,), 77, dtype=torch.uint8, device=DEV)
    logits = torch.full((nseq * HKV * 2,), float("nan"), dtype=torch.float32, device=DEV)
    cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    router(d, k, cu_t, MODE_FA, MODE_SSA, modes_out, logits)
    torch.cuda.synchronize()

    o = dec.o.double().cpu().numpy()
    lse = dec.lse.double().cpu().numpy()
    gz = logits.cpu().numpy().astype(np.float64).reshape(nseq, HKV, 2)
    gm = modes_out.cpu().numpy().reshape(nseq, HKV)
    kf, vf = bf16_bits_to_f64(base["k"]), bf16_bits_to_f64(base["v"])
    sane = _sane(MODES)
    for b, (s, n) in enumerate(seqs):
        if n == 0:
            assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b])), b
        else:
            Ob, LSEb = OD.decode(bf16_bits_to_f64(qn[b:b + 1]), kf[s:s + n], vf[s:s + n],
                                 np.array([0, n], dtype=np.int32), sane[b:b + 1], scale=cfg.softmax_scale,
                                 sink=cfg.ssa_sink, window=cfg.ssa_window)
            print(name, "decode", b, (s, n), PU.check_close(o[b].reshape(-1), Ob.reshape(-1), lse[b], LSEb[0],
                                                           f"malformed decode {name} seq {b}"), flush=True)
        om, oz = ORT.route(kf[s:s + n], np.array([0, n], dtype=np.int32), w, retrieval_mode=MODE_FA,
                           sparse_mode=MODE_SSA, head=100, tail=100)
        tol = 1e-4 * (1.0 + np.abs(oz[0]))
        assert np.all(np.abs(gz[b] - oz[0]) <= tol), (b, gz[b], oz[0])
        decided = np.abs(oz[0, :, 1] - oz[0, :, 0]) > 2 * tol.max(axis=-1)
        assert np.array_equal(gm[b][decided], om[0][decided]), b
