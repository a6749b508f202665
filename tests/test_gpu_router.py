"""GPU parity of the attention router (ea_route_heads) against the fp64 oracle.

Logits must agree within 1e-4 * (1 + |z|); the modes must be equal on every
head whose two logits differ by more than twice that bound (closer heads are
ties that either side may break, counted and reported).  End to end, the
modes the router writes on the device drive ea_hybrid_attn_prefill, whose
output must match the oracle's attention under the oracle's own routing.
"""

import numpy as np
import pytest
import torch

from hybrid_sparse_full_amd import ea as E
from hybrid_sparse_full_amd.layer import HybridPrefill, Router, bf16_tensor, desc_for, make_desc
from oracle import router as ORT
from synth import get_config, make_inputs, bf16_bits_to_f64, f32_to_bf16_bits, MODE_FA, MODE_SSA, MODE_XA
from synth.router_weights import make_router_weights
import parity_utils as PU

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _route_gpu(desc, weights, k_bits, cu, rm, sm, pool_head=100, pool_tail=100):
    r = Router(weights, DEV, pool_head, pool_tail)
    nseq, hkv = desc.num_seqs, desc.num_kv_heads
    modes = torch.full((nseq * hkv,), 255, dtype=torch.uint8, device=DEV)
    logits = torch.full((nseq * hkv * 2,), float("nan"), dtype=torch.float32, device=DEV)
    k = bf16_tensor(k_bits, DEV)
    cu_t = torch.from_numpy(np.ascontiguousarray(cu, dtype=np.int32)).to(DEV)
    r(desc, k, cu_t, rm, sm, modes, logits)
    torch.cuda.synchronize()
    return modes.cpu().numpy().reshape(nseq, hkv), logits.cpu().numpy().reshape(nseq, hkv, 2)


def _check(k_bits, cu, weights, rm, sm, gm, gz, pool_head=100, pool_tail=100):
    om, oz = ORT.route(bf16_bits_to_f64(k_bits), cu, weights, retrieval_mode=rm, sparse_mode=sm,
                       head=pool_head, tail=pool_tail)
    tol = 1e-4 * (1.0 + np.abs(oz))
    assert np.all(np.abs(gz - oz) <= tol), float(np.max(np.abs(gz - oz) / (1 + np.abs(oz))))
    margin = np.abs(oz[..., 1] - oz[..., 0])
    decided = margin > 2 * tol.max(axis=-1)
    assert np.array_equal(gm[decided], om[decided])
    assert set(np.unique(gm)) <= {rm, sm}
    ties = int((~decided).sum())
    print(f"router: {gm.size} heads, {ties} ties, modes {np.bincount(gm.reshape(-1), minlength=3)}",
          flush=True)
    return om


@pytest.mark.parametrize("D,hidden,pool", [(128, 512, (100, 100)), (64, 256, (100, 100)),
                                           (128, 1024, (7, 0)), (64, 100, (0, 33)),
                                           (128, 64, (0, 0))])
def test_router_matches_oracle(D, hidden, pool):
    seqlens = (0, 1, 150, 199, 200, 201, 1000, 4096)
    hkv = 4
    rng = np.random.Generator(np.random.PCG64(D + hidden))
    T = sum(seqlens)
    kf = rng.standard_normal((T, hkv, D), dtype=np.float32)
    # A per-(sequence, head) offset so that the pooled vectors differ.
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    for b in range(len(seqlens)):
        kf[cu[b]:cu[b + 1]] += rng.standard_normal((1, hkv, D), dtype=np.float32)
    k_bits = f32_to_bf16_bits(kf)
    w = make_router_weights(D, hidden, seed=hidden)
    d = make_desc(num_seqs=len(seqlens), total_tokens=T, max_seqlen=max(seqlens), num_q_heads=8,
                  num_kv_heads=hkv, head_dim=D, block=64)
    gm, gz = _route_gpu(d, w, k_bits, cu, MODE_FA, MODE_SSA, *pool)
    _check(k_bits, cu, w, MODE_FA, MODE_SSA, gm, gz, *pool)


def test_router_on_256k_keys():
    # Qwen3-8B-shaped keys at 262,144 tokens: the router reads 200 of them.
    inp = make_inputs(get_config("qwen8b-faxa-256k"))
    cfg = inp["cfg"]
    w = make_router_weights(cfg.head_dim, 4 * cfg.head_dim, seed=3)
    d = desc_for(cfg, inp["seqlens"])
    gm, gz = _route_gpu(d, w, inp["k"], inp["cu_seqlens"], MODE_FA, MODE_XA)
    _check(inp["k"], inp["cu_seqlens"], w, MODE_FA, MODE_XA, gm, gz)


def test_router_is_deterministic():
    inp = make_inputs(get_config("tiny-1k"))
    cfg = inp["cfg"]
    w = make_router_weights(cfg.head_dim, 4 * cfg.head_dim, seed=5)
    d = desc_for(cfg, inp["seqlens"])
    a = _route_gpu(d, w, inp["k"], inp["cu_seqlens"], MODE_XA, MODE_SSA)
    b = _route_gpu(d, w, inp["k"], inp["cu_seqlens"], MODE_XA, MODE_SSA)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("rm,sm", [(MODE_FA, MODE_SSA), (MODE_XA, MODE_SSA), (MODE_FA, MODE_XA)])
def test_routed_prefill_end_to_end(rm, sm):
    # Router on the device -> modes in device memory -> XA select -> prefill,
    # with no host round trip; the oracle routes and attends on its own.
    cfg = get_config("tiny-1k").with_(name="routed", seed=21, num_q_heads=8, num_kv_heads=4,
                                      head_dim=128, block=128, ssa_sink=64, ssa_window=200,
                                      xa_stride=8, seqlens=(1024, 384, 640),
                                      modes=((MODE_FA,) * 4,))
    inp = make_inputs(cfg)
    # Weight seed 212 routes 8 of the 12 (sequence, KV head) pairs to the
    # sparse mode, with every logit margin above 0.02.
    w = make_router_weights(cfg.head_dim, 4 * cfg.head_dim, seed=212)
    d = desc_for(cfg, inp["seqlens"])
    layer = HybridPrefill(d, inp["cu_seqlens"], None, device=DEV, mode_set=(rm, sm), block_mass=True)
    q, k, v = (bf16_tensor(inp[n], DEV) for n in ("q", "k", "v"))
    logits = torch.empty(d.num_seqs * d.num_kv_heads * 2, dtype=torch.float32, device=DEV)
    layer.route(Router(w, DEV), k, logits)
    layer(q, k, v)
    torch.cuda.synchronize()
    gm = layer.device_modes()
    om = _check(inp["k"], inp["cu_seqlens"], w, rm, sm, gm,
                logits.cpu().numpy().reshape(d.num_seqs, d.num_kv_heads, 2))
    assert np.array_equal(gm, om), "a tie decided this case differently; pick another seed"
    inp_o = dict(inp)
    inp_o["modes"] = om
    masks = PU.oracle_xa(inp_o)
    if masks:
        gout = dict(mask=layer.mask.cpu().numpy().view(np.uint32),
                    block_mass=layer.block_mass.cpu().numpy())
        PU.check_masks(gout, inp_o, masks)
    O, LSE = PU.oracle_full(inp_o, masks)
    T = int(inp["cu_seqlens"][-1])
    o = layer.o.float().cpu().numpy().astype(np.float64).reshape(T, -1)
    lse = layer.lse.cpu().numpy().astype(np.float64)
    res = PU.check_close(o, O.reshape(T, -1), lse, LSE, f"routed {rm}-{sm}")
    print(res, flush=True)
