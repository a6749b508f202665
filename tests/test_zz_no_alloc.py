"""ea_hybrid_attn_decode_noalloc (scratch in the library's own device array)
against ea_hybrid_attn_decode (caller's workspace), through the C ABI.

The two run the same kernels on the same inputs, so their outputs must be
bit-identical; the small cases are also checked against the fp64 decode
oracle.  Calls run back to back on one stream, a large step first and then a
smaller one, so the second call meets the scratch the first one left behind.
"""

import numpy as np
import pytest
import torch

from hybrid_sparse_full_amd import ea as E
from hybrid_sparse_full_amd.layer import HybridDecode, bf16_tensor, desc_for, make_desc
from oracle import decode as OD
from synth import get_config, make_inputs, bf16_bits_to_f64, MODE_FA, MODE_SSA
import parity_utils as PU

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _noalloc(desc, cu, modes, q, k, v):
    o = torch.full((desc.num_seqs, desc.num_q_heads, desc.head_dim), 7.0, dtype=torch.bfloat16,
                   device=DEV)
    lse = torch.full((desc.num_seqs, desc.num_q_heads), 7.0, dtype=torch.float32, device=DEV)
    E.ea_hybrid_attn_decode_noalloc(desc, q, k, v, cu, modes, o, lse)
    return o, lse


def _with_workspace(desc, cu_host, modes_host, q, k, v):
    dec = HybridDecode(desc, cu_host, modes_host, device=DEV)
    dec(q, k, v)
    return dec.o, dec.lse


def _small_case(seed, seqlens, hq=8, hkv=2):
    rng = np.random.default_rng(seed)
    modes = tuple(tuple(int(x) for x in r) for r in rng.integers(0, 3, size=(len(seqlens), hkv)))
    cfg = get_config("tiny-1k").with_(name=f"noalloc-{seed}", seed=seed, num_q_heads=hq,
                                      num_kv_heads=hkv, head_dim=128, block=128, ssa_sink=64,
                                      ssa_window=300, seqlens=tuple(seqlens), modes=modes)
    inp = make_inputs(cfg)
    cu = inp["cu_seqlens"]
    idx = np.maximum(cu[1:] - 1, 0)
    qn = inp["q"][idx].copy()
    qn[cu[1:] == cu[:-1]] = 0
    return inp, qn


def _check_small(inp, qn, o_na, lse_na, o_ws, lse_ws, tag):
    assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16)), tag
    assert torch.equal(lse_na.view(torch.int32), lse_ws.view(torch.int32)), tag
    cfg = inp["cfg"]
    O, LSE = OD.decode(bf16_bits_to_f64(qn), bf16_bits_to_f64(inp["k"]), bf16_bits_to_f64(inp["v"]),
                       inp["cu_seqlens"], inp["modes"], scale=cfg.softmax_scale, sink=cfg.ssa_sink,
                       window=cfg.ssa_window)
    o = o_na.float().cpu().numpy().astype(np.float64)
    lse = lse_na.cpu().numpy().astype(np.float64)
    keep = np.asarray(inp["seqlens"]) > 0
    assert np.all(o[~keep] == 0) and np.all(np.isneginf(lse[~keep]))
    res = PU.check_close(o[keep].reshape(-1), O[keep].reshape(-1), lse[keep], LSE[keep], tag)
    print(tag, res, flush=True)


def test_noalloc_equals_workspace_decode_large_then_small():
    # Call 1: 8 sequences of 64K cached tokens (Llama-3.1-8B shape, FA-SSA),
    # the plan path with split partials over most of the scratch.
    L, batch, Hq, Hkv, D = 65536, 8, 32, 8, 128
    desc = make_desc(num_seqs=batch, total_tokens=L * batch, max_seqlen=L, num_q_heads=Hq,
                     num_kv_heads=Hkv, head_dim=D, block=128, ssa_sink=128, ssa_window=2048)
    assert E.ea_workspace_bytes(desc, E.EA_OP_DECODE) <= E.EA_DECODE_NOALLOC_SCRATCH_BYTES
    gen = torch.Generator(device=DEV)
    gen.manual_seed(23)
    k = torch.randn((L * batch, Hkv, D), generator=gen, device=DEV).to(torch.bfloat16)
    v = torch.randn((L * batch, Hkv, D), generator=gen, device=DEV).to(torch.bfloat16)
    q = torch.randn((batch, Hq, D), generator=gen, device=DEV).to(torch.bfloat16)
    cu_host = (np.arange(batch + 1) * L).astype(np.int32)
    modes_host = np.tile(np.array([0, 1, 1, 0, 1, 1, 0, 1], dtype=np.uint8), (batch, 1))
    modes_host[1] = 1
    modes_host[2] = 2
    cu = torch.from_numpy(cu_host).to(DEV)
    modes = torch.from_numpy(modes_host.reshape(-1)).to(DEV)
    print("noalloc call 1: 8 x 64K", flush=True)
    o1, l1 = _noalloc(desc, cu, modes, q, k, v)
    o1w, l1w = _with_workspace(desc, cu_host, modes_host, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o1w.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l1w.view(torch.int32))
    assert torch.isfinite(l1).all()
    del k, v

    # Call 2, right after: a smaller ragged batch (empty and 1-token
    # sequences included), also checked against the oracle.
    inp, qn = _small_case(41, (1, 2, 63, 1000, 0, 1025, 3000))
    d2 = desc_for(inp["cfg"], inp["seqlens"])
    q2 = bf16_tensor(qn, DEV)
    k2, v2 = bf16_tensor(inp["k"], DEV), bf16_tensor(inp["v"], DEV)
    cu2 = torch.from_numpy(inp["cu_seqlens"].astype(np.int32)).to(DEV)
    m2 = torch.from_numpy(np.ascontiguousarray(inp["modes"], dtype=np.uint8).reshape(-1)).to(DEV)
    print("noalloc call 2: 7 ragged sequences", flush=True)
    o2, l2 = _noalloc(d2, cu2, m2, q2, k2, v2)
    o2w, l2w = _with_workspace(d2, inp["cu_seqlens"], inp["modes"], q2, k2, v2)
    torch.cuda.synchronize()
    _check_small(inp, qn, o2, l2, o2w, l2w, "noalloc after 8 x 64K")


def test_noalloc_two_small_calls_in_a_row():
    a, qa = _small_case(5, (2049, 700, 0, 64, 65, 1))
    b, qb = _small_case(6, (300, 17))
    outs = []
    for inp, qn in ((a, qa), (b, qb)):
        d = desc_for(inp["cfg"], inp["seqlens"])
        q = bf16_tensor(qn, DEV)
        k, v = bf16_tensor(inp["k"], DEV), bf16_tensor(inp["v"], DEV)
        cu = torch.from_numpy(inp["cu_seqlens"].astype(np.int32)).to(DEV)
        m = torch.from_numpy(np.ascontiguousarray(inp["modes"], dtype=np.uint8).reshape(-1)).to(DEV)
        print("noalloc small call", inp["cfg"].name, flush=True)
        o, l = _noalloc(d, cu, m, q, k, v)
        outs.append((inp, qn, o, l, d, q, k, v))
    torch.cuda.synchronize()
    for inp, qn, o, l, d, q, k, v in outs:
        ow, lw = _with_workspace(d, inp["cu_seqlens"], inp["modes"], q, k, v)
        torch.cuda.synchronize()
        _check_small(inp, qn, o, l, ow, lw, f"noalloc {inp['cfg'].name}")
