"""Concurrent calls on separate streams (include/ea.h: the library keeps no
state, so calls with distinct workspaces may overlap).

A prefill with XA selection and a decode step, each with its own buffers,
are issued on two streams (default priority) without synchronising between
them, twice over in an interleaved order; their outputs must equal those of
the same calls run one after another on one stream, bit for bit (the kernels
are deterministic).
"""

import numpy as np
import pytest
import torch

from hybrid_sparse_full_amd.layer import HybridDecode, HybridPrefill, bf16_tensor, desc_for
from synth import get_config, make_inputs, MODE_FA, MODE_SSA, MODE_XA

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def test_prefill_and_decode_on_two_streams():
    cfg = get_config("tiny-1k").with_(name="streams", seed=61, num_q_heads=8, num_kv_heads=4, head_dim=128,
                                      block=128, ssa_sink=64, ssa_window=300, xa_stride=8,
                                      seqlens=(2048, 1024, 640),
                                      modes=((MODE_XA, MODE_SSA, MODE_FA, MODE_SSA),
                                             (MODE_SSA, MODE_XA, MODE_SSA, MODE_FA),
                                             (MODE_FA, MODE_FA, MODE_XA, MODE_SSA)))
    inp = make_inputs(cfg)
    d = desc_for(cfg, inp["seqlens"])
    q, k, v = (bf16_tensor(inp[n], DEV) for n in ("q", "k", "v"))
    qd = q[torch.tensor(np.cumsum(inp["seqlens"]) - 1, device=DEV)].contiguous()
    pre = [HybridPrefill(d, inp["cu_seqlens"], inp["modes"], device=DEV, block_mass=True) for _ in range(2)]
    dec = [HybridDecode(d, inp["cu_seqlens"], inp["modes"], device=DEV) for _ in range(2)]
    torch.cuda.synchronize()

    # Reference: one after another on the current stream.
    pre[0](q, k, v)
    dec[0](qd, k, v)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (pre[0].o, pre[0].lse, pre[0].mask, dec[0].o, dec[0].lse)]

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for t in (pre[1].o, pre[1].lse, dec[1].o, dec[1].lse):
        t.fill_(float("nan"))
    pre[1].mask.fill_(-1)
    torch.cuda.synchronize()
    for _ in range(2):
        pre[1](q, k, v, stream=s1)
        dec[1](qd, k, v, stream=s2)
        dec[1](qd, k, v, stream=s2)
        pre[1](q, k, v, stream=s1)
    torch.cuda.synchronize()
    got = (pre[1].o, pre[1].lse, pre[1].mask, dec[1].o, dec[1].lse)
    for i, (a, b) in enumerate(zip(got, ref)):
        assert torch.equal(_bits(a), _bits(b)), f"output {i} differs when the calls overlap"
