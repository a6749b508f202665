"""Serial dispatch (split by mode, one single-mode layer per group, write
back) through the C ABI: bit-identical to the fused hybrid kernel, and
within tolerance of the fp64 oracle."""

import numpy as np
import pytest
import torch

from hybrid_sparse_full_amd import ea as E
from hybrid_sparse_full_amd.layer import bf16_tensor, desc_for
from synth import get_config, make_inputs, MODE_FA, MODE_SSA
import parity_utils as PU

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _serial(inp):
    cfg = inp["cfg"]
    desc = desc_for(cfg, inp["seqlens"])
    T, Hq, D = desc.total_tokens, desc.num_q_heads, desc.head_dim
    q, k, v = (bf16_tensor(inp[n], DEV) for n in ("q", "k", "v"))
    cu = torch.from_numpy(inp["cu_seqlens"].astype(np.int32)).to(DEV)
    o = torch.full((T, Hq, D), 3.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((Hq, T), 3.0, dtype=torch.float32, device=DEV)
    ws = torch.empty(E.ea_workspace_bytes(desc, E.EA_OP_PREFILL_SERIAL), dtype=torch.uint8, device=DEV)
    layer_modes = np.ascontiguousarray(inp["modes"][0], dtype=np.uint8)
    E.ea_hybrid_attn_prefill_serial(desc, q, k, v, cu, layer_modes, o, lse, ws)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _case(name, seqlens, row, hq, hkv, D=128, B=128, **kw):
    cfg = get_config("tiny-1k").with_(name=name, seed=13, num_q_heads=hq, num_kv_heads=hkv,
                                      head_dim=D, block=B, ssa_sink=64, ssa_window=300,
                                      seqlens=tuple(seqlens), modes=(tuple(row),), **kw)
    return make_inputs(cfg)


@pytest.mark.parametrize("hq,hkv,D,B,row", [
    (32, 8, 128, 128, (0, 1, 1, 0, 1, 1, 0, 1)),
    (8, 2, 64, 64, (1, 0)),
    (6, 3, 128, 64, (1, 0, 1)),          # G = 2
    (3, 3, 64, 128, (0, 1, 1)),          # G = 1: one head per workgroup
    (8, 4, 128, 128, (1, 1, 1, 1)),      # all sparse: the full group is empty
    (8, 4, 128, 128, (0, 0, 0, 0)),      # all full
])
def test_serial_dispatch_bitwise_equals_fused(hq, hkv, D, B, row):
    inp = _case(f"serial-{hq}-{hkv}", (3 * B + 17, 1, 0, 5 * B, 200), row, hq, hkv, D, B)
    o_s, l_s = _serial(inp)
    fused = PU.run_gpu(inp)
    assert np.array_equal(o_s, fused["o"]) and np.array_equal(l_s, fused["lse"])


def test_serial_dispatch_matches_oracle():
    inp = _case("serial-oracle", (1024, 777), (0, 1), 8, 2)
    o_s, l_s = _serial(inp)
    O, LSE = PU.oracle_full(inp, {})
    T = int(inp["cu_seqlens"][-1])
    res = PU.check_close(o_s.reshape(T, -1), O.reshape(T, -1), l_s, LSE, "serial dispatch")
    print("serial dispatch", res, flush=True)


def test_serial_dispatch_16k_layer_bitwise():
    # The Llama-3.1-8B-shaped 16K layer (3 FA + 5 SSA KV heads), as the bench runs it.
    inp = make_inputs(get_config("llama8b-fassa-16k"))
    o_s, l_s = _serial(inp)
    fused = PU.run_gpu(inp)
    assert np.array_equal(o_s, fused["o"]) and np.array_equal(l_s, fused["lse"])
