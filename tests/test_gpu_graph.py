"""The library's entry points under HIP graph capture.

Every entry point only launches kernels on the caller's stream (no memset,
copy, synchronisation or allocation), and every call starts with a kernel
that clears the counters it uses, so a captured call must replay exactly
what an eager call does.  Each test captures a chain of calls into one
torch.cuda.CUDAGraph, then replays it several times.  Before each replay the
outputs are overwritten with garbage, and the program does eager work of its
own with synchronisations in between.  Every replay must reproduce the eager
result bit for bit (the kernels are deterministic), and a replay on new input
values, copied into the captured buffers, must equal an eager call on them
and the fp64 oracle.
"""

import numpy as np
import pytest
import torch

from hybrid_sparse_full_amd import ea as E
from hybrid_sparse_full_amd.layer import HybridDecode, HybridPrefill, Router, bf16_tensor, desc_for, make_desc
from oracle import decode as OD
from synth import get_config, make_inputs, bf16_bits_to_f64, MODE_FA, MODE_SSA, MODE_XA
from synth.router_weights import make_router_weights
import parity_utils as PU

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
REPLAYS = 4
ROW_COUNT, BLOCK_MASS = 3, 5  # positions in the prefill test's output list


def _bits(t):
    """A tensor's raw bits, for bit-for-bit comparison (NaN-safe)."""
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32) if t.element_size() == 4 \
        else t.view(torch.int64) if t.element_size() == 8 else t.view(torch.uint8)


def _garble(tensors):
    for t in tensors:
        if t.is_floating_point():
            t.fill_(float("nan"))
        else:
            t.view(torch.uint8).fill_(0xA5)


def _unrelated_eager_work():
    a = torch.randn((512, 512), device=DEV)
    (a @ a).sum().item()
    torch.cuda.synchronize()


def _replay_and_compare(graph, outs, refs, tag, check=None):
    """`check`, if given, compares (outputs, references) itself; else every
    output must equal its reference bit for bit."""
    for r in range(REPLAYS):
        _garble(outs)
        _unrelated_eager_work()
        graph.replay()
        torch.cuda.synchronize()
        if check is not None:
            check(outs, refs, f"{tag}: replay {r}")
        else:
            for i, (t, ref) in enumerate(zip(outs, refs)):
                assert torch.equal(_bits(t), _bits(ref)), f"{tag}: replay {r}, output {i} differs from eager"
        print(f"{tag}: replay {r} equals eager", flush=True)


def _check_prefill(outs, refs, tag):
    """Every output bit for bit, except the block masses: those are written
    on the rows of XA heads (row_count > 0) only, and the other rows must be
    left as they were (here: the garbage)."""
    for i, (t, ref) in enumerate(zip(outs, refs)):
        if i == BLOCK_MASS:
            xa = refs[ROW_COUNT] > 0
            assert torch.equal(_bits(t[xa]), _bits(ref[xa])), f"{tag}: block masses of XA rows differ"
            assert bool(torch.isnan(t[~xa]).all()), f"{tag}: a row of a non-XA head was written"
        else:
            assert torch.equal(_bits(t), _bits(ref)), f"{tag}: output {i} differs from eager"


def _prefill_inputs(seed):
    cfg = get_config("tiny-1k").with_(name=f"graph-{seed}", seed=seed, num_q_heads=8, num_kv_heads=4,
                                      head_dim=128, block=128, ssa_sink=64, ssa_window=200, xa_stride=8,
                                      seqlens=(1024, 384, 640), modes=((MODE_FA,) * 4,))
    return make_inputs(cfg)


def test_routed_prefill_graph_replays_match_eager():
    # Router -> modes on the device -> XA scoring and selection -> prefill, in
    # one graph: 4 launches of routing, selection and attention per replay.
    inp = _prefill_inputs(31)
    d = desc_for(inp["cfg"], inp["seqlens"])
    layer = HybridPrefill(d, inp["cu_seqlens"], None, device=DEV, mode_set=(MODE_XA, MODE_SSA),
                          block_mass=True)
    router = Router(make_router_weights(128, 512, seed=212), DEV)
    q, k, v = (bf16_tensor(inp[n], DEV) for n in ("q", "k", "v"))
    logits = torch.empty(d.num_seqs * d.num_kv_heads * 2, dtype=torch.float32, device=DEV)

    def step():
        layer.route(router, k, logits)
        layer(q, k, v)

    outs = [layer.modes, logits, layer.mask, layer.row_count, layer.xa_pairs, layer.block_mass, layer.o,
            layer.lse]
    assert outs[ROW_COUNT] is layer.row_count and outs[BLOCK_MASS] is layer.block_mass
    step()
    torch.cuda.synchronize()
    refs = [t.clone() for t in outs]
    modes = layer.device_modes()
    assert (modes == MODE_XA).any() and (modes == MODE_SSA).any(), modes

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    _replay_and_compare(g, outs, refs, "routed prefill", _check_prefill)

    # New values in the captured input buffers: the replay must read them.
    inp2 = _prefill_inputs(32)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        t.copy_(bf16_tensor(inp2[n], DEV))
    _garble(outs)
    g.replay()
    torch.cuda.synchronize()
    got = [t.clone() for t in outs]
    assert not torch.equal(_bits(got[-2]), _bits(refs[-2])), "the replay ignored the new inputs"
    _garble(outs)
    step()
    torch.cuda.synchronize()
    _check_prefill(outs, got, "new inputs: eager against the replay")

    # ... and the replay's attention matches the oracle under the modes it routed.
    inp_o = dict(inp2)
    inp_o["modes"] = layer.device_modes()
    masks = PU.oracle_xa(inp_o)
    if masks:
        PU.check_masks(dict(mask=got[2].cpu().numpy().view(np.uint32), block_mass=got[5].cpu().numpy()),
                       inp_o, masks)
    O, LSE = PU.oracle_full(inp_o, masks)
    T = int(inp2["cu_seqlens"][-1])
    o = got[6].float().cpu().numpy().astype(np.float64).reshape(T, -1)
    lse = got[7].cpu().numpy().astype(np.float64)
    print(PU.check_close(o, O.reshape(T, -1), lse, LSE, "graph replay, new inputs"), flush=True)


def _decode_case(seqlens, seed, hq=32, hkv=8):
    rng = np.random.Generator(np.random.PCG64(seed))
    nseq = len(seqlens)
    cu = np.zeros(nseq + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    modes = rng.integers(0, 3, size=(nseq, hkv)).astype(np.uint8)
    desc = make_desc(num_seqs=nseq, total_tokens=int(cu[-1]), max_seqlen=int(max(seqlens)), num_q_heads=hq,
                     num_kv_heads=hkv, head_dim=128, block=128, ssa_sink=128, ssa_window=2048)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    T = int(cu[-1])
    k = torch.randn((T, hkv, 128), generator=gen, device=DEV).to(torch.bfloat16)
    v = torch.randn((T, hkv, 128), generator=gen, device=DEV).to(torch.bfloat16)
    q = torch.randn((nseq, hq, 128), generator=gen, device=DEV).to(torch.bfloat16)
    return desc, cu, modes, q, k, v


def test_decode_graph_replays_match_eager():
    # Two steps in one graph: 40 (sequence, KV head) units, where each wave
    # plans the step itself, and 96 units, where k_decode_plan runs first;
    # then the second step again through the allocation-free entry point.
    a = _decode_case((12000, 0, 3000, 17000, 65), seed=41)
    b = _decode_case(tuple(int(x) for x in np.random.Generator(np.random.PCG64(42)).integers(0, 7000, 12)),
                     seed=43)
    for desc, *_ in (a, b):
        assert E.ea_workspace_bytes(desc, E.EA_OP_DECODE) <= E.EA_DECODE_NOALLOC_SCRATCH_BYTES
    dec_a = HybridDecode(a[0], a[1], a[2], device=DEV)
    dec_b = HybridDecode(b[0], b[1], b[2], device=DEV)
    o_na = torch.empty_like(dec_b.o)
    lse_na = torch.empty_like(dec_b.lse)

    def step():
        dec_a(*a[3:])
        dec_b(*b[3:])
        E.ea_hybrid_attn_decode_noalloc(b[0], *b[3:], dec_b.cu, dec_b.modes, o_na, lse_na)

    outs = [dec_a.o, dec_a.lse, dec_b.o, dec_b.lse, o_na, lse_na]
    step()
    torch.cuda.synchronize()
    refs = [t.clone() for t in outs]
    assert torch.equal(_bits(o_na), _bits(dec_b.o)) and torch.equal(_bits(lse_na), _bits(dec_b.lse))

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    _replay_and_compare(g, outs, refs, "decode")

    # New queries: the replay must equal the oracle on the first step.
    gen = torch.Generator(device=DEV)
    gen.manual_seed(44)
    a[3].copy_(torch.randn(a[3].shape, generator=gen, device=DEV).to(torch.bfloat16))
    _garble(outs)
    g.replay()
    torch.cuda.synchronize()
    desc, cu, modes, q, k, v = a
    O, LSE = OD.decode(q.double().cpu().numpy(), k.double().cpu().numpy(), v.double().cpu().numpy(), cu, modes,
                       scale=128 ** -0.5, sink=128, window=2048)
    keep = np.diff(cu) > 0
    o = dec_a.o.double().cpu().numpy()
    lse = dec_a.lse.double().cpu().numpy()
    assert np.all(o[~keep] == 0) and np.all(np.isneginf(lse[~keep]))
    print(PU.check_close(o[keep].reshape(-1), O[keep].reshape(-1), lse[keep], LSE[keep], "decode graph replay"),
          flush=True)


def test_segmented_cache_decode_loop_graph():
    # A serving loop: every step appends one token per sequence to the
    # segmented cache and decodes it.  The descriptor holds the capacity (an
    # upper bound of the lengths), so one capture serves every step; between
    # replays only device buffers change: the lengths and the new k, v and q.
    # A twin cache driven by eager calls must match every replay bit for bit,
    # and the last step matches the oracle over each sequence's whole history.
    from hybrid_sparse_full_amd.layer import SegmentedDecodeCache
    nseq, Hq, Hkv, D, sink, window, steps = 3, 8, 2, 128, 16, 64, 6
    L0 = np.array([100, 37, 200])
    cap = L0 + steps
    modes = np.array([[MODE_FA, MODE_SSA], [MODE_SSA, MODE_XA], [MODE_SSA, MODE_SSA]], dtype=np.uint8)
    desc = make_desc(num_seqs=nseq, total_tokens=int(cap.sum()), max_seqlen=int(cap.max()), num_q_heads=Hq,
                     num_kv_heads=Hkv, head_dim=D, block=128, ssa_sink=sink, ssa_window=window)
    desc0 = make_desc(num_seqs=nseq, total_tokens=int(L0.sum()), max_seqlen=int(L0.max()), num_q_heads=Hq,
                      num_kv_heads=Hkv, head_dim=D, block=128, ssa_sink=sink, ssa_window=window)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(51)
    kh = [torch.randn((int(c), Hkv, D), generator=gen, device=DEV).to(torch.bfloat16) for c in cap]
    vh = [torch.randn((int(c), Hkv, D), generator=gen, device=DEV).to(torch.bfloat16) for c in cap]
    qs = torch.randn((steps, nseq, Hq, D), generator=gen, device=DEV).to(torch.bfloat16)

    def cu_of(lens):
        return torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)

    k0 = torch.cat([kh[b][:L0[b]] for b in range(nseq)])
    v0 = torch.cat([vh[b][:L0[b]] for b in range(nseq)])
    caches = [SegmentedDecodeCache(desc, modes, cap.astype(np.int32), device=DEV) for _ in range(2)]
    for c in caches:
        c.fill(desc0, k0, v0, cu_of(L0))
    ws = [torch.empty(E.ea_workspace_bytes(desc, E.EA_OP_DECODE), dtype=torch.uint8, device=DEV) for _ in range(2)]
    outs = [(torch.empty((nseq, Hq, D), dtype=torch.bfloat16, device=DEV),
             torch.empty((nseq, Hq), dtype=torch.float32, device=DEV)) for _ in range(2)]
    cu = torch.empty(nseq + 1, dtype=torch.int32, device=DEV)
    k_new = torch.empty((nseq, Hkv, D), dtype=torch.bfloat16, device=DEV)
    v_new = torch.empty_like(k_new)
    q = torch.empty((nseq, Hq, D), dtype=torch.bfloat16, device=DEV)

    def step(i):
        c, (o, lse) = caches[i], outs[i]
        c.append(desc, k_new, v_new, cu)
        c.decode(desc, q, cu, o, lse, ws[i])

    def set_inputs(s):
        lens = L0 + s + 1
        cu.copy_(cu_of(lens))
        for b in range(nseq):
            k_new[b].copy_(kh[b][lens[b] - 1])
            v_new[b].copy_(vh[b][lens[b] - 1])
        q.copy_(qs[s])
        torch.cuda.synchronize()
        return lens

    g = None
    for s in range(steps):
        lens = set_inputs(s)
        if g is None:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(0)
            torch.cuda.synchronize()
        _garble(list(outs[0]))
        g.replay()
        step(1)
        torch.cuda.synchronize()
        for a, b in zip(outs[0], outs[1]):
            assert torch.equal(_bits(a), _bits(b)), f"step {s}: the replay differs from the eager loop"
        print(f"cache loop step {s} (lengths {lens.tolist()}) replay equals eager", flush=True)
    kp = torch.cat([kh[b][:lens[b]] for b in range(nseq)]).double().cpu().numpy()
    vp = torch.cat([vh[b][:lens[b]] for b in range(nseq)]).double().cpu().numpy()
    O, LSE = OD.decode(qs[steps - 1].double().cpu().numpy(), kp, vp,
                       np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), modes,
                       scale=desc.softmax_scale, sink=sink, window=window)
    print(PU.check_close(outs[0][0].double().cpu().numpy().reshape(-1), O.reshape(-1),
                         outs[0][1].double().cpu().numpy(), LSE, "cache loop, last step"), flush=True)
