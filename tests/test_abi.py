"""CPU tests of the C ABI: exported symbols, workspace sizing, argument
validation (every case fails before any device work), and the host-side
sparsity ratios against the oracle."""

import ctypes
import os
import re

import numpy as np
import pytest

from hybrid_sparse_full_amd import ea as E
from oracle import ratios as OR
from synth import MODE_FA, MODE_SSA, MODE_XA

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # 16-byte aligned non-null address; never dereferenced here


def header_functions():
    src = open(os.path.join(ROOT, "include", "ea.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ea_[a-z_]+)\s*\(", src)))


def test_library_exports_every_header_symbol():
    names = header_functions()
    assert "ea_hybrid_attn_prefill" in names and "ea_sparsity_ratios" in names
    lib = E.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(E.EXPORTS)


def desc(**kw):
    base = dict(num_seqs=1, total_tokens=4096, max_seqlen=4096, num_q_heads=32, num_kv_heads=8,
                head_dim=128, block=128, softmax_scale=128 ** -0.5, ssa_sink=128, ssa_window=2048,
                xa_stride=8, xa_tau_num=9, xa_tau_den=10)
    base.update(kw)
    return E.AttnDesc(**base)


def test_workspace_sizes():
    d = desc()
    for op in (E.EA_OP_PREFILL, E.EA_OP_XA_SELECT):
        assert E.ea_workspace_bytes(d, op) > 0
    assert E.ea_workspace_bytes(d, 7) == 0
    assert E.ea_mask_words(d) == 1 and E.ea_mask_rows(d) == (4096 // 128 + 1) * 32
    big = desc(total_tokens=262144, max_seqlen=262144)
    assert E.ea_mask_words(big) == 64
    assert E.ea_workspace_bytes(big, E.EA_OP_PREFILL) > E.ea_workspace_bytes(d, E.EA_OP_PREFILL)
    assert E.ea_workspace_offset(d, E.EA_OP_PREFILL, "tiles") > 0
    assert E.ea_workspace_offset(d, E.EA_OP_PREFILL, "xa_lse") == -1
    assert E.ea_workspace_offset(d, E.EA_OP_XA_SELECT, "xa_lse") > 0


BAD = [
    (dict(num_q_heads=30), E.EA_ERR_INVALID_ARG),           # Hq % Hkv
    (dict(num_kv_heads=0), E.EA_ERR_INVALID_ARG),
    (dict(head_dim=96), E.EA_ERR_UNSUPPORTED),
    (dict(block=32), E.EA_ERR_UNSUPPORTED),
    (dict(ssa_window=0), E.EA_ERR_INVALID_ARG),
    (dict(ssa_sink=-1), E.EA_ERR_INVALID_ARG),
    (dict(xa_tau_num=11), E.EA_ERR_INVALID_ARG),            # tau > 1
    (dict(xa_tau_num=0), E.EA_ERR_INVALID_ARG),             # tau = 0
    (dict(xa_stride=3), E.EA_ERR_INVALID_ARG),              # stride does not divide block
    (dict(xa_stride=64), E.EA_ERR_UNSUPPORTED),             # B/S = 2
    (dict(softmax_scale=0.0), E.EA_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), E.EA_ERR_INVALID_ARG),
    (dict(max_seqlen=5000), E.EA_ERR_INVALID_ARG),          # longer than the batch
    (dict(num_seqs=2, max_seqlen=1000), E.EA_ERR_INVALID_ARG),  # 2 * 1000 < 4096
    (dict(num_seqs=0), E.EA_ERR_INVALID_ARG),
    (dict(xa_group=2), E.EA_ERR_INVALID_ARG),
    (dict(xa_group=1, num_q_heads=64), E.EA_ERR_UNSUPPORTED),   # G = 8: one mask per KV head needs G <= 4
]


@pytest.mark.parametrize("kw,code", BAD)
def test_prefill_rejects_bad_descriptor(kw, code):
    lib = E.lib()
    d = desc(**kw)
    st = lib.ea_hybrid_attn_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                    FAKE, FAKE, 1 << 40, None)
    assert st == code
    st = lib.ea_xa_block_select(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                FAKE, 1 << 40, None)
    assert st == code
    assert E.ea_workspace_bytes(d, E.EA_OP_PREFILL) == 0


def test_prefill_rejects_null_and_misaligned_and_small_workspace():
    lib = E.lib()
    d = desc()
    need = E.ea_workspace_bytes(d, E.EA_OP_PREFILL)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, need, None]
    assert lib.ea_hybrid_attn_prefill(None, *args) == E.EA_ERR_INVALID_ARG
    for i in (0, 1, 2, 3, 4, 6, 7):          # q k v cu modes o lse
        a = list(args)
        a[i] = None
        assert lib.ea_hybrid_attn_prefill(ctypes.byref(d), *a) == E.EA_ERR_INVALID_ARG, i
    for i in (0, 1, 2, 6):                   # q k v o need 16-byte alignment
        a = list(args)
        a[i] = FAKE + 2
        assert lib.ea_hybrid_attn_prefill(ctypes.byref(d), *a) == E.EA_ERR_INVALID_ARG, i
    a = list(args)
    a[9] = need - 1
    assert lib.ea_hybrid_attn_prefill(ctypes.byref(d), *a) == E.EA_ERR_WORKSPACE
    a = list(args)
    a[8] = None
    assert lib.ea_hybrid_attn_prefill(ctypes.byref(d), *a) == E.EA_ERR_WORKSPACE
    # Nothing to do: returns before any launch.
    d0 = desc(total_tokens=0, max_seqlen=0)
    need0 = E.ea_workspace_bytes(d0, E.EA_OP_PREFILL)
    assert lib.ea_hybrid_attn_prefill(ctypes.byref(d0), None, None, None, FAKE, FAKE, None, None,
                                      None, FAKE, need0, None) == E.EA_OK


def test_plan_and_run_reject_null_misaligned_and_small_workspace():
    lib = E.lib()
    d = desc()
    need = E.ea_workspace_bytes(d, E.EA_OP_PREFILL)
    plan = [FAKE, FAKE, FAKE, FAKE, None, FAKE, need, None]   # k v cu modes mask ws bytes stream
    run = [FAKE, FAKE, FAKE, FAKE, FAKE, need, None]          # q modes o lse ws bytes stream
    assert lib.ea_hybrid_attn_plan(None, *plan) == E.EA_ERR_INVALID_ARG
    assert lib.ea_hybrid_attn_run(None, *run) == E.EA_ERR_INVALID_ARG
    for i in (0, 1, 2, 3):                   # k v cu modes
        a = list(plan)
        a[i] = None
        assert lib.ea_hybrid_attn_plan(ctypes.byref(d), *a) == E.EA_ERR_INVALID_ARG, i
    for i in (0, 1, 2, 3):                   # q modes o lse
        a = list(run)
        a[i] = None
        assert lib.ea_hybrid_attn_run(ctypes.byref(d), *a) == E.EA_ERR_INVALID_ARG, i
    for i in (0, 1):                         # k v need 16-byte alignment
        a = list(plan)
        a[i] = FAKE + 2
        assert lib.ea_hybrid_attn_plan(ctypes.byref(d), *a) == E.EA_ERR_INVALID_ARG, i
    for i in (0, 2):                         # q o
        a = list(run)
        a[i] = FAKE + 2
        assert lib.ea_hybrid_attn_run(ctypes.byref(d), *a) == E.EA_ERR_INVALID_ARG, i
    a = list(plan)
    a[6] = need - 1
    assert lib.ea_hybrid_attn_plan(ctypes.byref(d), *a) == E.EA_ERR_WORKSPACE
    a = list(run)
    a[4] = None
    assert lib.ea_hybrid_attn_run(ctypes.byref(d), *a) == E.EA_ERR_WORKSPACE
    # A bad q, o or lse makes the one-call prefill fail before its plan runs.
    args = [None, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, need, None]
    assert lib.ea_hybrid_attn_prefill(ctypes.byref(d), *args) == E.EA_ERR_INVALID_ARG


def test_select_rejects_small_workspace_and_nulls():
    lib = E.lib()
    d = desc()
    need = E.ea_workspace_bytes(d, E.EA_OP_XA_SELECT)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, need, None]
    for i in (0, 1, 2, 3, 4, 5, 6):          # q k cu modes mask count pairs
        a = list(args)
        a[i] = None
        assert lib.ea_xa_block_select(ctypes.byref(d), *a) == E.EA_ERR_INVALID_ARG, i
    a = list(args)
    a[9] = need - 256
    assert lib.ea_xa_block_select(ctypes.byref(d), *a) == E.EA_ERR_WORKSPACE


def _ratios_c(d, cu, modes, sparse_mode, pairs):
    nseq, hkv = modes.shape
    msr, esr, rho, pw = np.zeros(nseq + 1), np.zeros(nseq + 1), np.zeros(nseq * hkv), np.zeros(1)
    E.ea_sparsity_ratios(d, np.ascontiguousarray(cu, np.int32), np.ascontiguousarray(modes, np.uint8),
                         sparse_mode, None if pairs is None else np.ascontiguousarray(pairs, np.int64),
                         msr, esr, rho, pw)
    return msr, esr, rho.reshape(nseq, hkv), pw[0]


@pytest.mark.parametrize("seed", range(6))
def test_sparsity_ratios_match_oracle(seed):
    rng = np.random.default_rng(seed)
    nseq = int(rng.integers(1, 6))
    hkv, G = 4, int(rng.choice([1, 2, 4]))
    seqlens = rng.integers(0, 3000, size=nseq)
    modes = rng.integers(0, 3, size=(nseq, hkv)).astype(np.uint8)
    sink, window = int(rng.integers(0, 300)), int(rng.integers(1, 2000))
    pairs = np.zeros((nseq, hkv * G), dtype=np.int64)
    for b in range(nseq):
        causal = int(seqlens[b]) * (int(seqlens[b]) + 1) // 2
        pairs[b] = rng.integers(0, causal + 1, size=hkv * G)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    d = desc(num_seqs=nseq, total_tokens=int(cu[-1]), max_seqlen=max(1, int(seqlens.max())),
             num_q_heads=hkv * G, num_kv_heads=hkv, ssa_sink=sink, ssa_window=window)
    sm = int(rng.integers(0, 3))
    msr, esr, rho, pw = _ratios_c(d, cu, modes, sm, pairs)
    ref = OR.sparsity_ratios(seqlens, modes, hkv * G, sink=sink, window=window, sparse_mode=sm,
                             xa_pairs=pairs)
    np.testing.assert_allclose(msr, ref["msr"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(esr, ref["esr"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(rho, ref["rho"], rtol=0, atol=1e-13)
    assert abs(pw - ref["esr_pairs"]) < 1e-13


def test_sparsity_ratios_rejects_bad_host_data():
    d = desc(num_seqs=2, total_tokens=300, max_seqlen=200)
    modes = np.array([[0, 1, 1, 1, 1, 1, 1, 1], [0, 1, 1, 1, 1, 1, 1, 1]], np.uint8)
    ok_cu = np.array([0, 100, 300], np.int32)
    _ratios_c(d, ok_cu, modes, MODE_SSA, None)
    for cu in ([1, 100, 300], [0, 100, 299], [0, 250, 300], [0, 150, 100]):
        with pytest.raises(E.EaError):
            _ratios_c(d, np.array(cu, np.int32), modes, MODE_SSA, None)
    bad = modes.copy()
    bad[0, 0] = 3
    with pytest.raises(E.EaError):
        _ratios_c(d, ok_cu, bad, MODE_SSA, None)
    xa = modes.copy()
    xa[1, 2] = MODE_XA
    with pytest.raises(E.EaError):                  # XA head but no pair counts
        _ratios_c(d, ok_cu, xa, MODE_SSA, None)
    pairs = np.zeros((2, 32), np.int64)
    pairs[1, 8] = 10 ** 9                           # more pairs than causal
    with pytest.raises(E.EaError):
        _ratios_c(d, ok_cu, xa, MODE_SSA, pairs)


def test_page_fact_ratios_through_c_abi():
    # 10 % of the causal pairs kept -> rho = 0.9 (Eq. 5 worked example).
    L = 1000
    d = desc(num_seqs=1, total_tokens=L, max_seqlen=L, num_q_heads=2, num_kv_heads=2)
    causal = L * (L + 1) // 2
    pairs = np.array([[causal // 10, 0]], np.int64)
    msr, esr, rho, pw = _ratios_c(d, np.array([0, L]), np.array([[MODE_XA, MODE_FA]], np.uint8),
                                  MODE_XA, pairs)
    assert abs(rho[0, 0] - 0.9) < 1e-12 and rho[0, 1] == 0 and msr[0] == 0.5


def _router_desc(**kw):
    base = dict(hidden=512, pool_head=100, pool_tail=100)
    base.update(kw)
    return E.RouterDesc(*([FAKE] * len(E.ROUTER_WEIGHTS)), base["hidden"], base["pool_head"],
                        base["pool_tail"])


def test_route_heads_rejects_bad_arguments():
    L = E.lib()
    d = desc()
    ok = dict(k=FAKE, cu=FAKE, rm=MODE_FA, sm=MODE_SSA, modes=FAKE, logits=FAKE)

    def call(rd, **kw):
        a = dict(ok)
        a.update(kw)
        return L.ea_route_heads(ctypes.byref(d), ctypes.byref(rd) if rd is not None else None,
                                a["k"], a["cu"], a["rm"], a["sm"], a["modes"], a["logits"], None)

    bad = E.EA_ERR_INVALID_ARG
    assert call(None) == bad
    assert call(_router_desc(hidden=0)) == bad
    assert call(_router_desc(hidden=1025)) == bad
    assert call(_router_desc(hidden=1028)) == bad
    assert call(_router_desc(hidden=6)) == bad
    assert call(_router_desc(pool_head=-1)) == bad
    assert call(_router_desc(pool_tail=-1)) == bad
    assert call(_router_desc(), rm=3) == bad
    assert call(_router_desc(), sm=7) == bad
    assert call(_router_desc(), cu=None) == bad
    assert call(_router_desc(), modes=None) == bad
    assert call(_router_desc(), k=None) == bad
    assert call(_router_desc(), k=FAKE + 2) == bad
    assert call(_router_desc(), logits=FAKE + 2) == bad
    rd = _router_desc()
    rd.w3 = None
    assert call(rd) == bad
    rd = _router_desc()
    rd.b4 = FAKE + 1
    assert call(rd) == bad
    rd = _router_desc()
    rd.w2 = FAKE + 4
    assert call(rd) == bad
    # A bad layer descriptor is rejected the same way as by the other calls.
    d = desc(head_dim=96)
    assert call(_router_desc()) == E.EA_ERR_UNSUPPORTED
    # No sequence: nothing to do, nothing touched.
    d = desc(num_seqs=0, total_tokens=0, max_seqlen=0)
    assert call(_router_desc(), modes=None, k=None) == E.EA_OK


def test_decode_rejects_bad_arguments_and_sizes_workspace():
    L = E.lib()
    d = desc()
    need = E.ea_workspace_bytes(d, E.EA_OP_DECODE)
    # fp32 partials: num_seqs * Hq * ceil(max_seqlen / split) * (d + 2) floats, plus
    # metadata and the wave list; 4096 tokens x 8 KV heads / 2048 waves -> split
    # 256, 16 splits
    assert need >= 4 * 1 * 32 * 16 * 130

    def call(dd=None, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, modes=FAKE, o=FAKE, lse=FAKE, ws=FAKE, n=need)
        a.update(kw)
        return L.ea_hybrid_attn_decode(ctypes.byref(dd or d), a["q"], a["k"], a["v"], a["cu"],
                                       a["modes"], a["o"], a["lse"], a["ws"], a["n"], None)

    bad = E.EA_ERR_INVALID_ARG
    for name in ("q", "k", "v", "cu", "modes", "o", "lse"):
        assert call(**{name: None}) == bad, name
    for name in ("q", "k", "v", "o"):
        assert call(**{name: FAKE + 2}) == bad, name
    assert call(lse=FAKE + 2) == bad
    assert call(ws=None) == E.EA_ERR_WORKSPACE
    assert call(n=need - 1) == E.EA_ERR_WORKSPACE
    assert call(desc(num_q_heads=34, num_kv_heads=2)) == E.EA_ERR_UNSUPPORTED   # G = 17
    assert call(desc(head_dim=96)) == E.EA_ERR_UNSUPPORTED
    empty = desc(num_seqs=0, total_tokens=0, max_seqlen=0)
    assert call(empty, q=None, k=None, v=None, o=None, lse=None,
                n=E.ea_workspace_bytes(empty, E.EA_OP_DECODE)) == E.EA_OK
    # More than 2^31 - 1 key-split waves: no workspace size, and the call says so.
    huge = desc(num_seqs=65535, total_tokens=2 ** 31 - 1, max_seqlen=2 ** 31 - 1,
                num_q_heads=16, num_kv_heads=16)
    assert E.ea_workspace_bytes(huge, E.EA_OP_DECODE) == 0
    assert call(huge) == E.EA_ERR_UNSUPPORTED


def test_workspace_sizes_do_not_wrap_near_int32_max():
    # The largest accepted batch (2^31 - 2^16 tokens) in one or two sequences,
    # a sink as long as the cache: every size is an honest upper bound (no
    # int32 wrap in ceil-divisions).
    T = E.EA_MAX_TOKENS
    for kw in (dict(num_seqs=2, num_q_heads=8, num_kv_heads=8),
               dict(num_seqs=1, num_q_heads=32, num_kv_heads=8, ssa_sink=T)):
        d = desc(total_tokens=T, max_seqlen=T, **kw)
        hkv, hq = kw["num_kv_heads"], kw["num_q_heads"]
        pre = E.ea_workspace_bytes(d, E.EA_OP_PREFILL)
        assert 2 * 2 * hkv * 128 * T <= pre < 2 ** 60          # packed K and V^T
        dec = E.ea_workspace_bytes(d, E.EA_OP_DECODE)
        # fp32 partials of splits of at least 512 keys, per (sequence, q-head)
        assert 4 * hq * (T // 4096) * 130 <= dec < 2 ** 40
        assert 0 < E.ea_workspace_bytes(d, E.EA_OP_XA_SELECT) < 2 ** 60


def test_select_rejects_rows_longer_than_12288_blocks():
    # The selector holds a block row in LDS: 12,288 blocks at most.
    lib = E.lib()
    for nb, code in ((12288, E.EA_ERR_WORKSPACE), (12289, E.EA_ERR_UNSUPPORTED)):
        d = desc(total_tokens=nb * 128, max_seqlen=nb * 128, num_seqs=1)
        st = lib.ea_xa_block_select(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                    0, None)
        assert st == code, (nb, st)


def test_token_limit_is_enforced_by_every_call():
    # One token past EA_MAX_TOKENS: every call that takes a descriptor
    # rejects it on the host, before touching a pointer.
    src = open(os.path.join(ROOT, "include", "ea.h")).read()
    m = re.search(r"#define EA_MAX_TOKENS (0x[0-9a-fA-F]+)", src)
    assert m and int(m.group(1), 16) == E.EA_MAX_TOKENS == 2 ** 31 - 2 ** 16
    lib = E.lib()
    ok = desc(total_tokens=E.EA_MAX_TOKENS, max_seqlen=E.EA_MAX_TOKENS, num_seqs=1)
    big = desc(total_tokens=E.EA_MAX_TOKENS + 1, max_seqlen=E.EA_MAX_TOKENS + 1, num_seqs=1)
    for op in (E.EA_OP_XA_SELECT, E.EA_OP_PREFILL, E.EA_OP_DECODE):
        assert E.ea_workspace_bytes(ok, op) > 0
        assert E.ea_workspace_bytes(big, op) == 0
    W = 1 << 62
    assert lib.ea_hybrid_attn_prefill(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                      FAKE, W, None) == E.EA_ERR_UNSUPPORTED
    assert lib.ea_xa_block_select(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                  FAKE, W, None) == E.EA_ERR_UNSUPPORTED
    assert lib.ea_hybrid_attn_plan(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, None, FAKE, W,
                                   None) == E.EA_ERR_UNSUPPORTED
    assert lib.ea_hybrid_attn_run(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, W,
                                  None) == E.EA_ERR_UNSUPPORTED
    assert lib.ea_hybrid_attn_decode(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, W,
                                     None) == E.EA_ERR_UNSUPPORTED
    assert lib.ea_hybrid_attn_decode_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                             None) == E.EA_ERR_UNSUPPORTED
    modes = np.zeros(8, dtype=np.uint8)
    assert lib.ea_hybrid_attn_prefill_serial(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, modes.ctypes.data,
                                             FAKE, FAKE, FAKE, W, None) == E.EA_ERR_UNSUPPORTED
    assert lib.ea_route_heads(ctypes.byref(big), ctypes.byref(_router_desc()), FAKE, FAKE, MODE_FA, MODE_SSA,
                              FAKE, FAKE, None) == E.EA_ERR_UNSUPPORTED
    for fn in (lib.ea_decode_cache_fill, lib.ea_decode_cache_append):
        assert fn(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, 100, FAKE, FAKE, None) == E.EA_ERR_UNSUPPORTED
    assert lib.ea_hybrid_attn_decode_cached(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, 100, FAKE, FAKE, FAKE,
                                            FAKE, FAKE, W, None) == E.EA_ERR_UNSUPPORTED
    seg = np.zeros(9, dtype=np.int64)
    assert lib.ea_decode_cache_layout(ctypes.byref(big), modes.ctypes.data,
                                      np.array([1], dtype=np.int32).ctypes.data,
                                      seg.ctypes.data) == E.EA_ERR_UNSUPPORTED
    cu = np.array([0, E.EA_MAX_TOKENS + 1], dtype=np.int32)
    out = [np.zeros(2), np.zeros(2), np.zeros(8), np.zeros(1)]
    assert lib.ea_sparsity_ratios(ctypes.byref(big), cu.ctypes.data, modes.ctypes.data, MODE_SSA, None,
                                  *[x.ctypes.data for x in out]) == E.EA_ERR_UNSUPPORTED


def test_decode_noalloc_rejects_before_any_device_work():
    # Every case below fails on the host, before the scratch lookup or a launch.
    L = E.lib()
    d = desc()

    def call(dd=None, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, modes=FAKE, o=FAKE, lse=FAKE)
        a.update(kw)
        return L.ea_hybrid_attn_decode_noalloc(ctypes.byref(dd or d), a["q"], a["k"], a["v"],
                                               a["cu"], a["modes"], a["o"], a["lse"], None)

    bad = E.EA_ERR_INVALID_ARG
    for name in ("q", "k", "v", "cu", "modes", "o", "lse"):
        assert call(**{name: None}) == bad, name
    for name in ("q", "k", "v", "o"):
        assert call(**{name: FAKE + 2}) == bad, name
    assert call(desc(num_q_heads=34, num_kv_heads=2)) == E.EA_ERR_UNSUPPORTED
    assert call(desc(head_dim=96)) == E.EA_ERR_UNSUPPORTED
    # A step whose scratch would exceed the library's array is refused:
    # 256 sequences of 64K cached tokens need about 131 MiB of fp32 partials.
    big = desc(num_seqs=256, total_tokens=256 * 65536, max_seqlen=65536)
    assert E.ea_workspace_bytes(big, E.EA_OP_DECODE) > E.EA_DECODE_NOALLOC_SCRATCH_BYTES
    assert call(big) == E.EA_ERR_WORKSPACE
    # The limit is the stated one: 8 sequences of 64K fit.
    fits = desc(num_seqs=8, total_tokens=8 * 65536, max_seqlen=65536)
    assert E.ea_workspace_bytes(fits, E.EA_OP_DECODE) <= E.EA_DECODE_NOALLOC_SCRATCH_BYTES
    # An empty batch has nothing to do.
    empty = desc(num_seqs=0, total_tokens=0, max_seqlen=0)
    assert call(empty, q=None, k=None, v=None, o=None, lse=None) == E.EA_OK


def test_noalloc_scratch_size_matches_header():
    src = open(os.path.join(ROOT, "include", "ea.h")).read()
    m = re.search(r"#define EA_DECODE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == E.EA_DECODE_NOALLOC_SCRATCH_BYTES


def test_serial_dispatch_rejects_before_any_device_work():
    L = E.lib()
    d = desc()
    need = E.ea_workspace_bytes(d, E.EA_OP_PREFILL_SERIAL)
    # Split copies of q, k, v, o and lse, plus one whole-layer prefill workspace.
    T, Hq, Hkv, D = 4096, 32, 8, 128
    assert need >= E.ea_workspace_bytes(d, E.EA_OP_PREFILL) + 2 * T * D * (2 * Hq + 2 * Hkv) + 4 * T * Hq
    modes = np.array([0, 1, 1, 0, 1, 1, 0, 1], dtype=np.uint8)

    def call(dd=None, m=modes, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, o=FAKE, lse=FAKE, ws=FAKE, n=need)
        a.update(kw)
        return L.ea_hybrid_attn_prefill_serial(ctypes.byref(dd or d), a["q"], a["k"], a["v"], a["cu"],
                                               None if m is None else m.ctypes.data, a["o"], a["lse"],
                                               a["ws"], a["n"], None)

    bad = E.EA_ERR_INVALID_ARG
    for name in ("q", "k", "v", "cu", "o", "lse"):
        assert call(**{name: None}) == bad, name
    assert call(m=None) == bad
    for name in ("q", "k", "v", "o"):
        assert call(**{name: FAKE + 8}) == bad, name
    assert call(m=np.array([0, 1, 1, 0, 1, 1, 0, 3], dtype=np.uint8)) == bad
    # The pages' serial baseline splits full and sliding-window heads; XA is not built for it.
    assert call(m=np.array([0, 1, 1, 0, 2, 1, 0, 1], dtype=np.uint8)) == E.EA_ERR_UNSUPPORTED
    assert call(ws=None) == E.EA_ERR_WORKSPACE
    assert call(n=need - 1) == E.EA_ERR_WORKSPACE
    assert call(desc(num_q_heads=512, num_kv_heads=8)) == E.EA_ERR_UNSUPPORTED
    empty = desc(num_seqs=0, total_tokens=0, max_seqlen=0)
    assert call(empty, q=None, k=None, v=None, o=None, lse=None,
                n=E.ea_workspace_bytes(empty, E.EA_OP_PREFILL_SERIAL)) == E.EA_OK


def test_decode_cache_layout_rows():
    # FA and XA segments hold the capacity; SSA segments sink + window rows at most.
    d = desc(num_seqs=3, total_tokens=3 * 1000, max_seqlen=1000, num_kv_heads=2, num_q_heads=4,
             ssa_sink=5, ssa_window=20)
    modes = np.array([0, 1, 1, 2, 1, 1], dtype=np.uint8)
    cap = np.array([1000, 7, 0], dtype=np.int32)
    seg = np.zeros(7, dtype=np.int64)
    E.ea_decode_cache_layout(d, modes, cap, seg)
    assert seg.tolist() == [0, 1000, 1025, 1032, 1039, 1039, 1039]
    with pytest.raises(E.EaError):
        E.ea_decode_cache_layout(d, modes, np.array([1, -1, 0], dtype=np.int32), seg)
    with pytest.raises(E.EaError):
        E.ea_decode_cache_layout(d, np.array([0, 1, 3, 0, 0, 0], dtype=np.uint8), cap, seg)


def test_decode_cache_calls_reject_before_any_device_work():
    L = E.lib()
    d = desc()
    bad = E.EA_ERR_INVALID_ARG
    for fn in (L.ea_decode_cache_fill, L.ea_decode_cache_append):
        def call(**kw):
            a = dict(k=FAKE, v=FAKE, cu=FAKE, modes=FAKE, seg=FAKE, rows=100, kc=FAKE, vc=FAKE)
            a.update(kw)
            return fn(ctypes.byref(d), a["k"], a["v"], a["cu"], a["modes"], a["seg"], a["rows"], a["kc"],
                      a["vc"], None)
        for name in ("k", "v", "cu", "modes", "seg", "kc", "vc"):
            assert call(**{name: None}) == bad, name
        assert call(rows=0) == bad and call(rows=-1) == bad
        assert call(kc=FAKE + 4) == bad
        assert fn(ctypes.byref(desc(num_seqs=9000, total_tokens=9000, max_seqlen=1)), FAKE, FAKE, FAKE,
                  FAKE, FAKE, 100, FAKE, FAKE, None) == E.EA_ERR_UNSUPPORTED
    need = E.ea_workspace_bytes(d, E.EA_OP_DECODE)

    def dec(**kw):
        a = dict(q=FAKE, kc=FAKE, vc=FAKE, seg=FAKE, rows=100, cu=FAKE, modes=FAKE, o=FAKE, lse=FAKE,
                 ws=FAKE, n=need)
        a.update(kw)
        return L.ea_hybrid_attn_decode_cached(ctypes.byref(d), a["q"], a["kc"], a["vc"], a["seg"], a["rows"],
                                              a["cu"], a["modes"], a["o"], a["lse"], a["ws"], a["n"], None)
    for name in ("q", "kc", "vc", "seg", "cu", "modes", "o", "lse"):
        assert dec(**{name: None}) == bad, name
    assert dec(rows=0) == bad
    assert dec(n=need - 1) == E.EA_ERR_WORKSPACE
