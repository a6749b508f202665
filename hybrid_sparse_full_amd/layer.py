"""Device-memory plumbing around the C ABI: one hybrid-head prefill layer.

`HybridPrefill` owns the workspaces and output buffers (torch tensors, so
torch's caching allocator provides device memory and streams) and calls the
device entry points in order: optionally ea_route_heads (modes written on the
device by the attention router), ea_xa_block_select when some head can be
XA, then ea_hybrid_attn_prefill.  `Router` holds the router weights on the
device.  All arithmetic happens inside libea.so.
"""

import math

import numpy as np
import torch

from . import ea as E


def make_desc(*, num_seqs, total_tokens, max_seqlen, num_q_heads, num_kv_heads, head_dim,
              block, softmax_scale=None, ssa_sink=128, ssa_window=2048, xa_stride=8,
              xa_tau=(9, 10), xa_group=0, xa_norm=0):
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    return E.AttnDesc(int(num_seqs), int(total_tokens), int(max_seqlen), int(num_q_heads),
                      int(num_kv_heads), int(head_dim), int(block), float(softmax_scale),
                      int(ssa_sink), int(ssa_window), int(xa_stride), int(xa_tau[0]),
                      int(xa_tau[1]), int(xa_group), int(xa_norm))


class Router:
    """The attention router's weights on the device and the ea_router_desc
    that points at them.  `weights` maps w1, b1, w2, b2, w3, b3, w4, b4 to
    arrays of shape [d, H], [H], [H, d], [d], [2d, H], [H], [H, 2], [2]."""

    def __init__(self, weights, device="cuda", pool_head=100, pool_tail=100):
        self.device = torch.device(device)
        self.t = {n: torch.from_numpy(np.ascontiguousarray(weights[n], dtype=np.float32)).to(self.device)
                  for n in E.ROUTER_WEIGHTS}
        self.hidden = int(self.t["w1"].shape[1])
        self.desc = E.RouterDesc(*[self.t[n].data_ptr() for n in E.ROUTER_WEIGHTS],
                                 self.hidden, int(pool_head), int(pool_tail))

    def __call__(self, attn_desc, k, cu_seqlens, retrieval_mode, sparse_mode, modes_out,
                 logits_out=None, stream=None):
        E.ea_route_heads(attn_desc, self.desc, k, cu_seqlens, retrieval_mode, sparse_mode,
                         modes_out, logits_out, stream)


class HybridPrefill:
    """One layer's buffers for a fixed descriptor.

    cu_seqlens and modes are given as host numpy arrays; they are copied to
    the device once here (the C ABI reads them on the device).  With
    modes=None the modes are left to `route` (the attention router writes
    them on the device); `mode_set` = (retrieval mode, sparse mode) then says
    which modes it may write.
    """

    def __init__(self, desc, cu_seqlens, modes, device="cuda", block_mass=False, mode_set=None):
        self.desc = desc
        self.device = torch.device(device)
        self.cu_host = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        self.cu = torch.from_numpy(self.cu_host).to(self.device)
        self.mode_set = tuple(int(x) for x in mode_set) if mode_set is not None else None
        if modes is None:
            if self.mode_set is None:
                raise ValueError("modes=None needs mode_set=(retrieval_mode, sparse_mode)")
            self.modes_host = None
            self.modes = torch.zeros(desc.num_seqs * desc.num_kv_heads, dtype=torch.uint8,
                                     device=self.device)
            self.has_xa = E.EA_MODE_XA in self.mode_set
        else:
            self.modes_host = np.ascontiguousarray(modes, dtype=np.uint8)
            self.modes = torch.from_numpy(self.modes_host.reshape(-1)).to(self.device)
            self.has_xa = bool((self.modes_host == E.EA_MODE_XA).any())
        T, Hq, D = desc.total_tokens, desc.num_q_heads, desc.head_dim
        self.o = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=self.device)
        self.lse = torch.empty((Hq, T), dtype=torch.float32, device=self.device)
        self.ws_prefill = torch.empty(E.ea_workspace_bytes(desc, E.EA_OP_PREFILL),
                                      dtype=torch.uint8, device=self.device)
        self.rows = E.ea_mask_rows(desc)
        self.words = E.ea_mask_words(desc)
        self.maxqb = -(-desc.max_seqlen // desc.block)
        self.mask = self.row_count = self.xa_pairs = self.block_mass = self.ws_select = None
        if self.has_xa:
            self.ws_select = torch.empty(E.ea_workspace_bytes(desc, E.EA_OP_XA_SELECT),
                                         dtype=torch.uint8, device=self.device)
            self.mask = torch.empty((self.rows, self.words), dtype=torch.int32, device=self.device)
            self.row_count = torch.empty(self.rows, dtype=torch.int32, device=self.device)
            self.xa_pairs = torch.empty(desc.num_seqs * Hq, dtype=torch.int64, device=self.device)
            if block_mass:
                self.block_mass = torch.zeros((self.rows, self.maxqb), dtype=torch.float32,
                                              device=self.device)

    def route(self, router, k, logits_out=None, stream=None):
        """Modes from the attention router, written on the device."""
        if self.mode_set is None:
            raise ValueError("route() needs mode_set=(retrieval_mode, sparse_mode)")
        router(self.desc, k, self.cu, self.mode_set[0], self.mode_set[1], self.modes,
               logits_out, stream)

    def device_modes(self):
        """The modes the kernels read, copied back to the host [num_seqs, Hkv]."""
        return self.modes.cpu().numpy().reshape(self.desc.num_seqs, self.desc.num_kv_heads)

    def select(self, q, k, stream=None):
        E.ea_xa_block_select(self.desc, q, k, self.cu, self.modes, self.mask, self.row_count,
                             self.xa_pairs, self.block_mass, self.ws_select, stream)

    def prefill(self, q, k, v, stream=None):
        E.ea_hybrid_attn_prefill(self.desc, q, k, v, self.cu, self.modes,
                                 self.mask if self.has_xa else None, self.o, self.lse,
                                 self.ws_prefill, stream)

    def plan(self, k, v, stream=None):
        E.ea_hybrid_attn_plan(self.desc, k, v, self.cu, self.modes,
                              self.mask if self.has_xa else None, self.ws_prefill, stream)

    def run(self, q, stream=None):
        E.ea_hybrid_attn_run(self.desc, q, self.modes, self.o, self.lse, self.ws_prefill, stream)

    def __call__(self, q, k, v, stream=None):
        if self.has_xa:
            self.select(q, k, stream)
        self.prefill(q, k, v, stream)
        return self.o, self.lse

    def ratios(self, sparse_mode):
        """Omega_MSR / Omega_ESR / rho on the host (needs the XA pair counts)."""
        modes_host = self.modes_host if self.modes_host is not None else self.device_modes()
        nseq, hkv = modes_host.shape
        msr = np.zeros(nseq + 1)
        esr = np.zeros(nseq + 1)
        rho = np.zeros(nseq * hkv)
        pw = np.zeros(1)
        pairs = None
        if self.has_xa:
            pairs = np.ascontiguousarray(self.xa_pairs.cpu().numpy())
        E.ea_sparsity_ratios(self.desc, self.cu_host, np.ascontiguousarray(modes_host), sparse_mode, pairs,
                             msr, esr, rho, pw)
        return dict(msr=msr, esr=esr, rho=rho.reshape(nseq, hkv), esr_pairs=float(pw[0]))


class HybridDecode:
    """Buffers of one decode step for a fixed descriptor: the descriptor
    describes the cache (cu_seqlens over the cached tokens, the current token
    included); q holds one new query per sequence."""

    def __init__(self, desc, cu_seqlens, modes, device="cuda"):
        self.desc = desc
        self.device = torch.device(device)
        self.cu = torch.from_numpy(np.ascontiguousarray(cu_seqlens, dtype=np.int32)).to(self.device)
        self.modes = torch.from_numpy(np.ascontiguousarray(modes, dtype=np.uint8).reshape(-1)).to(self.device)
        nseq, Hq, D = desc.num_seqs, desc.num_q_heads, desc.head_dim
        self.o = torch.empty((nseq, Hq, D), dtype=torch.bfloat16, device=self.device)
        self.lse = torch.empty((nseq, Hq), dtype=torch.float32, device=self.device)
        self.ws = torch.empty(max(1, E.ea_workspace_bytes(desc, E.EA_OP_DECODE)), dtype=torch.uint8,
                              device=self.device)

    def __call__(self, q, k, v, stream=None):
        E.ea_hybrid_attn_decode(self.desc, q, k, v, self.cu, self.modes, self.o, self.lse, self.ws,
                                stream)
        return self.o, self.lse


def bf16_tensor(bits, device):
    """uint16 bf16 bit patterns (numpy) -> torch bfloat16 on `device`."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def desc_for(cfg, seqlens):
    return make_desc(num_seqs=len(seqlens), total_tokens=int(np.sum(seqlens)),
                     max_seqlen=int(np.max(seqlens)) if len(seqlens) else 0,
                     num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads,
                     head_dim=cfg.head_dim, block=cfg.block, softmax_scale=cfg.softmax_scale,
                     ssa_sink=cfg.ssa_sink, ssa_window=cfg.ssa_window, xa_stride=cfg.xa_stride,
                     xa_tau=(cfg.tau_num, cfg.tau_den), xa_group=cfg.xa_group,
                     xa_norm=cfg.xa_norm)


class SegmentedDecodeCache:
    """Decode cache in which SSA heads keep only their sink and window keys
    (ea_decode_cache_layout / _fill / _append, ea_hybrid_attn_decode_cached).

    `capacity` (host, int32 [num_seqs]) is the length each sequence may reach;
    `modes` (host, [num_seqs, Hkv]) are the routing decisions the layout is
    built for.  The pools are [rows, d] bf16 for k and for v.
    """

    def __init__(self, desc, modes, capacity, device="cuda"):
        self.device = torch.device(device)
        self.desc = desc
        self.modes_host = np.ascontiguousarray(modes, dtype=np.uint8).reshape(-1)
        self.capacity = np.ascontiguousarray(capacity, dtype=np.int32)
        self.seg_host = np.zeros(self.modes_host.size + 1, dtype=np.int64)
        E.ea_decode_cache_layout(desc, self.modes_host, self.capacity, self.seg_host)
        self.rows = int(self.seg_host[-1])
        self.seg = torch.from_numpy(self.seg_host).to(self.device)
        self.modes = torch.from_numpy(self.modes_host).to(self.device)
        D = desc.head_dim
        self.k = torch.zeros((max(self.rows, 1), D), dtype=torch.bfloat16, device=self.device)
        self.v = torch.zeros((max(self.rows, 1), D), dtype=torch.bfloat16, device=self.device)

    def nbytes(self):
        return 2 * self.rows * self.desc.head_dim * 2

    def fill(self, desc, k, v, cu_seqlens_dev, stream=None):
        """From a packed [T, Hkv, d] k / v described by desc / cu_seqlens."""
        E.ea_decode_cache_fill(desc, k, v, cu_seqlens_dev, self.modes, self.seg, self.rows, self.k, self.v,
                               stream)

    def append(self, desc, k_new, v_new, cu_seqlens_dev, stream=None):
        """One token per sequence; desc / cu_seqlens give the lengths after it."""
        E.ea_decode_cache_append(desc, k_new, v_new, cu_seqlens_dev, self.modes, self.seg, self.rows,
                                 self.k, self.v, stream)

    def decode(self, desc, q, cu_seqlens_dev, o_out, lse_out, workspace, stream=None):
        E.ea_hybrid_attn_decode_cached(desc, q, self.k, self.v, self.seg, self.rows, cu_seqlens_dev,
                                       self.modes, o_out, lse_out, workspace, stream)
