"""ctypes binding of libea.so (include/ea.h), argument marshalling only.

Each function here has the name of the C entry point it wraps and does
nothing but convert arguments: torch tensors become raw pointers (data_ptr),
the stream defaults to torch's current stream, and a status other than EA_OK
raises EaError.  Every step of the computation runs in the HIP library.
There is no fallback: if libea.so is missing, loading it raises.
"""

import ctypes
import os

EA_OK = 0
EA_ERR_INVALID_ARG = 1
EA_ERR_UNSUPPORTED = 2
EA_ERR_WORKSPACE = 3
EA_ERR_HIP = 4

EA_MODE_FA = 0
EA_MODE_SSA = 1
EA_MODE_XA = 2

EA_OP_XA_SELECT = 0
EA_OP_PREFILL = 1
EA_OP_DECODE = 2
EA_OP_PREFILL_SERIAL = 3

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libea.so")

# Every symbol include/ea.h declares.
EXPORTS = (
    "ea_workspace_bytes", "ea_mask_rows", "ea_mask_words", "ea_workspace_offset",
    "ea_xa_block_select", "ea_hybrid_attn_prefill", "ea_hybrid_attn_plan", "ea_hybrid_attn_run",
    "ea_sparsity_ratios", "ea_route_heads", "ea_hybrid_attn_decode",
    "ea_hybrid_attn_decode_noalloc", "ea_hybrid_attn_prefill_serial", "ea_decode_cache_layout",
    "ea_decode_cache_fill", "ea_decode_cache_append", "ea_hybrid_attn_decode_cached",
    "ea_status_string",
)

# Size of the library-owned scratch of ea_hybrid_attn_decode_noalloc.
EA_DECODE_NOALLOC_SCRATCH_BYTES = 64 << 20
EA_MAX_TOKENS = 0x7FFF0000

# Router weight arrays in ea_router_desc order: Task MLP (w1, b1, w2, b2),
# Router MLP (w3, b3, w4, b4); fp32, row-major [in][out].
ROUTER_WEIGHTS = ("w1", "b1", "w2", "b2", "w3", "b3", "w4", "b4")


class EaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("block", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("ssa_sink", ctypes.c_int32), ("ssa_window", ctypes.c_int32),
        ("xa_stride", ctypes.c_int32), ("xa_tau_num", ctypes.c_int32),
        ("xa_tau_den", ctypes.c_int32), ("xa_group", ctypes.c_int32), ("xa_norm", ctypes.c_int32),
    ]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class RouterDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ROUTER_WEIGHTS] + [
        ("hidden", ctypes.c_int32), ("pool_head", ctypes.c_int32), ("pool_tail", ctypes.c_int32),
    ]


_lib = None


def lib():
    """Load libea.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m hybrid_sparse_full_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    D = ctypes.POINTER(AttnDesc)
    L.ea_workspace_bytes.argtypes = [D, ctypes.c_int]
    L.ea_workspace_bytes.restype = ctypes.c_size_t
    L.ea_mask_rows.argtypes = [D]
    L.ea_mask_rows.restype = ctypes.c_int64
    L.ea_mask_words.argtypes = [D]
    L.ea_mask_words.restype = ctypes.c_int32
    L.ea_workspace_offset.argtypes = [D, ctypes.c_int, ctypes.c_char_p]
    L.ea_workspace_offset.restype = ctypes.c_int64
    L.ea_xa_block_select.argtypes = [D, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.ea_xa_block_select.restype = ctypes.c_int
    L.ea_hybrid_attn_prefill.argtypes = [D, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.ea_hybrid_attn_prefill.restype = ctypes.c_int
    L.ea_hybrid_attn_plan.argtypes = [D, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.ea_hybrid_attn_plan.restype = ctypes.c_int
    L.ea_hybrid_attn_run.argtypes = [D, P, P, P, P, P, ctypes.c_size_t, P]
    L.ea_hybrid_attn_run.restype = ctypes.c_int
    L.ea_sparsity_ratios.argtypes = [D, P, P, ctypes.c_uint8, P, P, P, P, P]
    L.ea_sparsity_ratios.restype = ctypes.c_int
    L.ea_route_heads.argtypes = [D, ctypes.POINTER(RouterDesc), P, P, ctypes.c_uint8, ctypes.c_uint8,
                                 P, P, P]
    L.ea_route_heads.restype = ctypes.c_int
    L.ea_hybrid_attn_decode.argtypes = [D, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.ea_hybrid_attn_decode.restype = ctypes.c_int
    L.ea_hybrid_attn_decode_noalloc.argtypes = [D, P, P, P, P, P, P, P, P]
    L.ea_hybrid_attn_decode_noalloc.restype = ctypes.c_int
    L.ea_hybrid_attn_prefill_serial.argtypes = [D, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.ea_hybrid_attn_prefill_serial.restype = ctypes.c_int
    L.ea_decode_cache_layout.argtypes = [D, P, P, P]
    L.ea_decode_cache_layout.restype = ctypes.c_int
    L.ea_decode_cache_fill.argtypes = [D, P, P, P, P, P, ctypes.c_int64, P, P, P]
    L.ea_decode_cache_fill.restype = ctypes.c_int
    L.ea_decode_cache_append.argtypes = [D, P, P, P, P, P, ctypes.c_int64, P, P, P]
    L.ea_decode_cache_append.restype = ctypes.c_int
    L.ea_hybrid_attn_decode_cached.argtypes = [D, P, P, P, P, ctypes.c_int64, P, P, P, P, P,
                                               ctypes.c_size_t, P]
    L.ea_hybrid_attn_decode_cached.restype = ctypes.c_int
    L.ea_status_string.argtypes = [ctypes.c_int]
    L.ea_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def _ptr(x):
    """Raw address of a tensor / numpy array / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t):
    return t.numel() * t.element_size()


def status_string(status):
    return lib().ea_status_string(int(status)).decode()


def ea_workspace_bytes(desc, op):
    return int(lib().ea_workspace_bytes(ctypes.byref(desc), int(op)))


def ea_mask_rows(desc):
    return int(lib().ea_mask_rows(ctypes.byref(desc)))


def ea_mask_words(desc):
    return int(lib().ea_mask_words(ctypes.byref(desc)))


def ea_workspace_offset(desc, op, name):
    return int(lib().ea_workspace_offset(ctypes.byref(desc), int(op), name.encode()))


def ea_xa_block_select(desc, q, k, cu_seqlens, modes, mask_out, row_count_out, xa_pairs_out,
                       block_mass_out, workspace, stream=None):
    st = lib().ea_xa_block_select(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(cu_seqlens), _ptr(modes), _ptr(mask_out),
        _ptr(row_count_out), _ptr(xa_pairs_out), _ptr(block_mass_out), _ptr(workspace),
        _nbytes(workspace) if workspace is not None else 0, _stream(stream))
    if st != EA_OK:
        raise EaError(st, "ea_xa_block_select")


def ea_hybrid_attn_prefill(desc, q, k, v, cu_seqlens, modes, xa_mask, o_out, lse_out, workspace,
                           stream=None):
    st = lib().ea_hybrid_attn_prefill(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), _ptr(modes),
        _ptr(xa_mask), _ptr(o_out), _ptr(lse_out), _ptr(workspace),
        _nbytes(workspace) if workspace is not None else 0, _stream(stream))
    if st != EA_OK:
        raise EaError(st, "ea_hybrid_attn_prefill")


def ea_hybrid_attn_plan(desc, k, v, cu_seqlens, modes, xa_mask, workspace, stream=None):
    st = lib().ea_hybrid_attn_plan(
        ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(cu_seqlens), _ptr(modes), _ptr(xa_mask),
        _ptr(workspace), _nbytes(workspace) if workspace is not None else 0, _stream(stream))
    if st != EA_OK:
        raise EaError(st, "ea_hybrid_attn_plan")


def ea_hybrid_attn_run(desc, q, modes, o_out, lse_out, workspace, stream=None):
    st = lib().ea_hybrid_attn_run(
        ctypes.byref(desc), _ptr(q), _ptr(modes), _ptr(o_out), _ptr(lse_out), _ptr(workspace),
        _nbytes(workspace) if workspace is not None else 0, _stream(stream))
    if st != EA_OK:
        raise EaError(st, "ea_hybrid_attn_run")


def ea_hybrid_attn_prefill_serial(desc, q, k, v, cu_seqlens, layer_modes_host, o_out, lse_out,
                                  workspace, stream=None):
    """layer_modes_host: numpy uint8 [num_kv_heads] (host memory)."""
    st = lib().ea_hybrid_attn_prefill_serial(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), _ptr(layer_modes_host),
        _ptr(o_out), _ptr(lse_out), _ptr(workspace),
        _nbytes(workspace) if workspace is not None else 0, _stream(stream))
    if st != EA_OK:
        raise EaError(st, "ea_hybrid_attn_prefill_serial")


def ea_sparsity_ratios(desc, cu_seqlens_host, modes_host, sparse_mode, xa_pairs_host,
                       msr_out, esr_out, rho_out, esr_pair_weighted_out=None):
    """Host arrays (numpy, C-contiguous) in and out."""
    st = lib().ea_sparsity_ratios(
        ctypes.byref(desc), _ptr(cu_seqlens_host), _ptr(modes_host), int(sparse_mode),
        _ptr(xa_pairs_host), _ptr(msr_out), _ptr(esr_out), _ptr(rho_out),
        _ptr(esr_pair_weighted_out))
    if st != EA_OK:
        raise EaError(st, "ea_sparsity_ratios")


def ea_route_heads(desc, router_desc, k, cu_seqlens, retrieval_mode, sparse_mode, modes_out,
                   logits_out=None, stream=None):
    st = lib().ea_route_heads(
        ctypes.byref(desc), ctypes.byref(router_desc) if router_desc is not None else None,
        _ptr(k), _ptr(cu_seqlens), int(retrieval_mode), int(sparse_mode), _ptr(modes_out),
        _ptr(logits_out), _stream(stream))
    if st != EA_OK:
        raise EaError(st, "ea_route_heads")


def ea_hybrid_attn_decode(desc, q, k, v, cu_seqlens, modes, o_out, lse_out, workspace, stream=None):
    st = lib().ea_hybrid_attn_decode(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), _ptr(modes), _ptr(o_out),
        _ptr(lse_out), _ptr(workspace), _nbytes(workspace) if workspace is not None else 0,
        _stream(stream))
    if st != EA_OK:
        raise EaError(st, "ea_hybrid_attn_decode")


def ea_hybrid_attn_decode_noalloc(desc, q, k, v, cu_seqlens, modes, o_out, lse_out, stream=None):
    st = lib().ea_hybrid_attn_decode_noalloc(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), _ptr(modes), _ptr(o_out),
        _ptr(lse_out), _stream(stream))
    if st != EA_OK:
        raise EaError(st, "ea_hybrid_attn_decode_noalloc")


def ea_decode_cache_layout(desc, modes_host, capacity_host, seg_off_out):
    """Host arrays: modes uint8 [num_seqs*Hkv], capacity int32 [num_seqs],
    seg_off_out int64 [num_seqs*Hkv + 1] (written)."""
    st = lib().ea_decode_cache_layout(ctypes.byref(desc), _ptr(modes_host), _ptr(capacity_host),
                                      _ptr(seg_off_out))
    if st != EA_OK:
        raise EaError(st, "ea_decode_cache_layout")


def ea_decode_cache_fill(desc, k, v, cu_seqlens, modes, seg_off, cache_rows, k_cache, v_cache,
                         stream=None):
    st = lib().ea_decode_cache_fill(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(cu_seqlens), _ptr(modes),
                                    _ptr(seg_off), int(cache_rows), _ptr(k_cache), _ptr(v_cache),
                                    _stream(stream))
    if st != EA_OK:
        raise EaError(st, "ea_decode_cache_fill")


def ea_decode_cache_append(desc, k_new, v_new, cu_seqlens, modes, seg_off, cache_rows, k_cache,
                           v_cache, stream=None):
    st = lib().ea_decode_cache_append(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(cu_seqlens),
                                      _ptr(modes), _ptr(seg_off), int(cache_rows), _ptr(k_cache),
                                      _ptr(v_cache), _stream(stream))
    if st != EA_OK:
        raise EaError(st, "ea_decode_cache_append")


def ea_hybrid_attn_decode_cached(desc, q, k_cache, v_cache, seg_off, cache_rows, cu_seqlens, modes,
                                 o_out, lse_out, workspace, stream=None):
    st = lib().ea_hybrid_attn_decode_cached(
        ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seg_off), int(cache_rows),
        _ptr(cu_seqlens), _ptr(modes), _ptr(o_out), _ptr(lse_out), _ptr(workspace),
        _nbytes(workspace) if workspace is not None else 0, _stream(stream))
    if st != EA_OK:
        raise EaError(st, "ea_hybrid_attn_decode_cached")
