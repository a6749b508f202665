"""Workload descriptions for hybrid-head prefill attention.

Shapes follow the attention layers of Llama-3.1-8B and Qwen3-8B (32 query
heads, 8 KV heads, head dim 128) and the 8K-256K length range over which the
Elastic Attention pages evaluate (RULER, Table 11 of the paper-reading pages).
The per-head sparse settings come from the pages' Table 8 (sink/local 128/2048)
and from the XAttention parameters (block 128, stride 8, threshold 0.9) of the
workloads below.  Mode codes: 0 = FA (full causal attention, Eq. 1),
1 = SSA (attention sink + sliding window), 2 = XA (antidiagonal-scored
block-sparse attention).

Nothing here computes attention; these are only sizes, seeds and mode arrays.
"""

from dataclasses import dataclass, replace
from typing import Optional, Tuple

MODE_FA = 0
MODE_SSA = 1
MODE_XA = 2


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block: int
    ssa_sink: int
    ssa_window: int
    xa_stride: int = 8
    tau_num: int = 9
    tau_den: int = 10
    # XA masks: 0 = one per q-head; 1 = one per KV head (group-mean scores).
    xa_group: int = 0
    # XA block masses: 0 = softmax per reduced row then pooled (R2);
    # 1 = softmax over each block row of the raw block sums (R1).
    xa_norm: int = 0
    # Fixed sequence lengths, or None when they are drawn from the seed
    # (ragged batch: `ragged_count` lengths, each block * U{lo..hi}).
    seqlens: Optional[Tuple[int, ...]] = None
    ragged_count: int = 0
    ragged_blocks: Tuple[int, int] = (64, 512)
    # Per-(sequence, KV head) modes; one row per sequence, or a single row
    # broadcast to every sequence.  None means drawn from the seed.
    modes: Optional[Tuple[Tuple[int, ...], ...]] = None
    # Which mode fills the "sparse" slot of the {retrieval}-{sparse} mode set.
    sparse_mode: int = MODE_SSA
    # Drawn-mode settings: target per-sequence model sparsity ratios.
    omega_choices: Tuple[float, ...] = ()
    # Needle placement: "uniform" over all keys, or "clustered" inside
    # `needle_blocks_per_64k` random 128-token blocks per 65,536 keys.
    needle_layout: str = "uniform"
    needle_blocks_per_64k: int = 16
    needle_fraction: float = 0.01
    needle_gain: float = 3.0
    description: str = ""

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(self.head_dim) ** 0.5


def _row(fa=(), xa=(), n=8, rest=MODE_SSA):
    r = [rest] * n
    for h in fa:
        r[h] = MODE_FA
    for h in xa:
        r[h] = MODE_XA
    return (tuple(r),)


CONFIGS = {
    # Tiny single layer: 1 x 1024, 4/2 heads, d 64, modes [FA, SSA].
    "tiny-1k": Config(
        name="tiny-1k", seed=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
        block=64, ssa_sink=64, ssa_window=256, seqlens=(1024,),
        modes=((MODE_FA, MODE_SSA),),
        description="batch 1, seq 1024, 4 q / 2 KV heads, d 64, [FA, SSA], sink 64 window 256, block 64"),
    # Llama-3.1-8B-shaped FA-SSA layer at 16K: FA on KV heads {0,3,6}.
    "llama8b-fassa-16k": Config(
        name="llama8b-fassa-16k", seed=2, num_q_heads=32, num_kv_heads=8,
        head_dim=128, block=128, ssa_sink=128, ssa_window=2048,
        seqlens=(16384,), modes=_row(fa=(0, 3, 6)),
        description="batch 1, seq 16384, 32/8 heads, d 128, 3 FA + 5 SSA (sink 128, window 2048)"),
    # The same layout at 64K: the headline FA-SSA layer.
    "llama8b-fassa-64k": Config(
        name="llama8b-fassa-64k", seed=2, num_q_heads=32, num_kv_heads=8,
        head_dim=128, block=128, ssa_sink=128, ssa_window=2048,
        seqlens=(65536,), modes=_row(fa=(0, 3, 6)),
        description="batch 1, seq 65536, 32/8 heads, d 128, 3 FA + 5 SSA (sink 128, window 2048)"),
    # XA-SSA at 64K with clustered needles.
    "xassa-64k": Config(
        name="xassa-64k", seed=3, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block=128, ssa_sink=128, ssa_window=4096, xa_stride=8,
        seqlens=(65536,), modes=_row(xa=(0, 4)), sparse_mode=MODE_SSA,
        needle_layout="clustered", needle_blocks_per_64k=16,
        description="batch 1, seq 65536, 32/8 heads, d 128, XA {0,4} (block 128, stride 8, tau 0.9) + 6 SSA (sink 128, window 4096)"),
    # The same XA-SSA layer with one XA mask per KV head (group-mean scores).
    "xassa-64k-group": Config(
        name="xassa-64k-group", seed=3, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block=128, ssa_sink=128, ssa_window=4096, xa_stride=8, xa_group=1,
        seqlens=(65536,), modes=_row(xa=(0, 4)), sparse_mode=MODE_SSA,
        needle_layout="clustered", needle_blocks_per_64k=16,
        description="batch 1, seq 65536, 32/8 heads, d 128, XA {0,4} (block 128, stride 8, tau 0.9, one mask per KV head) + 6 SSA (sink 128, window 4096)"),
    # The same XA-SSA layer with the block masses taken from the raw block
    # sums (reading R1, for comparison).
    "xassa-64k-r1": Config(
        name="xassa-64k-r1", seed=3, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block=128, ssa_sink=128, ssa_window=4096, xa_stride=8, xa_norm=1,
        seqlens=(65536,), modes=_row(xa=(0, 4)), sparse_mode=MODE_SSA,
        needle_layout="clustered", needle_blocks_per_64k=16,
        description="batch 1, seq 65536, 32/8 heads, d 128, XA {0,4} (block 128, stride 8, tau 0.9, R1 block sums) + 6 SSA (sink 128, window 4096)"),
    # The same XA-SSA layer with the XA parameters of the pages' Table 8:
    # block 64 and stride 16 (4 reduced rows per block); kernel tiles of 64.
    "xassa-64k-b64s16": Config(
        name="xassa-64k-b64s16", seed=3, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block=64, ssa_sink=128, ssa_window=4096, xa_stride=16,
        seqlens=(65536,), modes=_row(xa=(0, 4)), sparse_mode=MODE_SSA,
        needle_layout="clustered", needle_blocks_per_64k=16,
        description="batch 1, seq 65536, 32/8 heads, d 128, XA {0,4} (block 64, stride 16, tau 0.9) + 6 SSA (sink 128, window 4096)"),
    # Qwen3-8B-shaped 256K prefill, two mode sets over the same tensors.
    "qwen8b-faxa-256k": Config(
        name="qwen8b-faxa-256k", seed=4, num_q_heads=32, num_kv_heads=8,
        head_dim=128, block=128, ssa_sink=128, ssa_window=4096, xa_stride=8,
        seqlens=(262144,), modes=_row(fa=(0, 4), rest=MODE_XA), sparse_mode=MODE_XA,
        needle_layout="clustered", needle_blocks_per_64k=16,
        description="batch 1, seq 262144, 32/8 heads, d 128, FA {0,4} + 6 XA (tau 0.9)"),
    "qwen8b-xassa-256k": Config(
        name="qwen8b-xassa-256k", seed=4, num_q_heads=32, num_kv_heads=8,
        head_dim=128, block=128, ssa_sink=128, ssa_window=4096, xa_stride=8,
        seqlens=(262144,), modes=_row(xa=(0, 4)), sparse_mode=MODE_SSA,
        needle_layout="clustered", needle_blocks_per_64k=16,
        description="batch 1, seq 262144, 32/8 heads, d 128, XA {0,4} + 6 SSA (sink 128, window 4096)"),
    # Ragged per-request routing: 8 sequences of 128 * U{64..512} tokens.
    "ragged-8x": Config(
        name="ragged-8x", seed=5, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block=128, ssa_sink=128, ssa_window=2048, xa_stride=8,
        ragged_count=8, ragged_blocks=(64, 512), modes=None, sparse_mode=MODE_SSA,
        omega_choices=(0.63, 0.68, 0.82, 0.85),
        description="8 sequences, lengths 128*U{64..512}, 32/8 heads, d 128; per-sequence modes with "
                    "Omega_MSR in {0.63,0.68,0.82,0.85}; retrieval heads alternate FA/XA, rest SSA (window 2048)"),
}


def get_config(name: str) -> Config:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown config {name!r}; known: {sorted(CONFIGS)}") from None
