"""Seeded synthetic inputs for paged KV-cache attention.

This module builds the inputs that both the GPU library and the CPU oracle
consume: request lengths, shuffled physical-block pools, block tables, slot
mappings and the q/K/V values.  It holds none of the attention arithmetic and
imports neither the GPU library nor the oracle.

Shapes and distributions follow the workloads on the source pages:
  * lengths: truncated lognormal, the "ShareGPT-like" synthetic shape the
    lecture simulators use (Lecture 16 "LLM Serving (1)", §0.4; Lecture 7
    "KV Cache Management", §3.3 and §4.4, final length mean 493);
  * physical blocks handed out from a pool in a seeded random order, so
    logically adjacent blocks are physically scattered (Lecture 7 §4.1);
  * block size 16, the default the pages settle on (Lecture 7 §4.4, Month 2
    "PagedAttention" §5.3).
No public dataset is read; these generators stand in for the ShareGPT-style
traces the pages cite.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

__all__ = [
    "lognormal_lengths", "shuffled_block_ids", "assign_block_tables", "slots_for_positions",
    "normal_f32", "round_to_bf16_bits", "bf16_bits_to_f32", "PagedLayout", "build_paged_layout",
    "kv_bytes_per_token", "block_bytes",
]


def lognormal_lengths(n: int, median: float, sigma: float, lo: int, hi: int, seed: int) -> np.ndarray:
    """n lengths ~ round(LogNormal(ln median, sigma)) clipped to [lo, hi] (int32)."""
    rng = np.random.default_rng(seed)
    x = rng.lognormal(mean=math.log(median), sigma=sigma, size=n)
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


def shuffled_block_ids(num_blocks: int, seed: int) -> np.ndarray:
    """A seeded random permutation of 0..num_blocks-1 (the free-list order)."""
    rng = np.random.default_rng(seed)
    return rng.permutation(num_blocks).astype(np.int32)


def assign_block_tables(seq_lens, block_size: int, free_ids: np.ndarray,
                        max_blocks_per_seq: Optional[int] = None) -> np.ndarray:
    """Give each sequence ceil(len / block_size) blocks, taken in order from free_ids.

    Returns int32 [B, max_blocks_per_seq]; unused entries are -1.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    need = (seq_lens + block_size - 1) // block_size
    width = int(max(int(need.max()) if len(need) else 0, 1)) if max_blocks_per_seq is None else max_blocks_per_seq
    if int(need.sum()) > len(free_ids):
        raise ValueError("pool too small: need %d blocks, have %d" % (int(need.sum()), len(free_ids)))
    tables = np.full((len(seq_lens), width), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(need):
        if n > width:
            raise ValueError("sequence %d needs %d blocks > table width %d" % (b, n, width))
        tables[b, :n] = free_ids[k:k + n]
        k += int(n)
    return tables


def slots_for_positions(table_row, positions, block_size: int) -> np.ndarray:
    """Slot ids (block * block_size + offset) for token positions of one sequence (int64)."""
    positions = np.asarray(positions, dtype=np.int64)
    table_row = np.asarray(table_row, dtype=np.int64)
    return table_row[positions // block_size] * block_size + positions % block_size


def normal_f32(shape, std: float, seed: int) -> np.ndarray:
    """i.i.d. N(0, std^2) float32 values from a seeded PCG64 stream."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16, round-to-nearest-even; returns the uint16 bit patterns.

    Input preparation only (the inputs are *defined* as these bf16 values).
    Inputs here are finite normal draws, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """K and V bytes one token occupies over all layers (Month 2 "PagedAttention" §2.1)."""
    return 2 * num_layers * num_kv_heads * head_dim * dtype_bytes


def block_bytes(block_size: int, num_kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """K plus V bytes of one physical block of one layer (Month 2 "PagedAttention" §5.2)."""
    return block_size * num_kv_heads * head_dim * dtype_bytes * 2


def swap_time_model(tokens: int, block_size: int, layers: int, kv_heads: int, head_dim: int, dtype_bytes: int,
                    bytes_per_s: float, per_copy_s: float):
    """The per-copy swap cost model (Lecture 7 "KV Cache Management" §6.2): every layer's K and V
    blocks are separate copies, each costing a fixed overhead plus its bytes over the link.
    Returns (copies, bytes per copy, seconds for one direction)."""
    blocks = -(-tokens // block_size)
    copies = layers * 2 * blocks
    per_copy = block_size * kv_heads * head_dim * dtype_bytes
    return copies, per_copy, copies * (per_copy_s + per_copy / bytes_per_s)


@dataclass
class PagedLayout:
    """Where every sequence's tokens live: lengths, block tables and the pool size."""
    seq_lens: np.ndarray          # int32 [B]
    block_tables: np.ndarray      # int32 [B, max_blocks_per_seq], -1 = unused
    num_blocks: int
    block_size: int
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.batch else 0


def build_paged_layout(seq_lens, block_size: int, seed: int, pool_factor: float = 1.25,
                       num_blocks: Optional[int] = None) -> PagedLayout:
    """Lengths -> shuffled pool of ceil(pool_factor * needed) blocks -> block tables."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    need = int(((seq_lens.astype(np.int64) + block_size - 1) // block_size).sum())
    if num_blocks is None:
        num_blocks = max(int(math.ceil(pool_factor * need)), 1)
    ids = shuffled_block_ids(num_blocks, seed)
    tables = assign_block_tables(seq_lens, block_size, ids)
    return PagedLayout(seq_lens=seq_lens, block_tables=tables, num_blocks=num_blocks,
                       block_size=block_size)
