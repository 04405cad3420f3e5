"""The synthetic workloads, seeded, shaped like the pages' examples.

  tiny_decode        4 sequences of {17, 64, 100, 203} tokens, Hq 8 / Hkv 2,
                     head_dim 64, fp32, 64 physical blocks in a seeded order.
  llama8b_decode     Llama-3.1-8B-shaped layer (Hq 32, Hkv 8, head_dim 128,
                     bf16), 64 sequences, truncated-lognormal lengths (median
                     390, clipped to [16, 4096]), shuffled pool 1.25x needed.
  shared_prefix      16 prompts x 512 tokens, 8 samples each sharing the
                     prompt blocks, 0-256 private tokens per sample, one new
                     token per sample; a 500-token prompt variant exercises
                     copy-on-write.
  llama70b_long      Llama-3.1-70B-shaped layer (Hq 64, Hkv 8), 8 sequences of
                     32768 tokens, split-K over 512-token partitions.
  llama70b_one_long  the same layer, one sequence of 131072 tokens: eight rows
                     cut into dozens of pieces each.
  chunked_prefill    16 sequences, 1024 cached tokens + a 512-token chunk.

Length model: the pages' lecture simulators use ShareGPT-like truncated
lognormal lengths (Lecture 16 "LLM Serving (1)" §0.4) with a final-length
mean of 493 (Lecture 7 "KV Cache Management" §4.4).  With median 390 the
lognormal sigma follows from mean = median * exp(sigma^2 / 2).

Values are i.i.d. normal; bf16 inputs are the round-to-nearest-even bf16 of
the fp32 draws.  Small problems draw on the host (numpy PCG64); the large
ones draw on the device (torch's generator on the GPU) and copy whatever the
oracle needs back to the host.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

from . import (PagedLayout, build_paged_layout, lognormal_lengths, normal_f32, round_to_bf16_bits,
               shuffled_block_ids, slots_for_positions)
from .block_manager import BlockManager

SIGMA_8B = math.sqrt(2.0 * math.log(493.0 / 390.0))


@dataclass
class DecodeWorkload:
    name: str
    layout: PagedLayout
    num_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str            # "f32" or "bf16"
    std: float
    seed: int
    partition_size: int = 0
    copies: List[Tuple[int, int]] = field(default_factory=list)   # CoW pairs, if any
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def block_size(self) -> int:
        return self.layout.block_size

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def cache_shape(self):
        return (self.layout.num_blocks, self.num_kv_heads, self.layout.block_size, self.head_dim)

    def q_shape(self):
        return (self.layout.batch, self.num_heads, self.head_dim)

    def kv_bytes(self) -> int:
        """Bytes of valid K and V rows (padding slots of last blocks excluded)."""
        return int(self.layout.seq_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * 2 * self.elem_bytes

    def algorithmic_bytes(self, out_bytes: int = 4) -> int:
        """K/V rows + q + out + the block-table entries read + seq_lens."""
        B = self.layout.batch
        nblk = (self.layout.seq_lens.astype(np.int64) + self.block_size - 1) // self.block_size
        return (self.kv_bytes() + B * self.num_heads * self.head_dim * (self.elem_bytes + out_bytes)
                + 4 * int(nblk.sum()) + 4 * B)

    def flops(self) -> int:
        return 4 * int(self.layout.seq_lens.astype(np.int64).sum()) * self.num_heads * self.head_dim


@dataclass
class PrefillWorkload:
    name: str
    layout: PagedLayout          # seq_lens = prefix + chunk
    chunk_lens: np.ndarray       # int32 [B]
    num_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    std: float
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def query_start_loc(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.chunk_lens)]).astype(np.int32)

    @property
    def num_query_tokens(self) -> int:
        return int(self.chunk_lens.sum())

    def chunk_slots(self) -> np.ndarray:
        """Slots of every chunk token, in query order (int64)."""
        out = []
        for b in range(self.layout.batch):
            S, n = int(self.layout.seq_lens[b]), int(self.chunk_lens[b])
            out.append(slots_for_positions(self.layout.block_tables[b], np.arange(S - n, S), self.layout.block_size))
        return np.concatenate(out).astype(np.int64)

    def flops(self) -> int:
        """Exact causal count: every (row, visible key) pair costs 4*D flops per query head."""
        keys = 0
        for S, n in zip(self.layout.seq_lens.astype(np.int64), self.chunk_lens.astype(np.int64)):
            keys += int(n * (S - n) + n * (n + 1) // 2)
        return 4 * keys * self.num_heads * self.head_dim


# ----------------------------------------------------------------------------- the configurations
def tiny_decode() -> DecodeWorkload:
    lay = build_paged_layout([17, 64, 100, 203], 16, seed=1, num_blocks=64)
    return DecodeWorkload("tiny_decode_fp32", lay, 8, 2, 64, "f32", 1.0, seed=1)


def llama8b_decode(batch: int = 64, seed: int = 2, block_size: int = 16, dtype: str = "bf16") -> DecodeWorkload:
    """The same lengths at any block size (the pool is 1.25x the blocks they need); dtype "f32" gives the
    same batch with fp32 K/V and q (the vector kernels' shape)."""
    lens = lognormal_lengths(batch, 390, SIGMA_8B, 16, 4096, seed=seed)
    lay = build_paged_layout(lens, block_size, seed=seed + 1000, pool_factor=1.25)
    name = "llama8b_decode_" + dtype + ("" if block_size == 16 else "_bs%d" % block_size)
    return DecodeWorkload(name, lay, 32, 8, 128, dtype, 0.5, seed=seed)


def llama70b_long(batch: int = 8, seq_len: int = 32768, seed: int = 4, block_size: int = 16) -> DecodeWorkload:
    lay = build_paged_layout([seq_len] * batch, block_size, seed=seed + 1000, pool_factor=1.0)
    name = "llama70b_long_bf16" + ("" if block_size == 16 else "_bs%d" % block_size)
    return DecodeWorkload(name, lay, 64, 8, 128, "bf16", 1.0, seed=seed, partition_size=512)


def llama70b_one_long(seq_len: int = 131072, seed: int = 6) -> DecodeWorkload:
    """One long request alone: a single sequence, so each of the 8 (sequence, KV head) rows spans many of
    the split's pieces."""
    lay = build_paged_layout([seq_len], 16, seed=seed + 1000, pool_factor=1.0)
    return DecodeWorkload("llama70b_one_long_bf16", lay, 64, 8, 128, "bf16", 1.0, seed=seed, partition_size=512)


def shared_prefix(prompts: int = 16, prompt_len: int = 512, samples: int = 8, max_private: int = 256,
                  seed: int = 3) -> DecodeWorkload:
    """Parallel sampling: every sample shares its prompt's blocks.

    Built with the block manager: prompt prefill, fork into `samples`, then
    each sample appends its private tokens and finally one new token.  The
    copy-on-write copies this causes are returned in ``copies`` (none when the
    prompt fills whole blocks).  ``extra`` holds the slots of the prompt
    tokens, of the private tokens and of the new tokens, in writing order.
    """
    rng = np.random.default_rng(seed)
    priv = rng.integers(0, max_private + 1, size=prompts * samples)
    bs = 16
    need = prompts * (prompt_len + bs) // bs + sum(int(u) // bs + 2 for u in priv) + 8
    nb = int(math.ceil(1.25 * need))
    mgr = BlockManager(nb, bs, free_order=shuffled_block_ids(nb, seed + 1000))
    prompt_slots, private_slots, new_slots, seqs = [], [], [], []
    for _ in range(prompts):
        s = mgr.new_sequence()
        prompt_slots.append(mgr.append(s, prompt_len))
        seqs.extend(mgr.fork(s, samples))
    copies_at_first_write = []
    for i, s in enumerate(seqs):
        n = int(priv[i])
        private_slots.append(mgr.append(s, n))
    copies_at_first_write = mgr.take_copies()
    for s in seqs:
        new_slots.append(mgr.append(s, 1)[0])
    copies_new = mgr.take_copies()
    lens = np.array([mgr.lengths[s] for s in seqs], np.int32)
    tables = mgr.table_array(seqs)
    lay = PagedLayout(seq_lens=lens, block_tables=tables, num_blocks=nb, block_size=bs)
    w = DecodeWorkload("shared_prefix_bf16_p%d" % prompt_len, lay, 32, 8, 128, "bf16", 0.5, seed=seed,
                       copies=copies_at_first_write + copies_new)
    w.extra = dict(prompt_slots=prompt_slots, private_slots=private_slots, new_slots=np.array(new_slots),
                   private_counts=priv, samples=samples, prompts=prompts, prompt_len=prompt_len,
                   copies_at_first_write=copies_at_first_write, copies_new=copies_new,
                   unique_blocks=mgr.blocks_in_use())
    return w


def chunked_prefill(batch: int = 16, prefix: int = 1024, chunk: int = 512, seed: int = 5,
                    block_size: int = 16) -> PrefillWorkload:
    lay = build_paged_layout([prefix + chunk] * batch, block_size, seed=seed + 1000, pool_factor=1.0)
    name = "chunked_prefill_bf16" + ("" if block_size == 16 else "_bs%d" % block_size)
    return PrefillWorkload(name, lay, np.full(batch, chunk, np.int32), 32, 8, 128, "bf16", 1.0, seed=seed)


# ----------------------------------------------------------------------------- values
def host_values(shape, std: float, seed: int, dtype: str) -> np.ndarray:
    """fp32 draws, or their bf16 bit patterns (uint16) for dtype 'bf16'."""
    x = normal_f32(shape, std, seed)
    return x if dtype == "f32" else round_to_bf16_bits(x)


def device_values(shape, std: float, seed: int, dtype: str, device="cuda"):
    """The same distribution drawn on the device with torch's seeded generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(std)
    return x if dtype == "f32" else x.to(torch.bfloat16)


# ----------------------------------------------------------------------------- mixed decoding modes
@dataclass
class MixedDecodeTrace:
    """Decode steps of one batch that mixes beam search, parallel sampling and
    greedy sequences (Lecture 7 "KV Cache Management" §5.1-§5.3: the kernels
    only see each row's list of physical blocks, so the modes share a batch).

    Row order is fixed: the beams of each beam group, then the samples of each
    sampling group, then the greedy rows.  Per step: ``copies`` (src, dst)
    pairs to run first, then every row's new token goes to ``slots[row]``, then
    attention over ``seq_lens`` through ``tables`` (all padded to one width)."""
    name: str
    num_blocks: int
    block_size: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    std: float
    seed: int
    modes: List[str]
    tables: List[np.ndarray]            # per step, int32 [B, W]
    seq_lens: List[np.ndarray]          # per step, int32 [B]
    slots: List[np.ndarray]             # per step, int64 [B]
    copies: List[List[Tuple[int, int]]]  # per step
    whole_copy_tokens: int = 0          # tokens a copy-the-parent scheme would have copied

    @property
    def batch(self) -> int:
        return len(self.modes)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def beam_parents(rng, k: int) -> np.ndarray:
    """Parents of the k new beams among the k old ones, drawn independently and
    uniformly: some old beams get several children and others none, as in a
    beam step (Lecture 7 §5.2).  With k = 4 this averages 4 - 4(1 - (3/4)^4)
    = 1.27 copy-on-write copies per step, close to the pages' demo (35 copies
    over 32 steps)."""
    return np.sort(rng.integers(0, k, size=k))


def mixed_decode_trace(beam_groups: int = 16, beam_width: int = 4, sample_groups: int = 8, samples: int = 4,
                       greedy: int = 32, steps: int = 32, block_size: int = 16, seed: int = 6,
                       beam_prompt: Optional[int] = None, sample_prompt: int = 100,
                       num_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128,
                       dtype: str = "bf16") -> MixedDecodeTrace:
    """Build the trace with the block manager.  Prompts: the beam groups' from the
    length model (or ``beam_prompt`` tokens each), the sampling groups' of
    ``sample_prompt`` tokens (a partially filled last block, so the first write
    copies it n - 1 times), greedy rows from the length model."""
    rng = np.random.default_rng(seed)
    bp = (lognormal_lengths(beam_groups, 390, SIGMA_8B, 16, 2048, seed=seed + 1) if beam_prompt is None
          else np.full(beam_groups, beam_prompt, np.int32))
    gl = lognormal_lengths(greedy, 390, SIGMA_8B, 16, 4096, seed=seed + 2)
    bs = block_size
    need = (sum(-(-int(L) // bs) + beam_width * (steps // bs + 2) for L in bp)
            + sample_groups * (-(-sample_prompt // bs) + samples * (steps // bs + 2))
            + sum(-(-int(L) // bs) + steps // bs + 2 for L in gl))
    nb = int(math.ceil(1.25 * need)) + 8
    mgr = BlockManager(nb, bs, free_order=shuffled_block_ids(nb, seed + 1000))
    groups = []                                        # (mode, [seq ids])
    for L in bp:
        s = mgr.new_sequence()
        mgr.append(s, int(L))
        groups.append(("beam", [s]))
    for _ in range(sample_groups):
        s = mgr.new_sequence()
        mgr.append(s, sample_prompt)
        groups.append(("sample", mgr.fork(s, samples)))
    for L in gl:
        s = mgr.new_sequence()
        mgr.append(s, int(L))
        groups.append(("greedy", [s]))
    mgr.take_copies()
    modes = []
    for mode, seqs in groups:
        modes += [mode] * (beam_width if mode == "beam" else len(seqs))
    whole = 0
    tables, lens, slots, copies = [], [], [], []
    for step in range(steps):
        rows = []
        for gi, (mode, seqs) in enumerate(groups):
            if mode == "beam":
                if step == 0:
                    new = mgr.fork(seqs[0], beam_width)     # the prompt fans out into k beams
                else:
                    par = beam_parents(rng, beam_width)
                    counts = np.bincount(par, minlength=beam_width)
                    new = []
                    for b, c in zip(seqs, counts):
                        if c == 0:
                            mgr.free_sequence(b)
                    for b, c in zip(seqs, counts):
                        if c > 0:
                            new += mgr.fork(b, int(c))
                # a copy-the-parent scheme copies every new beam's whole history
                whole += beam_width * mgr.lengths[new[0]] if step == 0 else sum(mgr.lengths[s] for s in new)
                groups[gi] = (mode, new)
                seqs = new
            rows += seqs
        step_slots = [mgr.append(s, 1)[0] for s in rows]
        copies.append(mgr.take_copies())
        slots.append(np.asarray(step_slots, np.int64))
        lens.append(np.asarray([mgr.lengths[s] for s in rows], np.int32))
        tables.append([list(mgr.tables[s]) for s in rows])
    width = max(len(t) for st in tables for t in st)
    tabs = []
    for st in tables:
        a = np.full((len(st), width), -1, np.int32)
        for i, t in enumerate(st):
            a[i, :len(t)] = t
        tabs.append(a)
    return MixedDecodeTrace("mixed_beam_sample_greedy", nb, bs, num_heads, num_kv_heads, head_dim, dtype, 0.5,
                            seed, modes, tabs, lens, slots, copies, whole)
