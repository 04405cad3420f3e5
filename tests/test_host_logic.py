"""Host-side logic against the pages' worked examples (golden fixtures) and
the oracle's write/copy semantics.  CPU only."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from synth.block_manager import BlockManager

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_slot_worked_example():
    g = load("slot_example.json")
    bs = g["block_size"]
    mgr = BlockManager(len(g["free_order"]), bs, free_order=g["free_order"])
    s = mgr.new_sequence()
    slots = mgr.append(s, g["prompt_tokens"])
    fill = [min(bs, g["prompt_tokens"] - i * bs) for i in range(len(mgr.tables[s]))]
    assert fill == g["expected_fill_after_prompt"]
    slots += mgr.append(s, g["generated_tokens"])
    assert slots == g["expected_slots"]
    assert mgr.tables[s] == g["expected_table"]
    # the same slots written by the oracle read back in order through the table
    D, Hkv = 3, 2
    key = synth.normal_f32((len(slots), Hkv, D), 1.0, 1)
    val = synth.normal_f32((len(slots), Hkv, D), 1.0, 2)
    kc = np.zeros((len(g["free_order"]), Hkv, bs, D), np.float32)
    vc = np.zeros_like(kc)
    oracle.kv_cache_write(key, val, kc, vc, slots)
    for t in range(len(slots)):
        blk = g["expected_table"][t // bs]
        np.testing.assert_array_equal(kc[blk, :, t % bs], key[t])
        np.testing.assert_array_equal(vc[blk, :, t % bs], val[t])


def test_cow_exercise5_counts():
    e = load("cow_counts.json")["exercise5"]
    n, prompt, gen, bs = e["n"], e["prompt"], e["generated"], e["block_size"]
    # without sharing: every sample holds its own copy of the prompt
    mgr = BlockManager(200, bs)
    for _ in range(n):
        s = mgr.new_sequence()
        mgr.append(s, prompt + gen)
    assert mgr.blocks_in_use() == e["blocks_without_sharing"]
    # with sharing: one prompt, forked into n, then each sample generates
    mgr = BlockManager(200, bs)
    s = mgr.new_sequence()
    mgr.append(s, prompt)
    samples = mgr.fork(s, n)
    for _ in range(gen):                      # samples advance one token at a time
        for x in samples:
            mgr.append(x, 1)
    assert mgr.blocks_in_use() == e["blocks_with_sharing"]
    assert len(mgr.take_copies()) == e["cow_copies"]


@pytest.mark.parametrize("case", load("cow_counts.json")["exercise4"]["cases"])
def test_cow_exercise4_n_minus_1(case):
    mgr = BlockManager(4096, case["block_size"])
    s = mgr.new_sequence()
    mgr.append(s, case["prompt"])
    samples = mgr.fork(s, case["n"])
    for x in samples:
        mgr.append(x, 1)
    copies = mgr.take_copies()
    assert len(copies) == case["cow_copies"]
    # every copy reads the one shared partial block and writes a fresh, distinct one
    assert len({d for _, d in copies}) == len(copies)
    assert len({src for src, _ in copies}) <= 1


def test_prompt100_split():
    e = load("cow_counts.json")["prompt100_split"]
    assert 100 // e["block_size"] == e["full_blocks"] and 100 % e["block_size"] == e["tokens_in_last"]


def test_free_returns_blocks_at_zero():
    mgr = BlockManager(64, 16)
    s = mgr.new_sequence()
    mgr.append(s, 40)
    kids = mgr.fork(s, 3)
    assert mgr.blocks_in_use() == 3
    mgr.free_sequence(kids[1])
    mgr.free_sequence(kids[2])
    assert mgr.blocks_in_use() == 3 and all(mgr.refcount[b] == 1 for b in mgr.tables[s])
    mgr.free_sequence(s)
    assert mgr.blocks_in_use() == 0 and len(mgr.free) == 64


def test_kv_byte_formulas():
    g = load("kv_bytes.json")
    for m in g["per_token"]:
        assert synth.kv_bytes_per_token(m["layers"], m["kv_heads"], m["head_dim"], m["dtype_bytes"]) == m["bytes"]
    b = g["block"]
    assert synth.block_bytes(b["block_size"], b["kv_heads"], b["head_dim"], b["dtype_bytes"]) == b["bytes"]


def test_oracle_kv_write_skips_negative_and_leaves_rest():
    NB, Hkv, bs, D = 6, 2, 4, 5
    kc = synth.round_to_bf16_bits(synth.normal_f32((NB, Hkv, bs, D), 1.0, 3))
    vc = synth.round_to_bf16_bits(synth.normal_f32((NB, Hkv, bs, D), 1.0, 4))
    k0, v0 = kc.copy(), vc.copy()
    key = synth.round_to_bf16_bits(synth.normal_f32((4, Hkv, D), 1.0, 5))
    val = synth.round_to_bf16_bits(synth.normal_f32((4, Hkv, D), 1.0, 6))
    slots = [7, -1, 0, 23]
    oracle.kv_cache_write(key, val, kc, vc, slots)
    touched = {(7 // bs, 7 % bs), (0, 0), (23 // bs, 23 % bs)}
    for blk in range(NB):
        for off in range(bs):
            if (blk, off) in touched:
                continue
            np.testing.assert_array_equal(kc[blk, :, off], k0[blk, :, off])
            np.testing.assert_array_equal(vc[blk, :, off], v0[blk, :, off])
    np.testing.assert_array_equal(kc[1, :, 3], key[0])
    np.testing.assert_array_equal(vc[5, :, 3], val[3])
    np.testing.assert_array_equal(kc[0, :, 0], key[2])


def test_oracle_block_copy_semantics():
    NB, Hkv, bs, D = 8, 3, 4, 6
    kc = synth.normal_f32((NB, Hkv, bs, D), 1.0, 7)
    vc = synth.normal_f32((NB, Hkv, bs, D), 1.0, 8)
    k0, v0 = kc.copy(), vc.copy()
    oracle.block_copy(kc, vc, [(1, 5), (2, 2), (0, 7)])
    np.testing.assert_array_equal(kc[5], k0[1])
    np.testing.assert_array_equal(vc[7], v0[0])
    for b in (0, 1, 2, 3, 4, 6):
        np.testing.assert_array_equal(kc[b], k0[b])
        np.testing.assert_array_equal(vc[b], v0[b])


def test_lognormal_lengths_shape():
    # the 8B decode workload's length model: median ~390, mean ~493 (sigma from the pages' mean)
    sigma = math.sqrt(2 * math.log(493 / 390))
    L = synth.lognormal_lengths(200000, 390, sigma, 16, 4096, seed=1234)
    assert abs(np.median(L) - 390) < 5
    assert abs(L.mean() - 493) < 6
    assert L.min() >= 16 and L.max() <= 4096


def test_layout_is_a_permutation_and_deterministic():
    lay = synth.build_paged_layout([17, 64, 100, 203], 16, seed=1, num_blocks=64)
    used = lay.block_tables[lay.block_tables >= 0]
    assert len(used) == 26 and len(set(used.tolist())) == 26
    lay2 = synth.build_paged_layout([17, 64, 100, 203], 16, seed=1, num_blocks=64)
    np.testing.assert_array_equal(lay.block_tables, lay2.block_tables)


def test_block_size_sweep_waste_accounting():
    """The sweep's fragmentation figure: unused slots of each sequence's last block."""
    import bench
    lay = synth.build_paged_layout([1, 16, 17, 0], 16, seed=3)
    assert bench.slot_waste(lay) == (15 + 0 + 15, 16 + 16 + 32)
    lay8 = synth.build_paged_layout([1, 16, 17, 0], 8, seed=3)
    assert bench.slot_waste(lay8) == (7 + 0 + 7, 8 + 16 + 24)
    # the sweep's decode workload keeps its lengths at every block size
    from synth import workloads as W
    base = W.llama8b_decode().layout.seq_lens
    for bs in (8, 32, 128):
        w = W.llama8b_decode(block_size=bs)
        assert np.array_equal(w.layout.seq_lens, base) and w.block_size == bs
        assert w.name.endswith("_bs%d" % bs)


def test_swap_cost_model_exercise6():
    """The pages' worked swap-vs-recompute example, through the model the swap benchmark reports."""
    g = load("swap_exercise6.json")
    m = g["model"]
    args = (m["layers"], m["kv_heads"], m["head_dim"], m["dtype_bytes"], g["pcie_bytes_per_s"], g["per_copy_s"])
    copies, per_copy, secs = synth.swap_time_model(g["tokens"], g["block_size"], *args)
    assert copies == g["copies"] and per_copy == g["bytes_per_copy"]
    assert round((g["per_copy_s"] + per_copy / g["pcie_bytes_per_s"]) * 1e6, 1) == g["us_per_copy"]
    assert round(secs * 1e3, 1) == g["swap_out_ms"]
    assert round(2 * secs * 1e3, 1) == g["swap_out_and_in_ms"]
    assert (2 * secs * 1e3 < g["recompute_ms"]) == g["swap_faster_than_recompute"]
    lo, hi = g["crossover_between_block_sizes"]
    assert 2 * synth.swap_time_model(g["tokens"], lo, *args)[2] * 1e3 > g["recompute_ms"]
    assert 2 * synth.swap_time_model(g["tokens"], hi, *args)[2] * 1e3 < g["recompute_ms"]


def test_oracle_swap_image_and_round_trip():
    """Swap-out packs K then V of each listed block; swap-in to other ids equals block copies."""
    NB, Hkv, bs, D = 9, 2, 4, 8
    for dt in ("f32", "bf16"):
        kc = synth.normal_f32((NB, Hkv, bs, D), 1.0, 11)
        vc = synth.normal_f32((NB, Hkv, bs, D), 1.0, 12)
        if dt == "bf16":
            kc, vc = synth.round_to_bf16_bits(kc), synth.round_to_bf16_bits(vc)
        ids = [4, 0, 7, 99, -2]
        img = oracle.swap_out(kc, vc, ids)
        nb = Hkv * bs * D * kc.itemsize
        assert img.shape == (5, 2, nb)
        for i, b in enumerate(ids[:3]):
            assert img[i, 0].tobytes() == kc[b].tobytes() and img[i, 1].tobytes() == vc[b].tobytes()
        assert not img[3:].any()                        # bad ids give zero pieces
        # swap in to other blocks == copying those blocks there
        k1, v1, k2, v2 = kc.copy(), vc.copy(), kc.copy(), vc.copy()
        new = [1, 5, 8]
        oracle.swap_in(k1, v1, new + [-1, NB], img)      # pieces 3 and 4: bad target ids, skipped
        oracle.block_copy(k2, v2, list(zip(ids[:3], new)))
        assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_beam_search_copy_counts():
    """Copy-the-parent beam search copies the closed-form 10,176 tokens (L7 §14 exercise 5);
    with forked blocks only shared, partially filled last blocks are copied, at most k - 1 per
    step, and each copy is the block the writer was about to write into."""
    from synth import workloads as W
    g = load("beam_copies.json")
    k, bs = g["beam_width"], g["block_size"]
    counts = []
    for seed in range(8):
        tr = W.mixed_decode_trace(beam_groups=1, beam_width=k, sample_groups=0, greedy=0, beam_prompt=g["prompt"],
                                  steps=g["steps"], block_size=bs, seed=seed)
        assert tr.whole_copy_tokens == g["whole_copy_tokens"]
        for step, (cp, slots, lens) in enumerate(zip(tr.copies, tr.slots, tr.seq_lens)):
            assert len(cp) <= k - 1
            if (g["prompt"] + step) % bs == 0:       # the new token opens a fresh block: nothing shared to copy
                assert not cp
            dsts = {d for _, d in cp}
            assert len(dsts) == len(cp) and not dsts & {s for s, _ in cp}
            for _, d in cp:                            # a copy's target receives this step's token
                assert d in set(int(s) // bs for s in slots)
        counts.append(sum(len(c) for c in tr.copies))
    # the demo's 35 copies (560 tokens) sit inside the spread of seeded trajectories
    assert min(counts) <= g["demo_paged_copies"] <= max(counts)
    assert g["demo_paged_copies"] * bs == g["demo_paged_copy_tokens"]
    assert all(c * bs * 10 < g["whole_copy_tokens"] for c in counts)
