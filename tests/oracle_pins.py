"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin takes the oracle module as an argument so the mutation test can run
the same pins against deliberately broken builds of the oracle.

What each pin rests on:
  brute_force      -- attention by the definition in pure-Python loops with
                      math.fsum and no max subtraction (tiny inputs only);
  torch_sdpa       -- torch's scaled_dot_product_attention in fp64 on the CPU
                      (a library routine; GQA via its own enable_gqa grouping);
  paged_vs_contig  -- paging changes where K/V live, not what is computed, for
                      any block size and permutation (Lecture 7 "KV Cache
                      Management" §4.2; Lecture 16 "LLM Serving (1)" §3.3);
  permutation_bits -- same block size, different physical permutation gives
                      bit-identical results (Lecture 7 §4.2);
  blockwise_online -- the pages' block loop with the online-softmax rescale
                      (Month 2 "PagedAttention" §5.4) and a partition merge
                      (Lecture 16 §3.3) equal the two-pass definition;
  gqa_as_mha       -- grouped-query attention equals multi-head attention over
                      KV heads replicated per group;
  closed_forms     -- softmax special cases with known answers;
  prefill_rows     -- a chunk of n rows equals the last n rows of full causal
                      attention; a chunk of one row equals decode;
  cache_vs_recompute -- decoding with the paged cache gives the same logits and
                      the same greedy tokens as recomputing without a cache
                      (Lecture 16 §1.1; Lecture 7 §4.2, block sizes 1/4/16/64);
  fp8_codec        -- E4M3 decode of all 256 codes and the quantiser (nearest,
                      ties to even, saturating at 448) against torch's
                      float8_e4m3fn conversions (a library routine), plus
                      codes with known values;
  fp8_attention    -- attention over an FP8 cache equals attention over the
                      dequantised values: exactly, through the fp32 path, when
                      the scales are powers of two; against torch SDPA in fp64
                      for other scales (decode and prefill);
  fp8_write        -- the quantising KV write stores torch's codes of
                      fp32(x) / fp32(scale) at the slots, and nothing else.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import synth
from synth.block_manager import BlockManager


# ----------------------------------------------------------------------------- helpers
def make_problem(lens, Hq, Hkv, D, bs, seed, dtype="f32", std=1.0, pool_factor=1.5):
    layout = synth.build_paged_layout(lens, bs, seed=seed, pool_factor=pool_factor)
    B = len(lens)
    shape = (layout.num_blocks, Hkv, bs, D)
    k = synth.normal_f32(shape, std, seed * 7 + 1)
    v = synth.normal_f32(shape, std, seed * 7 + 2)
    q = synth.normal_f32((B, Hq, D), std, seed * 7 + 3)
    if dtype == "bf16":
        k, v, q = (synth.round_to_bf16_bits(x) for x in (k, v, q))
    return layout, q, k, v


def to_f64(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def gather_contiguous(cache, table_row, L):
    """[L, Hkv, D] rows of one sequence, read through its block table (index copy, no math)."""
    NB, Hkv, bs, D = cache.shape
    out = np.empty((L, Hkv, D), dtype=cache.dtype)
    for t in range(L):
        out[t] = cache[table_row[t // bs], :, t % bs, :]
    return out


def repack(layout, k, v, new_bs, seed):
    """The same logical K/V stored with another block size and permutation."""
    B = layout.batch
    NB, Hkv, bs, D = k.shape
    new = synth.build_paged_layout(layout.seq_lens, new_bs, seed=seed, pool_factor=1.3)
    k2 = np.zeros((new.num_blocks, Hkv, new_bs, D), dtype=k.dtype)
    v2 = np.zeros_like(k2)
    for b in range(B):
        L = int(layout.seq_lens[b])
        ck = gather_contiguous(k, layout.block_tables[b], L)
        cv = gather_contiguous(v, layout.block_tables[b], L)
        for t in range(L):
            k2[new.block_tables[b, t // new_bs], :, t % new_bs, :] = ck[t]
            v2[new.block_tables[b, t // new_bs], :, t % new_bs, :] = cv[t]
    return new, k2, v2


def assert_close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, "%s: max abs err %.3e > %.1e" % (what, err, tol)


# ----------------------------------------------------------------------------- pins
def pin_brute_force(orc):
    """Tiny inputs against pure-Python attention (fsum, no max subtraction)."""
    lens = [5, 9, 1, 12]
    Hq, Hkv, D, bs = 4, 2, 8, 4
    layout, q, k, v = make_problem(lens, Hq, Hkv, D, bs, seed=11)
    scale = 1.0 / math.sqrt(D)
    out = orc.paged_decode(q, k, v, layout.block_tables, layout.seq_lens, scale)
    g = Hq // Hkv
    for b, L in enumerate(lens):
        K = gather_contiguous(k, layout.block_tables[b], L).astype(float)
        V = gather_contiguous(v, layout.block_tables[b], L).astype(float)
        for h in range(Hq):
            kh = h // g
            w = [math.exp(scale * math.fsum(float(q[b, h, d]) * K[t, kh, d] for d in range(D)))
                 for t in range(L)]
            Z = math.fsum(w)
            for d in range(D):
                ref = math.fsum(w[t] * V[t, kh, d] for t in range(L)) / Z
                assert abs(out[b, h, d] - ref) <= 1e-12, (b, h, d, out[b, h, d], ref)


def _sdpa(qc, Kc, Vc, scale, mask=None):
    """torch SDPA in fp64: qc [Hq, Tq, D], Kc/Vc [Hkv, Lk, D]."""
    q = torch.from_numpy(qc)[None]
    k = torch.from_numpy(Kc)[None]
    v = torch.from_numpy(Vc)[None]
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=m, scale=scale, enable_gqa=True)[0].numpy()


def pin_torch_sdpa_decode(orc):
    for dtype, (Hq, Hkv, D) in (("f32", (8, 2, 64)), ("bf16", (32, 8, 128)), ("f32", (6, 6, 16))):
        lens = [17, 64, 100, 203, 1, 16]
        layout, q, k, v = make_problem(lens, Hq, Hkv, D, 16, seed=5, dtype=dtype)
        scale = 1.0 / math.sqrt(D)
        out = orc.paged_decode(q, k, v, layout.block_tables, layout.seq_lens, scale)
        for b, L in enumerate(lens):
            K = to_f64(gather_contiguous(k, layout.block_tables[b], L)).transpose(1, 0, 2).copy()
            V = to_f64(gather_contiguous(v, layout.block_tables[b], L)).transpose(1, 0, 2).copy()
            ref = _sdpa(to_f64(q[b])[:, None, :].copy(), K, V, scale)[:, 0, :]
            assert_close(out[b], ref, 1e-12, "sdpa decode %s b=%d" % (dtype, b))


def pin_torch_sdpa_prefill(orc):
    Hq, Hkv, D, bs = 8, 2, 32, 16
    total = [40, 64, 17, 5]
    chunk = [13, 64, 1, 5]
    layout, _, k, v = make_problem(total, Hq, Hkv, D, bs, seed=9)
    qsl = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q = synth.normal_f32((int(qsl[-1]), Hq, D), 1.0, 99)
    scale = 0.3
    out = orc.paged_prefill(q, k, v, layout.block_tables, qsl, layout.seq_lens, scale)
    for b, (S, n) in enumerate(zip(total, chunk)):
        K = to_f64(gather_contiguous(k, layout.block_tables[b], S)).transpose(1, 0, 2).copy()
        V = to_f64(gather_contiguous(v, layout.block_tables[b], S)).transpose(1, 0, 2).copy()
        qc = to_f64(q[qsl[b]:qsl[b + 1]]).transpose(1, 0, 2).copy()
        pos = S - n + np.arange(n)
        mask = np.arange(S)[None, :] <= pos[:, None]
        ref = _sdpa(qc, K, V, scale, mask).transpose(1, 0, 2)
        assert_close(out[qsl[b]:qsl[b + 1]], ref, 1e-12, "sdpa prefill b=%d" % b)


def pin_paged_vs_contiguous(orc):
    lens = [17, 64, 100, 203]
    Hq, Hkv, D = 8, 2, 64
    layout, q, k, v = make_problem(lens, Hq, Hkv, D, 16, seed=1)
    scale = 0.125
    base = orc.paged_decode(q, k, v, layout.block_tables, layout.seq_lens, scale)
    for b, L in enumerate(lens):
        K = to_f64(gather_contiguous(k, layout.block_tables[b], L))
        V = to_f64(gather_contiguous(v, layout.block_tables[b], L))
        ref = orc.contiguous_attention(to_f64(q[b])[None], K, V, [L], scale)[0]
        assert_close(base[b], ref, 1e-13, "contiguous b=%d" % b)
    for new_bs in (1, 4, 16, 64, 256):
        lay2, k2, v2 = repack(layout, k, v, new_bs, seed=new_bs + 100)
        out = orc.paged_decode(q, k2, v2, lay2.block_tables, lay2.seq_lens, scale)
        assert_close(out, base, 1e-13, "block size %d" % new_bs)


def pin_permutation_bit_exact(orc):
    lens = [33, 7, 250]
    layout, q, k, v = make_problem(lens, 8, 4, 32, 16, seed=3, dtype="bf16")
    base = orc.paged_decode(q, k, v, layout.block_tables, layout.seq_lens, 0.2)
    lay2, k2, v2 = repack(layout, k, v, 16, seed=12345)
    assert not np.array_equal(lay2.block_tables, layout.block_tables)
    out = orc.paged_decode(q, k2, v2, lay2.block_tables, lay2.seq_lens, 0.2)
    assert np.array_equal(out, base), "permutation changed the bits"


def pin_blockwise_online(orc):
    lens = [1, 15, 16, 17, 100, 203, 512]
    Hq, Hkv, D = 4, 2, 16
    layout, q, k, v = make_problem(lens, Hq, Hkv, D, 16, seed=21)
    scale = 0.7
    ref = orc.paged_decode(q, k, v, layout.block_tables, layout.seq_lens, scale)
    rng = np.random.default_rng(4)
    for b, L in enumerate(lens):
        nblk = (L + 15) // 16
        for pb in (1, 2, 3, 32, 10 ** 6):
            order = np.arange(nblk, dtype=np.int32)
            for p0 in range(0, nblk, pb):
                seg = order[p0:p0 + pb]
                order[p0:p0 + pb] = seg[rng.permutation(len(seg))]
            for h in range(Hq):
                got = orc.blockwise_decode_row(q[b, h], k, v, layout.block_tables[b], L, h // 2,
                                               scale, partition_blocks=pb, visit_order=order)
                assert_close(got, ref[b, h], 1e-13, "blockwise b=%d pb=%d" % (b, pb))


def pin_gqa_as_mha(orc):
    lens = [20, 45]
    Hq, Hkv, D = 8, 2, 16
    g = Hq // Hkv
    layout, q, k, v = make_problem(lens, Hq, Hkv, D, 16, seed=8, dtype="bf16")
    gqa = orc.paged_decode(q, k, v, layout.block_tables, layout.seq_lens, 0.25)
    k_rep = np.repeat(k, g, axis=1).copy()
    v_rep = np.repeat(v, g, axis=1).copy()
    mha = orc.paged_decode(q, k_rep, v_rep, layout.block_tables, layout.seq_lens, 0.25)
    assert np.array_equal(gqa, mha)


def pin_closed_forms(orc):
    Hq, Hkv, D, bs = 4, 2, 8, 4
    # L = 1: the only weight is 1, out = v_0.
    layout, q, k, v = make_problem([1, 1], Hq, Hkv, D, bs, seed=31)
    out = orc.paged_decode(q, k, v, layout.block_tables, layout.seq_lens, 0.5)
    for b in range(2):
        for h in range(Hq):
            np.testing.assert_array_equal(out[b, h], v[layout.block_tables[b, 0], h // 2, 0].astype(np.float64))
    # all V rows equal c: out = c for any scores.
    layout, q, k, v = make_problem([13, 30], Hq, Hkv, D, bs, seed=32)
    c = synth.normal_f32((Hkv, D), 1.0, 77)
    v[:] = c[None, :, None, :]
    out = orc.paged_decode(q, k, v, layout.block_tables, layout.seq_lens, 0.5)
    for b in range(2):
        for h in range(Hq):
            assert_close(out[b, h], c[h // 2].astype(np.float64), 1e-14, "constant V")
    # scale = 0 (or q = 0): uniform weights, out = mean of V over the L tokens.
    layout, q, k, v = make_problem([13, 30], Hq, Hkv, D, bs, seed=33)
    for qq, sc in ((q, 0.0), (np.zeros_like(q), 0.9)):
        out = orc.paged_decode(qq, k, v, layout.block_tables, layout.seq_lens, sc)
        for b, L in enumerate([13, 30]):
            V = gather_contiguous(v, layout.block_tables[b], L).astype(np.float64)
            for h in range(Hq):
                assert_close(out[b, h], V[:, h // 2].mean(axis=0), 1e-14, "uniform weights")
    # one key aligned with q and huge: out -> that key's v.
    layout, q, k, v = make_problem([40], Hq, Hkv, D, bs, seed=34)
    t_star = 27
    blk, off = layout.block_tables[0, t_star // bs], t_star % bs
    for h in range(Hkv):
        k[blk, h, off] = 1000.0 * q[0, h * 2]
        q[0, h * 2 + 1] = q[0, h * 2]
    out = orc.paged_decode(q, k, v, layout.block_tables, layout.seq_lens, 1.0)
    for h in range(Hq):
        assert_close(out[0, h], v[blk, h // 2, off].astype(np.float64), 1e-12, "dominant key")
    # L = 0: all-zero row.
    layout, q, k, v = make_problem([0, 5], Hq, Hkv, D, bs, seed=35)
    out = orc.paged_decode(q, k, v, layout.block_tables, layout.seq_lens, 1.0)
    assert np.all(out[0] == 0.0)


def pin_prefill_rows(orc):
    Hq, Hkv, D, bs = 4, 2, 16, 16
    total = [50, 33]
    layout, _, k, v = make_problem(total, Hq, Hkv, D, bs, seed=41, dtype="bf16")
    q_full = synth.round_to_bf16_bits(synth.normal_f32((sum(total), Hq, D), 1.0, 42))
    qsl_full = np.array([0, 50, 83], np.int32)
    full = orc.paged_prefill(q_full, k, v, layout.block_tables, qsl_full, layout.seq_lens, 0.25)
    # rows S-n..S-1 of the full causal pass equal a chunk of n rows.
    for n0, n1 in ((7, 33), (1, 1), (50, 33)):
        qsl = np.array([0, n0, n0 + n1], np.int32)
        qc = np.concatenate([q_full[50 - n0:50], q_full[83 - n1:83]])
        out = orc.paged_prefill(qc, k, v, layout.block_tables, qsl, layout.seq_lens, 0.25)
        assert_close(out[:n0], full[50 - n0:50], 1e-13, "chunk rows seq0")
        assert_close(out[n0:], full[83 - n1:83], 1e-13, "chunk rows seq1")
    # a chunk of one row is a decode.
    qd = np.stack([q_full[49], q_full[82]])
    dec = orc.paged_decode(qd, k, v, layout.block_tables, layout.seq_lens, 0.25)
    one = orc.paged_prefill(qd, k, v, layout.block_tables, np.array([0, 1, 2], np.int32),
                            layout.seq_lens, 0.25)
    assert np.array_equal(dec, one)
    # full causal pass equals contiguous attention with a causal key count.
    for b, S in enumerate(total):
        K = to_f64(gather_contiguous(k, layout.block_tables[b], S))
        V = to_f64(gather_contiguous(v, layout.block_tables[b], S))
        ref = orc.contiguous_attention(to_f64(q_full[qsl_full[b]:qsl_full[b + 1]]), K, V,
                                       np.arange(1, S + 1), 0.25)
        assert_close(full[qsl_full[b]:qsl_full[b + 1]], ref, 1e-13, "causal contiguous")


def pin_cache_vs_recompute(orc, block_sizes=(1, 4, 16, 64), steps=20):
    """Single attention layer, 4 sequences, prefill + `steps` greedy decode steps."""
    vocab, dm, Hq, Hkv, D = 48, 24, 4, 2, 8
    E = synth.normal_f32((vocab, dm), 1.0, 500)
    Wq = synth.normal_f32((dm, Hq * D), 0.4, 501)
    Wk = synth.normal_f32((dm, Hkv * D), 0.4, 502)
    Wv = synth.normal_f32((dm, Hkv * D), 0.4, 503)
    Wo = synth.normal_f32((Hq * D, vocab), 0.4, 504)
    rng = np.random.default_rng(505)
    prompts = [list(rng.integers(0, vocab, size=n)) for n in (3, 11, 17, 30)]
    scale = 1.0 / math.sqrt(D)

    def proj(tokens, W, H):
        x = E[np.asarray(tokens)].astype(np.float64)
        return (x @ W.astype(np.float64)).astype(np.float32).reshape(len(tokens), H, D)

    def logits_of(attn_rows):
        return attn_rows.reshape(attn_rows.shape[0], Hq * D) @ Wo.astype(np.float64)

    # without a cache: recompute every K, V from scratch at each step
    ref_tokens, ref_logits = [], []
    for p in prompts:
        seq = list(p)
        lg_all = []
        for _ in range(steps + 1):
            K, V, Q = proj(seq, Wk, Hkv), proj(seq, Wv, Hkv), proj(seq[-1:], Wq, Hq)
            row = orc.contiguous_attention(Q.astype(np.float64), K, V, [len(seq)], scale)
            lg = logits_of(row)[0]
            lg_all.append(lg)
            seq.append(int(np.argmax(lg)))
        ref_tokens.append(seq)
        ref_logits.append(lg_all)

    for bs in block_sizes:
        nb = sum((len(p) + steps + bs) // bs + 1 for p in prompts) + 8
        mgr = BlockManager(nb, bs, free_order=synth.shuffled_block_ids(nb, bs + 600))
        kc = np.zeros((nb, Hkv, bs, D), np.float32)
        vc = np.zeros_like(kc)
        seqs = [mgr.new_sequence() for _ in prompts]
        toks = [list(p) for p in prompts]
        # prefill: write all prompt K/V, attend the prompt causally, keep the last row
        lgs = [[] for _ in prompts]
        for i, s in enumerate(seqs):
            slots = mgr.append(s, len(toks[i]))
            orc.kv_cache_write(proj(toks[i], Wk, Hkv), proj(toks[i], Wv, Hkv), kc, vc, slots)
        tables = mgr.table_array(seqs, width=64)
        lens = np.array([len(t) for t in toks], np.int32)
        qs = np.concatenate([proj(t, Wq, Hq) for t in toks])
        qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        out = orc.paged_prefill(qs, kc, vc, tables, qsl, lens, scale)
        for i in range(len(seqs)):
            lg = logits_of(out[qsl[i + 1] - 1:qsl[i + 1]])[0]
            lgs[i].append(lg)
            toks[i].append(int(np.argmax(lg)))
        # decode steps, all sequences in one batch
        for _ in range(steps):
            for i, s in enumerate(seqs):
                slot = mgr.append(s, 1)
                t = toks[i][-1:]
                orc.kv_cache_write(proj(t, Wk, Hkv), proj(t, Wv, Hkv), kc, vc, slot)
            tables = mgr.table_array(seqs, width=64)
            lens = np.array([mgr.lengths[s] for s in seqs], np.int32)
            qd = np.concatenate([proj(t[-1:], Wq, Hq) for t in toks])
            out = orc.paged_decode(qd, kc, vc, tables, lens, scale)
            for i in range(len(seqs)):
                lg = logits_of(out[i:i + 1])[0]
                lgs[i].append(lg)
                toks[i].append(int(np.argmax(lg)))
        for i in range(len(seqs)):
            assert toks[i] == ref_tokens[i], "greedy tokens differ at block size %d" % bs
            assert_close(np.array(lgs[i]), np.array(ref_logits[i]), 1e-12, "logits bs=%d" % bs)


def _torch_fp8_codes(x_f32):
    """torch's E4M3 codes of fp32 values after clamping to the finite range."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_fp8_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def pin_fp8_codec(orc):
    codes = np.arange(256, dtype=np.uint8)
    val = orc.fp8_decode(codes)
    ref = _torch_fp8_values(codes)
    assert np.array_equal(np.isnan(val), np.isnan(ref)) and np.isnan(val).sum() == 2
    ok = ~np.isnan(ref)
    assert np.array_equal(val[ok], ref[ok]) and np.array_equal(np.signbit(val[ok]), np.signbit(ref[ok]))
    # known codes: 1.0, the largest finite value, the smallest subnormal, ties to the even code
    known = {1.0: 0x38, 448.0: 0x7E, 2.0 ** -9: 0x01, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02,
             1.0625: 0x38, 1.1875: 0x3A, 1000.0: 0x7E, -1.0: 0xB8, -0.0: 0x80}
    xs = np.array(list(known), np.float32)
    assert orc.fp8_encode(xs).tolist() == list(known.values())
    # every midpoint between neighbouring codes, a hair either side, and random magnitudes
    pos = np.sort(ref[:127])
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(8)
    x = np.concatenate([pos, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                        np.nextafter(mids.astype(np.float32), np.float32(1e9)),
                        rng.lognormal(-3.0, 3.0, 20000), [449.0, 463.99, 464.0, 464.01, 1e30, 1e-30]]).astype(np.float32)
    x = np.concatenate([x, -x])
    assert np.array_equal(orc.fp8_encode(x), _torch_fp8_codes(x))


def _fp8_problem(lens, Hq, Hkv, D, bs, seed, ks, vs):
    layout, q, k, v = make_problem(lens, Hq, Hkv, D, bs, seed=seed)
    kc = _torch_fp8_codes(k / np.float32(ks))
    vc = _torch_fp8_codes(v / np.float32(vs))
    return layout, q, kc, vc


def pin_fp8_attention(orc):
    lens = [17, 64, 100, 5, 1]
    Hq, Hkv, D, bs = 8, 2, 64, 16
    for ks, vs in ((2.0 ** -6, 2.0 ** -5), (0.0123, 0.0377)):
        layout, q, kc, vc = _fp8_problem(lens, Hq, Hkv, D, bs, 21, ks, vs)
        out = orc.paged_decode(q, kc, vc, layout.block_tables, layout.seq_lens, 0.125, k_scale=ks, v_scale=vs)
        kd, vd = _torch_fp8_values(kc) * ks, _torch_fp8_values(vc) * vs
        if ks == 2.0 ** -6:
            # power-of-two scales: the dequantised values are exact in fp32
            ref = orc.paged_decode(q, kd.astype(np.float32), vd.astype(np.float32), layout.block_tables,
                                   layout.seq_lens, 0.125)
            assert_close(out, ref, 1e-15, "fp8 decode == fp32 decode of the dequantised cache")
        for b, L in enumerate(lens):
            K = gather_contiguous(kd, layout.block_tables[b], L).transpose(1, 0, 2).copy()
            V = gather_contiguous(vd, layout.block_tables[b], L).transpose(1, 0, 2).copy()
            ref = _sdpa(q[b].astype(np.float64)[:, None, :].copy(), K, V, 0.125)[:, 0, :]
            assert_close(out[b], ref, 1e-12, "fp8 decode vs sdpa b=%d" % b)
    # prefill: a chunk of 7 rows at the end of a 40-token sequence
    layout, _, kc, vc = _fp8_problem([40], Hq, Hkv, D, bs, 22, 0.02, 0.03)
    qp = synth.normal_f32((7, Hq, D), 1.0, 23)
    out = orc.paged_prefill(qp, kc, vc, layout.block_tables, np.array([0, 7], np.int32), layout.seq_lens, 0.125,
                            k_scale=0.02, v_scale=0.03)
    K = gather_contiguous(_torch_fp8_values(kc) * 0.02, layout.block_tables[0], 40).transpose(1, 0, 2).copy()
    V = gather_contiguous(_torch_fp8_values(vc) * 0.03, layout.block_tables[0], 40).transpose(1, 0, 2).copy()
    mask = np.arange(40)[None, :] <= (33 + np.arange(7))[:, None]
    ref = _sdpa(qp.astype(np.float64).transpose(1, 0, 2).copy(), K, V, 0.125, mask=mask).transpose(1, 0, 2)
    assert_close(out, ref, 1e-12, "fp8 prefill vs sdpa")


def pin_fp8_write(orc):
    NB, Hkv, bs, D, T = 7, 2, 4, 16, 9
    for dt in ("f32", "bf16"):
        key = synth.normal_f32((T, Hkv, D), 3.0, 31)
        val = synth.normal_f32((T, Hkv, D), 0.2, 32)
        if dt == "bf16":
            key, val = synth.round_to_bf16_bits(key), synth.round_to_bf16_bits(val)
        kc = np.full((NB, Hkv, bs, D), 0x55, np.uint8)
        vc = kc.copy()
        slots = np.array([3, 27, -1, 0, 12, 5, 26, 17, 8], np.int64)
        orc.kv_cache_write_fp8(key, val, kc, vc, slots, 0.011, 0.0007)
        kf = to_f64(key).astype(np.float32)
        vf = to_f64(val).astype(np.float32)
        touched = set()
        for t, s in enumerate(slots):
            if s < 0:
                continue
            touched.add((s // bs, s % bs))
            assert np.array_equal(kc[s // bs, :, s % bs], _torch_fp8_codes(kf[t] / np.float32(0.011)))
            assert np.array_equal(vc[s // bs, :, s % bs], _torch_fp8_codes(vf[t] / np.float32(0.0007)))
        for blk in range(NB):
            for off in range(bs):
                if (blk, off) not in touched:
                    assert (kc[blk, :, off] == 0x55).all() and (vc[blk, :, off] == 0x55).all()


ALL_PINS = [pin_brute_force, pin_torch_sdpa_decode, pin_torch_sdpa_prefill, pin_paged_vs_contiguous,
            pin_permutation_bit_exact, pin_blockwise_online, pin_gqa_as_mha, pin_closed_forms,
            pin_prefill_rows, pin_cache_vs_recompute, pin_fp8_codec, pin_fp8_attention, pin_fp8_write]
