"""GPU parity: the HIP kernels against the fp64 CPU oracle on identical seeded
inputs, called through the C ABI (via the thin binding).

Tolerances (max abs error): 1e-5 for fp32 KV, 2e-3 for bf16 KV (fp32 output;
a bf16 output is compared against the oracle rounded to bf16).  Slot writes
and block copies are compared bit for bit over the whole caches.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as W
from gpu_helpers import TOL, bf16_round_f64, max_err, out_to_f64, require_gpu, to_gpu, to_host, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    mod = require_gpu()
    oracle.build(force=False)
    return mod


def rand_problem(lens, Hq, Hkv, D, bs, dtype, seed, std=1.0, pool_factor=1.3):
    lay = synth.build_paged_layout(lens, bs, seed=seed, pool_factor=pool_factor)
    shape = (lay.num_blocks, Hkv, bs, D)
    k = W.host_values(shape, std, seed * 11 + 1, dtype)
    v = W.host_values(shape, std, seed * 11 + 2, dtype)
    q = W.host_values((len(lens), Hq, D), std, seed * 11 + 3, dtype)
    return lay, q, k, v


def gpu_decode(pa, lay, q, k, v, scale, out_dtype="f32", partition_size=0):
    torch = torch_mod()
    B, Hq, D = q.shape
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    bt = to_gpu(lay.block_tables.astype(np.int32))
    sl = to_gpu(lay.seq_lens.astype(np.int32))
    out = torch.empty((B, Hq, D), dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16, device="cuda")
    max_len = max(int(lay.seq_lens.max()), 1)
    wsb = pa.paged_attn_decode_workspace_size(B, Hq, k.shape[1], D, k.shape[2], max_len, partition_size)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    pa.paged_attn_decode(out, qg, kg, vg, bt, sl, scale, max_len, partition_size, ws)
    torch.cuda.synchronize()
    return out


# ----------------------------------------------------------------------------- kv_cache_write / block_copy
@pytest.mark.parametrize("dtype,D,bs", [("bf16", 128, 16), ("f32", 64, 16), ("bf16", 64, 8), ("f32", 128, 1)])
def test_kv_cache_write_bit_exact(pa, dtype, D, bs):
    Hkv, T = 4, 50
    NB = max(37, (2 * T + bs - 1) // bs)
    rng = np.random.default_rng(7)
    slots = rng.choice(NB * bs, size=T, replace=False).astype(np.int64)
    slots[[3, 17]] = -1                 # padding rows are skipped
    slots[25] = NB * bs + 5             # out of range: skipped
    kc = W.host_values((NB, Hkv, bs, D), 1.0, 1, dtype)
    vc = W.host_values((NB, Hkv, bs, D), 1.0, 2, dtype)
    key = W.host_values((T, Hkv, D), 1.0, 3, dtype)
    val = W.host_values((T, Hkv, D), 1.0, 4, dtype)
    kg, vg = to_gpu(kc), to_gpu(vc)
    pa.kv_cache_write(to_gpu(key), to_gpu(val), kg, vg, to_gpu(slots))
    torch_mod().cuda.synchronize()
    ok_slots = slots.copy()
    ok_slots[25] = -1
    oracle.kv_cache_write(key, val, kc, vc, ok_slots)
    assert np.array_equal(to_host(kg), kc)
    assert np.array_equal(to_host(vg), vc)


@pytest.mark.parametrize("dtype,Hkv,bs,D", [
    ("bf16", 8, 16, 128),     # 2048 16-byte chunks per block: two rounds of 4 per thread
    ("f32", 8, 16, 128),      # four rounds
    ("bf16", 5, 32, 128),     # 2560 chunks: two rounds and a tail of 512
    ("f32", 1, 8, 64),        # 128 chunks: the tail loop alone, half the threads idle
])
def test_block_copy_bit_exact(pa, dtype, Hkv, bs, D):
    NB = 40
    kc = W.host_values((NB, Hkv, bs, D), 1.0, 5, dtype)
    vc = W.host_values((NB, Hkv, bs, D), 1.0, 6, dtype)
    pairs = np.array([[1, 30], [2, 31], [7, 7], [9, 33], [0, 39], [12, NB + 3]], np.int64)
    kg, vg = to_gpu(kc), to_gpu(vc)
    pa.block_copy(kg, vg, to_gpu(pairs))
    torch_mod().cuda.synchronize()
    oracle.block_copy(kc, vc, pairs[:-1])
    assert np.array_equal(to_host(kg), kc)
    assert np.array_equal(to_host(vg), vc)


@pytest.mark.parametrize("dtype,bs,staging_blocks", [("bf16", 16, 3), ("f32", 8, 1000), ("bf16", 128, 1)])
def test_swap_out_in_bit_exact(pa, dtype, bs, staging_blocks):
    """Swap-out image and swap-in result against the oracle, bit for bit; the staging
    buffer forces several chunks; bad ids give zero pieces out and are skipped in."""
    torch = torch_mod()
    NB, Hkv, D = 40, 4, 128
    k = W.host_values((NB, Hkv, bs, D), 1.0, 31, dtype)
    v = W.host_values((NB, Hkv, bs, D), 1.0, 32, dtype)
    ids = np.array([17, 3, 39, 0, NB + 2, 25, 8, -1, 30, 11], np.int64)
    new = np.array([5, 6, 7, 9, 12, 13, 14, 15, 1, -4], np.int64)
    blk = Hkv * bs * D * k.itemsize
    kg, vg = to_gpu(k), to_gpu(v)
    staging = torch.empty(staging_blocks * 2 * blk, dtype=torch.uint8, device="cuda")
    host = torch.empty(len(ids) * 2 * blk, dtype=torch.uint8, pin_memory=True)
    host.fill_(0xCD)
    pa.kv_swap_out(kg, vg, to_gpu(ids), host, staging)
    torch.cuda.synchronize()
    img = oracle.swap_out(k, v, ids)
    assert np.array_equal(host.numpy().reshape(img.shape), img)
    # swap the image back into other blocks of the caches
    pa.kv_swap_in(kg, vg, to_gpu(new), host, staging)
    torch.cuda.synchronize()
    k2, v2 = k.copy(), v.copy()
    oracle.swap_in(k2, v2, new, img)
    assert np.array_equal(to_host(kg), k2) and np.array_equal(to_host(vg), v2)


def test_empty_calls_are_noops(pa):
    torch = torch_mod()
    kc = torch.zeros(4, 2, 16, 64, device="cuda")
    pa.kv_cache_write(torch.zeros(0, 2, 64, device="cuda"), torch.zeros(0, 2, 64, device="cuda"), kc,
                      kc.clone(), torch.zeros(0, dtype=torch.int64, device="cuda"))
    pa.block_copy(kc, kc.clone(), torch.zeros(0, 2, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert float(kc.abs().sum()) == 0.0


# ----------------------------------------------------------------------------- decode
def test_decode_tiny_fp32(pa):
    """The tiny fp32 configuration, also checked against contiguous attention."""
    w = W.tiny_decode()
    q = W.host_values(w.q_shape(), w.std, 101, w.dtype)
    k = W.host_values(w.cache_shape(), w.std, 102, w.dtype)
    v = W.host_values(w.cache_shape(), w.std, 103, w.dtype)
    ref = oracle.paged_decode(q, k, v, w.layout.block_tables, w.layout.seq_lens, w.scale)
    out = out_to_f64(gpu_decode(pa, w.layout, q, k, v, w.scale))
    assert max_err(out, ref) <= TOL["f32"], max_err(out, ref)
    for b, L in enumerate(w.layout.seq_lens):
        rows = [(w.layout.block_tables[b, t // 16], t % 16) for t in range(L)]
        Kc = np.stack([k[blk, :, off] for blk, off in rows]).astype(np.float64)
        Vc = np.stack([v[blk, :, off] for blk, off in rows]).astype(np.float64)
        cont = oracle.contiguous_attention(q[b:b + 1].astype(np.float64), Kc, Vc, [L], w.scale)[0]
        assert max_err(out[b], cont) <= TOL["f32"]


DECODE_CASES = [
    # dtype, D, Hq, Hkv, out, partition
    ("bf16", 128, 32, 8, "f32", 0),      # the 8B shape, MFMA path
    ("bf16", 128, 64, 8, "f32", 512),    # the 70B shape (group 8), MFMA path
    ("bf16", 128, 16, 16, "f32", 64),    # MHA (group 1), MFMA path
    ("bf16", 128, 32, 2, "f32", 128),    # group 16, MFMA path
    ("bf16", 128, 32, 8, "bf16", 256),   # bf16 output
    ("bf16", 64, 8, 2, "f32", 32),       # head_dim 64 bf16 (vector path)
    ("f32", 64, 8, 2, "f32", 48),        # fp32, vector path
    ("f32", 128, 12, 4, "f32", 0),       # fp32, head_dim 128
    ("bf16", 128, 24, 8, "f32", 16),     # group 3, one block per partition
]


@pytest.mark.parametrize("dtype,D,Hq,Hkv,out_dtype,part", DECODE_CASES)
def test_decode_parity(pa, dtype, D, Hq, Hkv, out_dtype, part):
    P = part or 256
    lens = [1, 2, 15, 16, 17, P - 1, P, P + 1, 2 * P + 1, 3 * P + 7, 40, 5]
    lay, q, k, v = rand_problem(lens, Hq, Hkv, D, 16, dtype, seed=D + Hq + Hkv + part)
    scale = 1.0 / math.sqrt(D)
    ref = oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, scale)
    out = out_to_f64(gpu_decode(pa, lay, q, k, v, scale, out_dtype, part))
    tol = TOL[dtype]
    if out_dtype == "bf16":
        # the output format's own rounding on top of the bar: round-to-nearest
        # into bf16 (8 significant bits) moves a value by at most 2^-8 of it
        excess = np.abs(out - ref) - (tol + (np.abs(ref) + tol) * 2.0 ** -8)
        assert excess.max() <= 0, "bf16 output off by %.3e beyond the bar" % excess.max()
        return
    err = max_err(out, ref)
    assert err <= tol, "max abs err %.3e" % err
    assert np.isfinite(out).all()


@pytest.mark.parametrize("dtype,bs", [("f32", 1), ("bf16", 8), ("bf16", 32), ("f32", 64)])
def test_decode_other_block_sizes(pa, dtype, bs):
    lens = [1, 7, 64, 65, 300]
    lay, q, k, v = rand_problem(lens, 8, 2, 64, bs, dtype, seed=bs + 50)
    ref = oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, 0.125)
    out = out_to_f64(gpu_decode(pa, lay, q, k, v, 0.125, "f32", 0))
    assert max_err(out, ref) <= TOL[dtype]


MFMA_BLOCK_SIZES = [8, 32, 64, 128]


@pytest.mark.parametrize("bs", MFMA_BLOCK_SIZES)
def test_decode_mfma_block_sizes(pa, bs):
    """bf16 / head_dim 128 at every block size the MFMA kernels walk in 16-token
    tiles: lengths around the block and tile edges, on the balanced split (auto
    and explicit pieces) and on the partition grid (one-tile pieces of a long row)."""
    lens = [0, 1, 7, 8, 9, 15, 16, 17, bs - 1, bs, bs + 1, 2 * bs + 3, 333, 1000]
    lay, q, k, v = rand_problem(lens, 32, 8, 128, bs, "bf16", seed=400 + bs)
    ref = oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, 0.09)
    for part in (0, max(bs, 64), 4 * bs, bs):
        out = out_to_f64(gpu_decode(pa, lay, q, k, v, 0.09, "f32", part))
        err = max_err(out, ref)
        assert err <= TOL["bf16"], (part, err)
        assert np.all(out[0] == 0)
    # a long row cut into one-tile pieces takes the partition grid
    lens = [3000, 5, 2049]
    lay, q, k, v = rand_problem(lens, 32, 8, 128, bs, "bf16", seed=500 + bs)
    ref = oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, 0.09)
    out = out_to_f64(gpu_decode(pa, lay, q, k, v, 0.09, "f32", bs))
    assert max_err(out, ref) <= TOL["bf16"]


@pytest.mark.parametrize("bs", [8, 64])
def test_decode_block_size_permutation_bit_exact(pa, bs):
    lens = [33, 700, 5, 1029]
    lay, q, k, v = rand_problem(lens, 32, 8, 128, bs, "bf16", seed=78)
    lay2 = synth.build_paged_layout(lens, bs, seed=4321, pool_factor=1.9)
    k2 = np.zeros((lay2.num_blocks,) + k.shape[1:], k.dtype)
    v2 = np.zeros_like(k2)
    for b, L in enumerate(lens):
        for j in range((L + bs - 1) // bs):
            k2[lay2.block_tables[b, j]] = k[lay.block_tables[b, j]]
            v2[lay2.block_tables[b, j]] = v[lay.block_tables[b, j]]
    for part in (0, 128):
        o1 = gpu_decode(pa, lay, q, k, v, 0.1, "f32", part).cpu().numpy()
        o2 = gpu_decode(pa, lay2, q, k2, v2, 0.1, "f32", part).cpu().numpy()
        assert np.array_equal(o1, o2), part


@pytest.mark.parametrize("bs", [8, 16, 64])
def test_decode_bad_table_entry_is_contained(pa, bs):
    """An out-of-range block id is masked, never dereferenced: the other
    sequences still match the oracle and every output is finite."""
    lens = [500, 300, 77, 1000]
    lay, q, k, v = rand_problem(lens, 32, 8, 128, bs, "bf16", seed=90 + bs)
    ref = oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, 0.1)
    bad = lay.block_tables.copy()
    bad[1, 3] = lay.num_blocks + 5
    bad[3, (1000 // bs) - 1] = -3
    lay_bad = synth.PagedLayout(seq_lens=lay.seq_lens, block_tables=bad, num_blocks=lay.num_blocks,
                                block_size=bs)
    for part in (0, 16 if bs <= 16 else bs):
        out = out_to_f64(gpu_decode(pa, lay_bad, q, k, v, 0.1, "f32", part))
        assert np.isfinite(out).all(), part
        for b in (0, 2):
            assert max_err(out[b], ref[b]) <= TOL["bf16"], (part, b)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_permutation_bit_exact(pa, dtype):
    """Same logical K/V under another physical permutation: identical bits."""
    D, Hq, Hkv = (128, 32, 8) if dtype == "bf16" else (64, 8, 2)
    lens = [33, 700, 5, 1029]
    lay, q, k, v = rand_problem(lens, Hq, Hkv, D, 16, dtype, seed=77)
    lay2 = synth.build_paged_layout(lens, 16, seed=12345, pool_factor=1.7)
    k2 = np.zeros((lay2.num_blocks,) + k.shape[1:], k.dtype)
    v2 = np.zeros_like(k2)
    for b, L in enumerate(lens):
        for j in range((L + 15) // 16):
            k2[lay2.block_tables[b, j]] = k[lay.block_tables[b, j]]
            v2[lay2.block_tables[b, j]] = v[lay.block_tables[b, j]]
    o1 = gpu_decode(pa, lay, q, k, v, 0.1, "f32", 128).cpu().numpy()
    o2 = gpu_decode(pa, lay2, q, k2, v2, 0.1, "f32", 128).cpu().numpy()
    assert np.array_equal(o1, o2)


def test_decode_partition_size_independence(pa):
    lens = [2000, 513, 1, 4096]
    lay, q, k, v = rand_problem(lens, 32, 8, 128, 16, "bf16", seed=91)
    ref = oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, 0.09)
    for part in (16, 64, 256, 512, 1024, 4096):
        out = out_to_f64(gpu_decode(pa, lay, q, k, v, 0.09, "f32", part))
        assert max_err(out, ref) <= TOL["bf16"], part


def test_decode_vector_default_pieces_many_rows(pa):
    """fp32 caches at the 8B shape's row count (64 sequences x 8 KV heads): with partition_size 0 the vector
    path takes long pieces (here 1024 tokens, so the longest rows split in two and go through the merge),
    and every row matches the oracle; explicit 256-token pieces agree with it to the same bar."""
    rng = np.random.default_rng(93)
    lens = [int(x) for x in rng.integers(1, 1100, size=60)] + [1, 1023, 1024, 1025]
    lay, q, k, v = rand_problem(lens, 32, 8, 128, 16, "f32", seed=93)
    ref = oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, 0.088)
    out = out_to_f64(gpu_decode(pa, lay, q, k, v, 0.088, "f32", 0))
    assert max_err(out, ref) <= TOL["f32"]
    out256 = out_to_f64(gpu_decode(pa, lay, q, k, v, 0.088, "f32", 256))
    assert max_err(out256, ref) <= TOL["f32"]
    assert np.isfinite(out).all()


def test_decode_zero_length_gives_zeros(pa):
    lens = [0, 20, 0]
    lay, q, k, v = rand_problem(lens, 32, 8, 128, 16, "bf16", seed=5)
    out = out_to_f64(gpu_decode(pa, lay, q, k, v, 0.1))
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    ref = oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, 0.1)
    assert max_err(out[1], ref[1]) <= TOL["bf16"]


def test_decode_deterministic(pa):
    lens = [100, 3000, 257]
    lay, q, k, v = rand_problem(lens, 32, 8, 128, 16, "bf16", seed=6)
    o1 = gpu_decode(pa, lay, q, k, v, 0.1).cpu().numpy()
    o2 = gpu_decode(pa, lay, q, k, v, 0.1).cpu().numpy()
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("bs", [16, 8])
def test_mixed_modes_trace(pa, bs):
    """Beam search, parallel sampling and greedy rows in one batch over 24 steps: every step's
    copy-on-write copies, new-token writes and decode match the oracle replaying the same trace."""
    torch = torch_mod()
    tr = W.mixed_decode_trace(beam_groups=3, beam_width=4, sample_groups=2, samples=3, greedy=3, steps=24,
                              block_size=bs, seed=9, num_heads=16, num_kv_heads=4)
    B, Hq, Hkv, D = tr.batch, tr.num_heads, tr.num_kv_heads, tr.head_dim
    k = W.host_values((tr.num_blocks, Hkv, bs, D), 0.5, 61, "bf16")
    v = W.host_values((tr.num_blocks, Hkv, bs, D), 0.5, 62, "bf16")
    q = W.host_values((B, Hq, D), 0.5, 63, "bf16")
    nk = W.host_values((B, Hkv, D), 0.5, 64, "bf16")
    nv = W.host_values((B, Hkv, D), 0.5, 65, "bf16")
    kg, vg, qg, nkg, nvg = to_gpu(k), to_gpu(v), to_gpu(q), to_gpu(nk), to_gpu(nv)
    max_len = int(max(int(x.max()) for x in tr.seq_lens))
    ws = torch.empty(max(pa.paged_attn_decode_workspace_size(B, Hq, Hkv, D, bs, max_len, 0), 1),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hq, D, device="cuda")
    assert sum(len(c) for c in tr.copies) > 0
    for s in range(len(tr.tables)):
        if tr.copies[s]:
            pa.block_copy(kg, vg, to_gpu(np.asarray(tr.copies[s], np.int64)))
            oracle.block_copy(k, v, tr.copies[s])
        pa.kv_cache_write(nkg, nvg, kg, vg, to_gpu(tr.slots[s]))
        oracle.kv_cache_write(nk, nv, k, v, tr.slots[s])
        pa.paged_attn_decode(out, qg, kg, vg, to_gpu(tr.tables[s]), to_gpu(tr.seq_lens[s]), tr.scale, max_len, 0, ws)
        ref = oracle.paged_decode(q, k, v, tr.tables[s], tr.seq_lens[s], tr.scale)
        assert max_err(out_to_f64(out), ref) <= TOL["bf16"], s
    assert np.array_equal(to_host(kg), k) and np.array_equal(to_host(vg), v)


# ----------------------------------------------------------------------------- prefill
def gpu_prefill(pa, lay, chunk_lens, q, k, v, scale, out_dtype="f32"):
    torch = torch_mod()
    qsl = np.concatenate([[0], np.cumsum(chunk_lens)]).astype(np.int32)
    Tq, Hq, D = q.shape
    out = torch.empty((Tq, Hq, D), dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16, device="cuda")
    pa.paged_attn_prefill_chunk(out, to_gpu(q), to_gpu(k), to_gpu(v), to_gpu(lay.block_tables.astype(np.int32)),
                                to_gpu(qsl), to_gpu(lay.seq_lens.astype(np.int32)), scale,
                                int(max(chunk_lens)), int(lay.seq_lens.max()))
    torch.cuda.synchronize()
    return out, qsl


PREFILL_CASES = [
    ("bf16", 128, 32, 8),     # 8B shape: MFMA path, 4 tokens x 4 heads per wave
    ("bf16", 128, 64, 8),     # group 8
    ("bf16", 128, 8, 8),      # group 1
    ("f32", 64, 8, 2),        # vector path
    ("bf16", 128, 24, 8),     # group 3: three one-head sub-groups on the MFMA kernel
    ("bf16", 128, 48, 4),     # group 12: three sub-groups of 4 heads
    ("bf16", 128, 32, 1),     # group 32: two sub-groups of 16 heads
    ("bf16", 128, 40, 8),     # group 5
    ("bf16", 64, 24, 8),      # head size 64, group 3: vector path
]


@pytest.mark.parametrize("dtype,D,Hq,Hkv", PREFILL_CASES)
def test_prefill_parity(pa, dtype, D, Hq, Hkv):
    total = [40, 64, 17, 5, 300, 1, 129]
    chunk = [13, 64, 1, 5, 37, 1, 128]     # chunks starting mid-block, at 0, and of one row
    lay, _, k, v = rand_problem(total, Hq, Hkv, D, 16, dtype, seed=D + Hq)
    q = W.host_values((sum(chunk), Hq, D), 1.0, 4242, dtype)
    qsl = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    scale = 1.0 / math.sqrt(D)
    ref = oracle.paged_prefill(q, k, v, lay.block_tables, qsl, lay.seq_lens, scale)
    out, _ = gpu_prefill(pa, lay, chunk, q, k, v, scale)
    err = max_err(out_to_f64(out), ref)
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_prefill_peaked_softmax(pa, dtype):
    """Scores three times sharper than N(0,1) (a few keys carry most of the weight), where rounding
    each weight once to fp16 for the PV product matters most: still within the bf16 bar, for short
    rows (1-5 visible keys) and long ones."""
    total = [1, 3, 5, 40, 300, 1029]
    chunk = [1, 3, 2, 13, 37, 129]
    Hq, Hkv, D, bs = 32, 8, 128, 16
    lay = synth.build_paged_layout(total, bs, seed=91, pool_factor=1.3)
    shape = (lay.num_blocks, Hkv, bs, D)
    q = W.host_values((sum(chunk), Hq, D), 3.0, 9103, "bf16")
    qsl = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    scale = 1.0 / math.sqrt(D)
    if dtype == "fp8":
        ks, vs = 0.0071, 0.0093
        k = oracle.fp8_encode(W.host_values(shape, 1.0, 9101, "f32") / np.float32(ks))
        v = oracle.fp8_encode(W.host_values(shape, 1.0, 9102, "f32") / np.float32(vs))
        ref = oracle.paged_prefill(q, k, v, lay.block_tables, qsl, lay.seq_lens, scale, k_scale=ks, v_scale=vs)
        out = torch_mod().full((sum(chunk), Hq, D), float("nan"), device="cuda")
        pa.paged_attn_prefill_chunk_fp8(out, to_gpu(q), to_gpu(k), to_gpu(v), ks, vs,
                                        to_gpu(lay.block_tables.astype(np.int32)), to_gpu(qsl),
                                        to_gpu(lay.seq_lens.astype(np.int32)), scale, int(max(chunk)), int(max(total)))
        torch_mod().cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
    else:
        k = W.host_values(shape, 1.0, 9101, "bf16")
        v = W.host_values(shape, 1.0, 9102, "bf16")
        ref = oracle.paged_prefill(q, k, v, lay.block_tables, qsl, lay.seq_lens, scale)
        out, _ = gpu_prefill(pa, lay, chunk, q, k, v, scale)
        got = out_to_f64(out)
    err = max_err(got, ref)
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("bs", MFMA_BLOCK_SIZES)
def test_prefill_mfma_block_sizes(pa, bs):
    total = [40, 64, 17, 5, 300, 1, 129, 2 * bs + 3]
    chunk = [13, 64, 1, 5, 37, 1, 128, bs + 2]
    lay, _, k, v = rand_problem(total, 32, 8, 128, bs, "bf16", seed=600 + bs)
    q = W.host_values((sum(chunk), 32, 128), 1.0, 4343 + bs, "bf16")
    qsl = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    ref = oracle.paged_prefill(q, k, v, lay.block_tables, qsl, lay.seq_lens, 0.088)
    out, _ = gpu_prefill(pa, lay, chunk, q, k, v, 0.088)
    err = max_err(out_to_f64(out), ref)
    assert err <= TOL["bf16"], err


def repack_blocks(lay, k, v, lens, bs, seed, pool_factor=1.8):
    """The same logical K/V under another physical block permutation (and a
    larger pool): every block of every sequence moved, with its unused tail
    slots, to the id a fresh seeded layout gives it; unused ids hold zeros."""
    lay2 = synth.build_paged_layout(lens, bs, seed=seed, pool_factor=pool_factor)
    k2 = np.zeros((lay2.num_blocks,) + k.shape[1:], k.dtype)
    v2 = np.zeros_like(k2)
    for b, L in enumerate(lens):
        for j in range((L + bs - 1) // bs):
            k2[lay2.block_tables[b, j]] = k[lay.block_tables[b, j]]
            v2[lay2.block_tables[b, j]] = v[lay.block_tables[b, j]]
    assert not np.array_equal(lay2.block_tables[:, :4], lay.block_tables[:, :4])
    return lay2, k2, v2


@pytest.mark.parametrize("kv,bs", [("bf16", 16), ("bf16", 8), ("fp8", 16), ("fp8", 8)])
def test_prefill_permutation_bit_exact(pa, kv, bs):
    """Paging changes where the KV lives, not what is computed (Lecture 7 §4.2; Lecture 16 §3.3): the
    chunked prefill over the same logical K/V in another physical permutation gives identical bits,
    for chunks that start mid-block, at 0, and span several query tiles."""
    torch = torch_mod()
    total = [40, 700, 17, 1029, 300, 1]
    chunk = [13, 200, 1, 129, 37, 1]
    Hq, Hkv, D = 32, 8, 128
    lay = synth.build_paged_layout(total, bs, seed=31 + bs, pool_factor=1.3)
    shape = (lay.num_blocks, Hkv, bs, D)
    if kv == "fp8":
        ks, vs = 0.0071, 0.0093
        k = oracle.fp8_encode(W.host_values(shape, 1.0, 811, "f32") / np.float32(ks))
        v = oracle.fp8_encode(W.host_values(shape, 1.0, 812, "f32") / np.float32(vs))
    else:
        k = W.host_values(shape, 1.0, 811, "bf16")
        v = W.host_values(shape, 1.0, 812, "bf16")
    q = W.host_values((sum(chunk), Hq, D), 1.0, 813, "bf16")
    qsl = to_gpu(np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32))
    lay2, k2, v2 = repack_blocks(lay, k, v, total, bs, seed=977 + bs)
    outs = []
    for L_, k_, v_ in ((lay, k, v), (lay2, k2, v2)):
        out = torch.full((sum(chunk), Hq, D), float("nan"), device="cuda")
        args = (to_gpu(L_.block_tables.astype(np.int32)), qsl, to_gpu(L_.seq_lens.astype(np.int32)), 0.0884,
                int(max(chunk)), int(max(total)))
        if kv == "fp8":
            pa.paged_attn_prefill_chunk_fp8(out, to_gpu(q), to_gpu(k_), to_gpu(v_), ks, vs, *args)
        else:
            pa.paged_attn_prefill_chunk(out, to_gpu(q), to_gpu(k_), to_gpu(v_), *args)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.isfinite(outs[0]).all()
    assert np.array_equal(outs[0], outs[1]), "max difference %.3g" % np.max(np.abs(outs[0] - outs[1]))
    # and the values are right
    qsl_h = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    kvs = dict(k_scale=ks, v_scale=vs) if kv == "fp8" else {}
    ref = oracle.paged_prefill(q, k, v, lay.block_tables, qsl_h, lay.seq_lens, 0.0884, **kvs)
    assert max_err(outs[0].astype(np.float64), ref) <= TOL["bf16"]


def test_prefill_one_row_equals_decode(pa):
    lens = [77, 300, 16]
    lay, q, k, v = rand_problem(lens, 32, 8, 128, 16, "bf16", seed=8)
    out_p, _ = gpu_prefill(pa, lay, [1, 1, 1], q, k, v, 0.1)
    out_d = gpu_decode(pa, lay, q, k, v, 0.1, "f32", 16 * 1024)
    # different wave splits round the weights differently: compare at the bf16 bar
    assert max_err(out_to_f64(out_p), out_to_f64(out_d)) <= TOL["bf16"]


# ----------------------------------------------------------------------------- balanced decode specifics
def test_decode_one_row_split_over_many_ranges(pa):
    """One KV head, one long row: fixed one- and three-tile pieces take the partition grid; the library's
    own split cuts the row over 313 one-tile ranges, whose merge shares the row out over those ranges."""
    lens = [5000]
    lay, q, k, v = rand_problem(lens, 16, 1, 128, 16, "bf16", seed=13)
    ref = oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, 0.088)
    for part in (16, 48, 0):
        out = out_to_f64(gpu_decode(pa, lay, q, k, v, 0.088, "f32", part))
        assert max_err(out, ref) <= TOL["bf16"], part


@pytest.mark.parametrize("lens,Hq,Hkv,bs,part", [
    ([5000], 8, 1, 16, 0),                 # one row over 313 ranges: 16-element chunks
    ([2000] * 7, 64, 8, 16, 0),            # 56 rows of 10-11 pieces: 64-element chunks, some workgroups take
                                           # two, many rows' first pieces in slot 1
    ([3000, 0, 1500, 7], 16, 16, 32, 0),   # group 1: 128 elements over a 256-thread workgroup
    ([2500, 900], 32, 2, 64, 0),           # group 16
    ([3000] * 4, 32, 8, 16, 256),          # a caller's 256-token pieces: 12 or 13 per row, fixed-size ranges
])
def test_decode_long_rows_shared_merge(pa, lens, Hq, Hkv, bs, part):
    """Rows cut into more than eight pieces: the merge deals each row's output elements out, in chunks of 16
    to 64, to the ranges holding the row, and its pieces to the threads of each; every output matches the
    oracle, empty rows are zero, and repeats are bit-identical."""
    torch = torch_mod()
    lay, q, k, v = rand_problem(lens, Hq, Hkv, 128, bs, "bf16", seed=31 + Hq + bs)
    ref = oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, 0.085)
    first = gpu_decode(pa, lay, q, k, v, 0.085, "f32", part)
    out = out_to_f64(first)
    assert max_err(out, ref) <= TOL["bf16"], max_err(out, ref)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(out[b] == 0)
    again = gpu_decode(pa, lay, q, k, v, 0.085, "f32", part)
    assert torch.equal(first, again)


@pytest.mark.parametrize("Hq,Hkv", [(32, 1), (96, 2), (48, 2), (40, 2), (17, 1), (64, 1)])
def test_decode_large_groups(pa, Hq, Hkv):
    """GQA groups above 16 query heads (32, 48, 24, 20, 17, 64): the balanced decode serves each as sub-groups
    of at most 16 heads (16, 16, 12, 10, 1 and 16 heads), each its own row over the same K/V; with a caller's
    pieces of more than 16 per row the vector kernels serve the group.  Every output matches the oracle."""
    lens = [0, 1, 17, 300, 1000, 2049, 5]
    lay, q, k, v = rand_problem(lens, Hq, Hkv, 128, 16, "bf16", seed=Hq + Hkv)
    ref = oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, 0.09)
    for part, odt in ((0, "f32"), (256, "bf16"), (16, "f32")):
        out = out_to_f64(gpu_decode(pa, lay, q, k, v, 0.09, odt, part))
        if odt == "bf16":
            excess = np.abs(out - ref) - (TOL["bf16"] + np.abs(ref) * 2.0 ** -8)
            assert excess.max() <= 0, (part, excess.max())
        else:
            assert max_err(out, ref) <= TOL["bf16"], (part, max_err(out, ref))
        assert np.all(out[0] == 0)


def test_decode_workspace_reuse_and_garbage(pa):
    """Stale or garbage workspace contents are ignored: every piece the merge reads was written earlier in
    the same call, so repeated calls on one workspace filled with garbage all match the oracle."""
    torch = torch_mod()
    lens = [300, 1, 0, 2048, 77, 0, 513]
    lay, q, k, v = rand_problem(lens, 32, 8, 128, 16, "bf16", seed=17)
    B, Hq, D = q.shape
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    bt, sl = to_gpu(lay.block_tables), to_gpu(lay.seq_lens)
    ref = oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, 0.1)
    wsb = pa.paged_attn_decode_workspace_size(B, Hq, 8, D, 16, 2048, 32)
    ws = torch.full((wsb,), 0xAB, dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hq, D, device="cuda")
    for rep in range(3):
        out.fill_(float("nan"))
        pa.paged_attn_decode(out, qg, kg, vg, bt, sl, 0.1, 2048, 32, ws)
        torch.cuda.synchronize()
        o = out_to_f64(out)
        assert np.isfinite(o).all(), rep
        assert max_err(o, ref) <= TOL["bf16"], rep
        assert np.all(o[2] == 0) and np.all(o[5] == 0)


def test_decode_partial_handoff_stress(pa):
    """Thousands of partial rows handed between workgroups on all XCDs, repeated: every repeat
    matches the oracle and is bit-identical to the first."""
    torch = torch_mod()
    lens = [4096, 3001, 4096, 17, 2500, 4096, 1, 3333]
    lay, q, k, v = rand_problem(lens, 64, 8, 128, 16, "bf16", seed=23)
    B, Hq, D = q.shape
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    bt, sl = to_gpu(lay.block_tables), to_gpu(lay.seq_lens)
    ref = oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, 0.09)
    for part in (16, 32, 0):
        wsb = pa.paged_attn_decode_workspace_size(B, Hq, 8, D, 16, 4096, part)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        out = torch.empty(B, Hq, D, device="cuda")
        first = None
        for rep in range(20):
            pa.paged_attn_decode(out, qg, kg, vg, bt, sl, 0.09, 4096, part, ws)
            o = out.cpu().numpy()
            if first is None:
                first = o.copy()
                assert max_err(o.astype(np.float64), ref) <= TOL["bf16"], part
            else:
                assert np.array_equal(o, first), (part, rep)
