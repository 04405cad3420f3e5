"""GPU: paged_attn_decode_append (the decode step with its KV write folded
in) against the same step done in two calls, kv_cache_write then
paged_attn_decode_planned, through the C ABI: outputs and both whole caches
bit for bit, and the output against the oracle (which writes the new rows
first, Lecture 7 §4.3 / §4.1).

Covered: bf16 caches on the balanced split (the folded path) at block sizes
16, 8 and 64, GQA groups 4 and 8, rows with no new token (slot -1), empty
rows, a new token at every offset of its tile, and a slot that names an
unused block instead of the appended position (the write still lands there;
that row then reads position L - 1 as it was); FP8 and fp32 caches (written
first, then decoded).
"""
import math

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as W
from gpu_helpers import TOL, max_err, out_to_f64, require_gpu, to_gpu, to_host, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    mod = require_gpu()
    oracle.build(force=False)
    return mod


def _setup(lens, Hq, Hkv, bs, dtype, seed, D=128):
    lay = synth.build_paged_layout(lens, bs, seed=seed, pool_factor=1.4)
    shape = (lay.num_blocks, Hkv, bs, D)
    qd = "bf16" if dtype in ("bf16", "fp8") else "f32"
    if dtype == "fp8":
        ks, vs = 0.0081, 0.0067
        k = oracle.fp8_encode(W.host_values(shape, 1.0, seed * 5 + 1, "f32") / np.float32(ks))
        v = oracle.fp8_encode(W.host_values(shape, 1.0, seed * 5 + 2, "f32") / np.float32(vs))
    else:
        ks = vs = None
        k = W.host_values(shape, 0.5, seed * 5 + 1, dtype)
        v = W.host_values(shape, 0.5, seed * 5 + 2, dtype)
    B = len(lens)
    q = W.host_values((B, Hq, D), 0.5, seed * 5 + 3, qd)
    nk = W.host_values((B, Hkv, D), 0.5, seed * 5 + 4, qd)
    nv = W.host_values((B, Hkv, D), 0.5, seed * 5 + 5, qd)
    # the appended position of every row with a token
    slots = np.array([synth.slots_for_positions(lay.block_tables[b], [L - 1], bs)[0] if L > 0 else -1
                      for b, L in enumerate(lens)], np.int64)
    return lay, q, k, v, nk, nv, slots, ks, vs


def _run(pa, lay, q, k, v, nk, nv, slots, ks, vs, fold):
    torch = torch_mod()
    B, Hq, D = q.shape
    Hkv, bs = k.shape[1], k.shape[2]
    kg, vg = to_gpu(k), to_gpu(v)
    if k.dtype == np.uint8:
        kvd = pa.PA_FP8_E4M3
    else:
        kvd = pa._dtype_code(kg)
    bt, sl = to_gpu(lay.block_tables.astype(np.int32)), to_gpu(lay.seq_lens.astype(np.int32))
    max_len = max(int(lay.seq_lens.max()), 1)
    wsb = pa.paged_attn_decode_workspace_size(B, Hq, Hkv, D, bs, max_len, 0)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    psize = pa.paged_attn_decode_plan_size(B, Hq, Hkv, D, bs, lay.block_tables.shape[1], max_len, 0, kvd)
    plan = torch.empty(psize, dtype=torch.uint8, device="cuda") if psize else None
    pa.paged_attn_decode_plan(plan, kg, bt, sl, Hq, max_len, 0)
    out = torch.full((B, Hq, D), float("nan"), device="cuda")
    qg, nkg, nvg, sg = to_gpu(q), to_gpu(nk), to_gpu(nv), to_gpu(slots)
    scale = 1.0 / math.sqrt(D)
    kw = dict(k_scale=ks, v_scale=vs) if ks is not None else {}
    if fold:
        pa.paged_attn_decode_append(out, qg, nkg, nvg, sg, kg, vg, plan, bt, sl, scale, max_len, 0, ws, **kw)
    else:
        if ks is not None:
            pa.kv_cache_write_fp8(nkg, nvg, kg, vg, sg, ks, vs)
        else:
            pa.kv_cache_write(nkg, nvg, kg, vg, sg)
        pa.paged_attn_decode_planned(out, qg, kg, vg, plan, bt, sl, scale, max_len, 0, ws, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), to_host(kg), to_host(vg), scale


CASES = [
    # dtype, block size, Hq, Hkv
    ("bf16", 16, 32, 8),
    ("bf16", 8, 32, 8),
    ("bf16", 64, 64, 8),
    ("fp8", 16, 32, 8),
    ("f32", 16, 8, 2),
    ("bf16", 16, 32, 1),    # a group of 32 (sub-groups): written first, then attended
]


@pytest.mark.parametrize("dtype,bs,Hq,Hkv", CASES)
def test_decode_append_equals_write_then_decode(pa, dtype, bs, Hq, Hkv):
    rng = np.random.default_rng(bs + Hq)
    lens = [int(x) for x in rng.integers(1, 1500, size=30)]
    lens += [16 * i + o for i, o in enumerate(range(16))]   # the new token at every offset of its tile
    lens += [0, 1, 2, 4096, 17]
    lay, q, k, v, nk, nv, slots, ks, vs = _setup(lens, Hq, Hkv, bs, dtype, seed=bs + 7)
    slots[3] = -1                                            # no new token for row 3
    # row 5's slot names a block no row uses: the write lands there, row 5 reads position L - 1 as it was
    used = set(int(x) for b, L in enumerate(lens) for x in lay.block_tables[b, :(L + bs - 1) // bs])
    free = [x for x in range(lay.num_blocks) if x not in used]
    assert free
    slots[5] = free[0] * bs + 3
    o1, k1, v1, scale = _run(pa, lay, q, k, v, nk, nv, slots, ks, vs, fold=True)
    o2, k2, v2, _ = _run(pa, lay, q, k, v, nk, nv, slots, ks, vs, fold=False)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2), "caches differ"
    assert np.array_equal(o1, o2), "outputs differ: max %.3g" % np.nanmax(np.abs(o1 - o2))
    # against the oracle: write first, then attend
    kh, vh = k.copy(), v.copy()
    if dtype == "fp8":
        oracle.kv_cache_write_fp8(nk[slots >= 0], nv[slots >= 0], kh, vh, slots[slots >= 0], ks, vs)
        ref = oracle.paged_decode(q, kh, vh, lay.block_tables, lay.seq_lens, scale, k_scale=ks, v_scale=vs)
    else:
        oracle.kv_cache_write(nk, nv, kh, vh, slots)
        ref = oracle.paged_decode(q, kh, vh, lay.block_tables, lay.seq_lens, scale)
    assert np.array_equal(k1, kh) and np.array_equal(v1, vh), "caches differ from the oracle's write"
    assert max_err(o1.astype(np.float64), ref) <= TOL["f32" if dtype == "f32" else "bf16"]


def test_decode_append_few_long_rows(pa):
    """Two long sequences of 8 KV heads, each row cut into dozens of pieces: the folded step (its merge shares
    every row out over the row's ranges and writes the new rows) against the two-call step and the oracle."""
    lens = [3000, 1201]
    lay, q, k, v, nk, nv, slots, ks, vs = _setup(lens, 64, 8, 16, "bf16", seed=61)
    o1, k1, v1, scale = _run(pa, lay, q, k, v, nk, nv, slots, ks, vs, fold=True)
    o2, k2, v2, _ = _run(pa, lay, q, k, v, nk, nv, slots, ks, vs, fold=False)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2), "caches differ"
    assert np.array_equal(o1, o2), "outputs differ: max %.3g" % np.nanmax(np.abs(o1 - o2))
    kh, vh = k.copy(), v.copy()
    oracle.kv_cache_write(nk, nv, kh, vh, slots)
    ref = oracle.paged_decode(q, kh, vh, lay.block_tables, lay.seq_lens, scale)
    assert max_err(o1.astype(np.float64), ref) <= TOL["bf16"]


def test_decode_append_full_config(pa):
    """The 8B-shaped decode step (64 lognormal rows) folded, in the configuration bench.py times, against the
    two-call step: bit-identical output and caches."""
    w = W.llama8b_decode()
    lens = w.layout.seq_lens
    B, Hq, Hkv, D = w.layout.batch, w.num_heads, w.num_kv_heads, w.head_dim
    k = W.host_values(w.cache_shape(), w.std, 901, "bf16")
    v = W.host_values(w.cache_shape(), w.std, 902, "bf16")
    q = W.host_values((B, Hq, D), w.std, 903, "bf16")
    nk = W.host_values((B, Hkv, D), w.std, 904, "bf16")
    nv = W.host_values((B, Hkv, D), w.std, 905, "bf16")
    slots = np.array([synth.slots_for_positions(w.layout.block_tables[b], [lens[b] - 1], 16)[0] for b in range(B)],
                     np.int64)
    o1, k1, v1, _ = _run(pa, w.layout, q, k, v, nk, nv, slots, None, None, fold=True)
    o2, k2, v2, _ = _run(pa, w.layout, q, k, v, nk, nv, slots, None, None, fold=False)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    assert np.array_equal(o1, o2)
