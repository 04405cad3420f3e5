"""GPU: parity at the full benchmark configurations, in the launch
configuration bench.py times (decode: one plan per step, the planned call,
library-chosen partitioning; prefill: the MFMA grid).  Decode is checked on
every row of every batch; the chunked prefill on two rows of every 32-row
query tile of every sequence (one tile is one workgroup's work), at offsets
that vary from tile to tile so every wave and column group is covered.  The
oracle computes the rows one at a time, spread over host threads (its
ctypes calls release the interpreter lock).

Inputs come from the same seeded generators as the benchmark (device draws,
copied to the host for the oracle).  Shapes: Llama-3.1-8B-shaped decode (64
lognormal rows, Hq 32 / Hkv 8), the 70B-shaped 8 x 32K decode (Hq 64 / Hkv 8),
parallel sampling over shared prompts, and the 16 x (1024 + 512) chunked
prefill, in bf16 and with FP8 caches."""
import concurrent.futures
import os

import numpy as np
import pytest

import oracle
from synth import workloads as W
from gpu_helpers import TOL, max_err, require_gpu, to_host, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    mod = require_gpu()
    oracle.build(force=False)
    return mod


def _fp8_pool(torch, shape, std, seed):
    """FP8 E4M3 codes of N(0, std) draws under one per-tensor scale max|x| / 448."""
    x = W.device_values(shape, std, seed, "f32")
    s = float(x.abs().max()) / 448.0
    codes = (x / s).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, s


def _decode_planned(pa, torch, w, K, V, q, partition=0, k_scale=1.0, v_scale=1.0, fp8=False):
    B, Hq, Hkv, D = w.layout.batch, w.num_heads, w.num_kv_heads, w.head_dim
    lens = w.layout.seq_lens
    max_len = int(lens.max())
    bt = torch.from_numpy(w.layout.block_tables).cuda()
    sl = torch.from_numpy(lens.astype(np.int32)).cuda()
    out = torch.full((B, Hq, D), float("nan"), device="cuda", dtype=torch.float32)
    wsb = pa.paged_attn_decode_workspace_size(B, Hq, Hkv, D, w.block_size, max_len, partition)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    kvd = pa.PA_FP8_E4M3 if fp8 else pa._dtype_code(K)
    psize = pa.paged_attn_decode_plan_size(B, Hq, Hkv, D, w.block_size, w.layout.block_tables.shape[1], max_len,
                                           partition, kvd)
    if psize > 0:
        plan = torch.empty(psize, dtype=torch.uint8, device="cuda")
        pa.paged_attn_decode_plan(plan, K, bt, sl, Hq, max_len, partition)
        pa.paged_attn_decode_planned(out, q, K, V, plan, bt, sl, w.scale, max_len, partition, ws,
                                     k_scale=k_scale, v_scale=v_scale)
    elif fp8:
        pa.paged_attn_decode_fp8(out, q, K, V, k_scale, v_scale, bt, sl, w.scale, max_len, partition, ws)
    else:
        pa.paged_attn_decode(out, q, K, V, bt, sl, w.scale, max_len, partition, ws)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def _check_decode_rows(w, got, qh, Kh, Vh, tol, k_scale=None, v_scale=None):
    """Every row of the batch against the oracle, rows spread over threads."""
    lens = w.layout.seq_lens
    assert np.isfinite(got).all()

    def one(b):
        ref = oracle.paged_decode(qh[b:b + 1], Kh, Vh, w.layout.block_tables[b:b + 1], lens[b:b + 1], w.scale,
                                  k_scale=k_scale, v_scale=v_scale)
        return b, max_err(got[b:b + 1], ref)

    order = [int(b) for b in np.argsort(-lens)]  # longest first keeps the pool busy
    with concurrent.futures.ThreadPoolExecutor(max_workers=_threads()) as ex:
        errs = dict(ex.map(one, order))
    worst = max(errs, key=errs.get)
    assert errs[worst] <= tol, "row %d (length %d): max abs error %.3g" % (worst, lens[worst], errs[worst])
    return errs


DECODE_CONFIGS = [
    # workload, partition
    ("llama8b_decode", 0),
    ("llama70b_long", 0),
    ("llama70b_long", 512),
    ("shared_prefix", 0),
]


@pytest.mark.parametrize("name,partition", DECODE_CONFIGS)
def test_full_config_decode_bf16(pa, name, partition):
    torch = torch_mod()
    w = getattr(W, name)()
    shape = w.cache_shape()
    K = W.device_values(shape, w.std, w.seed * 1000, w.dtype)
    V = W.device_values(shape, w.std, w.seed * 1000 + 1, w.dtype)
    q = W.device_values(w.q_shape(), w.std, w.seed * 1000 - 1, w.dtype)
    got = _decode_planned(pa, torch, w, K, V, q, partition)
    qh, Kh, Vh = to_host(q), to_host(K), to_host(V)
    del K, V
    errs = _check_decode_rows(w, got, qh, Kh, Vh, TOL["bf16"])
    print("%s partition %d: %d rows, max abs error %.3e" % (name, partition, len(errs), max(errs.values())))


@pytest.mark.parametrize("name", ["llama8b_decode", "llama70b_long"])
def test_full_config_decode_fp8(pa, name):
    torch = torch_mod()
    w = getattr(W, name)()
    shape = w.cache_shape()
    K, ks = _fp8_pool(torch, shape, w.std, w.seed * 1000)
    V, vs = _fp8_pool(torch, shape, w.std, w.seed * 1000 + 1)
    q = W.device_values(w.q_shape(), w.std, w.seed * 1000 - 1, "bf16")
    got = _decode_planned(pa, torch, w, K, V, q, 0, ks, vs, fp8=True)
    qh, Kh, Vh = to_host(q), to_host(K), to_host(V)
    del K, V
    errs = _check_decode_rows(w, got, qh, Kh, Vh, TOL["bf16"], k_scale=ks, v_scale=vs)
    print("%s fp8: %d rows, max abs error %.3e" % (name, len(errs), max(errs.values())))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_full_config_chunked_prefill(pa, kv):
    torch = torch_mod()
    w = W.chunked_prefill()
    lay = w.layout
    B, Hq, Hkv, D = lay.batch, w.num_heads, w.num_kv_heads, w.head_dim
    shape = (lay.num_blocks, Hkv, lay.block_size, D)
    if kv == "fp8":
        K, ks = _fp8_pool(torch, shape, w.std, w.seed * 1000)
        V, vs = _fp8_pool(torch, shape, w.std, w.seed * 1000 + 1)
    else:
        K = W.device_values(shape, w.std, w.seed * 1000, w.dtype)
        V = W.device_values(shape, w.std, w.seed * 1000 + 1, w.dtype)
        ks = vs = None
    qsl_h = w.query_start_loc
    Tq = int(qsl_h[-1])
    q = W.device_values((Tq, Hq, D), w.std, w.seed * 1000 - 1, "bf16")
    out = torch.full((Tq, Hq, D), float("nan"), device="cuda", dtype=torch.float32)
    bt = torch.from_numpy(lay.block_tables).cuda()
    qsl = torch.from_numpy(qsl_h.astype(np.int32)).cuda()
    sl = torch.from_numpy(lay.seq_lens.astype(np.int32)).cuda()
    mq, ms = int(w.chunk_lens.max()), int(lay.seq_lens.max())
    if kv == "fp8":
        pa.paged_attn_prefill_chunk_fp8(out, q, K, V, ks, vs, bt, qsl, sl, w.scale, mq, ms)
    else:
        pa.paged_attn_prefill_chunk(out, q, K, V, bt, qsl, sl, w.scale, mq, ms)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all()
    qh, Kh, Vh = to_host(q), to_host(K), to_host(V)
    kvs = dict(k_scale=ks, v_scale=vs) if kv == "fp8" else {}
    # two rows of every 32-row query tile of every sequence (a tile is one
    # workgroup: 4 waves x 2 column groups x 4 chunk tokens of the 4-head
    # group), at offsets that move from tile to tile, plus each sequence's
    # first and last chunk row
    tile_rows = 32
    cases = []
    for b in range(B):
        n = int(w.chunk_lens[b])
        rows = {0, n - 1}
        for t in range((n + tile_rows - 1) // tile_rows):
            for extra in (0, 17):
                i = t * tile_rows + (b * 5 + t * 11 + extra) % tile_rows
                if i < n:
                    rows.add(i)
        cases += [(b, i) for i in sorted(rows)]

    def one(case):
        b, i = case
        S, n = int(lay.seq_lens[b]), int(w.chunk_lens[b])
        r = int(qsl_h[b]) + i
        ref = oracle.paged_prefill(qh[r:r + 1], Kh, Vh, lay.block_tables[b:b + 1], np.array([0, 1], np.int32),
                                   np.array([S - n + i + 1], np.int32), w.scale, **kvs)
        return case, max_err(got[r:r + 1], ref)

    with concurrent.futures.ThreadPoolExecutor(max_workers=_threads()) as ex:
        errs = dict(ex.map(one, cases))
    worst = max(errs, key=errs.get)
    print("chunked prefill %s: %d rows checked, max abs error %.3e" % (kv, len(errs), errs[worst]))
    assert len(cases) >= 2 * B * (int(w.chunk_lens.min()) // tile_rows)
    assert errs[worst] <= TOL["bf16"], "sequence %d chunk row %d: max abs error %.3g" % (worst + (errs[worst],))
