"""GPU: parity at the full benchmark configurations, in the launch
configuration bench.py times (decode: one plan per step, the planned call,
library-chosen partitioning; prefill: the MFMA grid), on sampled rows that
the oracle computes one at a time.

Inputs come from the same seeded generators as the benchmark (device draws,
copied to the host for the oracle).  Shapes: Llama-3.1-8B-shaped decode (64
lognormal rows, Hq 32 / Hkv 8), the 70B-shaped 8 x 32K decode (Hq 64 / Hkv 8),
parallel sampling over shared prompts, and the 16 x (1024 + 512) chunked
prefill, in bf16 and with FP8 caches."""
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


def _check_decode_rows(w, got, qh, Kh, Vh, rows, tol, k_scale=None, v_scale=None):
    lens = w.layout.seq_lens
    assert np.isfinite(got).all()
    for b in rows:
        ref = oracle.paged_decode(qh[b:b + 1], Kh, Vh, w.layout.block_tables[b:b + 1], lens[b:b + 1], w.scale,
                                  k_scale=k_scale, v_scale=v_scale)
        err = max_err(got[b:b + 1], ref)
        assert err <= tol, "row %d (length %d): max abs error %.3g" % (b, lens[b], err)


def _sample_rows(lens, n, seed):
    """The longest and the shortest row, plus n - 2 others drawn with a seed."""
    order = np.argsort(lens)
    rng = np.random.default_rng(seed)
    rest = rng.choice(order[1:-1], size=min(n - 2, len(order) - 2), replace=False)
    return [int(order[-1]), int(order[0])] + [int(x) for x in rest]


DECODE_CONFIGS = [
    # workload, partition, sampled rows
    ("llama8b_decode", 0, 10),
    ("llama70b_long", 0, 2),
    ("llama70b_long", 512, 2),
    ("shared_prefix", 0, 10),
]


@pytest.mark.parametrize("name,partition,nrows", DECODE_CONFIGS)
def test_full_config_decode_bf16(pa, name, partition, nrows):
    torch = torch_mod()
    w = getattr(W, name)()
    shape = w.cache_shape()
    K = W.device_values(shape, w.std, w.seed * 1000, w.dtype)
    V = W.device_values(shape, w.std, w.seed * 1000 + 1, w.dtype)
    q = W.device_values(w.q_shape(), w.std, w.seed * 1000 - 1, w.dtype)
    got = _decode_planned(pa, torch, w, K, V, q, partition)
    qh, Kh, Vh = to_host(q), to_host(K), to_host(V)
    del K, V
    _check_decode_rows(w, got, qh, Kh, Vh, _sample_rows(w.layout.seq_lens, nrows, w.seed), TOL["bf16"])


@pytest.mark.parametrize("name,nrows", [("llama8b_decode", 8), ("llama70b_long", 2)])
def test_full_config_decode_fp8(pa, name, nrows):
    torch = torch_mod()
    w = getattr(W, name)()
    shape = w.cache_shape()
    K, ks = _fp8_pool(torch, shape, w.std, w.seed * 1000)
    V, vs = _fp8_pool(torch, shape, w.std, w.seed * 1000 + 1)
    q = W.device_values(w.q_shape(), w.std, w.seed * 1000 - 1, "bf16")
    got = _decode_planned(pa, torch, w, K, V, q, 0, ks, vs, fp8=True)
    qh, Kh, Vh = to_host(q), to_host(K), to_host(V)
    del K, V
    _check_decode_rows(w, got, qh, Kh, Vh, _sample_rows(w.layout.seq_lens, nrows, w.seed), TOL["bf16"],
                       k_scale=ks, v_scale=vs)


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
    # rows of three sequences: the first chunk row, a middle one, the last one
    for b in (0, B // 2, B - 1):
        S, n = int(lay.seq_lens[b]), int(w.chunk_lens[b])
        for i in (0, n // 2 + 3, n - 1):
            r = int(qsl_h[b]) + i
            ref = oracle.paged_prefill(qh[r:r + 1], Kh, Vh, lay.block_tables[b:b + 1], np.array([0, 1], np.int32),
                                       np.array([S - n + i + 1], np.int32), w.scale, **kvs)
            err = max_err(got[r:r + 1], ref)
            assert err <= TOL["bf16"], "sequence %d chunk row %d: max abs error %.3g" % (b, i, err)
