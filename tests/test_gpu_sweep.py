"""GPU: a seeded sweep over the decode and chunked-prefill configuration space, against the oracle.

Each case draws its configuration from a fixed seed: the cache dtype (bf16, FP8 E4M3, fp32), the head size,
the block size (the MFMA sizes and others), the KV heads and the GQA group (1 to 32, divisors of 16 or not),
the sequence count and a length mix (empty rows, one token, block and tile edges, long rows), the caller's
partition size or the library's, the output dtype and, for decode, the call form (plain, planned, or with the
step's write folded in).  Every output is compared with the oracle at the parity bar: max abs error 2e-3 for
bf16 and FP8 caches, 1e-5 for fp32, plus the output's own bf16 rounding for bf16 outputs; rows with no tokens
must be exactly zero.  The cases are drawn once, so a failure names a reproducible seed."""
import math

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as W
from gpu_helpers import TOL, out_to_f64, require_gpu, to_gpu, to_host, torch_mod

pytestmark = pytest.mark.gpu

MFMA_BS = [8, 16, 32, 64, 128]
GROUPS = [1, 2, 3, 4, 6, 8, 12, 16, 24, 32]


@pytest.fixture(scope="module")
def pa():
    mod = require_gpu()
    oracle.build(force=False)
    return mod


def _lengths(rng, n, bs, longest):
    out = []
    for _ in range(n):
        u = rng.random()
        if u < 0.08:
            out.append(0)
        elif u < 0.25:
            out.append(int(rng.integers(1, 18)))
        elif u < 0.45:  # next to a block or tile edge
            e = int(rng.choice([bs, 16, 2 * bs, 4 * bs, 256]))
            out.append(max(1, e * int(rng.integers(1, 5)) + int(rng.integers(-1, 2))))
        else:
            out.append(int(rng.integers(1, longest + 1)))
    return out


def _config(seed, prefill):
    rng = np.random.default_rng(20_000 + 97 * seed + (1 if prefill else 0))
    kv = str(rng.choice(["bf16", "bf16", "fp8", "f32"]))
    D = 128 if kv == "fp8" else int(rng.choice([64, 128, 128]))
    bs = int(rng.choice(MFMA_BS)) if kv == "fp8" or rng.random() < 0.75 else int(rng.choice([1, 4, 24]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice(GROUPS))
    while Hkv * g > 128:
        Hkv //= 2
    B = int(rng.integers(1, 9 if prefill else 25))
    lens = _lengths(rng, B, bs, 1200 if prefill else 3000)
    out_dtype = str(rng.choice(["f32", "bf16"]))
    return rng, kv, D, bs, Hkv, g, B, lens, out_dtype


def _caches(lay, Hkv, D, kv, seed, ks, vs):
    shape = (lay.num_blocks, Hkv, lay.block_size, D)
    if kv == "fp8":
        k = oracle.fp8_encode(W.host_values(shape, 1.0, seed * 7 + 1, "f32") / np.float32(ks))
        v = oracle.fp8_encode(W.host_values(shape, 1.0, seed * 7 + 2, "f32") / np.float32(vs))
    else:
        k = W.host_values(shape, 1.0, seed * 7 + 1, kv)
        v = W.host_values(shape, 1.0, seed * 7 + 2, kv)
    return k, v


def _check(out, ref, kv, out_dtype, empty_rows, what):
    tol = TOL["f32" if kv == "f32" else "bf16"]
    slack = np.abs(ref) * 2.0 ** -8 if out_dtype == "bf16" else 0.0
    excess = np.abs(out - ref) - (tol + slack)
    assert np.isfinite(out).all(), what
    assert excess.max() <= 0, (what, float(excess.max()))
    for r in empty_rows:
        assert np.all(out[r] == 0), (what, "row %d" % r)


@pytest.mark.parametrize("seed", range(24))
def test_decode_sweep(pa, seed):
    torch = torch_mod()
    rng, kv, D, bs, Hkv, g, B, lens, out_dtype = _config(seed, prefill=False)
    Hq = Hkv * g
    mode = str(rng.choice(["plain", "planned", "append"]))
    part = 0
    # FP8 has MFMA kernels only: a group above 16 needs the library's balanced split
    if rng.random() < 0.4 and not (kv == "fp8" and g > 16):
        part = bs * int(rng.choice([1, 2, 4, 16, 64]))
    ks, vs = (float(rng.uniform(0.004, 0.05)), float(rng.uniform(0.004, 0.05))) if kv == "fp8" else (1.0, 1.0)
    what = dict(seed=seed, kv=kv, D=D, bs=bs, Hq=Hq, Hkv=Hkv, lens=lens, part=part, mode=mode, out=out_dtype)
    print("case", what, flush=True)
    lay = synth.build_paged_layout(lens, bs, seed=seed + 500, pool_factor=1.4)
    k, v = _caches(lay, Hkv, D, kv, seed, ks, vs)
    qd = "f32" if kv == "f32" else "bf16"
    q = W.host_values((B, Hq, D), 1.0, seed * 7 + 3, qd)
    scale = 1.0 / math.sqrt(D)
    max_len = max(max(lens), 1)
    kw = dict(k_scale=ks, v_scale=vs) if kv == "fp8" else {}
    kh, vh = k.copy(), v.copy()
    kg, vg = to_gpu(k), to_gpu(v)
    bt = to_gpu(lay.block_tables.astype(np.int32))
    sl = to_gpu(lay.seq_lens.astype(np.int32))
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out = torch.full((B, Hq, D), float("nan"), dtype=odt, device="cuda")
    wsb = pa.paged_attn_decode_workspace_size(B, Hq, Hkv, D, bs, max_len, part)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    kvd = {"bf16": pa.PA_BF16, "fp8": pa.PA_FP8_E4M3, "f32": pa.PA_F32}[kv]
    if mode == "plain":
        if kv == "fp8":
            pa.paged_attn_decode_fp8(out, to_gpu(q), kg, vg, ks, vs, bt, sl, scale, max_len, part, ws)
        else:
            pa.paged_attn_decode(out, to_gpu(q), kg, vg, bt, sl, scale, max_len, part, ws)
    else:
        psz = pa.paged_attn_decode_plan_size(B, Hq, Hkv, D, bs, lay.block_tables.shape[1], max_len, part, kvd)
        # (only the balanced split takes a plan; other paths get none and run as the plain call)
        plan = torch.full((psz,), 0x5A, dtype=torch.uint8, device="cuda") if psz else None
        pa.paged_attn_decode_plan(plan, kg, bt, sl, Hq, max_len, part)
        if mode == "planned":
            pa.paged_attn_decode_planned(out, to_gpu(q), kg, vg, plan, bt, sl, scale, max_len, part, ws, **kw)
        else:
            nd = "f32" if kv == "f32" else "bf16"
            nk = W.host_values((B, Hkv, D), 1.0, seed * 7 + 4, nd)
            nv = W.host_values((B, Hkv, D), 1.0, seed * 7 + 5, nd)
            slots = np.array([synth.slots_for_positions(lay.block_tables[b], [L - 1], bs)[0] if L > 0 else -1
                              for b, L in enumerate(lens)], np.int64)
            pa.paged_attn_decode_append(out, to_gpu(q), to_gpu(nk), to_gpu(nv), to_gpu(slots), kg, vg, plan, bt, sl,
                                        scale, max_len, part, ws, **kw)
            if kv == "fp8":
                ok = slots >= 0
                oracle.kv_cache_write_fp8(nk[ok], nv[ok], kh, vh, slots[ok], ks, vs)
            else:
                oracle.kv_cache_write(nk, nv, kh, vh, slots)
    torch.cuda.synchronize()
    if mode == "append":
        assert np.array_equal(to_host(kg), kh) and np.array_equal(to_host(vg), vh), ("caches", what)
    ref = oracle.paged_decode(q, kh, vh, lay.block_tables, lay.seq_lens, scale, **kw)
    _check(out_to_f64(out), ref, kv, out_dtype, [b for b, L in enumerate(lens) if L == 0], what)


@pytest.mark.parametrize("seed", range(12))
def test_prefill_sweep(pa, seed):
    torch = torch_mod()
    rng, kv, D, bs, Hkv, g, B, lens, out_dtype = _config(seed, prefill=True)
    Hq = Hkv * g
    lens = [max(L, 1) for L in lens]
    chunk = []
    for L in lens:
        u = rng.random()
        chunk.append(L if u < 0.25 else 1 if u < 0.4 else int(rng.integers(1, L + 1)))
    ks, vs = (float(rng.uniform(0.004, 0.05)), float(rng.uniform(0.004, 0.05))) if kv == "fp8" else (1.0, 1.0)
    what = dict(seed=seed, kv=kv, D=D, bs=bs, Hq=Hq, Hkv=Hkv, lens=lens, chunk=chunk, out=out_dtype)
    print("case", what, flush=True)
    lay = synth.build_paged_layout(lens, bs, seed=seed + 900, pool_factor=1.4)
    k, v = _caches(lay, Hkv, D, kv, seed + 50, ks, vs)
    qd = "f32" if kv == "f32" else "bf16"
    q = W.host_values((sum(chunk), Hq, D), 1.0, seed * 7 + 6, qd)
    qsl = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    scale = 1.0 / math.sqrt(D)
    kw = dict(k_scale=ks, v_scale=vs) if kv == "fp8" else {}
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out = torch.full((sum(chunk), Hq, D), float("nan"), dtype=odt, device="cuda")
    bt = to_gpu(lay.block_tables.astype(np.int32))
    sl = to_gpu(lay.seq_lens.astype(np.int32))
    if kv == "fp8":
        pa.paged_attn_prefill_chunk_fp8(out, to_gpu(q), to_gpu(k), to_gpu(v), ks, vs, bt, to_gpu(qsl), sl, scale,
                                        int(max(chunk)), int(max(lens)))
    else:
        pa.paged_attn_prefill_chunk(out, to_gpu(q), to_gpu(k), to_gpu(v), bt, to_gpu(qsl), sl, scale,
                                    int(max(chunk)), int(max(lens)))
    torch.cuda.synchronize()
    ref = oracle.paged_prefill(q, k, v, lay.block_tables, qsl, lay.seq_lens, scale, **kw)
    _check(out_to_f64(out), ref, kv, out_dtype, [], what)
