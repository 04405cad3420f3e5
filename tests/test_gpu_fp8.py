"""GPU parity of the FP8 (E4M3) KV-cache calls against the fp64 oracle.

The quantising write is compared byte for byte over whole caches; attention
over FP8 caches is held to the bf16 bar (2e-3 max abs error, fp32 output),
since it computes exactly as on a bf16 cache holding the codes' values.
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


def fp8_problem(lens, Hq, Hkv, D, bs, seed, ks, vs, pool_factor=1.3):
    """Codes of N(0, 1) K and V at scales ks, vs (the oracle's quantiser), bf16 q."""
    lay = synth.build_paged_layout(lens, bs, seed=seed, pool_factor=pool_factor)
    shape = (lay.num_blocks, Hkv, bs, D)
    kc = oracle.fp8_encode(W.host_values(shape, 1.0, seed * 13 + 1, "f32") / np.float32(ks))
    vc = oracle.fp8_encode(W.host_values(shape, 1.0, seed * 13 + 2, "f32") / np.float32(vs))
    q = W.host_values((len(lens), Hq, D), 1.0, seed * 13 + 3, "bf16")
    return lay, q, kc, vc


def gpu_decode_fp8(pa, lay, q, kc, vc, ks, vs, scale, out_dtype="f32", partition_size=0):
    torch = torch_mod()
    B, Hq, D = q.shape
    out = torch.empty((B, Hq, D), dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16, device="cuda")
    max_len = max(int(lay.seq_lens.max()), 1)
    wsb = pa.paged_attn_decode_workspace_size(B, Hq, kc.shape[1], D, kc.shape[2], max_len, partition_size)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    pa.paged_attn_decode_fp8(out, to_gpu(q), to_gpu(kc), to_gpu(vc), ks, vs, to_gpu(lay.block_tables.astype(np.int32)),
                             to_gpu(lay.seq_lens.astype(np.int32)), scale, max_len, partition_size, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("src,bs", [("bf16", 16), ("f32", 16), ("bf16", 8), ("f32", 64)])
def test_kv_cache_write_fp8_bit_exact(pa, src, bs):
    """Every code the GPU writes is the oracle's: ties, subnormals, saturation, both signs."""
    torch = torch_mod()
    Hkv, D, T = 4, 128, 70
    NB = max(40, (2 * T + bs - 1) // bs)
    rng = np.random.default_rng(3)
    # magnitudes spread over the whole E4M3 range and beyond, in units of the scale
    ks, vs = 0.0173, 0.00091
    kx = (rng.standard_normal((T, Hkv, D)) * np.exp(rng.uniform(-12, 7, (T, Hkv, D))) * ks).astype(np.float32)
    vx = (rng.standard_normal((T, Hkv, D)) * np.exp(rng.uniform(-12, 7, (T, Hkv, D))) * vs).astype(np.float32)
    # values near the small codes and the subnormal range
    kx[0, 0, :64] = (oracle.fp8_decode(np.arange(64, dtype=np.uint8)) + 2.0 ** -10) * ks
    if src == "bf16":
        kx, vx = synth.round_to_bf16_bits(kx), synth.round_to_bf16_bits(vx)
    slots = rng.choice(NB * bs, size=T, replace=False).astype(np.int64)
    slots[[5, 40]] = -1
    slots[11] = NB * bs + 3
    kc = np.full((NB, Hkv, bs, D), 0x5A, np.uint8)
    vc = kc.copy()
    kg, vg = to_gpu(kc), to_gpu(vc)
    pa.kv_cache_write_fp8(to_gpu(kx), to_gpu(vx), kg, vg, to_gpu(slots), ks, vs)
    torch.cuda.synchronize()
    ok = (slots >= 0) & (slots < NB * bs)
    oracle.kv_cache_write_fp8(kx[ok], vx[ok], kc, vc, slots[ok], ks, vs)
    gk, gv = to_host(kg), to_host(vg)
    assert np.array_equal(gk, kc), int((gk != kc).sum())
    assert np.array_equal(gv, vc), int((gv != vc).sum())


def test_kv_cache_write_fp8_exact_ties(pa):
    """With a power-of-two scale every midpoint between codes is exact: ties go to the even code."""
    torch = torch_mod()
    mids = (oracle.fp8_decode(np.arange(126, dtype=np.uint8)) + oracle.fp8_decode(np.arange(1, 127, dtype=np.uint8))) / 2
    x = np.concatenate([mids, -mids, [448.0, 460.0, 464.0, 500.0, 1e30, -1e30]]).astype(np.float32)
    n = ((x.size + 127) // 128) * 128
    x = np.concatenate([x, np.zeros(n - x.size, np.float32)]).reshape(n // 128, 1, 128) * np.float32(0.25)
    T = x.shape[0]
    kc = np.zeros((T, 1, 1, 128), np.uint8)
    vc = kc.copy()
    kg, vg = to_gpu(kc), to_gpu(vc)
    slots = np.arange(T, dtype=np.int64)
    pa.kv_cache_write_fp8(to_gpu(x), to_gpu(x), kg, vg, to_gpu(slots), 0.25, 0.25)
    torch.cuda.synchronize()
    oracle.kv_cache_write_fp8(x, x, kc, vc, slots, 0.25, 0.25)
    assert np.array_equal(to_host(kg), kc) and np.array_equal(to_host(vg), vc)


FP8_DECODE_CASES = [
    # Hq, Hkv, bs, out, partition
    (32, 8, 16, "f32", 0),
    (32, 1, 16, "f32", 0),      # a group of 32: two sub-groups of 16 heads
    (48, 2, 32, "bf16", 0),     # groups of 24: two sub-groups of 12
    (64, 8, 16, "f32", 512),
    (16, 16, 16, "f32", 64),
    (32, 2, 16, "f32", 128),
    (32, 8, 16, "bf16", 256),
    (32, 8, 8, "f32", 0),
    (32, 8, 64, "f32", 64),
    (24, 8, 32, "f32", 32),
]


@pytest.mark.parametrize("Hq,Hkv,bs,out_dtype,part", FP8_DECODE_CASES)
def test_decode_fp8_parity(pa, Hq, Hkv, bs, out_dtype, part):
    P = part or 256
    lens = [1, 2, 15, 16, 17, P - 1, P, P + 1, 2 * P + 1, 3 * P + 7, 40, 0, 5]
    ks, vs = 0.0123, 0.0291
    lay, q, kc, vc = fp8_problem(lens, Hq, Hkv, 128, bs, seed=Hq + Hkv + bs + part, ks=ks, vs=vs)
    scale = 1.0 / math.sqrt(128)
    ref = oracle.paged_decode(q, kc, vc, lay.block_tables, lay.seq_lens, scale, k_scale=ks, v_scale=vs)
    out = out_to_f64(gpu_decode_fp8(pa, lay, q, kc, vc, ks, vs, scale, out_dtype, part))
    tol = TOL["bf16"]
    if out_dtype == "bf16":
        excess = np.abs(out - ref) - (tol + (np.abs(ref) + tol) * 2.0 ** -8)
        assert excess.max() <= 0, excess.max()
    else:
        assert max_err(out, ref) <= tol, max_err(out, ref)
    assert np.all(out[11] == 0)


def test_decode_fp8_long_rows_partition_grid(pa):
    """Rows cut into many one-tile pieces take the partition grid and its merge; the library's own split of
    the same rows (dozens of pieces each) the balanced kernel and its shared merge."""
    lens = [3000, 7, 2049]
    lay, q, kc, vc = fp8_problem(lens, 32, 8, 128, 16, seed=71, ks=0.05, vs=0.004)
    ref = oracle.paged_decode(q, kc, vc, lay.block_tables, lay.seq_lens, 0.09, k_scale=0.05, v_scale=0.004)
    for part in (16, 0):
        out = out_to_f64(gpu_decode_fp8(pa, lay, q, kc, vc, 0.05, 0.004, 0.09, "f32", part))
        assert max_err(out, ref) <= TOL["bf16"], part


def test_decode_fp8_equals_bf16_on_decoded_values(pa):
    """With scales 1, FP8 decode matches bf16 decode of the codes' values (the codes widen
    to bf16 exactly; only the order of the dims inside the fp32 QK sums differs)."""
    lens = [100, 1, 513]
    lay, q, kc, vc = fp8_problem(lens, 32, 8, 128, 16, seed=5, ks=1.0, vs=1.0)
    kb = synth.round_to_bf16_bits(oracle.fp8_decode(kc).astype(np.float32))
    vb = synth.round_to_bf16_bits(oracle.fp8_decode(vc).astype(np.float32))
    torch = torch_mod()
    out_b = torch.empty(3, 32, 128, device="cuda")
    ws = torch.empty(max(pa.paged_attn_decode_workspace_size(3, 32, 8, 128, 16, 513, 0), 1), dtype=torch.uint8,
                     device="cuda")
    pa.paged_attn_decode(out_b, to_gpu(q), to_gpu(kb), to_gpu(vb), to_gpu(lay.block_tables), to_gpu(lay.seq_lens),
                         0.1, 513, 0, ws)
    out_f = gpu_decode_fp8(pa, lay, q, kc, vc, 1.0, 1.0, 0.1)
    assert max_err(out_to_f64(out_f), out_to_f64(out_b)) <= 1e-5


@pytest.mark.parametrize("Hq,Hkv,bs", [(32, 8, 16), (64, 8, 16), (8, 8, 32), (32, 8, 8), (24, 8, 16), (32, 1, 16)])
def test_prefill_fp8_parity(pa, Hq, Hkv, bs):
    torch = torch_mod()
    total = [40, 64, 17, 5, 300, 1, 129]
    chunk = [13, 64, 1, 5, 37, 1, 128]
    ks, vs = 0.0211, 0.0177
    lay, _, kc, vc = fp8_problem(total, Hq, Hkv, 128, bs, seed=Hq + bs, ks=ks, vs=vs)
    q = W.host_values((sum(chunk), Hq, 128), 1.0, 4545 + bs, "bf16")
    qsl = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    ref = oracle.paged_prefill(q, kc, vc, lay.block_tables, qsl, lay.seq_lens, 0.088, k_scale=ks, v_scale=vs)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    pa.paged_attn_prefill_chunk_fp8(out, to_gpu(q), to_gpu(kc), to_gpu(vc), ks, vs, to_gpu(lay.block_tables),
                                    to_gpu(qsl), to_gpu(lay.seq_lens), 0.088, int(max(chunk)), int(lay.seq_lens.max()))
    torch.cuda.synchronize()
    assert max_err(out_to_f64(out), ref) <= TOL["bf16"], max_err(out_to_f64(out), ref)


def test_fp8_block_copy_and_swap(pa):
    """The byte-moving calls take FP8 caches like any other dtype."""
    torch = torch_mod()
    NB, Hkv, bs, D = 20, 8, 16, 128
    kc = oracle.fp8_encode(W.host_values((NB, Hkv, bs, D), 1.0, 81, "f32") * np.float32(30))
    vc = oracle.fp8_encode(W.host_values((NB, Hkv, bs, D), 1.0, 82, "f32") * np.float32(30))
    kg, vg = to_gpu(kc), to_gpu(vc)
    pairs = np.array([[3, 9], [0, 17]], np.int64)
    pa.block_copy(kg, vg, to_gpu(pairs))
    oracle.block_copy(kc, vc, pairs)
    ids = np.array([9, 4, 17], np.int64)
    host = torch.empty(pa.swap_host_bytes(kg, 3), dtype=torch.uint8, pin_memory=True)
    staging = torch.empty(2 * Hkv * bs * D, dtype=torch.uint8, device="cuda")
    pa.kv_swap_out(kg, vg, to_gpu(ids), host, staging)
    torch.cuda.synchronize()
    assert np.array_equal(host.numpy().reshape(3, 2, -1), oracle.swap_out(kc, vc, ids))
    assert np.array_equal(to_host(kg), kc) and np.array_equal(to_host(vg), vc)
