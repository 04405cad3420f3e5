"""GPU: decode plans.  A plan made once from seq_lens and the block tables and
reused by the attention of several layers gives results bit-identical to the
unplanned call, on every path the plan covers."""
import math

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as W
from gpu_helpers import TOL, max_err, out_to_f64, require_gpu, to_gpu, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    mod = require_gpu()
    oracle.build(force=False)
    return mod


def _case(lens, Hq, Hkv, bs, kv, seed, layers=3):
    lay = synth.build_paged_layout(lens, bs, seed=seed, pool_factor=1.3)
    shape = (lay.num_blocks, Hkv, bs, 128)
    if kv == "fp8":
        K = [oracle.fp8_encode(W.host_values(shape, 1.0, seed + 10 * l, "f32") * np.float32(40)) for l in range(layers)]
        V = [oracle.fp8_encode(W.host_values(shape, 1.0, seed + 10 * l + 1, "f32") * np.float32(40)) for l in range(layers)]
    else:
        K = [W.host_values(shape, 1.0, seed + 10 * l, "bf16") for l in range(layers)]
        V = [W.host_values(shape, 1.0, seed + 10 * l + 1, "bf16") for l in range(layers)]
    q = W.host_values((len(lens), Hq, 128), 1.0, seed + 7, "bf16")
    return lay, q, K, V


PLAN_CASES = [
    # lens, Hq, Hkv, bs, kv, partition, out
    ("lognormal64", 32, 8, 16, "bf16", 0, "f32"),
    ("lognormal100", 32, 8, 16, "bf16", 0, "f32"),     # more than 64 sequences: the LDS scan
    ("mixed", 64, 8, 16, "bf16", 512, "f32"),          # fixed-size ranges
    ("mixed", 32, 8, 8, "bf16", 0, "bf16"),
    ("mixed", 32, 4, 64, "fp8", 0, "f32"),
    ("mixed", 16, 16, 32, "fp8", 256, "f32"),
    ("few_long", 64, 8, 16, "bf16", 0, "f32"),       # rows of dozens of pieces: the shared merge
    ("few_long", 8, 1, 16, "fp8", 0, "bf16"),
    ("few_long", 8, 8, 32, "bf16", 0, "f32"),        # group 1
    ("mixed", 32, 1, 16, "bf16", 0, "f32"),          # a group of 32: two sub-groups of 16 heads
    ("mixed", 96, 2, 16, "fp8", 0, "bf16"),          # groups of 48: three sub-groups
]


def _lens(kind):
    if kind == "lognormal64":
        return list(synth.lognormal_lengths(64, 390, 0.685, 16, 2048, seed=3))
    if kind == "lognormal100":
        return list(synth.lognormal_lengths(100, 200, 0.685, 1, 1024, seed=4))
    if kind == "few_long":
        return [3000, 0, 1500, 7]
    return [0, 1, 15, 16, 17, 300, 1000, 0, 63, 64, 65, 2049, 5]


@pytest.mark.parametrize("kind,Hq,Hkv,bs,kv,part,out_dtype", PLAN_CASES)
def test_planned_decode_bit_identical(pa, kind, Hq, Hkv, bs, kv, part, out_dtype):
    torch = torch_mod()
    lens = _lens(kind)
    lay, q, K, V = _case(lens, Hq, Hkv, bs, kv, seed=len(lens) + bs + part)
    B = len(lens)
    max_len = max(int(lay.seq_lens.max()), 1)
    kvd = pa.PA_FP8_E4M3 if kv == "fp8" else pa.PA_BF16
    bt, sl, qg = to_gpu(lay.block_tables), to_gpu(lay.seq_lens), to_gpu(q)
    psize = pa.paged_attn_decode_plan_size(B, Hq, Hkv, 128, bs, lay.block_tables.shape[1], max_len, part, kvd)
    assert psize > 0
    plan = torch.full((psize,), 0x7F, dtype=torch.uint8, device="cuda")  # contents on entry are ignored
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    wsb = pa.paged_attn_decode_workspace_size(B, Hq, Hkv, 128, bs, max_len, part)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    kg0 = to_gpu(K[0])
    pa.paged_attn_decode_plan(plan, kg0, bt, sl, Hq, max_len, part)
    ks, vs = (0.025, 0.025) if kv == "fp8" else (1.0, 1.0)
    for l in range(len(K)):
        kg, vg = to_gpu(K[l]), to_gpu(V[l])
        a = torch.empty(B, Hq, 128, dtype=odt, device="cuda")
        b = torch.empty(B, Hq, 128, dtype=odt, device="cuda")
        if kv == "fp8":
            pa.paged_attn_decode_fp8(a, qg, kg, vg, ks, vs, bt, sl, 0.09, max_len, part, ws)
        else:
            pa.paged_attn_decode(a, qg, kg, vg, bt, sl, 0.09, max_len, part, ws)
        pa.paged_attn_decode_planned(b, qg, kg, vg, plan, bt, sl, 0.09, max_len, part, ws, k_scale=ks, v_scale=vs)
        torch.cuda.synchronize()
        assert torch.equal(a, b), (l, float((a.float() - b.float()).abs().max()))
        if l == 0:
            kw = dict(k_scale=ks, v_scale=vs) if kv == "fp8" else {}
            ref = oracle.paged_decode(q, K[0], V[0], lay.block_tables, lay.seq_lens, 0.09, **kw)
            err = np.abs(out_to_f64(b) - ref) - (TOL["bf16"] + (np.abs(ref) * 2.0 ** -8 if out_dtype == "bf16" else 0))
            assert err.max() <= 0, err.max()


def test_plan_not_needed_for_vector_path(pa):
    """fp32 / head_dim 64 decode is not split by ranges: no plan, and the planned call runs as the plain one."""
    torch = torch_mod()
    lens = [5, 40, 300]
    lay = synth.build_paged_layout(lens, 16, seed=2, pool_factor=1.3)
    k = W.host_values((lay.num_blocks, 2, 16, 64), 1.0, 1, "f32")
    v = W.host_values((lay.num_blocks, 2, 16, 64), 1.0, 2, "f32")
    q = W.host_values((3, 8, 64), 1.0, 3, "f32")
    assert pa.paged_attn_decode_plan_size(3, 8, 2, 64, 16, lay.block_tables.shape[1], 300, 0, pa.PA_F32) == 0
    bt, sl = to_gpu(lay.block_tables), to_gpu(lay.seq_lens)
    wsb = pa.paged_attn_decode_workspace_size(3, 8, 2, 64, 16, 300, 0)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    a = torch.empty(3, 8, 64, device="cuda")
    b = torch.empty(3, 8, 64, device="cuda")
    pa.paged_attn_decode_plan(None, to_gpu(k), bt, sl, 8, 300)
    pa.paged_attn_decode(a, to_gpu(q), to_gpu(k), to_gpu(v), bt, sl, 0.125, 300, 0, ws)
    pa.paged_attn_decode_planned(b, to_gpu(q), to_gpu(k), to_gpu(v), None, bt, sl, 0.125, 300, 0, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert max_err(out_to_f64(b), oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, 0.125)) <= TOL["f32"]
