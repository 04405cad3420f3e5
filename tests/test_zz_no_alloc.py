"""GPU: the decode entry point that allocates nothing (its workspace is the
library's built-in device scratch) against paged_attn_decode with a
caller-allocated workspace, through the C ABI.

Both calls run the same kernels, so the outputs must be bit-identical.  Two
calls in a row on one stream, the second with a smaller batch, check that
what the first call left in the shared scratch does not leak into the second.
Covered: the balanced split (the library's default) with GQA groups 4 and 8,
and the partition grid with its merge kernel (fixed short partitions of long
rows), plus a rejected oversized call.
"""
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


def _problem(lens, Hq, Hkv, seed, bs=16, D=128):
    lay = synth.build_paged_layout(lens, bs, seed=seed, pool_factor=1.3)
    shape = (lay.num_blocks, Hkv, bs, D)
    k = W.host_values(shape, 0.5, seed * 7 + 1, "bf16")
    v = W.host_values(shape, 0.5, seed * 7 + 2, "bf16")
    q = W.host_values((len(lens), Hq, D), 0.5, seed * 7 + 3, "bf16")
    return lay, q, k, v


def _both(pa, lay, q, k, v, partition):
    """(no-alloc output, allocated-workspace output) for one problem, on one stream."""
    torch = torch_mod()
    B, Hq, D = q.shape
    Hkv, bs = k.shape[1], k.shape[2]
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    bt, sl = to_gpu(lay.block_tables.astype(np.int32)), to_gpu(lay.seq_lens.astype(np.int32))
    max_len = int(lay.seq_lens.max())
    scale = 1.0 / math.sqrt(D)
    a = torch.full((B, Hq, D), float("nan"), device="cuda")
    pa.paged_attn_decode_noalloc(a, qg, kg, vg, bt, sl, scale, max_len, partition)
    wsb = pa.paged_attn_decode_workspace_size(B, Hq, Hkv, D, bs, max_len, partition)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    b = torch.full((B, Hq, D), float("nan"), device="cuda")
    pa.paged_attn_decode(b, qg, kg, vg, bt, sl, scale, max_len, partition, ws)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy(), scale


@pytest.mark.parametrize("Hq,Hkv,partition", [(32, 8, 0), (64, 8, 0), (32, 8, 128)])
def test_noalloc_matches_allocated_decode_two_calls(pa, Hq, Hkv, partition):
    rng = np.random.default_rng(Hq + partition)
    big = [int(x) for x in rng.integers(1, 3000, size=40)] + [0, 4096, 17]
    small = [5, 300, 0, 1000, 64]
    for lens, seed in ((big, 11), (small, 12)):  # the second call is the smaller one
        lay, q, k, v = _problem(lens, Hq, Hkv, seed)
        got, ref_gpu, scale = _both(pa, lay, q, k, v, partition)
        assert np.isfinite(got).all()
        assert np.array_equal(got, ref_gpu), "no-alloc decode differs from the allocated-workspace call"
        ref = oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, scale)
        assert max_err(out_to_f64(torch_mod().from_numpy(got)), ref) <= TOL["bf16"]


def test_noalloc_rejects_oversized_call(pa):
    torch = torch_mod()
    x = torch.zeros(1, device="cuda")
    B, Hq, Hkv, D, bs, max_len, part = 2048, 64, 8, 128, 16, 1 << 20, 16
    assert pa.paged_attn_decode_workspace_size(B, Hq, Hkv, D, bs, max_len, part) > pa.PA_NOALLOC_SCRATCH_BYTES
    import ctypes
    st = pa.lib.paged_attn_decode_noalloc(ctypes.c_void_p(x.data_ptr()), 0, ctypes.c_void_p(x.data_ptr()),
                                          ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(x.data_ptr()), 1,
                                          ctypes.c_void_p(x.data_ptr()), 1 << 16, ctypes.c_void_p(x.data_ptr()),
                                          B, Hq, Hkv, D, bs, 1 << 20, max_len, 0.1, part, ctypes.c_void_p(0))
    assert st == -6, st
    torch.cuda.synchronize()
