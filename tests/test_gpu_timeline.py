"""GPU: the timestamp build (libpagedattn_timeline.so) gives the release
build's results bit for bit and records, for every workgroup of the balanced
decode's planned kernels, its stamps in the order the kernel passes them.

The call is paged_attn_decode_append on a ragged batch (the folded step the
benchmark times), through the C ABI of each build."""
import math

import numpy as np
import pytest

import synth
from synth import workloads as W
from gpu_helpers import require_gpu, to_gpu, to_host, torch_mod

pytestmark = pytest.mark.gpu


def _run(pa, lib, lay, q, k, v, nk, nv, slots):
    torch = torch_mod()
    B, Hq, D = q.shape
    Hkv, bs = k.shape[1], k.shape[2]
    max_len = int(lay.seq_lens.max())
    with pa.using_library(lib):
        kg, vg = to_gpu(k), to_gpu(v)
        bt, sl = to_gpu(lay.block_tables.astype(np.int32)), to_gpu(lay.seq_lens.astype(np.int32))
        ws = torch.empty(max(pa.paged_attn_decode_workspace_size(B, Hq, Hkv, D, bs, max_len, 0), 1),
                         dtype=torch.uint8, device="cuda")
        plan = torch.empty(pa.paged_attn_decode_plan_size(B, Hq, Hkv, D, bs, lay.block_tables.shape[1], max_len, 0,
                                                          pa.PA_BF16), dtype=torch.uint8, device="cuda")
        out = torch.full((B, Hq, D), float("nan"), device="cuda")
        pa.paged_attn_decode_plan(plan, kg, bt, sl, Hq, max_len, 0)
        pa.paged_attn_decode_append(out, to_gpu(q), to_gpu(nk), to_gpu(nv), to_gpu(slots), kg, vg, plan, bt, sl,
                                    1.0 / math.sqrt(D), max_len, 0, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy(), to_host(kg), to_host(vg)


def test_timeline_build_matches_release_and_orders_its_stamps():
    pa = require_gpu()
    tlib = pa.load_timeline_library()
    pa.timeline(tlib, pa.PA_TIMELINE_ROWS, clear=True)
    rng = np.random.default_rng(41)
    lens = [int(x) for x in rng.integers(1, 2000, size=40)] + [0, 1, 17, 3000]
    lay = synth.build_paged_layout(lens, 16, seed=43, pool_factor=1.3)
    shape = (lay.num_blocks, 8, 16, 128)
    k = W.host_values(shape, 0.5, 431, "bf16")
    v = W.host_values(shape, 0.5, 432, "bf16")
    B = len(lens)
    q = W.host_values((B, 32, 128), 0.5, 433, "bf16")
    nk = W.host_values((B, 8, 128), 0.5, 434, "bf16")
    nv = W.host_values((B, 8, 128), 0.5, 435, "bf16")
    slots = np.array([synth.slots_for_positions(lay.block_tables[b], [L - 1], 16)[0] if L else -1
                      for b, L in enumerate(lens)], np.int64)
    o1, k1, v1 = _run(pa, pa.lib, lay, q, k, v, nk, nv, slots)
    o2, k2, v2 = _run(pa, tlib, lay, q, k, v, nk, nv, slots)
    assert np.array_equal(o1, o2) and np.array_equal(k1, k2) and np.array_equal(v1, v2)
    main, merge = pa.timeline(tlib, pa.PA_TIMELINE_ROWS, clear=True)
    ids = np.nonzero(main[:, 0])[0]
    assert len(ids) > 0 and np.array_equal(ids, np.arange(len(ids))), "stamps from workgroups 0 .. G-1"
    m = main[ids].astype(np.int64)
    assert (m > 0).all(), "every point of every workgroup stamped"
    # one thread's stamps, and stamps on the two sides of a barrier, are ordered; a wave's stream end and
    # thread 0's stamp after the staging barrier are taken by different waves (1 us of slack: 100 ticks)
    assert (m[:, 1] >= m[:, 0]).all() and (m[:, 2:6].min(1) >= m[:, 1] - 100).all()
    assert (m[:, 6] >= m[:, 2:6].max(1)).all() and (m[:, 7] >= m[:, 6]).all()
    g = merge[: len(ids)].astype(np.int64)
    assert (g > 0).all() and (g[:, 1] >= g[:, 0]).all()
    assert not merge[len(ids):].any() and not main[len(ids):].any()
    # cleared
    main2, merge2 = pa.timeline(tlib, 16, clear=False)
    assert not main2.any() and not merge2.any()
