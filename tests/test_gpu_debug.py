"""GPU: the debug build (libpagedattn_debug.so) records what the kernels'
bounds checks mask, and nothing else.

Every bad id below is masked or skipped by the kernels in both builds (never
dereferenced; the release build's tests check the same calls for
containment); the debug build must also set the matching bit of
pa_debug_flags.  Clean calls (the same shapes as the parity tests) must set
no bit and give the release build's results bit for bit.
"""
import ctypes
import math

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as W
from gpu_helpers import TOL, max_err, require_gpu, to_gpu, to_host, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    pa = require_gpu()
    oracle.build(force=False)
    dlib = pa.load_debug_library()
    pa.debug_flags(dlib, clear=True)
    return pa, dlib


def P(t):
    return ctypes.c_void_p(t.data_ptr())


N = ctypes.c_void_p(0)


def _write(lib, key, value, kc, vc, slots):
    NB, Hkv, bs, D = kc.shape
    return lib.kv_cache_write(P(key), P(value), P(kc), P(vc), P(slots), key.shape[0], NB, Hkv, bs, D,
                              1 if kc.dtype == torch_mod().bfloat16 else 0, N)


def _decode(lib, out, q, kc, vc, bt, sl, max_len, part, ws):
    NB, Hkv, bs, D = kc.shape
    B, Hq, _ = q.shape
    return lib.paged_attn_decode(P(out), 0, P(q), P(kc), P(vc), 1, P(bt), bt.shape[1], P(sl), B, Hq, Hkv, D, bs, NB,
                                 int(max_len), 0.09, int(part), P(ws), ws.numel(), N)


def _prefill(lib, out, q, kc, vc, bt, qsl, sl, max_q, max_len):
    NB, Hkv, bs, D = kc.shape
    Tq, Hq, _ = q.shape
    return lib.paged_attn_prefill_chunk(P(out), 0, P(q), P(kc), P(vc), 1, P(bt), bt.shape[1], P(qsl), P(sl),
                                        sl.shape[0], Tq, Hq, Hkv, D, bs, NB, int(max_q), int(max_len), 0.09, N)


def _decode_problem(lens, bs=16, seed=3):
    lay = synth.build_paged_layout(lens, bs, seed=seed, pool_factor=1.3)
    shape = (lay.num_blocks, 8, bs, 128)
    k = W.host_values(shape, 0.5, seed * 3 + 1, "bf16")
    v = W.host_values(shape, 0.5, seed * 3 + 2, "bf16")
    q = W.host_values((len(lens), 32, 128), 0.5, seed * 3 + 3, "bf16")
    return lay, q, k, v


def test_clean_calls_set_no_flag_and_match_release(libs):
    pa, dlib = libs
    torch = torch_mod()
    lens = [33, 700, 5, 1029, 0, 1, 300]
    lay, q, k, v = _decode_problem(lens)
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    bt, sl = to_gpu(lay.block_tables.astype(np.int32)), to_gpu(lay.seq_lens.astype(np.int32))
    outs = []
    for lib in (pa.lib, dlib):
        for part in (0, 32):
            ws = torch.empty(max(pa.paged_attn_decode_workspace_size(len(lens), 32, 8, 128, 16, 1029, part), 1),
                             dtype=torch.uint8, device="cuda")
            out = torch.empty(len(lens), 32, 128, device="cuda")
            assert _decode(lib, out, qg, kg, vg, bt, sl, 1029, part, ws) == 0
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[2]) and np.array_equal(outs[1], outs[3])
    # a clean write and copy
    nk = to_gpu(W.host_values((len(lens), 8, 128), 0.5, 71, "bf16"))
    slots = to_gpu(np.array([synth.slots_for_positions(lay.block_tables[b], [L - 1], 16)[0] if L else -1
                             for b, L in enumerate(lens)], np.int64))
    assert _write(dlib, nk, nk, kg, vg, slots) == 0
    pairs = to_gpu(np.array([[1, 2], [3, 3], [5, 6]], np.int64))
    assert dlib.block_copy(P(kg), P(vg), P(pairs), 3, kg.shape[0], 8, 16, 128, 1, N) == 0
    # a clean prefill
    total, chunk = [40, 300, 17], [13, 37, 1]
    lay2, _, k2, v2 = _decode_problem(total, seed=5)
    q2 = to_gpu(W.host_values((sum(chunk), 32, 128), 0.5, 72, "bf16"))
    qsl = to_gpu(np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32))
    out2 = torch.empty(sum(chunk), 32, 128, device="cuda")
    assert _prefill(dlib, out2, q2, to_gpu(k2), to_gpu(v2), to_gpu(lay2.block_tables.astype(np.int32)), qsl,
                    to_gpu(lay2.seq_lens.astype(np.int32)), max(chunk), max(total)) == 0
    assert pa.debug_flags(dlib) == 0


def test_bad_ids_set_their_flags(libs):
    pa, dlib = libs
    torch = torch_mod()
    bits = pa.DEBUG_BITS
    lens = [500, 300, 77, 1000]
    lay, q, k, v = _decode_problem(lens, seed=9)
    qg, kg, vg = to_gpu(q), to_gpu(k), to_gpu(v)
    NB = lay.num_blocks
    sl = to_gpu(lay.seq_lens.astype(np.int32))
    ref = oracle.paged_decode(q, k, v, lay.block_tables, lay.seq_lens, 0.09)
    # a block-table entry out of range: masked, flagged (balanced split and partition grid)
    bad = lay.block_tables.copy()
    bad[1, 3] = NB + 5
    for part in (0, 16):
        ws = torch.empty(max(pa.paged_attn_decode_workspace_size(4, 32, 8, 128, 16, 1000, part), 1),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty(4, 32, 128, device="cuda")
        assert _decode(dlib, out, qg, kg, vg, to_gpu(bad.astype(np.int32)), sl, 1000, part, ws) == 0
        got = out.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all()
        assert max_err(got[0], ref[0]) <= TOL["bf16"] and max_err(got[3], ref[3]) <= TOL["bf16"]
        assert pa.debug_flags(dlib) == bits["block_range"], part
    # a length past the call's bound: clamped, flagged
    ws = torch.empty(max(pa.paged_attn_decode_workspace_size(4, 32, 8, 128, 16, 1000, 0), 1), dtype=torch.uint8,
                     device="cuda")
    long_sl = to_gpu(np.array([500, 300, 77, 5000], np.int32))
    out = torch.empty(4, 32, 128, device="cuda")
    assert _decode(dlib, out, qg, kg, vg, to_gpu(lay.block_tables.astype(np.int32)), long_sl, 1000, 0, ws) == 0
    assert pa.debug_flags(dlib) & bits["len_clamped"]
    # slots: out of range, then duplicated
    nk = to_gpu(W.host_values((4, 8, 128), 0.5, 73, "bf16"))
    assert _write(dlib, nk, nk, kg, vg, to_gpu(np.array([3, NB * 16 + 2, -1, 7], np.int64))) == 0
    assert pa.debug_flags(dlib) == bits["slot_range"]
    assert _write(dlib, nk, nk, kg, vg, to_gpu(np.array([3, 9, 3, -1], np.int64))) == 0
    assert pa.debug_flags(dlib) == bits["slot_dup"]
    # copy pairs: out of range, then a dst that is another pair's src
    pr = to_gpu(np.array([[1, 2], [NB + 1, 4]], np.int64))
    assert dlib.block_copy(P(kg), P(vg), P(pr), 2, NB, 8, 16, 128, 1, N) == 0
    assert pa.debug_flags(dlib) == bits["pair_range"]
    pr = to_gpu(np.array([[1, 2], [2, 4]], np.int64))
    assert dlib.block_copy(P(kg), P(vg), P(pr), 2, NB, 8, 16, 128, 1, N) == 0
    assert pa.debug_flags(dlib) == bits["pair_conflict"]
    # swap ids out of range
    ids = to_gpu(np.array([2, NB + 9], np.int64))
    staging = torch.empty(2 * 2 * 8 * 16 * 128 * 2, dtype=torch.uint8, device="cuda")
    host = torch.empty(2 * 2 * 8 * 16 * 128 * 2, dtype=torch.uint8, pin_memory=True)
    assert dlib.kv_swap_out(P(kg), P(vg), P(ids), 2, ctypes.c_void_p(host.data_ptr()), P(staging),
                            staging.numel(), NB, 8, 16, 128, 1, N) == 0
    assert pa.debug_flags(dlib) == bits["swap_range"]
    # prefill: a bad table entry, then a query_start_loc past the query rows
    total, chunk = [40, 300, 17], [13, 37, 1]
    lay2, _, k2, v2 = _decode_problem(total, seed=11)
    q2 = to_gpu(W.host_values((sum(chunk), 32, 128), 0.5, 74, "bf16"))
    sl2 = to_gpu(lay2.seq_lens.astype(np.int32))
    qsl = to_gpu(np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32))
    bt2 = lay2.block_tables.copy()
    bt2[1, 2] = -7
    out2 = torch.empty(sum(chunk), 32, 128, device="cuda")
    assert _prefill(dlib, out2, q2, to_gpu(k2), to_gpu(v2), to_gpu(bt2.astype(np.int32)), qsl, sl2, max(chunk),
                    max(total)) == 0
    assert np.isfinite(out2.cpu().numpy()).all()
    assert pa.debug_flags(dlib) == bits["block_range"]
    bad_qsl = to_gpu(np.array([0, 13, 50, 60], np.int32))  # the last sequence runs past the 51 query rows
    assert _prefill(dlib, out2, q2, to_gpu(k2), to_gpu(v2), to_gpu(lay2.block_tables.astype(np.int32)), bad_qsl,
                    sl2, 10, max(total)) == 0
    assert pa.debug_flags(dlib) & bits["query_loc"]
    assert pa.debug_flags(dlib) == 0  # cleared
