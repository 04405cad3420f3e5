"""The calls under HIP-graph capture: a graph holding a slot write, a decode
(stream-K main + merge kernels), a chunked prefill and a block copy is
replayed several times, with eager work and synchronisations between the
replays, and every replay must reproduce the eager results bit for bit.  The
oracle checks the eager results themselves, so the replays are tied to it."""
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


def test_graph_replays_match_eager(pa):
    torch = torch_mod()
    lens = [1, 17, 300, 1000, 64, 257, 33, 900]
    B, Hq, Hkv, D, bs = len(lens), 32, 8, 128, 16
    lay = synth.build_paged_layout(lens, bs, seed=77, pool_factor=1.5)
    shape = (lay.num_blocks, Hkv, bs, D)
    k0 = W.host_values(shape, 1.0, 7701, "bf16")
    v0 = W.host_values(shape, 1.0, 7702, "bf16")
    q = W.host_values((B, Hq, D), 1.0, 7703, "bf16")
    newk = W.host_values((B, Hkv, D), 1.0, 7704, "bf16")
    newv = W.host_values((B, Hkv, D), 1.0, 7705, "bf16")
    # the new token of every sequence goes to its last position
    slots = np.array([lay.block_tables[b, (L - 1) // bs] * bs + (L - 1) % bs for b, L in enumerate(lens)], np.int64)
    # a chunk of the last 8 rows of every sequence longer than 8
    chunk = np.array([min(8, L) for L in lens], np.int32)
    qsl = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    qp = W.host_values((int(qsl[-1]), Hq, D), 1.0, 7706, "bf16")
    # copy the last block of sequence 2 onto a free block
    used = set(int(x) for x in lay.block_tables.ravel() if x >= 0)
    free = next(i for i in range(lay.num_blocks) if i not in used)
    pairs = np.array([[lay.block_tables[2, (lens[2] - 1) // bs], free]], np.int64)

    kg, vg = to_gpu(k0), to_gpu(v0)
    qg, qpg = to_gpu(q), to_gpu(qp)
    nkg, nvg = to_gpu(newk), to_gpu(newv)
    sg, pg = to_gpu(slots), to_gpu(pairs)
    bt, sl = to_gpu(lay.block_tables.astype(np.int32)), to_gpu(lay.seq_lens.astype(np.int32))
    qslg = to_gpu(qsl)
    out_d = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    out_p = torch.empty((int(qsl[-1]), Hq, D), dtype=torch.float32, device="cuda")
    max_len = int(max(lens))
    wsb = pa.paged_attn_decode_workspace_size(B, Hq, Hkv, D, bs, max_len, 0)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(D)

    def work():
        pa.kv_cache_write(nkg, nvg, kg, vg, sg)
        pa.paged_attn_decode(out_d, qg, kg, vg, bt, sl, scale, max_len, 0, ws)
        pa.paged_attn_prefill_chunk(out_p, qpg, kg, vg, bt, qslg, sl, scale, int(chunk.max()), max_len)
        pa.block_copy(kg, vg, pg)

    # eager reference, itself checked against the oracle
    work()
    torch.cuda.synchronize()
    ref_d, ref_p = out_d.clone(), out_p.clone()
    ref_k, ref_v = kg.clone(), vg.clone()
    k1, v1 = k0.copy(), v0.copy()
    oracle.kv_cache_write(newk, newv, k1, v1, slots)
    oracle.block_copy(k1, v1, pairs)
    assert np.array_equal(to_host(ref_k), k1) and np.array_equal(to_host(ref_v), v1)
    assert max_err(out_to_f64(ref_d), oracle.paged_decode(q, k1, v1, lay.block_tables, lay.seq_lens, scale)) \
        <= TOL["bf16"]
    assert max_err(out_to_f64(ref_p), oracle.paged_prefill(qp, k1, v1, lay.block_tables, qsl, lay.seq_lens,
                                                           scale)) <= TOL["bf16"]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work between replays: clobber the outputs and the workspace,
        # and run another decode into a different buffer
        out_d.fill_(float("nan"))
        out_p.fill_(-1.0)
        ws.fill_(0xA5)
        other = torch.empty_like(out_d)
        pa.paged_attn_decode(other, qg, kg, vg, bt, sl, 0.5 * scale, max_len, 0, ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_d, ref_d), "decode differs on replay %d" % rep
        assert torch.equal(out_p, ref_p), "prefill differs on replay %d" % rep
        assert torch.equal(kg, ref_k) and torch.equal(vg, ref_v), "caches differ on replay %d" % rep
