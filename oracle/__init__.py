"""CPU oracle for paged KV-cache attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package.  The GPU library never links or calls it,
and this package imports nothing from the GPU library.

The arithmetic lives in ``oracle.c`` (fp64, plain definition; see its header
for the passages of the source pages it follows).  This module only marshals
numpy arrays into it.

Array conventions
-----------------
* bf16 data is passed as ``numpy.uint16`` arrays holding the raw bf16 bit
  patterns; fp32 data as ``numpy.float32``; FP8 E4M3 caches as ``numpy.uint8``
  codes (with a K scale and a V scale).  q, K and V share one dtype, except
  that an FP8 cache is read with fp32 or bf16 queries.
* Caches are ``[num_blocks, Hkv, block_size, D]``; q for decode is
  ``[B, Hq, D]``; q for prefill is ``[Tq, Hq, D]``.
* Attention outputs come back as ``numpy.float64``.

Parity status of each function (what pins it) is listed in the design notes
and checked by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dbl_p = ctypes.POINTER(ctypes.c_double)
_i32_p = ctypes.POINTER(ctypes.c_int32)
_i64_p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc -O2 (no fast-math) into liboracle.so."""
    global _lib
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def use_library(path):
    """Swap in another build of oracle.c (the mutation tests use this); returns the previous one."""
    global _lib
    prev = _lib
    _lib = None if path is None else _bind(ctypes.CDLL(path))
    return prev


def restore_library(prev):
    global _lib
    _lib = prev


def _bind(lib):
    lib.oracle_kv_cache_write.argtypes = [_vp, _vp, _vp, _vp, _i64_p] + [ctypes.c_int] * 6
    lib.oracle_block_copy.argtypes = [_vp, _vp, _i64_p] + [ctypes.c_int] * 6
    lib.oracle_paged_decode.argtypes = ([_dbl_p, _vp, _vp, _vp, ctypes.c_int, _i32_p, ctypes.c_int,
                                         _i32_p] + [ctypes.c_int] * 6 + [ctypes.c_double])
    lib.oracle_paged_prefill.argtypes = ([_dbl_p, _vp, _vp, _vp, ctypes.c_int, _i32_p, ctypes.c_int,
                                          _i32_p, _i32_p] + [ctypes.c_int] * 6 + [ctypes.c_double])
    lib.oracle_contiguous_attention.argtypes = ([_dbl_p, _dbl_p, _dbl_p, _dbl_p, _i32_p]
                                                + [ctypes.c_int] * 5 + [ctypes.c_double])
    lib.oracle_blockwise_decode_row.argtypes = ([_dbl_p, _vp, ctypes.c_int64, _vp, _vp, ctypes.c_int,
                                                 _i32_p] + [ctypes.c_int] * 6
                                                + [ctypes.c_double, ctypes.c_int, _i32_p])
    lib.oracle_kv_cache_write_fp8.argtypes = ([_vp, _vp, ctypes.c_int, _vp, _vp, _i64_p] + [ctypes.c_int] * 5
                                              + [ctypes.c_float, ctypes.c_float])
    lib.oracle_paged_decode_ex.argtypes = ([_dbl_p, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, ctypes.c_double,
                                            ctypes.c_double, _i32_p, ctypes.c_int, _i32_p]
                                           + [ctypes.c_int] * 6 + [ctypes.c_double])
    lib.oracle_paged_prefill_ex.argtypes = ([_dbl_p, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, ctypes.c_double,
                                             ctypes.c_double, _i32_p, ctypes.c_int, _i32_p, _i32_p]
                                            + [ctypes.c_int] * 6 + [ctypes.c_double])
    lib.oracle_fp8_decode.argtypes = [_vp, _dbl_p, ctypes.c_int64]
    lib.oracle_fp8_decode.restype = None
    lib.oracle_fp8_encode.argtypes = [_vp, _vp, ctypes.c_int64]
    lib.oracle_fp8_encode.restype = None
    lib.oracle_swap_out.argtypes = [_vp, _vp, _i64_p, ctypes.c_int, _vp] + [ctypes.c_int] * 5
    lib.oracle_swap_in.argtypes = [_vp, _vp, _i64_p, ctypes.c_int, _vp] + [ctypes.c_int] * 5
    for name in ("oracle_kv_cache_write", "oracle_kv_cache_write_fp8", "oracle_paged_decode_ex",
                 "oracle_paged_prefill_ex", "oracle_block_copy", "oracle_swap_out", "oracle_swap_in",
                 "oracle_paged_decode",
                 "oracle_paged_prefill", "oracle_contiguous_attention",
                 "oracle_blockwise_decode_row"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.uint8:
        return 2
    raise TypeError("oracle takes float32, uint16 (bf16 bit patterns) or uint8 (fp8 E4M3 codes), got %s"
                    % a.dtype)


def _c(a, dtype=None):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError("%s failed with code %d" % (what, rc))


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of float32 or bf16-bit arrays to float64."""
    return bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def kv_cache_write(key, value, k_cache, v_cache, slot_mapping):
    """In-place scatter of key/value [T, Hkv, D] rows into the caches."""
    lib = _load()
    NB, Hkv, bs, D = k_cache.shape
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    key, value = _c(key), _c(value)
    dt = _dtype_code(k_cache)
    assert key.dtype == k_cache.dtype == value.dtype == v_cache.dtype
    T = key.shape[0]
    slots = _c(slot_mapping, np.int64)
    rc = lib.oracle_kv_cache_write(key.ctypes.data, value.ctypes.data, k_cache.ctypes.data,
                                   v_cache.ctypes.data, slots.ctypes.data_as(_i64_p), T, NB, Hkv,
                                   bs, D, dt)
    _check(rc, "oracle_kv_cache_write")


def block_copy(k_cache, v_cache, pairs):
    """In-place copy of whole blocks (all KV heads) for each (src, dst) pair."""
    lib = _load()
    NB, Hkv, bs, D = k_cache.shape
    pairs = _c(np.asarray(pairs).reshape(-1, 2), np.int64)
    rc = lib.oracle_block_copy(k_cache.ctypes.data, v_cache.ctypes.data,
                               pairs.ctypes.data_as(_i64_p), pairs.shape[0], NB, Hkv, bs, D,
                               _dtype_code(k_cache))
    _check(rc, "oracle_block_copy")


def swap_out(k_cache, v_cache, ids) -> np.ndarray:
    """Host image of blocks ``ids``: uint8 [n, 2, block_bytes] (K then V per block; zeros for a bad id)."""
    lib = _load()
    NB, Hkv, bs, D = k_cache.shape
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    ids = _c(np.asarray(ids).reshape(-1), np.int64)
    blk_bytes = Hkv * bs * D * k_cache.itemsize
    host = np.empty((ids.shape[0], 2, blk_bytes), np.uint8)
    rc = lib.oracle_swap_out(k_cache.ctypes.data, v_cache.ctypes.data, ids.ctypes.data_as(_i64_p), ids.shape[0],
                             host.ctypes.data, NB, Hkv, bs, D, _dtype_code(k_cache))
    _check(rc, "oracle_swap_out")
    return host


def swap_in(k_cache, v_cache, ids, host):
    """In-place: piece i of the host image goes to block ids[i] of both caches (a bad id is skipped)."""
    lib = _load()
    NB, Hkv, bs, D = k_cache.shape
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    ids = _c(np.asarray(ids).reshape(-1), np.int64)
    host = _c(host, np.uint8)
    assert host.size >= ids.shape[0] * 2 * Hkv * bs * D * k_cache.itemsize
    rc = lib.oracle_swap_in(k_cache.ctypes.data, v_cache.ctypes.data, ids.ctypes.data_as(_i64_p), ids.shape[0],
                            host.ctypes.data, NB, Hkv, bs, D, _dtype_code(k_cache))
    _check(rc, "oracle_swap_in")


def _kv_args(q, k_cache, v_cache, k_scale, v_scale):
    """dtype codes and scales of one attention call; an FP8 cache needs both scales."""
    kd = _dtype_code(k_cache)
    assert k_cache.dtype == v_cache.dtype
    if kd == 2:
        assert k_scale is not None and v_scale is not None, "an FP8 cache needs k_scale and v_scale"
        assert q.dtype in (np.float32, np.uint16)
        return _dtype_code(q), kd, float(k_scale), float(v_scale)
    assert q.dtype == k_cache.dtype and k_scale is None and v_scale is None
    return kd, kd, 1.0, 1.0


def paged_decode(q, k_cache, v_cache, block_tables, seq_lens, scale, k_scale=None, v_scale=None):
    """fp64 [B, Hq, D] decode attention through the block tables (FP8 caches: value(code) * scale)."""
    lib = _load()
    q, k_cache, v_cache = _c(q), _c(k_cache), _c(v_cache)
    NB, Hkv, bs, D = k_cache.shape
    B, Hq, Dq = q.shape
    assert Dq == D
    qd, kd, ks, vs = _kv_args(q, k_cache, v_cache, k_scale, v_scale)
    bt = _c(block_tables, np.int32)
    sl = _c(seq_lens, np.int32)
    out = np.zeros((B, Hq, D), np.float64)
    rc = lib.oracle_paged_decode_ex(out.ctypes.data_as(_dbl_p), q.ctypes.data, qd, k_cache.ctypes.data,
                                    v_cache.ctypes.data, kd, ks, vs, bt.ctypes.data_as(_i32_p),
                                    bt.shape[1], sl.ctypes.data_as(_i32_p), B, Hq, Hkv, D, bs, NB,
                                    float(scale))
    _check(rc, "oracle_paged_decode")
    return out


def paged_prefill(q, k_cache, v_cache, block_tables, query_start_loc, seq_lens, scale, k_scale=None,
                  v_scale=None):
    """fp64 [Tq, Hq, D] causal chunk attention over the paged cache."""
    lib = _load()
    q, k_cache, v_cache = _c(q), _c(k_cache), _c(v_cache)
    NB, Hkv, bs, D = k_cache.shape
    Tq, Hq, Dq = q.shape
    assert Dq == D
    qd, kd, ks, vs = _kv_args(q, k_cache, v_cache, k_scale, v_scale)
    bt = _c(block_tables, np.int32)
    qsl = _c(query_start_loc, np.int32)
    sl = _c(seq_lens, np.int32)
    B = sl.shape[0]
    assert qsl.shape[0] == B + 1 and qsl[-1] <= Tq
    out = np.zeros((Tq, Hq, D), np.float64)
    rc = lib.oracle_paged_prefill_ex(out.ctypes.data_as(_dbl_p), q.ctypes.data, qd, k_cache.ctypes.data,
                                     v_cache.ctypes.data, kd, ks, vs, bt.ctypes.data_as(_i32_p),
                                     bt.shape[1], qsl.ctypes.data_as(_i32_p), sl.ctypes.data_as(_i32_p),
                                     B, Hq, Hkv, D, bs, NB, float(scale))
    _check(rc, "oracle_paged_prefill")
    return out


def fp8_decode(codes) -> np.ndarray:
    """fp64 values of E4M3 codes (uint8)."""
    lib = _load()
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib.oracle_fp8_decode(c.ctypes.data, out.ctypes.data_as(_dbl_p), c.size)
    return out


def fp8_encode(x) -> np.ndarray:
    """E4M3 codes (uint8) of fp32 values: nearest, ties to even, saturating at 448."""
    lib = _load()
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib.oracle_fp8_encode(x.ctypes.data, out.ctypes.data, x.size)
    return out


def kv_cache_write_fp8(key, value, k_cache, v_cache, slot_mapping, k_scale, v_scale):
    """In-place: key/value [T, Hkv, D] (fp32 or bf16 bits) quantised into the uint8 FP8 caches."""
    lib = _load()
    NB, Hkv, bs, D = k_cache.shape
    assert k_cache.dtype == v_cache.dtype == np.uint8
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    key, value = _c(key), _c(value)
    assert key.dtype == value.dtype
    slots = _c(slot_mapping, np.int64)
    rc = lib.oracle_kv_cache_write_fp8(key.ctypes.data, value.ctypes.data, _dtype_code(key), k_cache.ctypes.data,
                                       v_cache.ctypes.data, slots.ctypes.data_as(_i64_p), key.shape[0], NB, Hkv,
                                       bs, D, float(k_scale), float(v_scale))
    _check(rc, "oracle_kv_cache_write_fp8")


def contiguous_attention(q, K, V, n_keys, scale):
    """fp64 attention over contiguous K,V [Lk, Hkv, D]; q [Tq, Hq, D]; row i sees n_keys[i] keys."""
    lib = _load()
    q, K, V = _c(q, np.float64), _c(K, np.float64), _c(V, np.float64)
    Tq, Hq, D = q.shape
    Lk, Hkv, _ = K.shape
    nk = _c(n_keys, np.int32)
    assert nk.shape[0] == Tq
    out = np.zeros((Tq, Hq, D), np.float64)
    rc = lib.oracle_contiguous_attention(out.ctypes.data_as(_dbl_p), q.ctypes.data_as(_dbl_p),
                                         K.ctypes.data_as(_dbl_p), V.ctypes.data_as(_dbl_p),
                                         nk.ctypes.data_as(_i32_p), Tq, Lk, Hq, Hkv, D, float(scale))
    _check(rc, "oracle_contiguous_attention")
    return out


def blockwise_decode_row(q_row, k_cache, v_cache, table, n_keys, kh, scale,
                         partition_blocks=1 << 30, visit_order=None):
    """The pages' block loop with online softmax for one query row (fp64 [D])."""
    lib = _load()
    q_row = _c(q_row)
    k_cache, v_cache = _c(k_cache), _c(v_cache)
    NB, Hkv, bs, D = k_cache.shape
    table = _c(table, np.int32)
    order = None if visit_order is None else _c(visit_order, np.int32)
    out = np.zeros(D, np.float64)
    rc = lib.oracle_blockwise_decode_row(out.ctypes.data_as(_dbl_p), q_row.ctypes.data, 0,
                                         k_cache.ctypes.data, v_cache.ctypes.data,
                                         _dtype_code(q_row), table.ctypes.data_as(_i32_p),
                                         int(n_keys), int(kh), Hkv, D, bs, NB, float(scale),
                                         int(min(partition_blocks, 1 << 30)),
                                         None if order is None else order.ctypes.data_as(_i32_p))
    _check(rc, "oracle_blockwise_decode_row")
    return out
