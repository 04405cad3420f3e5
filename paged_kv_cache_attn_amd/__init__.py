"""PagedAttention for AMD MI355X: Python binding of libpagedattn.so.

Thin argument marshalling over the C ABI in ``include/paged_attn.h``: every
step of the computation runs in the library's HIP kernels.  PyTorch supplies
device memory and the stream (``torch.cuda.current_stream()``).  The functions
have the C ABI's names; sizes are read from the tensors' shapes.

There is no fallback: if the library is missing, the first call (or the
first access to ``lib``) raises ImportError, and every call checks that its
tensors live on a GPU.  Importing the package itself never loads the library,
so ``python -m paged_kv_cache_attn_amd.build`` works on a fresh tree.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "PA_F32", "PA_BF16", "PagedAttnError", "lib", "library_path", "pa_status_string",
    "pa_abi_version", "kv_cache_write", "paged_attn_decode_workspace_size", "paged_attn_decode",
    "paged_attn_prefill_chunk", "block_copy", "kv_swap_out", "kv_swap_in", "swap_host_bytes",
    "kv_cache_write_fp8", "paged_attn_decode_fp8", "paged_attn_prefill_chunk_fp8", "PA_FP8_E4M3",
    "paged_attn_decode_plan_size", "paged_attn_decode_plan", "paged_attn_decode_planned",
    "paged_attn_decode_noalloc", "PA_NOALLOC_SCRATCH_BYTES", "paged_attn_decode_append", "EXPORTED_SYMBOLS",
    "load_debug_library", "debug_flags", "DEBUG_BITS", "load_timeline_library", "timeline", "using_library",
]

PA_F32 = 0
PA_BF16 = 1
PA_FP8_E4M3 = 2
PA_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024  # the library's built-in decode scratch (include/paged_attn.h)

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")
debug_library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn_debug.so")
timeline_library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn_timeline.so")
PA_TIMELINE_ROWS = 4096  # workgroup ids with timestamps (include/paged_attn.h)

EXPORTED_SYMBOLS = ("pa_status_string", "pa_abi_version", "kv_cache_write",
                    "paged_attn_decode_workspace_size", "paged_attn_decode",
                    "paged_attn_prefill_chunk", "block_copy", "kv_swap_out", "kv_swap_in",
                    "kv_cache_write_fp8", "paged_attn_decode_fp8", "paged_attn_prefill_chunk_fp8",
                    "paged_attn_decode_plan_size", "paged_attn_decode_plan", "paged_attn_decode_planned",
                    "paged_attn_decode_noalloc", "paged_attn_decode_append", "pa_debug_flags", "pa_timeline")


class PagedAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (status %d)" % (fn, pa_status_string(status), status))
        self.status = status


def _load(path=None):
    path = path or library_path
    if not os.path.exists(path):
        raise ImportError("%s is not built (run `python -m paged_kv_cache_attn_amd.build`); "
                          "there is no fallback path" % os.path.basename(path))
    L = ctypes.CDLL(path)
    vp, i32, i64p, i32p = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p
    L.pa_status_string.argtypes = [ctypes.c_int]
    L.pa_status_string.restype = ctypes.c_char_p
    L.pa_abi_version.argtypes = []
    L.pa_abi_version.restype = ctypes.c_int
    L.pa_debug_flags.argtypes = [ctypes.POINTER(ctypes.c_uint), ctypes.c_int]
    L.pa_debug_flags.restype = ctypes.c_int
    L.pa_timeline.argtypes = [vp, vp, i32, i32]
    L.pa_timeline.restype = ctypes.c_int
    L.kv_cache_write.argtypes = [vp, vp, vp, vp, vp] + [i32] * 6 + [vp]
    L.kv_cache_write.restype = ctypes.c_int
    L.paged_attn_decode_workspace_size.argtypes = [i32] * 7
    L.paged_attn_decode_workspace_size.restype = ctypes.c_size_t
    L.paged_attn_decode.argtypes = ([vp, i32, vp, vp, vp, i32, vp, i32, vp] + [i32] * 7
                                    + [ctypes.c_float, i32, vp, ctypes.c_size_t, vp])
    L.paged_attn_decode.restype = ctypes.c_int
    L.paged_attn_prefill_chunk.argtypes = ([vp, i32, vp, vp, vp, i32, vp, i32, vp, vp] + [i32] * 9
                                           + [ctypes.c_float, vp])
    L.paged_attn_prefill_chunk.restype = ctypes.c_int
    L.block_copy.argtypes = [vp, vp, vp] + [i32] * 6 + [vp]
    L.block_copy.restype = ctypes.c_int
    f32 = ctypes.c_float
    L.kv_cache_write_fp8.argtypes = [vp, vp, i32, vp, vp, vp] + [i32] * 5 + [f32, f32, vp]
    L.kv_cache_write_fp8.restype = ctypes.c_int
    L.paged_attn_decode_fp8.argtypes = ([vp, i32, vp, vp, vp, f32, f32, vp, i32, vp] + [i32] * 7
                                        + [f32, i32, vp, ctypes.c_size_t, vp])
    L.paged_attn_decode_fp8.restype = ctypes.c_int
    L.paged_attn_prefill_chunk_fp8.argtypes = ([vp, i32, vp, vp, vp, f32, f32, vp, i32, vp, vp] + [i32] * 9
                                               + [f32, vp])
    L.paged_attn_prefill_chunk_fp8.restype = ctypes.c_int
    L.paged_attn_decode_plan_size.argtypes = [i32] * 9
    L.paged_attn_decode_plan_size.restype = ctypes.c_size_t
    L.paged_attn_decode_plan.argtypes = [vp, ctypes.c_size_t, i32, vp, i32, vp] + [i32] * 8 + [vp]
    L.paged_attn_decode_plan.restype = ctypes.c_int
    L.paged_attn_decode_planned.argtypes = ([vp, i32, vp, vp, vp, i32, f32, f32, vp, ctypes.c_size_t, vp, i32, vp]
                                            + [i32] * 7 + [f32, i32, vp, ctypes.c_size_t, vp])
    L.paged_attn_decode_planned.restype = ctypes.c_int
    L.paged_attn_decode_append.argtypes = ([vp, i32, vp, vp, vp, vp, vp, vp, i32, f32, f32, vp, ctypes.c_size_t,
                                            vp, i32, vp] + [i32] * 7 + [f32, i32, vp, ctypes.c_size_t, vp])
    L.paged_attn_decode_append.restype = ctypes.c_int
    L.paged_attn_decode_noalloc.argtypes = ([vp, i32, vp, vp, vp, i32, vp, i32, vp] + [i32] * 7
                                            + [ctypes.c_float, i32, vp])
    L.paged_attn_decode_noalloc.restype = ctypes.c_int
    L.kv_swap_out.argtypes = [vp, vp, vp, i32, vp, vp, ctypes.c_size_t] + [i32] * 5 + [vp]
    L.kv_swap_out.restype = ctypes.c_int
    L.kv_swap_in.argtypes = [vp, vp, vp, i32, vp, vp, ctypes.c_size_t] + [i32] * 5 + [vp]
    L.kv_swap_in.restype = ctypes.c_int
    return L


_lib = None


def _L():
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def __getattr__(name):
    if name == "lib":
        return _L()
    raise AttributeError(name)


def pa_status_string(status: int) -> str:
    return _L().pa_status_string(int(status)).decode()


def pa_abi_version() -> int:
    return int(_L().pa_abi_version())


# ----------------------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PA_FP8_E4M3
    raise TypeError("unsupported dtype %s (float32, bfloat16, or uint8 / float8_e4m3fn codes)" % t.dtype)


def _fp8_cache(t, name: str):
    if _dtype_code(t) != PA_FP8_E4M3:
        raise TypeError("%s must hold E4M3 codes (uint8 or float8_e4m3fn), got %s" % (name, t.dtype))
    return _dev(t, name)


def _dev(t, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (no CPU path exists)" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, status: int):
    if status != 0:
        raise PagedAttnError(fn, status)


# ----------------------------------------------------------------------------- the calls
def kv_cache_write(key, value, k_cache, v_cache, slot_mapping, stream=None):
    """Scatter key/value [T, Hkv, D] into the [NB, Hkv, bs, D] caches at slot_mapping (int64)."""
    torch = _torch()
    NB, Hkv, bs, D = k_cache.shape
    T = key.shape[0]
    if tuple(key.shape) != (T, Hkv, D) or key.shape != value.shape or k_cache.shape != v_cache.shape:
        raise ValueError("shape mismatch: key %s value %s cache %s" % (tuple(key.shape), tuple(value.shape),
                                                                      tuple(k_cache.shape)))
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    dt = _dtype_code(k_cache)
    if not (key.dtype == value.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("key, value and caches must share one dtype")
    st = _L().kv_cache_write(_dev(key, "key"), _dev(value, "value"), _dev(k_cache, "k_cache"),
                            _dev(v_cache, "v_cache"), _dev(slot_mapping, "slot_mapping", torch.int64),
                            T, NB, Hkv, bs, D, dt, _stream(stream))
    _check("kv_cache_write", st)


def paged_attn_decode_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                                     block_size: int, max_seq_len: int, partition_size: int = 0) -> int:
    return int(_L().paged_attn_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                                    max_seq_len, partition_size))


def paged_attn_decode(out, q, k_cache, v_cache, block_tables, seq_lens, scale: float, max_seq_len: int,
                      partition_size: int = 0, workspace=None, stream=None):
    """out[B, Hq, D] (fp32 or bf16) = decode attention of q[B, Hq, D] over the paged caches.

    ``workspace`` is a uint8 GPU tensor of at least
    ``paged_attn_decode_workspace_size(B, Hq, Hkv, D, block_size, max_seq_len, partition_size)``
    bytes (may be None when that is 0).
    """
    torch = _torch()
    NB, Hkv, bs, D = k_cache.shape
    B, Hq, Dq = q.shape
    if Dq != D or tuple(out.shape) != (B, Hq, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_tables must be [B, max_blocks], seq_lens [B]")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q and caches must share one dtype")
    ws_ptr, ws_bytes = ctypes.c_void_p(0), 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    st = _L().paged_attn_decode(_dev(out, "out"), _dtype_code(out), _dev(q, "q"), _dev(k_cache, "k_cache"),
                               _dev(v_cache, "v_cache"), _dtype_code(k_cache),
                               _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
                               _dev(seq_lens, "seq_lens", torch.int32), B, Hq, Hkv, D, bs, NB,
                               int(max_seq_len), float(scale), int(partition_size), ws_ptr, ws_bytes,
                               _stream(stream))
    _check("paged_attn_decode", st)


def paged_attn_prefill_chunk(out, q, k_cache, v_cache, block_tables, query_start_loc, seq_lens,
                             scale: float, max_query_len: int, max_seq_len: int, stream=None):
    """out[Tq, Hq, D] = causal chunk attention of q[Tq, Hq, D] over cached prefix + chunk."""
    torch = _torch()
    NB, Hkv, bs, D = k_cache.shape
    Tq, Hq, Dq = q.shape
    B = seq_lens.shape[0]
    if Dq != D or tuple(out.shape) != (Tq, Hq, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or tuple(query_start_loc.shape) != (B + 1,):
        raise ValueError("block_tables must be [B, max_blocks], query_start_loc [B+1]")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q and caches must share one dtype")
    st = _L().paged_attn_prefill_chunk(_dev(out, "out"), _dtype_code(out), _dev(q, "q"),
                                      _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                      _dtype_code(k_cache), _dev(block_tables, "block_tables", torch.int32),
                                      block_tables.shape[1],
                                      _dev(query_start_loc, "query_start_loc", torch.int32),
                                      _dev(seq_lens, "seq_lens", torch.int32), B, Tq, Hq, Hkv, D, bs, NB,
                                      int(max_query_len), int(max_seq_len), float(scale), _stream(stream))
    _check("paged_attn_prefill_chunk", st)


def block_copy(k_cache, v_cache, pairs, stream=None):
    """Copy whole blocks K[dst] = K[src], V[dst] = V[src] for pairs [N, 2] (int64)."""
    torch = _torch()
    NB, Hkv, bs, D = k_cache.shape
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [N, 2]")
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("caches must match")
    st = _L().block_copy(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(pairs, "pairs", torch.int64),
                        pairs.shape[0], NB, Hkv, bs, D, _dtype_code(k_cache), _stream(stream))
    _check("block_copy", st)


def swap_host_bytes(k_cache, num_ids: int) -> int:
    """Bytes of host memory kv_swap_out fills for num_ids blocks of these caches (K then V per block)."""
    NB, Hkv, bs, D = k_cache.shape
    return int(num_ids) * 2 * Hkv * bs * D * k_cache.element_size()


def _swap(fn: str, k_cache, v_cache, block_ids, host, staging, stream):
    torch = _torch()
    NB, Hkv, bs, D = k_cache.shape
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("caches must match")
    if block_ids.dim() != 1:
        raise ValueError("block_ids must be [num_ids]")
    n = block_ids.shape[0]
    if host.is_cuda or not host.is_contiguous():
        raise ValueError("the host buffer must be a contiguous CPU tensor (pinned for an asynchronous call)")
    if host.numel() * host.element_size() < swap_host_bytes(k_cache, n):
        raise ValueError("host buffer too small: %d < %d bytes" % (host.numel() * host.element_size(),
                                                                   swap_host_bytes(k_cache, n)))
    st = getattr(_L(), fn)(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                           _dev(block_ids, "block_ids", torch.int64), n, ctypes.c_void_p(host.data_ptr()),
                           _dev(staging, "staging"), staging.numel() * staging.element_size(), NB, Hkv, bs, D,
                           _dtype_code(k_cache), _stream(stream))
    _check(fn, st)


def kv_swap_out(k_cache, v_cache, block_ids, host_dst, staging, stream=None):
    """Copy blocks block_ids (GPU int64) of both caches into host_dst (CPU, pinned), K then V per block,
    through the GPU staging buffer (uint8, at least 2 blocks' bytes)."""
    _swap("kv_swap_out", k_cache, v_cache, block_ids, host_dst, staging, stream)


def kv_swap_in(k_cache, v_cache, block_ids, host_src, staging, stream=None):
    """Write the pieces of host_src (as kv_swap_out packs them) to blocks block_ids of both caches."""
    _swap("kv_swap_in", k_cache, v_cache, block_ids, host_src, staging, stream)


# ----------------------------------------------------------------------------- FP8 (E4M3) caches
def kv_cache_write_fp8(key, value, k_cache, v_cache, slot_mapping, k_scale: float, v_scale: float, stream=None):
    """Quantise key/value [T, Hkv, D] (fp32 or bf16) into the FP8 caches [NB, Hkv, bs, D] at slot_mapping."""
    torch = _torch()
    NB, Hkv, bs, D = k_cache.shape
    T = key.shape[0]
    if tuple(key.shape) != (T, Hkv, D) or key.shape != value.shape or k_cache.shape != v_cache.shape:
        raise ValueError("shape mismatch")
    if key.dtype != value.dtype:
        raise TypeError("key and value must share one dtype")
    st = _L().kv_cache_write_fp8(_dev(key, "key"), _dev(value, "value"), _dtype_code(key),
                                _fp8_cache(k_cache, "k_cache"), _fp8_cache(v_cache, "v_cache"),
                                _dev(slot_mapping, "slot_mapping", torch.int64), T, NB, Hkv, bs, D,
                                float(k_scale), float(v_scale), _stream(stream))
    _check("kv_cache_write_fp8", st)


def paged_attn_decode_fp8(out, q, k_cache, v_cache, k_scale: float, v_scale: float, block_tables, seq_lens,
                          scale: float, max_seq_len: int, partition_size: int = 0, workspace=None, stream=None):
    """paged_attn_decode over FP8 caches; q is bf16 [B, Hq, D]."""
    torch = _torch()
    NB, Hkv, bs, D = k_cache.shape
    B, Hq, Dq = q.shape
    if Dq != D or tuple(out.shape) != (B, Hq, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    ws_ptr, ws_bytes = ctypes.c_void_p(0), 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    st = _L().paged_attn_decode_fp8(_dev(out, "out"), _dtype_code(out), _dev(q, "q", torch.bfloat16),
                                   _fp8_cache(k_cache, "k_cache"), _fp8_cache(v_cache, "v_cache"),
                                   float(k_scale), float(v_scale), _dev(block_tables, "block_tables", torch.int32),
                                   block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32), B, Hq, Hkv, D,
                                   bs, NB, int(max_seq_len), float(scale), int(partition_size), ws_ptr, ws_bytes,
                                   _stream(stream))
    _check("paged_attn_decode_fp8", st)


def paged_attn_prefill_chunk_fp8(out, q, k_cache, v_cache, k_scale: float, v_scale: float, block_tables,
                                 query_start_loc, seq_lens, scale: float, max_query_len: int, max_seq_len: int,
                                 stream=None):
    """paged_attn_prefill_chunk over FP8 caches; q is bf16 [Tq, Hq, D]."""
    torch = _torch()
    NB, Hkv, bs, D = k_cache.shape
    Tq, Hq, Dq = q.shape
    B = seq_lens.shape[0]
    if Dq != D or tuple(out.shape) != (Tq, Hq, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    st = _L().paged_attn_prefill_chunk_fp8(_dev(out, "out"), _dtype_code(out), _dev(q, "q", torch.bfloat16),
                                          _fp8_cache(k_cache, "k_cache"), _fp8_cache(v_cache, "v_cache"),
                                          float(k_scale), float(v_scale),
                                          _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
                                          _dev(query_start_loc, "query_start_loc", torch.int32),
                                          _dev(seq_lens, "seq_lens", torch.int32), B, Tq, Hq, Hkv, D, bs, NB,
                                          int(max_query_len), int(max_seq_len), float(scale), _stream(stream))
    _check("paged_attn_prefill_chunk_fp8", st)


# ----------------------------------------------------------------------------- decode plans
def paged_attn_decode_plan_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                                max_blocks_per_seq: int, max_seq_len: int, partition_size: int = 0,
                                kv_dtype: int = PA_BF16) -> int:
    return int(_L().paged_attn_decode_plan_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                               max_blocks_per_seq, max_seq_len, partition_size, kv_dtype))


def paged_attn_decode_plan(plan, k_cache, block_tables, seq_lens, num_heads: int, max_seq_len: int,
                           partition_size: int = 0, stream=None):
    """Fill `plan` (uint8 GPU tensor, may be None when the plan size is 0) for decodes over caches shaped
    like k_cache (its dtype picks the kernel family) with these block tables and lengths."""
    torch = _torch()
    NB, Hkv, bs, D = k_cache.shape
    B = seq_lens.shape[0]
    pptr, pbytes = ctypes.c_void_p(0), 0
    if plan is not None:
        pptr, pbytes = _dev(plan, "plan"), plan.numel() * plan.element_size()
    st = _L().paged_attn_decode_plan(pptr, pbytes, _dtype_code(k_cache),
                                    _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
                                    _dev(seq_lens, "seq_lens", torch.int32), B, num_heads, Hkv, D, bs, NB,
                                    int(max_seq_len), int(partition_size), _stream(stream))
    _check("paged_attn_decode_plan", st)


def paged_attn_decode_planned(out, q, k_cache, v_cache, plan, block_tables, seq_lens, scale: float,
                              max_seq_len: int, partition_size: int = 0, workspace=None, k_scale: float = 1.0,
                              v_scale: float = 1.0, stream=None):
    """paged_attn_decode (or its FP8 form, by the caches' dtype) reading its split from `plan`."""
    torch = _torch()
    NB, Hkv, bs, D = k_cache.shape
    B, Hq, Dq = q.shape
    if Dq != D or tuple(out.shape) != (B, Hq, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    pptr, pbytes = ctypes.c_void_p(0), 0
    if plan is not None:
        pptr, pbytes = _dev(plan, "plan"), plan.numel() * plan.element_size()
    ws_ptr, ws_bytes = ctypes.c_void_p(0), 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    st = _L().paged_attn_decode_planned(_dev(out, "out"), _dtype_code(out), _dev(q, "q"), _dev(k_cache, "k_cache"),
                                       _dev(v_cache, "v_cache"), _dtype_code(k_cache), float(k_scale),
                                       float(v_scale), pptr, pbytes, _dev(block_tables, "block_tables", torch.int32),
                                       block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32), B, Hq, Hkv, D,
                                       bs, NB, int(max_seq_len), float(scale), int(partition_size), ws_ptr,
                                       ws_bytes, _stream(stream))
    _check("paged_attn_decode_planned", st)


def paged_attn_decode_append(out, q, key, value, slot_mapping, k_cache, v_cache, plan, block_tables, seq_lens,
                             scale: float, max_seq_len: int, partition_size: int = 0, workspace=None,
                             k_scale: float = 1.0, v_scale: float = 1.0, stream=None):
    """One decode step of one layer: key/value [B, Hkv, D] (the new token's rows) written at slot_mapping [B]
    (int64) and the decode over the caches (dtype picks bf16 / fp32 / FP8), the plan from
    paged_attn_decode_plan.  Same result as kv_cache_write(_fp8) followed by paged_attn_decode_planned."""
    torch = _torch()
    NB, Hkv, bs, D = k_cache.shape
    B, Hq, Dq = q.shape
    if Dq != D or tuple(out.shape) != (B, Hq, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if tuple(key.shape) != (B, Hkv, D) or value.shape != key.shape or tuple(slot_mapping.shape) != (B,):
        raise ValueError("key/value must be [B, Hkv, D] and slot_mapping [B]")
    if key.dtype != q.dtype or value.dtype != q.dtype:
        raise TypeError("key and value must have q's dtype")
    pptr, pbytes = ctypes.c_void_p(0), 0
    if plan is not None:
        pptr, pbytes = _dev(plan, "plan"), plan.numel() * plan.element_size()
    ws_ptr, ws_bytes = ctypes.c_void_p(0), 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    st = _L().paged_attn_decode_append(_dev(out, "out"), _dtype_code(out), _dev(q, "q"), _dev(key, "key"),
                                      _dev(value, "value"), _dev(slot_mapping, "slot_mapping", torch.int64),
                                      _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dtype_code(k_cache),
                                      float(k_scale), float(v_scale), pptr, pbytes,
                                      _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
                                      _dev(seq_lens, "seq_lens", torch.int32), B, Hq, Hkv, D, bs, NB,
                                      int(max_seq_len), float(scale), int(partition_size), ws_ptr, ws_bytes,
                                      _stream(stream))
    _check("paged_attn_decode_append", st)


# ----------------------------------------------------------------------------- no allocation
def paged_attn_decode_noalloc(out, q, k_cache, v_cache, block_tables, seq_lens, scale: float, max_seq_len: int,
                              partition_size: int = 0, stream=None):
    """paged_attn_decode with the library's built-in device scratch instead of a workspace (for callers that
    cannot allocate).  Calls that may overlap on one GPU race on that scratch; calls on one stream do not."""
    torch = _torch()
    NB, Hkv, bs, D = k_cache.shape
    B, Hq, Dq = q.shape
    if Dq != D or tuple(out.shape) != (B, Hq, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_tables must be [B, max_blocks], seq_lens [B]")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q and caches must share one dtype")
    st = _L().paged_attn_decode_noalloc(_dev(out, "out"), _dtype_code(out), _dev(q, "q"), _dev(k_cache, "k_cache"),
                                       _dev(v_cache, "v_cache"), _dtype_code(k_cache),
                                       _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
                                       _dev(seq_lens, "seq_lens", torch.int32), B, Hq, Hkv, D, bs, NB,
                                       int(max_seq_len), float(scale), int(partition_size), _stream(stream))
    _check("paged_attn_decode_noalloc", st)


# ----------------------------------------------------------------------------- debug build
# Bits of pa_debug_flags (include/paged_attn.h).
DEBUG_BITS = {"slot_range": 1 << 0, "slot_dup": 1 << 1, "block_range": 1 << 2, "pair_range": 1 << 3,
              "pair_conflict": 1 << 4, "len_clamped": 1 << 5, "query_loc": 1 << 6, "swap_range": 1 << 7,
              "plan": 1 << 8}


def load_debug_library():
    """The debug build (libpagedattn_debug.so) as a ctypes library with the same signatures, for calling
    directly; its kernels also record what their bounds checks mask (read with debug_flags)."""
    return _load(debug_library_path)


def load_timeline_library():
    """The timestamp build (libpagedattn_timeline.so) as a ctypes library with the same signatures; its
    balanced-decode kernels record per-workgroup timestamps (read with timeline)."""
    return _load(timeline_library_path)


class using_library:
    """Route the call wrappers of this module through another build of the library (the debug or the
    timestamp build) inside a `with` block."""

    def __init__(self, lib):
        self.lib, self.saved = lib, None

    def __enter__(self):
        global _lib
        self.saved, _lib = _lib, self.lib
        return self.lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def timeline(lib, rows: int, clear: bool = True):
    """pa_timeline of `lib` (waits for the device): the stamps of workgroup ids 0 .. rows - 1 as numpy uint64
    arrays, main kernel [rows, 8] and merge kernel [rows, 2] (points in include/paged_attn.h)."""
    import numpy as np
    main = np.zeros((rows, 8), np.uint64)
    merge = np.zeros((rows, 2), np.uint64)
    _check("pa_timeline", lib.pa_timeline(main.ctypes.data_as(ctypes.c_void_p),
                                          merge.ctypes.data_as(ctypes.c_void_p), int(rows), int(bool(clear))))
    return main, merge


def debug_flags(lib, clear: bool = True) -> int:
    """pa_debug_flags of `lib` (waits for the device): the OR of the recorded bits (DEBUG_BITS)."""
    v = ctypes.c_uint(0)
    _check("pa_debug_flags", lib.pa_debug_flags(ctypes.byref(v), int(bool(clear))))
    return int(v.value)
