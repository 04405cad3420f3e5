"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and its host-side argument checks return the documented
codes before anything is launched."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")
LIB = os.path.join(ROOT, "paged_kv_cache_attn_amd", "libpagedattn.so")
DEBUG_LIB = os.path.join(ROOT, "paged_kv_cache_attn_amd", "libpagedattn_debug.so")
TIMELINE_LIB = os.path.join(ROOT, "paged_kv_cache_attn_amd", "libpagedattn_timeline.so")

PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE = 0, -1, -2, -3, -4
PA_ERR_SCRATCH = -6


@pytest.fixture(scope="module")
def pa():
    if not os.path.exists(LIB):
        from paged_kv_cache_attn_amd import build as b
        b.build()
    import paged_kv_cache_attn_amd as pkg
    pkg.lib  # loads the library
    return pkg


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"PA_EXPORT\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("kv_cache_write", "paged_attn_decode", "paged_attn_prefill_chunk", "block_copy",
              "paged_attn_decode_workspace_size", "pa_status_string", "pa_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(pa):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(pa.lib, n)
    assert set(pa.EXPORTED_SYMBOLS) == set(declared_functions())


@pytest.mark.parametrize("variant", ["debug", "timeline"])
def test_variant_library_exports_every_declared_symbol(pa, variant):
    path = DEBUG_LIB if variant == "debug" else TIMELINE_LIB
    if not os.path.exists(path):
        from paged_kv_cache_attn_amd import build as b
        b.build(debug=variant == "debug", timeline=variant == "timeline")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in declared_functions():
        assert n in exported, n


def test_debug_flags_release_and_debug(pa):
    """The release build has no flag words: pa_debug_flags stores 0 and says so; the debug build refuses a
    NULL destination before it touches the GPU.  The bits match the header."""
    v = ctypes.c_uint(7)
    assert pa.lib.pa_debug_flags(ctypes.byref(v), 1) == PA_ERR_UNSUPPORTED and v.value == 0
    dlib = pa.load_debug_library()
    assert dlib.pa_debug_flags(None, 1) == PA_ERR_NULL
    text = open(HEADER).read()
    for name, bit in pa.DEBUG_BITS.items():
        m = re.search(r"#define PA_DEBUG_%s \(1u << (\d+)\)" % name.upper(), text)
        assert m and (1 << int(m.group(1))) == bit, name


def test_timeline_release_and_timestamp_build(pa):
    """The release build records no timestamps and says so; the timestamp build refuses NULL destinations
    and a row count outside 1 .. PA_TIMELINE_ROWS before it touches the GPU."""
    m = (ctypes.c_uint64 * 16)()
    g = (ctypes.c_uint64 * 4)()
    assert pa.lib.pa_timeline(m, g, 2, 0) == PA_ERR_UNSUPPORTED
    tlib = pa.load_timeline_library()
    assert tlib.pa_timeline(None, g, 2, 0) == PA_ERR_NULL
    assert tlib.pa_timeline(m, None, 2, 0) == PA_ERR_NULL
    assert tlib.pa_timeline(m, g, 0, 0) == PA_ERR_SHAPE
    assert tlib.pa_timeline(m, g, pa.PA_TIMELINE_ROWS + 1, 0) == PA_ERR_SHAPE
    assert re.search(r"#define PA_TIMELINE_ROWS %d\b" % pa.PA_TIMELINE_ROWS, open(HEADER).read())


def test_abi_version_and_status_strings(pa):
    v = int(re.search(r"#define PA_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert pa.pa_abi_version() == v
    assert pa.pa_status_string(0) == "ok"
    for code in (-1, -2, -3, -4, -5, -6):
        s = pa.pa_status_string(code)
        assert s and s != "unknown status"
    assert pa.pa_status_string(12345) == "unknown status"


P = ctypes.c_void_p(0x1000)  # non-NULL dummy: these calls must fail before touching it
N = ctypes.c_void_p(0)


def test_kv_cache_write_validation(pa):
    f = pa.lib.kv_cache_write
    assert f(P, P, P, P, P, -1, 10, 8, 16, 128, 1, N) == PA_ERR_SHAPE
    assert f(P, P, P, P, P, 4, 0, 8, 16, 128, 1, N) == PA_ERR_SHAPE
    assert f(P, P, P, P, P, 4, 10, 8, 16, 128, 7, N) == PA_ERR_UNSUPPORTED
    assert f(P, P, P, P, P, 4, 10, 8, 16, 4, 1, N) == PA_ERR_UNSUPPORTED      # 8-byte rows
    assert f(N, P, P, P, P, 4, 10, 8, 16, 128, 1, N) == PA_ERR_NULL
    assert f(P, P, P, P, N, 4, 10, 8, 16, 128, 1, N) == PA_ERR_NULL
    assert f(N, N, N, N, N, 0, 10, 8, 16, 128, 1, N) == PA_OK                 # empty: no-op


def _dec(pa, **kw):
    a = dict(out=P, out_dtype=0, q=P, k=P, v=P, kv_dtype=1, bt=P, maxblk=8, sl=P, B=2, Hq=8, Hkv=2,
             D=128, bs=16, NB=64, max_len=128, scale=0.1, part=0, ws=N, ws_bytes=0)
    a.update(kw)
    return pa.lib.paged_attn_decode(a["out"], a["out_dtype"], a["q"], a["k"], a["v"], a["kv_dtype"], a["bt"],
                                    a["maxblk"], a["sl"], a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["NB"],
                                    a["max_len"], a["scale"], a["part"], a["ws"], a["ws_bytes"], N)


def test_decode_validation(pa):
    assert _dec(pa, Hq=6, Hkv=4) == PA_ERR_SHAPE
    assert _dec(pa, B=-1) == PA_ERR_SHAPE
    assert _dec(pa, D=96) == PA_ERR_UNSUPPORTED
    assert _dec(pa, kv_dtype=3) == PA_ERR_UNSUPPORTED
    assert _dec(pa, out_dtype=2) == PA_ERR_UNSUPPORTED
    assert _dec(pa, NB=0) == PA_ERR_SHAPE
    assert _dec(pa, part=24) == PA_ERR_SHAPE                                  # not a block multiple
    for bad in (0.0, -0.5, float("inf"), float("nan")):
        assert _dec(pa, scale=bad) == PA_ERR_SHAPE                            # scale finite and > 0
    assert _dec(pa, q=N) == PA_ERR_NULL
    assert _dec(pa, bt=N) == PA_ERR_NULL
    # 4096 tokens in 256-token partitions need a workspace
    assert _dec(pa, max_len=4096, maxblk=256) == PA_ERR_WORKSPACE
    need = pa.paged_attn_decode_workspace_size(2, 8, 2, 128, 16, 4096, 0)
    assert _dec(pa, max_len=4096, maxblk=256, ws=P, ws_bytes=need - 1) == PA_ERR_WORKSPACE
    assert _dec(pa, B=0) == PA_OK


def _dec_noalloc(pa, **kw):
    a = dict(out=P, out_dtype=0, q=P, k=P, v=P, kv_dtype=1, bt=P, maxblk=8, sl=P, B=2, Hq=8, Hkv=2,
             D=128, bs=16, NB=64, max_len=128, scale=0.1, part=0)
    a.update(kw)
    return pa.lib.paged_attn_decode_noalloc(a["out"], a["out_dtype"], a["q"], a["k"], a["v"], a["kv_dtype"],
                                            a["bt"], a["maxblk"], a["sl"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                            a["bs"], a["NB"], a["max_len"], a["scale"], a["part"], N)


def test_decode_noalloc_validation(pa):
    """The no-allocation decode checks its arguments as paged_attn_decode does, and refuses (before touching
    the GPU) a call that needs more workspace than its built-in scratch holds."""
    assert _dec_noalloc(pa, Hq=6, Hkv=4) == PA_ERR_SHAPE
    assert _dec_noalloc(pa, D=96) == PA_ERR_UNSUPPORTED
    assert _dec_noalloc(pa, kv_dtype=2) == PA_ERR_UNSUPPORTED          # FP8 caches: not this call
    assert _dec_noalloc(pa, part=24) == PA_ERR_SHAPE
    assert _dec_noalloc(pa, scale=float("nan")) == PA_ERR_SHAPE
    assert _dec_noalloc(pa, q=N) == PA_ERR_NULL
    assert _dec_noalloc(pa, B=0) == PA_OK
    # 2048 rows of 64 heads, 1M tokens cut into 16-token partitions: the partition grid would need
    # terabytes of workspace
    big = dict(B=2048, Hq=64, Hkv=8, max_len=1 << 20, maxblk=1 << 16, part=16)
    assert pa.paged_attn_decode_workspace_size(2048, 64, 8, 128, 16, 1 << 20, 16) > pa.PA_NOALLOC_SCRATCH_BYTES
    assert _dec_noalloc(pa, **big) == PA_ERR_SCRATCH
    # the binding's constant is the header's
    m = re.search(r"#define PA_NOALLOC_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", open(HEADER).read())
    assert int(m.group(1)) << 20 == pa.PA_NOALLOC_SCRATCH_BYTES
    # the upper bound of the headline 8B shape fits, and so does 512-token partitioning of 8 x 32K rows of
    # 64 heads (the partition grid: 8 * 64 * 64 partial rows)
    assert pa.paged_attn_decode_workspace_size(64, 32, 8, 128, 16, 4096, 0) <= pa.PA_NOALLOC_SCRATCH_BYTES
    assert pa.paged_attn_decode_workspace_size(8, 64, 8, 128, 16, 32768, 512) <= pa.PA_NOALLOC_SCRATCH_BYTES


def _a256(x):
    return (x + 255) // 256 * 256


def test_decode_workspace_size(pa):
    f = pa.paged_attn_decode_workspace_size
    # 8B shape, library choice: 512 balanced ranges, 2 partial slots each, plus a 16-byte descriptor each
    B, Hq, Hkv, D, bs = 64, 32, 8, 128, 16
    g = Hq // Hkv
    ranges = 512
    streamk = _a256(ranges * 2 * g * D * 4) + _a256(ranges * 2 * g * 2 * 4) + _a256(ranges * 16)
    # the vector kernels' pieces: the longest power of two (256 .. 4096 tokens) that keeps
    # 512 rows x ceil(4096 / piece) >= 1024 workgroups: 2048 tokens, 2 per row
    grid = _a256(B * Hq * 2 * D * 4) + _a256(B * Hq * 2 * 2 * 4)
    assert f(B, Hq, Hkv, D, bs, 4096, 0) == max(streamk, grid)
    # few rows: the vector pieces stay at 256 tokens (8 rows x 8 pieces of 512 < 1024), so the
    # workspace covers 16 pieces per row
    assert f(4, 8, 2, 64, 16, 4096, 0) >= _a256(4 * 8 * 16 * 64 * 4) + _a256(4 * 8 * 16 * 2 * 4)
    # fixed 512-token pieces on 32K-token rows: 64 pieces per row, so the partition grid
    B, Hq, Hkv = 8, 64, 8
    grid = _a256(B * Hq * 64 * D * 4) + _a256(B * Hq * 64 * 2 * 4)
    assert f(B, Hq, Hkv, D, bs, 32768, 512) == grid
    # fixed 4096-token pieces on the same rows: 8 pieces per row, the balanced split
    g = Hq // Hkv
    ranges = B * Hkv * (32768 // 16) // 256
    streamk = _a256(ranges * 2 * g * D * 4) + _a256(ranges * 2 * g * 2 * 4) + _a256(ranges * 16)
    grid = _a256(B * Hq * 8 * D * 4) + _a256(B * Hq * 8 * 2 * 4)
    assert f(B, Hq, Hkv, D, bs, 32768, 4096) == max(streamk, grid)
    # tiny problem, explicit 64-token pieces: fewer ranges than the default
    t_up = 4 * 2 * 13
    ranges = (t_up + 3) // 4
    assert f(4, 8, 2, 64, 16, 203, 64) == (_a256(ranges * 2 * 4 * 64 * 4) + _a256(ranges * 2 * 4 * 2 * 4)
                                           + _a256(ranges * 16))
    assert f(0, 8, 2, 64, 16, 100, 0) == 0
    assert f(4, 8, 3, 64, 16, 100, 0) == 0          # invalid group
    assert f(4, 8, 2, 64, 16, 100, 24) == 0         # partition not a block multiple


def test_prefill_validation(pa):
    f = pa.lib.paged_attn_prefill_chunk
    # out, odt, q, k, v, kvdt, bt, maxblk, qsl, sl, B, Tq, Hq, Hkv, D, bs, NB, maxq, maxlen, scale, stream
    args = [P, 0, P, P, P, 1, P, 8, P, P, 2, 32, 8, 2, 128, 16, 64, 16, 128, 0.1, N]
    a = list(args); a[13] = 3                                  # Hkv does not divide Hq
    assert f(*a) == PA_ERR_SHAPE
    a = list(args); a[14] = 80
    assert f(*a) == PA_ERR_UNSUPPORTED
    a = list(args); a[8] = N
    assert f(*a) == PA_ERR_NULL
    a = list(args); a[17] = -1
    assert f(*a) == PA_ERR_SHAPE
    a = list(args); a[11] = -1
    assert f(*a) == PA_ERR_SHAPE
    a = list(args); a[17] = 0
    assert f(*a) == PA_OK


def test_block_copy_validation(pa):
    f = pa.lib.block_copy
    assert f(P, P, P, -1, 64, 8, 16, 128, 1, N) == PA_ERR_SHAPE
    assert f(P, P, N, 3, 64, 8, 16, 128, 1, N) == PA_ERR_NULL
    assert f(P, P, P, 3, 64, 8, 16, 128, 9, N) == PA_ERR_UNSUPPORTED
    assert f(N, N, N, 0, 64, 8, 16, 128, 1, N) == PA_OK


def test_swap_validation(pa):
    # k, v, ids, n, host, staging, staging_bytes, NB, Hkv, bs, D, dtype, stream
    blk = 8 * 16 * 128 * 2
    for f in (pa.lib.kv_swap_out, pa.lib.kv_swap_in):
        args = [P, P, P, 3, P, P, 2 * blk, 64, 8, 16, 128, 1, N]
        a = list(args); a[3] = -1
        assert f(*a) == PA_ERR_SHAPE
        a = list(args); a[11] = 9
        assert f(*a) == PA_ERR_UNSUPPORTED
        a = list(args); a[10] = 4          # 4 bf16 = 8 bytes: not a multiple of 16
        assert f(*a) == PA_ERR_UNSUPPORTED
        for i in (0, 1, 2, 4):
            a = list(args); a[i] = N
            assert f(*a) == PA_ERR_NULL
        a = list(args); a[5] = N
        assert f(*a) == PA_ERR_WORKSPACE
        a = list(args); a[6] = 2 * blk - 1
        assert f(*a) == PA_ERR_WORKSPACE
        assert f(N, N, N, 0, N, N, 0, 64, 8, 16, 128, 1, N) == PA_OK


def test_fp8_validation(pa):
    f = pa.lib.kv_cache_write_fp8
    # key, value, src_dtype, k, v, slots, T, NB, Hkv, bs, D, ks, vs, stream
    args = [P, P, 1, P, P, P, 4, 64, 8, 16, 128, 0.5, 0.5, N]
    assert f(*args[:6], -1, *args[7:]) == PA_ERR_SHAPE
    assert f(*args[:11], 0.0, 0.5, N) == PA_ERR_SHAPE
    assert f(*args[:11], 0.5, float("nan"), N) == PA_ERR_SHAPE
    assert f(*args[:11], float("inf"), 0.5, N) == PA_ERR_SHAPE
    assert f(P, P, 2, *args[3:]) == PA_ERR_UNSUPPORTED          # the source must be fp32 or bf16
    assert f(*args[:10], 40, 0.5, 0.5, N) == PA_ERR_UNSUPPORTED  # head_dim not a multiple of 16
    assert f(N, *args[1:]) == PA_ERR_NULL
    assert f(N, N, 1, N, N, N, 0, 64, 8, 16, 128, 0.5, 0.5, N) == PA_OK
    d = pa.lib.paged_attn_decode_fp8
    # out, out_dtype, q, k, v, ks, vs, bt, maxblk, sl, B, Hq, Hkv, D, bs, NB, max_len, scale, part, ws, wsb, stream
    base = [P, 0, P, P, P, 0.5, 0.5, P, 16, P, 4, 32, 8, 128, 16, 64, 256, 0.1, 64, N, 0, N]
    def dec(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return d(*a)
    assert dec(a5=-1.0) == PA_ERR_SHAPE
    assert dec(a13=64) == PA_ERR_UNSUPPORTED                  # FP8 serves head_dim 128 only
    assert dec(a14=4) == PA_ERR_UNSUPPORTED                   # and the MFMA block sizes
    # a group of 17 runs as 17 one-head sub-groups on the balanced split (so this call, without its
    # workspace, is refused for that); with a caller's 16-token pieces on 8K-token rows (512 per row, the
    # partition grid) it has no FP8 kernel
    assert dec(a11=136, a12=8) == PA_ERR_WORKSPACE
    assert dec(a11=136, a12=8, a8=512, a16=8192, a18=16) == PA_ERR_UNSUPPORTED
    assert dec(a11=128, a12=8, a8=512, a16=8192, a18=16) == PA_ERR_WORKSPACE  # group 16: the MFMA grid
    assert dec(a1=2) == PA_ERR_UNSUPPORTED                    # out cannot be FP8
    assert dec(a2=N) == PA_ERR_NULL
    assert dec(a10=0) == PA_OK
    pf = pa.lib.paged_attn_prefill_chunk_fp8
    # out, out_dtype, q, k, v, ks, vs, bt, maxblk, qsl, sl, B, Tq, Hq, Hkv, D, bs, NB, maxq, maxlen, scale, stream
    pbase = [P, 0, P, P, P, 0.5, 0.5, P, 16, P, P, 4, 8, 24, 8, 128, 16, 64, 4, 256, 0.1, N]
    assert pf(*pbase[:15], 64, *pbase[16:]) == PA_ERR_UNSUPPORTED   # FP8 serves head_dim 128 only
    assert pf(*pbase[:16], 4, *pbase[17:]) == PA_ERR_UNSUPPORTED    # and the MFMA block sizes
    pbase[13] = 32
    assert pf(*pbase[:6], 0.0, *pbase[7:]) == PA_ERR_SHAPE
    assert pf(*pbase[:11], 0, *pbase[12:]) == PA_OK
    # the plain calls refuse the FP8 code for their KV
    assert pa.lib.paged_attn_decode(P, 0, P, P, P, 2, P, 16, P, 4, 32, 8, 128, 16, 64, 256, 0.1, 64, N, 0, N) \
        == PA_ERR_UNSUPPORTED


def test_plan_validation(pa):
    size = pa.lib.paged_attn_decode_plan_size
    # B, Hq, Hkv, D, bs, maxblk, max_len, part, kv_dtype
    n = size(64, 32, 8, 128, 16, 128, 2048, 0, 1)
    assert n > 0 and n % 256 == 0
    assert size(64, 32, 8, 128, 16, 128, 2048, 0, 2) == n     # FP8 plans the same split
    assert size(64, 32, 8, 64, 16, 128, 2048, 0, 1) == 0      # head_dim 64: vector path, no plan
    assert size(64, 32, 8, 128, 16, 128, 2048, 0, 0) == 0     # fp32: vector path
    assert size(0, 32, 8, 128, 16, 128, 2048, 0, 1) == 0
    assert size(64, 30, 8, 128, 16, 128, 2048, 0, 1) == 0     # Hq not a multiple of Hkv
    assert size(64, 32, 8, 128, 16, 128, 2048, 24, 1) == 0    # partition not a block multiple
    plan = pa.lib.paged_attn_decode_plan
    # plan, bytes, kv_dtype, bt, maxblk, sl, B, Hq, Hkv, D, bs, NB, max_len, part, stream
    args = [P, n, 1, P, 128, P, 64, 32, 8, 128, 16, 4096, 2048, 0, N]
    assert plan(*args[:2], 7, *args[3:]) == PA_ERR_UNSUPPORTED
    assert plan(N, *args[1:]) == PA_ERR_WORKSPACE
    assert plan(P, n - 1, *args[2:]) == PA_ERR_WORKSPACE
    assert plan(*args[:3], N, *args[4:]) == PA_ERR_NULL
    assert plan(*args[:6], 0, *args[7:]) == PA_OK
    assert plan(N, 0, 1, N, 128, N, 64, 32, 8, 64, 16, 4096, 2048, 0, N) == PA_OK   # nothing to plan
    run = pa.lib.paged_attn_decode_planned
    # out, odt, q, k, v, kvdt, ks, vs, plan, bytes, bt, maxblk, sl, B, Hq, Hkv, D, bs, NB, max_len, scale, part,
    # ws, wsb, stream
    need = pa.paged_attn_decode_workspace_size(64, 32, 8, 128, 16, 2048, 0)
    r = [P, 0, P, P, P, 1, 1.0, 1.0, P, n, P, 128, P, 64, 32, 8, 128, 16, 4096, 2048, 0.1, 0, P, need, N]
    assert run(*r[:8], N, *r[9:]) == PA_ERR_WORKSPACE
    assert run(*r[:9], n - 1, *r[10:]) == PA_ERR_WORKSPACE
    assert run(*r[:5], 3, *r[6:]) == PA_ERR_UNSUPPORTED
    assert run(*r[:13], 0, *r[14:]) == PA_OK


def test_decode_append_validation(pa):
    f = pa.lib.paged_attn_decode_append
    n = pa.lib.paged_attn_decode_plan_size(64, 32, 8, 128, 16, 128, 2048, 0, 1)
    need = pa.paged_attn_decode_workspace_size(64, 32, 8, 128, 16, 2048, 0)
    # out, odt, q, key, value, slots, k, v, kvdt, ks, vs, plan, bytes, bt, maxblk, sl, B, Hq, Hkv, D, bs, NB,
    # max_len, scale, part, ws, wsb, stream
    a = [P, 0, P, P, P, P, P, P, 1, 1.0, 1.0, P, n, P, 128, P, 64, 32, 8, 128, 16, 4096, 2048, 0.1, 0, P, need, N]

    def call(**kw):
        b = list(a)
        for i, v in kw.items():
            b[int(i[1:])] = v
        return f(*b)

    assert call(a3=N) == PA_ERR_NULL          # key
    assert call(a4=N) == PA_ERR_NULL          # value
    assert call(a5=N) == PA_ERR_NULL          # slot_mapping
    assert call(a8=7) == PA_ERR_UNSUPPORTED
    assert call(a11=N) == PA_ERR_WORKSPACE    # the plan
    assert call(a26=16) == PA_ERR_WORKSPACE      # far below what the split needs
    assert call(a17=30) == PA_ERR_SHAPE       # Hq not a multiple of Hkv
    assert call(a16=0) == PA_OK               # no sequences: nothing to write or read


def test_binding_refuses_cpu_tensors(pa):
    import torch
    k = torch.zeros(4, 2, 16, 64)
    with pytest.raises(ValueError, match="GPU"):
        pa.kv_cache_write(torch.zeros(1, 2, 64), torch.zeros(1, 2, 64), k, k.clone(),
                          torch.zeros(1, dtype=torch.int64))
