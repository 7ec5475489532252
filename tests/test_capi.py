"""C-ABI checks that need no GPU: the library loads, exports every function
include/kvq.h declares, sizes planes as the block format prescribes, and
rejects bad arguments on the host before any device work is queued.

The cases here only use argument combinations that fail validation, so no
HIP call is ever reached."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

kvq = pytest.importorskip("decode_attention_rotate_amd")
from decode_attention_rotate_amd import _capi  # noqa: E402

if not os.path.exists(_capi.LIB_PATH):
    pytest.skip("libkvq.so not built", allow_module_level=True)

L = _capi.lib()
FAKE = 0x10000          # aligned, never dereferenced (validation fails first)
FAKE_MISALIGNED = 0x10008


def _header_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text))


def test_exports_every_declared_function():
    declared = _header_functions()
    assert declared == set(_capi.EXPORTS)
    for name in declared:
        assert hasattr(L, name)


def test_ceiling_library_exports_its_header():
    # the benchmark's read-bandwidth probes live in a library of their own
    if not os.path.exists(_capi.CEILING_PATH):
        pytest.skip("libkvq_ceiling.so not built")
    declared = _header_functions(os.path.join(ROOT, "include", "kvq_ceiling.h"))
    assert declared == set(_capi.CEILING_EXPORTS)
    C = _capi.ceiling_lib()
    assert C.kvq_ceiling_sink_words(4, 3) == 4 * 3 * 512
    # invalid arguments are refused before any launch
    assert C.kvq_ceiling_stream(None, 1024, 4, 4, 0, FAKE, None) == -1
    assert C.kvq_ceiling_stream(FAKE, 1000, 4, 4, 0, FAKE, None) == -1
    assert C.kvq_ceiling_stream(FAKE, 1024, 4, 3, 0, FAKE, None) == -1
    args = _capi.KvqCeilingTilesArgs(FAKE, FAKE, FAKE, FAKE, 2, 10, 8192, 4096, 512)
    assert C.kvq_ceiling_tiles(ctypes.byref(args), 4, 3, 0, FAKE, None) == -1
    assert C.kvq_ceiling_tiles(ctypes.byref(args), 4, 1, 4, FAKE, None) == -1
    bad = _capi.KvqCeilingTilesArgs(FAKE, FAKE, FAKE, FAKE, 2, 10, 8192, 16384, 512)
    assert C.kvq_ceiling_tiles(ctypes.byref(bad), 4, 1, 0, FAKE, None) == -1


def test_status_strings():
    for code in range(-6, 1):
        assert isinstance(kvq.kvq_status_str(code), str) and kvq.kvq_status_str(code)


@pytest.mark.parametrize("d,rot", [(64, 1), (128, 1), (256, 1), (32, 0), (96, 0), (192, 1)])
def test_default_rotation_rule(d, rot):
    # velog.io post, section "application and background": on for head_dim
    # >= 64 and a multiple of 64
    c = kvq.kvq_config_default(2, 4, d, 1000)
    assert (c.rotate_k, c.rotate_v) == (rot, rot)
    assert (c.k_bits, c.v_bits, c.tail_len) == (4, 4, 0)


def test_config_check():
    c = kvq.kvq_config_default(2, 4, 128, 1000)
    assert kvq.kvq_config_check(c) == 0
    c.k_bits, c.v_bits = 6, 6                       # q6_0
    assert kvq.kvq_config_check(c) == 0
    for field, val, want in (("head_dim", 320, -2), ("head_dim", 32, -2), ("k_bits", 7, -2),
                             ("v_bits", 3, -2), ("batch", 0, -1), ("batch", 257, -1),
                             ("tail_len", -1, -1), ("max_ctx", 0, -1), ("rotate_k", 2, -1),
                             ("k_min", 2, -1), ("v_min", -1, -1),
                             # int32 positions: the capacity rounded up to a
                             # tile, plus slack, must stay below 2^31
                             ("max_ctx", 2147483647, -1), ("max_ctx", 2147483647 - 64, -1)):
        bad = kvq.kvq_config_default(2, 4, 128, 1000)
        setattr(bad, field, val)
        assert kvq.kvq_config_check(bad) == want, field
    # scale-and-min blocks exist at 4 and 5 bits only (q4_1, q5_1)
    for kb, vb, km, vm, want in ((4, 5, 1, 1, 0), (5, 8, 1, 0, 0), (8, 4, 0, 1, 0),
                                 (6, 4, 1, 0, -2), (4, 8, 0, 1, -2)):
        m = kvq.kvq_config_default(2, 4, 128, 1000)
        m.k_bits, m.v_bits, m.k_min, m.v_min = kb, vb, km, vm
        assert kvq.kvq_config_check(m) == want, (kb, vb, km, vm)


@pytest.mark.parametrize("d", (64, 128, 192, 256))
@pytest.mark.parametrize("kb,vb", ((4, 4), (8, 4), (5, 4), (8, 8), (5, 5), (6, 6)))
def test_plane_bytes(d, kb, vb):
    B, H, max_ctx, T = 3, 2, 1000, 16
    c = kvq.kvq_config(B, H, d, max_ctx, kb, vb, T)
    cap = 1024
    pad = lambda r: (r + 15) // 16 * 16
    assert kvq.kvq_plane_bytes(c, kvq.KVQ_K_CODES) == B * H * cap * pad(d * kb // 8)
    # V codes sit in element-major 64-token tiles with no row padding
    assert kvq.kvq_plane_bytes(c, kvq.KVQ_V_CODES) == B * H * cap * d * vb // 8
    assert kvq.kvq_plane_bytes(c, kvq.KVQ_K_SCALES) == B * H * cap * (d // 32) * 2
    assert kvq.kvq_plane_bytes(c, kvq.KVQ_K_TAIL) == B * H * T * d * 2
    # codes + scales per token-head: 32*b/8 + 2 bytes per 32 elements
    for b, plane in ((kb, kvq.KVQ_K_CODES), (vb, kvq.KVQ_V_CODES)):
        if (d * b // 8) % 16 == 0 or plane == kvq.KVQ_V_CODES:
            per_tok = (kvq.kvq_plane_bytes(c, plane) + kvq.kvq_plane_bytes(c, kvq.KVQ_K_SCALES)) / (B * H * cap)
            assert per_tok == (d // 32) * (32 * b // 8 + 2)


def test_workspace_bytes():
    c = kvq.kvq_config(8, 8, 128, 65536, 8, 4, 1024)
    ws = kvq.kvq_decode_workspace_bytes(c, 40)
    assert ws > 8 * 40 * 128 * 4
    assert kvq.kvq_decode_workspace_bytes(c, 12) == 0     # not a multiple of 8
    assert kvq.kvq_decode_workspace_bytes(c, 4) == 0


def _cache(ptr=FAKE, tail=FAKE):
    return _capi.KvqCache(ptr, FAKE, FAKE, FAKE, tail, tail)


def _lens(*v):
    return (ctypes.c_int32 * len(v))(*v)


def _append(c, cache, n_new, lens, k=FAKE, v=FAKE, dtype=0):
    return L.kvq_rotate_quantize_append(ctypes.byref(c), ctypes.byref(cache), k, v, dtype,
                                        n_new, lens, None)


def test_append_validation():
    c = kvq.kvq_config(2, 2, 128, 100, 4, 4, 0)
    assert _append(c, _cache(), 10, _lens(91, 0)) == _capi.KVQ_ERR_CAPACITY
    assert _append(c, _cache(), 1, _lens(-1, 0)) == _capi.KVQ_ERR_INVALID
    assert _append(c, _cache(), -1, _lens(0, 0)) == _capi.KVQ_ERR_INVALID
    assert _append(c, _cache(0), 1, _lens(0, 0)) == _capi.KVQ_ERR_INVALID
    assert _append(c, _cache(FAKE_MISALIGNED), 1, _lens(0, 0)) == _capi.KVQ_ERR_ALIGN
    assert _append(c, _cache(), 1, _lens(0, 0), k=FAKE_MISALIGNED) == _capi.KVQ_ERR_ALIGN
    assert _append(c, _cache(), 1, _lens(0, 0), k=0) == _capi.KVQ_ERR_INVALID
    assert _append(c, _cache(), 1, _lens(0, 0), dtype=7) == _capi.KVQ_ERR_INVALID
    assert _append(c, _cache(), 0, _lens(0, 0)) == _capi.KVQ_OK      # no-op, no device work
    ct = kvq.kvq_config(2, 2, 128, 100, 4, 4, 8)
    assert _append(ct, _cache(tail=0), 1, _lens(0, 0)) == _capi.KVQ_ERR_INVALID
    bad = kvq.kvq_config_default(2, 2, 128, 100)
    bad.k_bits = 3
    assert _append(bad, _cache(), 1, _lens(0, 0)) == _capi.KVQ_ERR_UNSUPPORTED


def _decode(c, hq, lens, ws_bytes=1 << 40, sm=0.1, q=FAKE, out=FAKE, cache=None):
    cache = cache or _cache()
    return L.kvq_decode_attention(ctypes.byref(c), ctypes.byref(cache), q, 0, hq, sm, lens,
                                  out, FAKE, ws_bytes, None)


def test_decode_grid_limit():
    # 11 query heads per KV head run as 11 chunks of one head: with 10000 KV
    # heads the grid's y size (KV head x chunk) would exceed 65535
    c = kvq.kvq_config(1, 10000, 128, 100, 8, 4, 0)
    assert kvq.kvq_config_check(c) == 0
    assert _decode(c, 110000, _lens(50)) == _capi.KVQ_ERR_INVALID
    big = kvq.kvq_config(1, 8, 128, 2147483647 - 128, 8, 4, 0)
    assert kvq.kvq_config_check(big) == 0


def test_static_workspace_decode_validation():
    # the entry point for callers that cannot allocate: host checks first,
    # then a call whose partials would not fit the static workspace is
    # refused before any device work
    B = 256
    c = kvq.kvq_config(B, 8, 256, 70000, 8, 8, 0)
    assert kvq.kvq_decode_workspace_bytes(c, 64) > _capi.KVQ_STATIC_WORKSPACE_BYTES
    lens = _lens(*([65536] * B))
    f = L.kvq_decode_attention_static
    assert f(ctypes.byref(c), ctypes.byref(_cache()), FAKE, 0, 64, 0.1, lens, FAKE, None) == \
        _capi.KVQ_ERR_WORKSPACE
    small = kvq.kvq_config(2, 4, 128, 100, 8, 4, 0)
    assert f(ctypes.byref(small), ctypes.byref(_cache()), 0, 0, 8, 0.1, _lens(5, 5), FAKE, None) == \
        _capi.KVQ_ERR_INVALID
    assert f(ctypes.byref(small), ctypes.byref(_cache()), FAKE, 0, 6, 0.1, _lens(5, 5), FAKE, None) == \
        _capi.KVQ_ERR_INVALID
    assert f(ctypes.byref(small), ctypes.byref(_cache()), FAKE, 0, 8, 0.1, _lens(5, 101), FAKE, None) == \
        _capi.KVQ_ERR_CAPACITY
    assert f(ctypes.byref(small), ctypes.byref(_cache()), FAKE_MISALIGNED, 0, 8, 0.1, _lens(5, 5), FAKE,
             None) == _capi.KVQ_ERR_ALIGN


def test_decode_step_validation():
    # the fused append-and-attend call: the append's and the decode's host
    # checks, all before any device work
    c = kvq.kvq_config(2, 4, 128, 100, 8, 4, 16)
    f = L.kvq_decode_step

    def step(lens, k=FAKE, v=FAKE, q=FAKE, hq=8, kvdt=0, qdt=0, ws=1 << 40, cache=None, cfg=c):
        return f(ctypes.byref(cfg), ctypes.byref(cache or _cache()), k, v, kvdt, q, qdt, hq, 0.1,
                 lens, FAKE, FAKE, ws, None)
    assert step(_lens(100, 0)) == _capi.KVQ_ERR_CAPACITY
    assert step(_lens(-1, 0)) == _capi.KVQ_ERR_INVALID
    assert step(_lens(5, 5), k=0) == _capi.KVQ_ERR_INVALID
    assert step(_lens(5, 5), v=FAKE_MISALIGNED) == _capi.KVQ_ERR_ALIGN
    assert step(_lens(5, 5), kvdt=3) == _capi.KVQ_ERR_INVALID
    assert step(_lens(5, 5), qdt=3) == _capi.KVQ_ERR_INVALID
    assert step(_lens(5, 5), hq=6) == _capi.KVQ_ERR_INVALID
    assert step(_lens(5, 5), q=0) == _capi.KVQ_ERR_INVALID
    assert step(_lens(5, 5), ws=16) == _capi.KVQ_ERR_WORKSPACE
    assert step(_lens(5, 5), cache=_cache(tail=0)) == _capi.KVQ_ERR_INVALID
    bad = kvq.kvq_config_default(2, 4, 128, 100)
    bad.v_bits = 7
    assert step(_lens(5, 5), cfg=bad) == _capi.KVQ_ERR_UNSUPPORTED


def test_decode_validation():
    c = kvq.kvq_config(2, 4, 128, 100, 8, 4, 0)
    assert _decode(c, 6, _lens(5, 5)) == _capi.KVQ_ERR_INVALID      # 6 % 4 != 0
    assert _decode(c, 2, _lens(5, 5)) == _capi.KVQ_ERR_INVALID
    assert _decode(c, 8, _lens(0, 5)) == _capi.KVQ_ERR_INVALID      # empty sequence
    assert _decode(c, 8, _lens(5, 101)) == _capi.KVQ_ERR_CAPACITY
    assert _decode(c, 8, _lens(5, 5), sm=float("nan")) == _capi.KVQ_ERR_INVALID
    assert _decode(c, 8, _lens(5, 5), ws_bytes=100) == _capi.KVQ_ERR_WORKSPACE
    assert _decode(c, 8, _lens(5, 5), q=FAKE_MISALIGNED, ws_bytes=100) == _capi.KVQ_ERR_ALIGN
    assert _decode(c, 8, _lens(5, 5), out=0) == _capi.KVQ_ERR_INVALID


def test_dequantize_validation():
    c = kvq.kvq_config(2, 4, 128, 100, 8, 4, 0)
    lens = _lens(10, 20)
    deq = lambda which, b, t0, t1, space=0, out=FAKE: L.kvq_dequantize(
        ctypes.byref(c), ctypes.byref(_cache()), which, b, t0, t1, lens, space, out, None)
    assert deq(2, 0, 0, 5) == _capi.KVQ_ERR_INVALID
    assert deq(0, 2, 0, 5) == _capi.KVQ_ERR_INVALID
    assert deq(0, 0, 5, 4) == _capi.KVQ_ERR_INVALID
    assert deq(0, 0, 0, 11) == _capi.KVQ_ERR_INVALID
    assert deq(0, 0, 0, 5, space=3) == _capi.KVQ_ERR_INVALID
    assert deq(0, 0, 0, 5, out=FAKE_MISALIGNED) == _capi.KVQ_ERR_ALIGN
    assert deq(0, 0, 0, 5, out=0) == _capi.KVQ_ERR_INVALID
    assert deq(0, 0, 3, 3, out=0) == _capi.KVQ_OK                    # empty range


def test_prefill_workspace_bytes():
    c = kvq.kvq_config(1, 8, 128, 65536, 8, 4, 1024)
    ws = kvq.kvq_prefill_workspace_bytes(c, 40, 512)
    assert ws >= 512 * 40 * (128 + 2) * 4                   # at least one split per row
    assert kvq.kvq_prefill_workspace_bytes(c, 40, 1) <= ws
    assert kvq.kvq_prefill_workspace_bytes(c, 12, 16) == 0    # not a multiple of 8
    assert kvq.kvq_prefill_workspace_bytes(c, 40, 0) == 0


def _prefill(c, hq, n_q, lens, ws_bytes=1 << 40, sm=0.1, q=FAKE, out=FAKE):
    return L.kvq_prefill_attention(ctypes.byref(c), ctypes.byref(_cache()), q, 0, hq, n_q, sm,
                                   lens, out, FAKE, ws_bytes, None)


def test_prefill_validation():
    c = kvq.kvq_config(2, 4, 128, 100, 8, 4, 0)
    assert _prefill(c, 6, 4, _lens(5, 5)) == _capi.KVQ_ERR_INVALID    # 6 % 4 != 0
    assert _prefill(c, 8, 0, _lens(5, 5)) == _capi.KVQ_ERR_INVALID    # no query
    assert _prefill(c, 8, 6, _lens(5, 9)) == _capi.KVQ_ERR_INVALID    # length below n_q
    assert _prefill(c, 8, 4, _lens(5, 101)) == _capi.KVQ_ERR_CAPACITY
    assert _prefill(c, 8, 4, _lens(5, 5), sm=float("inf")) == _capi.KVQ_ERR_INVALID
    assert _prefill(c, 8, 4, _lens(5, 5), ws_bytes=100) == _capi.KVQ_ERR_WORKSPACE
    assert _prefill(c, 8, 4, _lens(5, 5), q=FAKE_MISALIGNED) == _capi.KVQ_ERR_ALIGN
    assert _prefill(c, 8, 4, _lens(5, 5), out=0) == _capi.KVQ_ERR_INVALID


@pytest.mark.parametrize("d", (64, 128, 192, 256))
def test_plane_bytes_scale_and_min(d):
    # an (s, m) fp16 pair per block: q5_1 costs 32*5/8 + 4 = 24 bytes per 32
    # elements, 37.5 % of bf16 (the aiwitness.kr table's q5_1 row)
    B, H, cap = 2, 3, 1024
    c = kvq.kvq_config(B, H, d, 1000, 5, 4, 0, k_min=True, v_min=False)
    assert kvq.kvq_plane_bytes(c, kvq.KVQ_K_SCALES) == B * H * cap * (d // 32) * 4
    assert kvq.kvq_plane_bytes(c, kvq.KVQ_V_SCALES) == B * H * cap * (d // 32) * 2
    c = kvq.kvq_config(B, H, d, 1000, 5, 5, 0, k_min=True, v_min=True)
    per_tok = (kvq.kvq_plane_bytes(c, kvq.KVQ_V_CODES) + kvq.kvq_plane_bytes(c, kvq.KVQ_V_SCALES)) / (B * H * cap)
    assert per_tok / (2 * d) == 0.375


def test_config_layout_and_sign_seed():
    # fourteen 32-bit fields: sign_seed, then k_min, v_min, page_pool,
    # outliers last; all 0 by default (plain Sylvester matrix, absmax blocks,
    # contiguous, no outlier channels)
    assert ctypes.sizeof(_capi.KvqConfig) == 56
    assert _capi.KvqConfig.sign_seed.offset == 36 and _capi.KvqConfig.v_min.offset == 44
    assert _capi.KvqConfig.page_pool.offset == 48 and _capi.KvqConfig.outliers.offset == 52
    c = kvq.kvq_config_default(1, 1, 128, 64)
    assert c.sign_seed == 0 and c.k_min == 0 and c.v_min == 0 and c.page_pool == 0
    assert c.outliers == 0
    c2 = kvq.kvq_config(1, 1, 128, 64, sign_seed=0xFFFFFFFF)
    assert c2.sign_seed == 0xFFFFFFFF


def test_cache_struct_layout():
    # six plane pointers, the page table, four outlier planes, the lists
    assert ctypes.sizeof(_capi.KvqCache) == 12 * 8
    assert _capi.KvqCache.page_table.offset == 48
    assert _capi.KvqCache.k_out_codes.offset == 56 and _capi.KvqCache.outlier_idx.offset == 88


@pytest.mark.parametrize("kb,vb", ((4, 4), (8, 4), (5, 6), (8, 8)))
def test_outlier_config_and_planes(kb, vb):
    # 32 channels per plane and KV head: K codes [tile][64][32] bytes, V
    # codes in element-major 8-bit tiles of a 32-element head (the same
    # size), one fp16 scale per position; the other planes keep their sizes
    B, H, max_ctx = 3, 2, 1000
    c = kvq.kvq_config(B, H, 128, max_ctx, kb, vb, outliers=32)
    plain = kvq.kvq_config(B, H, 128, max_ctx, kb, vb)
    cap = 1024
    assert kvq.kvq_plane_bytes(c, _capi.KVQ_K_OUT_CODES) == B * H * cap * 32
    assert kvq.kvq_plane_bytes(c, _capi.KVQ_V_OUT_CODES) == B * H * cap * 32
    assert kvq.kvq_plane_bytes(c, _capi.KVQ_K_OUT_SCALES) == B * H * cap * 2
    assert kvq.kvq_plane_bytes(c, _capi.KVQ_V_OUT_SCALES) == B * H * cap * 2
    for p in (kvq.KVQ_K_CODES, kvq.KVQ_V_CODES, kvq.KVQ_K_SCALES, kvq.KVQ_V_SCALES):
        assert kvq.kvq_plane_bytes(c, p) == kvq.kvq_plane_bytes(plain, p)
    for p in (_capi.KVQ_K_OUT_CODES, _capi.KVQ_V_OUT_SCALES):
        assert kvq.kvq_plane_bytes(plain, p) == 0
    paged = kvq.kvq_config(B, H, 128, max_ctx, kb, vb, page_pool=37, outliers=32)
    assert kvq.kvq_plane_bytes(paged, _capi.KVQ_K_OUT_CODES) == 37 * H * 64 * 32
    assert kvq.kvq_plane_bytes(paged, _capi.KVQ_V_OUT_SCALES) == 37 * H * 64 * 2
    # the workspace grows by the outlier channels' partial sums
    assert kvq.kvq_decode_workspace_bytes(c, 8) > kvq.kvq_decode_workspace_bytes(plain, 8)


def test_outlier_validation():
    base = kvq.kvq_config_default(2, 2, 128, 100)
    for field, val, want in (("outliers", 16, -1), ("outliers", -32, -1), ("outliers", 64, -1),
                             ("tail_len", 8, -2), ("head_dim", 64, -2), ("k_min", 1, -2),
                             ("v_min", 1, -2)):
        c = kvq.kvq_config_default(2, 2, 128, 100)
        c.outliers = 32
        setattr(c, field, val)
        assert kvq.kvq_config_check(c) == want, (field, val)
    c = kvq.kvq_config(2, 2, 128, 100, outliers=32)
    assert kvq.kvq_config_check(c) == 0 and kvq.kvq_config_check(base) == 0
    ch = _cache(tail=0)
    # no outlier planes or lists: refused before any launch
    assert _append(c, ch, 1, _lens(0, 0)) == _capi.KVQ_ERR_INVALID
    assert _decode(c, 4, _lens(1, 1), cache=ch) == _capi.KVQ_ERR_INVALID
    for name in ("k_out_codes", "k_out_scales", "v_out_codes", "v_out_scales"):
        setattr(ch, name, FAKE)
    assert _decode(c, 4, _lens(1, 1), cache=ch) == _capi.KVQ_ERR_INVALID   # no lists
    ch.outlier_idx = FAKE + 2
    assert _decode(c, 4, _lens(1, 1), cache=ch) == _capi.KVQ_ERR_ALIGN
    ch.v_out_codes = FAKE_MISALIGNED
    ch.outlier_idx = FAKE
    assert _decode(c, 4, _lens(1, 1), cache=ch) == _capi.KVQ_ERR_ALIGN
    ch.v_out_codes = FAKE
    # prefill is not built with outlier channels
    assert L.kvq_prefill_attention(ctypes.byref(c), ctypes.byref(ch), FAKE, 0, 4, 1,
                                   ctypes.c_float(0.1), _lens(1, 1), FAKE, FAKE, 1 << 40,
                                   None) == _capi.KVQ_ERR_UNSUPPORTED
    # n_new = 0 and an empty read-back queue nothing: accepted
    assert _append(c, ch, 0, _lens(0, 0)) == 0
    assert L.kvq_dequantize(ctypes.byref(c), ctypes.byref(ch), 1, 0, 0, 0, _lens(1, 1), 1, FAKE,
                            None) == 0


@pytest.mark.parametrize("d,kb,vb,km", [(64, 4, 4, 0), (128, 8, 4, 0), (192, 5, 6, 0),
                                        (256, 5, 4, 1)])
def test_plane_bytes_paged(d, kb, vb, km):
    # a pool of P pages holds P tiles of 64 positions per KV head; the tail
    # planes keep their per-sequence size
    B, H, T, P = 3, 2, 16, 37
    flat = kvq.kvq_config(B, H, d, 1000, kb, vb, T, k_min=km)
    paged = kvq.kvq_config(B, H, d, 1000, kb, vb, T, k_min=km, page_pool=P)
    tiles = (1000 + 63) // 64
    for plane in (kvq.KVQ_K_CODES, kvq.KVQ_V_CODES, kvq.KVQ_K_SCALES, kvq.KVQ_V_SCALES):
        per_tile = kvq.kvq_plane_bytes(flat, plane) // (B * H * tiles)
        assert kvq.kvq_plane_bytes(flat, plane) == B * H * tiles * per_tile
        assert kvq.kvq_plane_bytes(paged, plane) == P * H * per_tile
    for plane in (kvq.KVQ_K_TAIL, kvq.KVQ_V_TAIL):
        assert kvq.kvq_plane_bytes(paged, plane) == kvq.kvq_plane_bytes(flat, plane) == B * H * T * d * 2
    assert kvq.page_table_tiles(paged) == tiles


def _paged_cache(table):
    c = _cache()
    c.page_table = table
    return c


def test_paged_validation():
    c = kvq.kvq_config(2, 2, 128, 100, 4, 4, 0, page_pool=8)
    bad = kvq.kvq_config_default(2, 2, 128, 100)
    bad.page_pool = -1
    assert kvq.kvq_config_check(bad) == _capi.KVQ_ERR_INVALID
    assert kvq.kvq_plane_bytes(bad, kvq.KVQ_K_CODES) == 0
    # no page table, or one not 4-byte aligned: rejected before any launch
    assert _append(c, _paged_cache(0), 1, _lens(0, 0)) == _capi.KVQ_ERR_INVALID
    assert _append(c, _paged_cache(FAKE + 2), 1, _lens(0, 0)) == _capi.KVQ_ERR_ALIGN
    assert _decode(c, 4, _lens(1, 1), cache=_paged_cache(0)) == _capi.KVQ_ERR_INVALID
    assert _decode(c, 4, _lens(1, 1), cache=_paged_cache(FAKE + 1)) == _capi.KVQ_ERR_ALIGN
    out = FAKE
    assert L.kvq_dequantize(ctypes.byref(c), ctypes.byref(_paged_cache(0)), 0, 0, 0, 1,
                            _lens(1, 1), 0, out, None) == _capi.KVQ_ERR_INVALID
    # a table 4-byte aligned but not 16 is accepted (validation passes; n_new = 0
    # queues nothing)
    assert _append(c, _paged_cache(FAKE + 4), 0, _lens(0, 0)) == _capi.KVQ_OK
    # the table is ignored by contiguous caches
    flat = kvq.kvq_config(2, 2, 128, 100, 4, 4, 0)
    assert _append(flat, _paged_cache(0), 0, _lens(0, 0)) == _capi.KVQ_OK
