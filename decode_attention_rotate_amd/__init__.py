"""kvq: rotated low-bit KV cache and decode attention for MI355X (gfx950).

Thin Python binding over the C ABI in include/kvq.h.  Every step of the hot
path runs in the HIP kernels of libkvq.so; this module only marshals
arguments.  PyTorch supplies device memory and the current HIP stream.

    cfg   = kvq_config(batch, n_kv_heads, head_dim, max_ctx, k_bits=8, v_bits=4,
                       tail_len=1024)
    cache = KVCache(cfg, device="cuda")
    kvq_rotate_quantize_append(cfg, cache, k_new, v_new, seq_len)
    out   = kvq_decode_attention(cfg, cache, q, seq_len)
    x     = kvq_dequantize(cfg, cache, which=0, b=0, t0=0, t1=n, seq_len=seq_len)
"""

import ctypes
import math

from . import _capi
from ._capi import (KvqConfig, KvqCache, KvqError, KVQ_BF16, KVQ_F32,
                    KVQ_K_CODES, KVQ_K_SCALES, KVQ_V_CODES, KVQ_V_SCALES,
                    KVQ_K_TAIL, KVQ_V_TAIL, KVQ_K_OUT_CODES, KVQ_K_OUT_SCALES,
                    KVQ_V_OUT_CODES, KVQ_V_OUT_SCALES, KVQ_MAX_BATCH, KVQ_PAGE_TOKENS,
                    KVQ_STATIC_WORKSPACE_BYTES, LIB_PATH)

__all__ = [
    "KvqConfig", "KvqCache", "KvqError", "KVCache", "kvq_config",
    "kvq_config_default", "kvq_config_check", "kvq_plane_bytes",
    "kvq_decode_workspace_bytes", "kvq_rotate_quantize_append",
    "kvq_decode_attention", "kvq_dequantize", "kvq_status_str",
    "kvq_profile_decode_events", "kvq_prefill_workspace_bytes", "kvq_prefill_attention",
    "kvq_decode_attention_static", "KVQ_STATIC_WORKSPACE_BYTES", "kvq_decode_step",
    "KVQ_PAGE_TOKENS", "LIB_PATH",
]


def _torch():
    import torch
    return torch


def kvq_config_default(batch, n_kv_heads, head_dim, max_ctx):
    return _capi.lib().kvq_config_default(batch, n_kv_heads, head_dim, max_ctx)


def kvq_config(batch, n_kv_heads, head_dim, max_ctx, k_bits=4, v_bits=4,
               tail_len=0, rotate_k=None, rotate_v=None, sign_seed=0, k_min=False,
               v_min=False, page_pool=0, outliers=0):
    """kvq_config_default with fields overridden; validated by the library.
    k_min / v_min select scale-and-min blocks (q4_1 / q5_1 at 4 / 5 bits);
    page_pool > 0 makes a paged cache of that many 64-position pages;
    outliers = 32 keeps 32 outlier channels per plane and KV head at 8 bits
    (KVCache then needs their channel lists)."""
    c = kvq_config_default(batch, n_kv_heads, head_dim, max_ctx)
    c.k_bits, c.v_bits, c.tail_len = k_bits, v_bits, tail_len
    if rotate_k is not None:
        c.rotate_k = int(rotate_k)
    if rotate_v is not None:
        c.rotate_v = int(rotate_v)
    c.sign_seed = int(sign_seed) & 0xFFFFFFFF
    c.k_min, c.v_min = int(k_min), int(v_min)
    c.page_pool = int(page_pool)
    c.outliers = int(outliers)
    _capi.check(_capi.lib().kvq_config_check(ctypes.byref(c)), "kvq_config")
    return c


def kvq_config_check(cfg):
    return _capi.lib().kvq_config_check(ctypes.byref(cfg))


def kvq_plane_bytes(cfg, plane):
    return _capi.lib().kvq_plane_bytes(ctypes.byref(cfg), plane)


def kvq_decode_workspace_bytes(cfg, n_q_heads):
    return _capi.lib().kvq_decode_workspace_bytes(ctypes.byref(cfg), n_q_heads)


def kernel_elapsed_ms(before, after):
    """Elapsed ms between two torch.cuda.Event objects that
    kvq_profile_decode_events had the library record."""
    return _capi.event_elapsed_ms(before.cuda_event, after.cuda_event)


__all__ += ["kernel_elapsed_ms"]


def kvq_status_str(status):
    return _capi.status_str(status)


def kvq_profile_decode_events(before, after):
    """Bind two torch.cuda.Event objects to the split-K (or matrix-core
    prefill) kernel of later decode and prefill calls on this thread, so they
    take that kernel's own start and end; pass None, None to stop."""
    if before is None or after is None:
        _capi.lib().kvq_profile_decode_events(None, None)
        return
    # torch creates the underlying hipEvent on the first record(); record once
    # so both handles exist (the library's later records overwrite the times)
    for ev in (before, after):
        if not ev.cuda_event:
            ev.record()
    _capi.lib().kvq_profile_decode_events(ctypes.c_void_p(before.cuda_event),
                                          ctypes.c_void_p(after.cuda_event))


def page_table_tiles(cfg):
    """Row length of a paged cache's page table: ceil(max_ctx / 64)."""
    return (cfg.max_ctx + KVQ_PAGE_TOKENS - 1) // KVQ_PAGE_TOKENS


__all__ += ["page_table_tiles"]


class KVCache:
    """Device planes of one cache, allocated zeroed with torch (uint8).

    For a paged configuration (cfg.page_pool > 0) the code and scale planes
    are the page pool and `page_table` is the int32 device tensor
    [batch][ceil(max_ctx/64)] mapping each sequence's 64-position tiles to
    pages; the caller fills it (the planes keep a reference to it)."""

    PLANES = (("k_codes", KVQ_K_CODES), ("k_scales", KVQ_K_SCALES),
              ("v_codes", KVQ_V_CODES), ("v_scales", KVQ_V_SCALES),
              ("k_tail", KVQ_K_TAIL), ("v_tail", KVQ_V_TAIL),
              ("k_out_codes", _capi.KVQ_K_OUT_CODES), ("k_out_scales", _capi.KVQ_K_OUT_SCALES),
              ("v_out_codes", _capi.KVQ_V_OUT_CODES), ("v_out_scales", _capi.KVQ_V_OUT_SCALES))

    def __init__(self, cfg, device="cuda", page_table=None, outlier_idx=None):
        """outlier_idx (cfg.outliers > 0): the channel lists, int32 device
        tensor [2][n_kv_heads][32] (K's, then V's)."""
        torch = _torch()
        self.cfg = cfg
        self.planes = {}
        ptrs = {}
        self.page_table = None
        if cfg.page_pool > 0:
            if page_table is None:
                raise ValueError("a paged cache needs a page_table")
            want = (cfg.batch, page_table_tiles(cfg))
            if (page_table.dtype != torch.int32 or tuple(page_table.shape) != want
                    or not page_table.is_cuda or not page_table.is_contiguous()):
                raise ValueError("page_table must be a contiguous int32 device tensor of shape %s"
                                 % (want,))
            self.page_table = page_table
            ptrs["page_table"] = page_table.data_ptr()
        self.outlier_idx = None
        if cfg.outliers > 0:
            want = (2, cfg.n_kv_heads, cfg.outliers)
            if (outlier_idx is None or outlier_idx.dtype != torch.int32
                    or tuple(outlier_idx.shape) != want or not outlier_idx.is_cuda
                    or not outlier_idx.is_contiguous()):
                raise ValueError("outliers need outlier_idx, a contiguous int32 device tensor "
                                 "of shape %s" % (want,))
            self.outlier_idx = outlier_idx
            ptrs["outlier_idx"] = outlier_idx.data_ptr()
        for name, pid in self.PLANES:
            nbytes = kvq_plane_bytes(cfg, pid)
            optional = (name.endswith("tail") and cfg.tail_len == 0) or \
                ("_out_" in name and cfg.outliers == 0)
            if nbytes == 0 and optional:
                self.planes[name] = None
                ptrs[name] = None
                continue
            if nbytes == 0:
                raise KvqError(_capi.KVQ_ERR_INVALID, "kvq_plane_bytes(%s)" % name)
            t = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            self.planes[name] = t
            ptrs[name] = t.data_ptr()
        self.struct = KvqCache(**ptrs)

    def __getitem__(self, name):
        return self.planes[name]

    def sequence(self, b):
        """(config, cache) of sequence b alone over the same device memory:
        batch 1, the same page pool, row b of the page table and sequence b's
        tail slots, so calls can run on one sequence of a paged cache (for
        instance appends of a length the others do not share).  Paged caches
        only."""
        cfg = self.cfg
        if cfg.page_pool <= 0:
            raise ValueError("sequence views need a paged cache")
        if not 0 <= b < cfg.batch:
            raise IndexError("sequence %d of %d" % (b, cfg.batch))
        one = KvqConfig.from_buffer_copy(cfg)
        one.batch = 1
        view = KVCache.__new__(KVCache)
        view.cfg = one
        view.page_table = self.page_table[b:b + 1]
        view.planes = dict(self.planes)
        tail_bytes = cfg.n_kv_heads * cfg.tail_len * cfg.head_dim * 2
        ptrs = {"page_table": view.page_table.data_ptr()}
        if self.outlier_idx is not None:
            ptrs["outlier_idx"] = self.outlier_idx.data_ptr()
        for name, _ in self.PLANES:
            t = self.planes[name]
            if t is None:
                ptrs[name] = None
            elif name.endswith("tail"):
                view.planes[name] = t[b * tail_bytes:(b + 1) * tail_bytes]
                ptrs[name] = view.planes[name].data_ptr()
            else:
                ptrs[name] = t.data_ptr()
        view.struct = KvqCache(**ptrs)
        return one, view


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KVQ_BF16
    if t.dtype == torch.float32:
        return KVQ_F32
    raise TypeError("inputs must be torch.bfloat16 or torch.float32, got %s" % t.dtype)


def _lens(seq_len, batch):
    vals = [int(x) for x in seq_len]
    if len(vals) != batch:
        raise ValueError("seq_len must have %d entries" % batch)
    return (ctypes.c_int32 * batch)(*vals)


def _device_tensor(t, what):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous device tensor" % what)


def kvq_rotate_quantize_append(cfg, cache, k_new, v_new, seq_len, stream=None):
    """Append k_new/v_new [B][n_new][Hkv][d] at positions seq_len[b].. ."""
    _device_tensor(k_new, "k_new")
    _device_tensor(v_new, "v_new")
    if k_new.shape != v_new.shape or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must match in shape and dtype")
    B, n_new, H, d = k_new.shape
    if (B, H, d) != (cfg.batch, cfg.n_kv_heads, cfg.head_dim):
        raise ValueError("k_new shape %s does not match the configuration" % (tuple(k_new.shape),))
    st = _capi.lib().kvq_rotate_quantize_append(
        ctypes.byref(cfg), ctypes.byref(cache.struct), k_new.data_ptr(), v_new.data_ptr(),
        _dtype_code(k_new), n_new, _lens(seq_len, cfg.batch), _stream(stream))
    _capi.check(st, "kvq_rotate_quantize_append")


def kvq_decode_attention(cfg, cache, q, seq_len, sm_scale=None, out=None,
                         workspace=None, stream=None):
    """Decode attention for q [B][Hq][d]; returns float32 [B][Hq][d]."""
    torch = _torch()
    _device_tensor(q, "q")
    B, Hq, d = q.shape
    if (B, d) != (cfg.batch, cfg.head_dim):
        raise ValueError("q shape %s does not match the configuration" % (tuple(q.shape),))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _device_tensor(out, "out")
    need = kvq_decode_workspace_bytes(cfg, Hq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = _capi.lib().kvq_decode_attention(
        ctypes.byref(cfg), ctypes.byref(cache.struct), q.data_ptr(), _dtype_code(q), Hq,
        float(sm_scale), _lens(seq_len, cfg.batch), out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _capi.check(st, "kvq_decode_attention")
    return out


def kvq_decode_step(cfg, cache, k_new, v_new, q, seq_len, sm_scale=None, out=None,
                    workspace=None, stream=None):
    """One decode step: append k_new / v_new [B][1][Hkv][d] at positions
    seq_len[b] (lengths before the step), then attend q [B][Hq][d] over the
    seq_len[b] + 1 positions; returns float32 [B][Hq][d].  The caller
    advances its lengths afterwards."""
    torch = _torch()
    for t, name in ((k_new, "k_new"), (v_new, "v_new"), (q, "q")):
        _device_tensor(t, name)
    B, Hq, d = q.shape
    if (B, d) != (cfg.batch, cfg.head_dim) or tuple(k_new.shape) != (B, 1, cfg.n_kv_heads, d) \
            or tuple(v_new.shape) != tuple(k_new.shape) or v_new.dtype != k_new.dtype:
        raise ValueError("shapes q %s, k_new %s, v_new %s do not match the configuration"
                         % (tuple(q.shape), tuple(k_new.shape), tuple(v_new.shape)))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _device_tensor(out, "out")
    need = kvq_decode_workspace_bytes(cfg, Hq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = _capi.lib().kvq_decode_step(
        ctypes.byref(cfg), ctypes.byref(cache.struct), k_new.data_ptr(), v_new.data_ptr(),
        _dtype_code(k_new), q.data_ptr(), _dtype_code(q), Hq, float(sm_scale),
        _lens(seq_len, cfg.batch), out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _capi.check(st, "kvq_decode_step")
    return out


def kvq_decode_attention_static(cfg, cache, q, seq_len, sm_scale=None, out=None, stream=None):
    """kvq_decode_attention with the library's static device workspace (no
    workspace argument, nothing allocated by the library); calls on one GPU
    share that workspace and must not overlap.  Returns float32 [B][Hq][d]."""
    torch = _torch()
    _device_tensor(q, "q")
    B, Hq, d = q.shape
    if (B, d) != (cfg.batch, cfg.head_dim):
        raise ValueError("q shape %s does not match the configuration" % (tuple(q.shape),))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _device_tensor(out, "out")
    st = _capi.lib().kvq_decode_attention_static(
        ctypes.byref(cfg), ctypes.byref(cache.struct), q.data_ptr(), _dtype_code(q), Hq,
        float(sm_scale), _lens(seq_len, cfg.batch), out.data_ptr(), _stream(stream))
    _capi.check(st, "kvq_decode_attention_static")
    return out


def kvq_prefill_workspace_bytes(cfg, n_q_heads, n_q):
    return _capi.lib().kvq_prefill_workspace_bytes(ctypes.byref(cfg), n_q_heads, n_q)


def kvq_prefill_attention(cfg, cache, q, seq_len, sm_scale=None, out=None,
                          workspace=None, stream=None):
    """Chunked prefill attention for q [B][n_q][Hq][d], the queries of the
    last n_q positions of each sequence (already appended); returns float32
    [B][n_q][Hq][d]."""
    torch = _torch()
    _device_tensor(q, "q")
    B, n_q, Hq, d = q.shape
    if (B, d) != (cfg.batch, cfg.head_dim):
        raise ValueError("q shape %s does not match the configuration" % (tuple(q.shape),))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, n_q, Hq, d), dtype=torch.float32, device=q.device)
    _device_tensor(out, "out")
    need = kvq_prefill_workspace_bytes(cfg, Hq, n_q)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = _capi.lib().kvq_prefill_attention(
        ctypes.byref(cfg), ctypes.byref(cache.struct), q.data_ptr(), _dtype_code(q), Hq, n_q,
        float(sm_scale), _lens(seq_len, cfg.batch), out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _capi.check(st, "kvq_prefill_attention")
    return out


def kvq_dequantize(cfg, cache, which, b, t0, t1, seq_len, space=0, out=None, stream=None):
    """float32 [t1-t0][Hkv][d] read back from the K (0) or V (1) cache."""
    torch = _torch()
    dev = cache["k_codes"].device
    if out is None:
        out = torch.empty((max(t1 - t0, 0), cfg.n_kv_heads, cfg.head_dim),
                          dtype=torch.float32, device=dev)
    _device_tensor(out, "out")
    st = _capi.lib().kvq_dequantize(
        ctypes.byref(cfg), ctypes.byref(cache.struct), which, b, t0, t1,
        _lens(seq_len, cfg.batch), space, out.data_ptr(), _stream(stream))
    _capi.check(st, "kvq_dequantize")
    return out
