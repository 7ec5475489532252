"""ctypes declarations of the kvq C ABI (include/kvq.h).

Loads libkvq.so from this package directory and fails loudly when it is
missing: there is no fallback implementation."""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")
CEILING_PATH = os.path.join(_HERE, "libkvq_ceiling.so")

KVQ_OK = 0
KVQ_ERR_INVALID = -1
KVQ_ERR_UNSUPPORTED = -2
KVQ_ERR_CAPACITY = -3
KVQ_ERR_ALIGN = -4
KVQ_ERR_HIP = -5
KVQ_ERR_WORKSPACE = -6

KVQ_BF16 = 0
KVQ_F32 = 1

KVQ_K_CODES, KVQ_K_SCALES, KVQ_V_CODES, KVQ_V_SCALES, KVQ_K_TAIL, KVQ_V_TAIL = range(6)
KVQ_K_OUT_CODES, KVQ_K_OUT_SCALES, KVQ_V_OUT_CODES, KVQ_V_OUT_SCALES = range(6, 10)
OUTLIER_CHANNELS = 32
KVQ_MAX_BATCH = 256
KVQ_PAGE_TOKENS = 64

EXPORTS = (
    "kvq_config_default", "kvq_config_check", "kvq_plane_bytes",
    "kvq_decode_workspace_bytes", "kvq_rotate_quantize_append",
    "kvq_decode_attention", "kvq_dequantize", "kvq_status_str",
    "kvq_profile_decode_events", "kvq_prefill_workspace_bytes",
    "kvq_prefill_attention", "kvq_decode_attention_static", "kvq_decode_step",
)
KVQ_STATIC_WORKSPACE_BYTES = 33554432


CEILING_EXPORTS = ("kvq_ceiling_stream", "kvq_ceiling_tiles", "kvq_ceiling_sink_words")


class KvqConfig(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "n_kv_heads", "head_dim", "k_bits", "v_bits", "tail_len",
        "max_ctx", "rotate_k", "rotate_v")] + [("sign_seed", ctypes.c_uint32),
                                               ("k_min", ctypes.c_int32), ("v_min", ctypes.c_int32),
                                               ("page_pool", ctypes.c_int32),
                                               ("outliers", ctypes.c_int32)]

    def __repr__(self):
        return "KvqConfig(%s)" % ", ".join(
            "%s=%d" % (f, getattr(self, f)) for f, _ in self._fields_)


class KvqCache(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "k_codes", "k_scales", "v_codes", "v_scales", "k_tail", "v_tail", "page_table",
        "k_out_codes", "k_out_scales", "v_out_codes", "v_out_scales", "outlier_idx")]


class KvqCeilingTilesArgs(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in ("k_codes", "v_codes", "k_scales", "v_scales")] + [
        (name, ctypes.c_int32) for name in ("units", "tiles", "k_tile_bytes", "v_tile_bytes",
                                            "s_tile_bytes")]


class KvqError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, status_str(status), status))


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime with the same soname as the system
        # one; importing torch first makes libkvq.so bind to that copy, so the
        # process runs a single runtime and torch's streams and allocations are
        # valid in kvq calls.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libkvq.so is not built (%s); run python -m decode_attention_rotate_amd.build"
                % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.POINTER, ctypes.c_int32, ctypes.c_size_t
        CFG, CACHE = P(KvqConfig), P(KvqCache)
        vp = ctypes.c_void_p
        sig = {
            "kvq_config_default": (KvqConfig, [I32, I32, I32, I32]),
            "kvq_config_check": (I32, [CFG]),
            "kvq_plane_bytes": (SZ, [CFG, I32]),
            "kvq_decode_workspace_bytes": (SZ, [CFG, I32]),
            "kvq_rotate_quantize_append": (I32, [CFG, CACHE, vp, vp, I32, I32, P(I32), vp]),
            "kvq_decode_attention": (I32, [CFG, CACHE, vp, I32, I32, ctypes.c_float, P(I32),
                                           vp, vp, SZ, vp]),
            "kvq_decode_step": (I32, [CFG, CACHE, vp, vp, I32, vp, I32, I32, ctypes.c_float, P(I32),
                                      vp, vp, SZ, vp]),
            "kvq_decode_attention_static": (I32, [CFG, CACHE, vp, I32, I32, ctypes.c_float,
                                                  P(I32), vp, vp]),
            "kvq_prefill_workspace_bytes": (SZ, [CFG, I32, I32]),
            "kvq_prefill_attention": (I32, [CFG, CACHE, vp, I32, I32, I32, ctypes.c_float,
                                            P(I32), vp, vp, SZ, vp]),
            "kvq_dequantize": (I32, [CFG, CACHE, I32, I32, I32, I32, P(I32), I32, vp, vp]),
            "kvq_status_str": (ctypes.c_char_p, [I32]),
            "kvq_profile_decode_events": (None, [vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


_ceiling = None


def ceiling_lib():
    """The read-bandwidth probe library (include/kvq_ceiling.h); measurement
    only, loaded by the benchmark."""
    global _ceiling
    if _ceiling is None:
        import torch  # noqa: F401  (same HIP runtime as torch, see lib())
        if not os.path.exists(CEILING_PATH):
            raise ImportError("libkvq_ceiling.so is not built (%s)" % CEILING_PATH)
        L = ctypes.CDLL(CEILING_PATH)
        P, I32, SZ, vp = ctypes.POINTER, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
        sig = {
            "kvq_ceiling_stream": (I32, [vp, SZ, I32, I32, I32, vp, vp]),
            "kvq_ceiling_tiles": (I32, [P(KvqCeilingTilesArgs), I32, I32, I32, vp, vp]),
            "kvq_ceiling_sink_words": (SZ, [I32, I32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _ceiling = L
    return _ceiling


def event_elapsed_ms(before, after):
    """Milliseconds between two hipEvent_t handles (ints) recorded by the
    library, read through the HIP runtime libkvq.so is bound to."""
    lib()
    hip = ctypes.CDLL("libamdhip64.so.7")
    ms = ctypes.c_float()
    err = hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(before), ctypes.c_void_p(after))
    if err != 0:
        raise RuntimeError("hipEventElapsedTime failed with HIP error %d" % err)
    return ms.value


def status_str(status):
    return lib().kvq_status_str(status).decode()


def check(status, what):
    if status != KVQ_OK:
        raise KvqError(status, what)
