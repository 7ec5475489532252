"""Helpers for the GPU parity tests: run the HIP path and the CPU oracle on
the same seeded inputs and compare.  Imported by test_gpu_*.py only."""

import sys

import numpy as np
import torch

import decode_attention_rotate_amd as kvq
from oracle import OracleCache, decode_reference, pages_to_contiguous, padded_row_bytes
from oracle.blockquant import bf16_bits_to_f32, v_tile_bytes

DEV = "cuda"


def say(*msg):
    """Name the GPU step about to run, flushed, so a crash log shows it."""
    print("[gpu]", *msg, flush=True)
    sys.stdout.flush()


def to_device(x, dtype):
    """numpy inputs (bf16 bit patterns or float32) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def to_values(x, dtype):
    """numpy inputs -> float32 values (bf16 widened exactly)."""
    return bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, np.float32)


def gpu_planes(cache, cfg, table=None):
    """Device planes as numpy arrays shaped like OracleCache.physical(); a
    paged cache's pool is gathered into that layout through `table` (numpy
    [B][tiles], -1 for tiles that hold no positions)."""
    B, H, d, T = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.tail_len
    cap = (cfg.max_ctx + 63) // 64 * 64
    out = {}
    for p in ("k", "v"):
        bits = cfg.k_bits if p == "k" else cfg.v_bits
        minf = cfg.k_min if p == "k" else cfg.v_min
        codes = cache[p + "_codes"].cpu().numpy()
        scales = cache[p + "_scales"].cpu().numpy().view(np.uint16)
        if cfg.page_pool > 0:
            ct = 64 * padded_row_bytes(d, bits) if p == "k" else v_tile_bytes(d, bits)
            codes = pages_to_contiguous(codes, table, H, ct)
            scales = pages_to_contiguous(scales, table, H, 64 * (d // 32) * (2 if minf else 1))
        out[p + "_codes"] = codes.reshape(B, H, -1)
        # one fp16 per block, or an (s, m) pair for scale-and-min blocks
        out[p + "_scales"] = scales.reshape(B, H, cap, -1)
        if T > 0:
            out[p + "_tail"] = cache[p + "_tail"].cpu().numpy().view(np.uint16).reshape(B, H, T, d)
        else:
            out[p + "_tail"] = np.zeros((B, H, 0, d), np.uint16)
    return out


class Pair:
    """A device cache and the oracle cache fed the same appends."""

    def __init__(self, B, H, d, kb, vb, T, max_ctx, rotate_k=True, rotate_v=True, sign_seed=0,
                 k_min=False, v_min=False, page_pool=0, table=None):
        self.cfg = kvq.kvq_config(B, H, d, max_ctx, kb, vb, T, rotate_k, rotate_v, sign_seed,
                                  k_min, v_min, page_pool)
        self.table = None
        dev_table = None
        if page_pool > 0:
            self.table = np.asarray(table, dtype=np.int32)
            dev_table = torch.from_numpy(self.table).to(DEV)
        self.cache = kvq.KVCache(self.cfg, DEV, page_table=dev_table)
        self.orc = OracleCache(B, H, d, kb, vb, T, max_ctx, rotate_k, rotate_v, sign_seed,
                               k_min, v_min)
        self.lens = np.zeros(B, dtype=np.int64)

    def append(self, k, v, dtype, lens=None):
        lens = self.lens if lens is None else np.asarray(lens, dtype=np.int64)
        say("append", self.cfg, "n_new=%d" % k.shape[1], "lens=%s" % list(lens))
        kvq.kvq_rotate_quantize_append(self.cfg, self.cache, to_device(k, dtype),
                                       to_device(v, dtype), lens)
        torch.cuda.synchronize()
        self.orc.append(k, v, lens, dtype=dtype)
        self.lens = lens + k.shape[1]

    def compare_planes(self):
        got = gpu_planes(self.cache, self.cfg, self.table)
        want = self.orc.physical()
        for key in want:
            a, b = got[key], want[key]
            assert a.shape == b.shape, key
            if not np.array_equal(a, b):
                bad = np.argwhere(a != b)
                raise AssertionError("%s differs at %d places, first %s: gpu %s oracle %s"
                                     % (key, len(bad), bad[0], a[tuple(bad[0])], b[tuple(bad[0])]))
        return got

    def decode(self, q, dtype, lens=None, sm_scale=None):
        lens = self.lens if lens is None else lens
        say("decode", self.cfg, "Hq=%d" % q.shape[1], "lens=%s" % list(lens))
        out = kvq.kvq_decode_attention(self.cfg, self.cache, to_device(q, dtype), lens,
                                       sm_scale=sm_scale)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64)


def attention_errors(got, planes, qv, lens, cfg, sm_scale=None, heads=None):
    """Per-(b, h) relative L2 error of got against the float64 oracle
    evaluated on the given (device-produced) planes."""
    ref = decode_reference(planes, qv, lens, cfg.n_kv_heads, cfg.head_dim, cfg.k_bits,
                           cfg.v_bits, cfg.tail_len, sm_scale=sm_scale,
                           rotate_k=bool(cfg.rotate_k), rotate_v=bool(cfg.rotate_v),
                           heads=heads, sign_seed=cfg.sign_seed, k_min=bool(cfg.k_min),
                           v_min=bool(cfg.v_min))
    errs = {}
    B, Hq, _ = qv.shape
    for b in range(B):
        for h in range(Hq):
            if heads is not None and (b, h) not in set(heads):
                continue
            errs[(b, h)] = rel_l2(got[b, h], ref[b, h])
    return errs


def rel_l2(got, ref):
    """Relative L2 error of one output vector; infinite when the output is not
    finite, the absolute error when the exact output is the zero vector."""
    got = np.asarray(got, dtype=np.float64)
    if not np.all(np.isfinite(got)):
        return np.inf
    den = np.linalg.norm(ref)
    return np.linalg.norm(got - ref) / (den if den > 0 else 1.0)


def fill_lengths(pair, w, n_list, dtype):
    """Append workload tokens so sequence b ends with length n_list[b] (at
    most two distinct lengths): one append for everyone, then a second one
    that restarts the shorter sequences (a sequence given length 0 starts
    afresh)."""
    import workloads
    nmax = max(n_list)
    k = workloads.kv_numpy(w, 1, 0, nmax)
    v = workloads.kv_numpy(w, 2, 0, nmax)
    short = [n for n in n_list if n < nmax]
    if not short:
        pair.append(k, v, dtype)
        return
    m = min(short)
    assert all(x in (nmax, m) for x in n_list), "two distinct lengths supported"
    pair.append(k[:, : nmax - m], v[:, : nmax - m], dtype)
    lens = [nmax - m if n == nmax else 0 for n in n_list]
    pair.append(k[:, nmax - m:], v[:, nmax - m:], dtype, lens=lens)
