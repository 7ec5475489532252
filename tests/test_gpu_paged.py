"""GPU parity of the paged cache layout (reading R24): the code and scale
planes are a pool of 64-position pages shared by all sequences, mapped by a
device page table.  Every kernel (bulk, small and one-token appends, decode,
prefill, read-back) must give the bytes and results of the contiguous
layout: planes gathered through the table are bit-exact with the oracle,
pages the table does not name stay untouched, and attention is within
relative L2 1e-3 of the float64 oracle on the device-produced cache."""

import numpy as np
import pytest

import workloads
from gpu_common import Pair, say, to_device, to_values, attention_errors, gpu_planes
from oracle import dequantize_reference, prefill_reference

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _table(B, max_ctx, lens_final, pool, seed):
    """A shuffled assignment of distinct pages to the tiles each sequence
    will hold; tiles past a sequence's final length get -1."""
    tiles = (max_ctx + 63) // 64
    need = [(n + 63) // 64 for n in lens_final]
    perm = np.random.default_rng(seed).permutation(pool)
    assert sum(need) <= pool
    table = np.full((B, tiles), -1, np.int32)
    k = 0
    for b in range(B):
        table[b, : need[b]] = perm[k: k + need[b]]
        k += need[b]
    return table


def _untouched(pair):
    """Pool pages no table entry names must still be zero."""
    used = set(int(x) for x in pair.table.reshape(-1) if x >= 0)
    free = [p for p in range(pair.cfg.page_pool) if p not in used]
    H = pair.cfg.n_kv_heads
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        pool = pair.cache[name].cpu().numpy().reshape(pair.cfg.page_pool, H, -1)
        assert not pool[free].any(), name


CASES = [
    # d, kb, vb, k_min, v_min, T, dtype, B, H, chunks (per sequence the same), pool slack
    (128, 8, 4, False, False, 16, "bf16", 2, 2, [150, 1, 1, 70, 1], 5),
    (128, 4, 4, False, False, 0, "f32", 3, 1, [64, 200, 1, 3], 0),
    (64, 5, 8, False, False, 8, "bf16", 2, 3, [33, 1, 90], 2),
    (256, 5, 4, False, False, 0, "bf16", 2, 2, [130, 1, 1], 4),
    (192, 6, 5, False, False, 4, "bf16", 1, 2, [100, 1, 29], 3),
    (128, 4, 5, True, True, 12, "bf16", 2, 2, [77, 1, 60], 1),
    (256, 5, 4, True, True, 0, "bf16", 1, 2, [70, 1, 30], 2),
    (192, 8, 5, False, True, 6, "f32", 2, 1, [65, 1, 40], 3),
]


def _cid(c):
    d, kb, vb, km, vm, T, dt, B, H, ch, sl = c
    return "d%d-k%d%s-v%d%s-T%d-%s-B%d-H%d" % (d, kb, "m" if km else "", vb, "m" if vm else "",
                                            T, dt, B, H)


def _paged_pair(case, lens_final, max_ctx):
    d, kb, vb, km, vm, T, dtype, B, H, chunks, slack = case
    tiles_used = sum((n + 63) // 64 for n in lens_final)
    pool = tiles_used + slack
    table = _table(B, max_ctx, lens_final, pool, seed=d + kb)
    return Pair(B, H, d, kb, vb, T, max_ctx, k_min=km, v_min=vm, page_pool=pool, table=table)


@pytest.mark.parametrize("case", CASES, ids=[_cid(c) for c in CASES])
def test_paged_append_and_dequantize_bit_exact(case):
    """Adversarial rows (zero, subnormal-scale, saturating and tied blocks)
    through bulk, small and one-token appends of a shuffled pool."""
    import torch
    import decode_attention_rotate_amd as kvq
    d, kb, vb, km, vm, T, dtype, B, H, chunks, slack = case
    n = sum(chunks)
    pair = _paged_pair(case, [n] * B, n + 70)
    gen = workloads.shifted_numpy if (km or vm) else workloads.adversarial_numpy
    for i, c in enumerate(chunks):
        pair.append(gen(i + 1, (B, c, H, d), dtype), gen(500 + i, (B, c, H, d), dtype), dtype)
    planes = pair.compare_planes()
    _untouched(pair)
    b = B - 1
    for which, bits, mf in ((0, kb, km), (1, vb, vm)):
        for space in (0, 1):
            say("paged dequantize", which, space)
            out = kvq.kvq_dequantize(pair.cfg, pair.cache, which, b, 0, n, pair.lens,
                                     space).cpu().numpy()
            torch.cuda.synchronize()
            want = dequantize_reference(planes, which, b, 0, n, n, H, d, bits, T, space,
                                        minf=mf)
            assert np.array_equal(out.view(np.uint32), want.view(np.uint32)), (which, space)


@pytest.mark.parametrize("case", CASES, ids=[_cid(c) for c in CASES])
def test_paged_decode_attention(case):
    """Workload-shaped inputs (normal values, outlier channels, channel
    offsets for scale-and-min blocks) appended in the same chunks; decode
    attention over the paged cache against the float64 oracle."""
    d, kb, vb, km, vm, T, dtype, B, H, chunks, slack = case
    n = sum(chunks)
    w = workloads.workload("small", B=B, Hkv=H, Hq=2 * H, d=d, k_bits=kb, v_bits=vb, tail=T,
                           dtype=dtype, bias=1.0 if (km or vm) else 0.0)
    pair = _paged_pair(case, [n] * B, n + 70)
    t0 = 0
    for c in chunks:
        pair.append(workloads.kv_numpy(w, 1, t0, t0 + c), workloads.kv_numpy(w, 2, t0, t0 + c),
                    dtype)
        t0 += c
    planes = pair.compare_planes()
    q = workloads.q_numpy(w)
    got = pair.decode(q, dtype)
    errs = attention_errors(got, planes, to_values(q, dtype), pair.lens, pair.cfg)
    worst = max(errs.values())
    say("paged decode worst rel L2 %.3e" % worst)
    assert worst <= TOL


@pytest.mark.parametrize("name,over", [("long", dict(Hq=10, tail=32)),
                                       ("huge", dict(Hq=8, tail=0))], ids=["d128-k8v4-T32", "d256-k5v4"])
def test_paged_ragged_lengths_share_a_pool(name, over):
    """Sequences of very different lengths in a pool smaller than the
    contiguous layout would need (the point of paging), each appended on its
    own through a one-sequence view; decode and prefill over the whole
    batch."""
    import torch
    import decode_attention_rotate_amd as kvq
    from oracle import OracleCache
    w = workloads.workload(name, B=3, Hkv=2, **over)
    B, H, d, T, kb, vb = 3, 2, w["d"], w["tail"], w["k_bits"], w["v_bits"]
    lens = [700, 64, 230]
    max_ctx = 1000
    need = sum((n + 63) // 64 for n in lens)
    pool = need + 2
    assert pool < B * ((max_ctx + 63) // 64)
    table = _table(B, max_ctx, lens, pool, seed=11)
    cfg = kvq.kvq_config(B, H, d, max_ctx, kb, vb, T, page_pool=pool)
    cache = kvq.KVCache(cfg, "cuda", page_table=torch.from_numpy(table).cuda())
    k = workloads.kv_numpy(w, 1, 0, max(lens))
    v = workloads.kv_numpy(w, 2, 0, max(lens))
    want = []
    for b in range(B):
        cfg1, view = cache.sequence(b)
        orc = OracleCache(1, H, d, kb, vb, T, max_ctx)
        n = lens[b]
        cuts = [0, n // 2, n - 3, n - 2, n - 1, n]     # a bulk, a small and one-token appends
        for t0, t1 in zip(cuts[:-1], cuts[1:]):
            if t1 <= t0:
                continue
            kk, vv = k[b:b + 1, t0:t1], v[b:b + 1, t0:t1]
            say("paged append, sequence", b, "positions", t0, t1)
            kvq.kvq_rotate_quantize_append(cfg1, view, to_device(kk, w["dtype"]),
                                           to_device(vv, w["dtype"]), [t0])
            orc.append(kk, vv, [t0], dtype=w["dtype"])
        want.append(orc.physical())
    torch.cuda.synchronize()
    planes = gpu_planes(cache, cfg, table)
    for key in planes:
        ref = np.concatenate([wb[key] for wb in want], axis=0)
        assert np.array_equal(planes[key], ref), key
    q = workloads.q_numpy(w)
    say("paged ragged decode lens=%s" % lens)
    got = kvq.kvq_decode_attention(cfg, cache, to_device(q, w["dtype"]), lens).cpu().numpy()
    errs = attention_errors(got.astype(np.float64), planes, to_values(q, w["dtype"]), lens, cfg)
    say("paged ragged decode worst rel L2 %.3e" % max(errs.values()))
    assert max(errs.values()) <= TOL
    n_q = 40
    qp = workloads.prefill_q_numpy(w, n_q)
    say("paged prefill n_q=%d lens=%s" % (n_q, lens))
    pre = kvq.kvq_prefill_attention(cfg, cache, to_device(qp, w["dtype"]), lens).cpu().numpy()
    ref = prefill_reference(planes, to_values(qp, w["dtype"]), lens, H, d, kb, vb, T)
    torch.cuda.synchronize()
    err = np.linalg.norm(pre - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    say("paged prefill worst rel L2 %.3e" % err.max())
    assert err.max() <= TOL


def test_paged_entries_outside_the_pool_are_not_followed():
    """A table entry outside [0, page_pool) is never dereferenced: the append
    writes nothing for its positions and the other pages keep their bytes."""
    import torch
    import decode_attention_rotate_amd as kvq
    B, H, d = 2, 2, 128
    max_ctx = 256
    pool = 6
    table = np.array([[0, 1, -1, -1], [2, 9, -1, -1]], np.int32)   # 9 >= pool
    pair = Pair(B, H, d, 8, 4, 0, max_ctx, page_pool=pool, table=table)
    k = workloads.adversarial_numpy(1, (B, 100, H, d))
    v = workloads.adversarial_numpy(2, (B, 100, H, d))
    say("paged append with an entry outside the pool")
    kvq.kvq_rotate_quantize_append(pair.cfg, pair.cache, to_device(k, "bf16"),
                                   to_device(v, "bf16"), [0, 0])
    torch.cuda.synchronize()
    pair.orc.append(k, v, [0, 0], dtype="bf16")
    want = pair.orc.physical()
    got = gpu_planes(pair.cache, pair.cfg, np.where(table < pool, table, -1))
    # tiles with valid pages match; pages 3..5 stay zero
    for key in ("k_codes", "v_codes", "k_scales", "v_scales"):
        g, wnt = got[key].reshape(B, H, 4, -1), want[key].reshape(B, H, 4, -1)
        assert np.array_equal(g[0, :, :2], wnt[0, :, :2]), key
        assert np.array_equal(g[1, :, :1], wnt[1, :, :1]), key
        poolv = pair.cache[key].cpu().numpy().reshape(pool, H, -1)
        assert not poolv[3:].any(), key
    # attention and read-back still run and stay finite
    q = workloads.adversarial_numpy(5, (B, 4, d))
    out = pair.decode(q, "bf16", lens=[100, 100])
    assert np.all(np.isfinite(out))
    x = kvq.kvq_dequantize(pair.cfg, pair.cache, 0, 1, 0, 100, [100, 100], 0).cpu().numpy()
    assert np.all(np.isfinite(x))
