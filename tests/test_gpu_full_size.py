"""GPU parity at the full benchmark sizes, in the launch configuration that
bench.py times: the cache is filled with 8192-token appends, then decode steps
append one token and attend.  The oracle checks sampled outputs one by one:

* codes and fp16 scales of sampled 64-token windows of sampled (sequence, KV
  head) units, bit-exact against the oracle quantizer applied to the same
  input values (rotation, bf16 rounding when there is a tail, absmax blocks);
* the bf16 tail rows of those units, bit-exact;
* the attention outputs of those units' query heads, relative L2 <= 1e-3
  against the float64 oracle evaluated on the device cache of the unit, after
  the fill and after a decode step;
* the bulk append as the benchmark times it (32768 tokens per sequence in one
  call): every code and scale of sampled units, bit-exact.

Inputs come from the device generators of workloads.py; the windows the oracle
needs are regenerated and copied to the host."""

import numpy as np
import pytest
import torch

import workloads
import decode_attention_rotate_amd as kvq
from gpu_common import say
from oracle import rotate_f32, quantize_blocks, decode_reference, prefill_reference
from oracle.blockquant import (bf16_round, bf16_bits_to_f32, f32_to_bf16_bits, padded_row_bytes,
                               v_tile_bytes)
from oracle.kvcache import plane_codes

pytestmark = pytest.mark.gpu

FILL = 8192
TOL = 1e-3
DEV = "cuda"

# workload, sampled (sequence, KV head) units
CASES = [
    ("mid", [(3, 5), (15, 0)]),
    ("long", [(2, 7), (7, 1)]),
    ("huge", [(0, 3), (31, 1)]),
]


def host_values(t):
    """Device bf16/fp32 tensor -> float32 numpy values."""
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.float().cpu().numpy()


def unit_planes(cache, cfg, b, g):
    """Device planes of unit (b, g) shaped as a one-sequence, one-head cache."""
    B, H, d, T = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.tail_len
    cap = (cfg.max_ctx + 63) // 64 * 64
    out = {}
    for p in ("k", "v"):
        out[p + "_codes"] = cache[p + "_codes"].view(B, H, -1)[b, g].cpu().numpy()[None, None]
        sc = cache[p + "_scales"].view(B, H, -1)[b, g].cpu().numpy().view(np.uint16)
        out[p + "_scales"] = sc.reshape(1, 1, cap, d // 32)
        if T > 0:
            tl = cache[p + "_tail"].view(B, H, -1)[b, g].cpu().numpy().view(np.uint16)
            out[p + "_tail"] = tl.reshape(1, 1, T, d)
        else:
            out[p + "_tail"] = np.zeros((1, 1, 0, d), np.uint16)
    return out


def window_codes(planes, p, d, bits, t0, t1):
    """Codes of tokens [t0, t1) (t0 a multiple of 64) of a unit plane."""
    tile = 64 * padded_row_bytes(d, bits) if p == "k" else v_tile_bytes(d, bits)
    plane = planes[p + "_codes"][0, 0]
    sub = plane[(t0 // 64) * tile: ((t1 + 63) // 64) * tile]
    return plane_codes(sub, d, bits, t1 - t0, p)


def check_unit_bytes(w, planes, b, g, n):
    """Bit-exact codes, scales and tail rows of unit (b, g) on sampled windows."""
    d, T = w["d"], w["tail"]
    nt = min(n, T) if T > 0 else 0
    nq = n - nt
    starts = sorted({0, (nq // 2) // 64 * 64, max(0, (nq - 64) // 64 * 64)})
    for role, p, bits in ((1, "k", w["k_bits"]), (2, "v", w["v_bits"])):
        for t0 in starts:
            t1 = min(nq, t0 + 64)
            if t1 <= t0:
                continue
            x = host_values(workloads.kv_torch(w, role, t0, t1, DEV, torch)[b, :, g])
            y = rotate_f32(x)
            if T > 0:
                y = bf16_round(y)
            codes, scales = quantize_blocks(y, bits)
            got = window_codes(planes, p, d, bits, t0, t1)
            assert np.array_equal(got, codes), (p, b, g, t0, t1)
            assert np.array_equal(planes[p + "_scales"][0, 0, t0:t1], scales), (p, b, g, t0)
        if nt:
            x = host_values(workloads.kv_torch(w, role, nq, n, DEV, torch)[b, :, g])
            want = f32_to_bf16_bits(rotate_f32(x))
            slots = np.arange(nq, n) % T
            assert np.array_equal(planes[p + "_tail"][0, 0, slots], want), (p, b, g, "tail")


def check_unit_attention(w, cache, cfg, out, q, b, g, n):
    G = w["Hq"] // w["Hkv"]
    planes = unit_planes(cache, cfg, b, g)
    qv = host_values(q[b, g * G:(g + 1) * G])[None]
    ref = decode_reference(planes, qv, [n], 1, w["d"], w["k_bits"], w["v_bits"], w["tail"])
    got = out[b, g * G:(g + 1) * G].cpu().numpy()
    err = np.linalg.norm(got - ref[0], axis=-1) / np.linalg.norm(ref[0], axis=-1)
    say("unit", (b, g), "worst rel L2 %.3e" % err.max())
    assert err.max() <= TOL, (b, g, err)
    return planes


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,units", CASES, ids=[c[0] for c in CASES])
def test_full_size_sampled(name, units):
    w = workloads.workload(name)
    B, Hkv, Hq, d, n = w["B"], w["Hkv"], w["Hq"], w["d"], w["n"]
    steps = 2
    cfg = kvq.kvq_config(B, Hkv, d, n + steps + 64, w["k_bits"], w["v_bits"], w["tail"])
    cache = kvq.KVCache(cfg, DEV)
    lens = [0] * B
    for t0 in range(0, n, FILL):
        t1 = min(n, t0 + FILL)
        say(name, "fill", t0, t1)
        k = workloads.kv_torch(w, 1, t0, t1, DEV, torch)
        v = workloads.kv_torch(w, 2, t0, t1, DEV, torch)
        kvq.kvq_rotate_quantize_append(cfg, cache, k, v, lens)
        lens = [x + (t1 - t0) for x in lens]
        del k, v
    torch.cuda.synchronize()
    ws = torch.zeros(kvq.kvq_decode_workspace_bytes(cfg, Hq), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)

    say(name, "decode after fill")
    q = workloads.q_torch(w, 0, DEV, torch)
    kvq.kvq_decode_attention(cfg, cache, q, lens, out=out, workspace=ws)
    torch.cuda.synchronize()
    for b, g in units:
        planes = check_unit_attention(w, cache, cfg, out, q, b, g, n)
        check_unit_bytes(w, planes, b, g, n)

    # decode steps as the benchmark runs them: one kvq_decode_step call
    # appends the token and attends over the cache that holds it
    for s in range(1, steps + 1):
        say(name, "decode step", s)
        q = workloads.q_torch(w, s, DEV, torch)
        kvq.kvq_decode_step(cfg, cache, workloads.new_tokens_torch(w, 1, s, DEV, torch),
                            workloads.new_tokens_torch(w, 2, s, DEV, torch), q, lens, out=out,
                            workspace=ws)
        lens = [x + 1 for x in lens]
        torch.cuda.synchronize()
    for b, g in units:
        check_unit_attention(w, cache, cfg, out, q, b, g, n + steps)


@pytest.mark.timeout(600)
def test_outliers_full_size_sampled():
    """The long workload without a tail and with 32 outlier channels per
    plane and KV head, at full size: sampled windows of the rest's and the
    outliers' codes and scales bit-exact against the oracle's split
    quantizer, and the attention of sampled units within 1e-3 of the
    float64 split-form reference on the device planes."""
    from oracle.outliers import quantize_rows_outliers, decode_reference_outliers
    w = workloads.workload("long", tail=0)
    B, Hkv, Hq, d, n = w["B"], w["Hkv"], w["Hq"], w["d"], w["n"]
    kb, vb = w["k_bits"], w["v_bits"]
    lists = workloads.outlier_lists(w)
    units = [(2, 7), (7, 1)]
    steps = 2
    cfg = kvq.kvq_config(B, Hkv, d, n + steps + 64, kb, vb, 0, outliers=32)
    cache = kvq.KVCache(cfg, DEV, outlier_idx=torch.from_numpy(lists).to(DEV))
    lens = [0] * B
    for t0 in range(0, n, FILL):
        t1 = min(n, t0 + FILL)
        say("outliers fill", t0, t1)
        kvq.kvq_rotate_quantize_append(cfg, cache, workloads.kv_torch(w, 1, t0, t1, DEV, torch),
                                       workloads.kv_torch(w, 2, t0, t1, DEV, torch), lens)
        lens = [x + (t1 - t0) for x in lens]
    ws = torch.zeros(kvq.kvq_decode_workspace_bytes(cfg, Hq), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)
    for s in range(1, steps + 1):
        say("outliers decode step", s)
        q = workloads.q_torch(w, s, DEV, torch)
        kvq.kvq_decode_step(cfg, cache, workloads.new_tokens_torch(w, 1, s, DEV, torch),
                            workloads.new_tokens_torch(w, 2, s, DEV, torch), q, lens, out=out,
                            workspace=ws)
        lens = [x + 1 for x in lens]
        torch.cuda.synchronize()
    cap = (cfg.max_ctx + 63) // 64 * 64
    G = Hq // Hkv
    for b, g in units:
        planes = unit_planes(cache, cfg, b, g)
        for p in ("k", "v"):
            planes[p + "_out_codes"] = cache[p + "_out_codes"].view(B, Hkv, -1)[b, g].cpu().numpy()[None, None]
            planes[p + "_out_scales"] = (cache[p + "_out_scales"].view(B, Hkv, -1)[b, g].cpu().numpy()
                                         .view(np.uint16).reshape(1, 1, cap))
        # bytes of sampled windows of the fill
        for role, p, bits, pl in ((1, "k", kb, 0), (2, "v", vb, 1)):
            for t0 in (0, (n // 2) // 64 * 64, n - 64):
                x = host_values(workloads.kv_torch(w, role, t0, t0 + 64, DEV, torch)[b, :, g])
                parts = quantize_rows_outliers(x, lists[pl, g], bits)
                got = window_codes(planes, p, d, bits, t0, t0 + 64)
                assert np.array_equal(got, parts["rest_codes"]), (p, b, g, t0)
                assert np.array_equal(planes[p + "_scales"][0, 0, t0:t0 + 64], parts["rest_scales"]), (p, b, g, t0)
                assert np.array_equal(planes[p + "_out_scales"][0, 0, t0:t0 + 64], parts["out_scales"][:, 0]), \
                    (p, b, g, t0, "outlier scales")
                if p == "k":
                    oc = planes["k_out_codes"][0, 0].view(np.int8).reshape(-1, 32)[t0:t0 + 64]
                else:
                    from oracle.blockquant import vtiles_to_codes
                    oc = vtiles_to_codes(planes["v_out_codes"][0, 0], t0 + 64, 32, 8)[t0:t0 + 64]
                assert np.array_equal(oc, parts["out_codes"]), (p, b, g, t0, "outlier codes")
        qv = host_values(q[b, g * G:(g + 1) * G])[None]
        ref = decode_reference_outliers(planes, qv, [n + steps], 1, d, kb, vb, lists[0, g:g + 1],
                                        lists[1, g:g + 1])
        got = out[b, g * G:(g + 1) * G].cpu().numpy()
        err = np.linalg.norm(got - ref[0], axis=-1) / np.linalg.norm(ref[0], axis=-1)
        say("outliers unit", (b, g), "worst rel L2 %.3e" % err.max())
        assert err.max() <= TOL, (b, g, err)


@pytest.mark.timeout(600)
def test_prefill_full_size_sampled():
    # the prefill measurement's shape: batch 1, 40 query / 8 KV heads, K8 V4,
    # tail 1024, a 512-token chunk appended after 65024 cached tokens; sampled
    # rows (first, middle, last query of the chunk; two heads each of two KV
    # heads) against the oracle on the device cache
    w = workloads.workload("long", B=1)
    Hkv, Hq, d, n, n_q = w["Hkv"], w["Hq"], w["d"], w["n"], 512
    n0 = n - n_q
    cfg = kvq.kvq_config(1, Hkv, d, n, w["k_bits"], w["v_bits"], w["tail"])
    cache = kvq.KVCache(cfg, DEV)
    for t0 in range(0, n0, FILL):
        t1 = min(n0, t0 + FILL)
        say("prefill full size fill", t0, t1)
        kvq.kvq_rotate_quantize_append(cfg, cache, workloads.kv_torch(w, 1, t0, t1, DEV, torch),
                                       workloads.kv_torch(w, 2, t0, t1, DEV, torch), [t0])
    kvq.kvq_rotate_quantize_append(cfg, cache, workloads.kv_torch(w, 1, n0, n, DEV, torch),
                                   workloads.kv_torch(w, 2, n0, n, DEV, torch), [n0])
    q = workloads.prefill_q_torch(w, n_q, 0, DEV, torch)
    say("prefill full size attention")
    out = kvq.kvq_prefill_attention(cfg, cache, q, [n])
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.all(np.isfinite(out))
    qv = host_values(q)
    G = Hq // Hkv
    for g in (2, 7):
        planes = unit_planes(cache, cfg, 0, g)
        heads = (g * G, g * G + G - 1)
        rows = [(0, i, h - g * G) for i in (0, 255, 511) for h in heads]
        ref = prefill_reference(planes, qv[:, :, g * G:(g + 1) * G], [n], 1, d, w["k_bits"],
                                w["v_bits"], w["tail"], rows=rows)
        for b, i, hl in rows:
            got = out[0, i, g * G + hl]
            err = np.linalg.norm(got - ref[0, i, hl]) / np.linalg.norm(ref[0, i, hl])
            say("prefill full size row", (i, g * G + hl), "rel L2 %.3e" % err)
            assert err <= TOL, (i, g, hl, err)


@pytest.mark.timeout(600)
def test_bulk_append_full_size_sampled():
    """The bulk append the benchmark times: batch 16, 8 KV heads, head_dim
    128, K4 V4, no tail, 32768 new tokens per sequence in one call.  Every
    code and scale of sampled (sequence, KV head) units, bit-exact against
    the oracle quantizer on the same input values; a second call at the same
    positions rewrites the same bytes."""
    w = workloads.workload("mid")
    B, Hkv, d, n = w["B"], w["Hkv"], w["d"], w["n"]
    kb, vb = w["k_bits"], w["v_bits"]
    cfg = kvq.kvq_config(B, Hkv, d, n, kb, vb, 0)
    cache = kvq.KVCache(cfg, DEV)
    k = workloads.kv_torch(w, 1, 0, n, DEV, torch)
    v = workloads.kv_torch(w, 2, 0, n, DEV, torch)
    say("bulk append", B, n)
    kvq.kvq_rotate_quantize_append(cfg, cache, k, v, [0] * B)
    torch.cuda.synchronize()
    first = {p: cache[p].clone() for p in ("k_codes", "k_scales", "v_codes", "v_scales")}
    say("bulk append again at the same positions")
    kvq.kvq_rotate_quantize_append(cfg, cache, k, v, [0] * B)
    torch.cuda.synchronize()
    for p, t in first.items():
        assert torch.equal(cache[p], t), p
    for b, g in ((0, 0), (9, 5), (15, 7)):
        planes = unit_planes(cache, cfg, b, g)
        for src, p, bits in ((k, "k", kb), (v, "v", vb)):
            say("unit", (b, g), p)
            x = host_values(src[b, :, g])
            codes, scales = quantize_blocks(rotate_f32(x), bits)
            got = window_codes(planes, p, d, bits, 0, n)
            assert np.array_equal(got, codes), (p, b, g)
            assert np.array_equal(planes[p + "_scales"][0, 0, :n], scales), (p, b, g)
