"""GPU parity of the scale-and-min blocks q4_1 / q5_1 (x = u * s + m per
32-element block; sizes per the aiwitness.kr table's q5_1 rows), alone and
mixed with the absmax formats: planes and read-back bit-exact, decode and
prefill attention within relative L2 1e-3 of the float64 oracle on the
device-produced cache.  Inputs are shifted off zero so that blocks are
asymmetric (constant rows give zero-range blocks)."""

import numpy as np
import pytest

import workloads
from gpu_common import Pair, say, to_device, to_values, attention_errors, gpu_planes
from oracle import dequantize_reference, prefill_reference

pytestmark = pytest.mark.gpu

TOL = 1e-3

APPEND_CASES = [
    # d, kb, vb, k_min, v_min, T, dtype, B, H, chunks, rotate
    (64, 4, 4, True, True, 0, "f32", 1, 2, [256], False),
    (128, 5, 5, True, True, 0, "bf16", 2, 4, [130, 70], True),
    (128, 4, 5, False, True, 16, "bf16", 2, 4, [100, 1, 1, 40], True),
    (256, 5, 8, True, False, 8, "f32", 1, 2, [5, 90, 3], True),
    (256, 8, 4, False, True, 0, "bf16", 2, 2, [129, 63], False),
    (64, 6, 5, False, True, 4, "bf16", 2, 2, [3, 3, 70], True),
    (128, 4, 4, True, False, 64, "bf16", 1, 4, [10, 200, 1, 70], False),
]


def _case_id(c):
    d, kb, vb, km, vm, T, dt, B, H, ch, rot = c
    fk = "q%d_%d" % (kb, 1 if km else 0)
    fv = "q%d_%d" % (vb, 1 if vm else 0)
    return "d%d-%s-%s-T%d-%s-B%d-H%d-%s" % (d, fk, fv, T, dt, B, H, "rot" if rot else "norot")


@pytest.mark.parametrize("case", APPEND_CASES, ids=[_case_id(c) for c in APPEND_CASES])
def test_min_append_bit_exact(case):
    d, kb, vb, km, vm, T, dtype, B, H, chunks, rot = case
    pair = Pair(B, H, d, kb, vb, T, sum(chunks) + 7, rot, rot, k_min=km, v_min=vm)
    seed = 0
    for c in chunks:
        seed += 1
        pair.append(workloads.shifted_numpy(seed, (B, c, H, d), dtype),
                    workloads.shifted_numpy(1000 + seed, (B, c, H, d), dtype), dtype)
    pair.compare_planes()


@pytest.mark.parametrize("case", [(128, 5, 4, True, True, 8, "bf16", 2, 2, None, True),
                                  (64, 4, 5, True, True, 0, "f32", 2, 2, None, False),
                                  (256, 8, 5, False, True, 3, "bf16", 1, 2, None, True)],
                         ids=["d128-q5_1-q4_1-T8", "d64-q4_1-q5_1-T0", "d256-q8_0-q5_1-T3"])
def test_min_one_token_appends_bit_exact(case):
    # decode-step appends across V groups, a tile and every tail slot
    d, kb, vb, km, vm, T, dtype, B, H, _, rot = case
    pair = Pair(B, H, d, kb, vb, T, 120, rot, rot, k_min=km, v_min=vm)
    pair.append(workloads.shifted_numpy(1, (B, 13, H, d), dtype),
                workloads.shifted_numpy(2, (B, 13, H, d), dtype), dtype)
    for s in range(75):
        pair.append(workloads.shifted_numpy(100 + s, (B, 1, H, d), dtype),
                    workloads.shifted_numpy(300 + s, (B, 1, H, d), dtype), dtype)
    pair.compare_planes()


@pytest.mark.parametrize("case", APPEND_CASES[:5], ids=[_case_id(c) for c in APPEND_CASES[:5]])
def test_min_dequantize_bit_exact(case):
    import torch
    import decode_attention_rotate_amd as kvq
    d, kb, vb, km, vm, T, dtype, B, H, chunks, rot = case
    n = sum(chunks)
    pair = Pair(B, H, d, kb, vb, T, n, rot, rot, k_min=km, v_min=vm)
    pair.append(workloads.shifted_numpy(7, (B, n, H, d), dtype),
                workloads.shifted_numpy(8, (B, n, H, d), dtype), dtype)
    planes = gpu_planes(pair.cache, pair.cfg)
    for which, bits, mf in ((0, kb, km), (1, vb, vm)):
        for space in (0, 1):
            for b in range(B):
                t0, t1 = n // 3, n
                say("dequantize", which, b, t0, t1, space)
                got = kvq.kvq_dequantize(pair.cfg, pair.cache, which, b, t0, t1,
                                         pair.lens, space).cpu().numpy()
                torch.cuda.synchronize()
                want = dequantize_reference(planes, which, b, t0, t1, n, H, d, bits, T,
                                            space, rotate=rot, minf=mf)
                assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
                    (which, space, b)


def _fill(pair, w, lens, dtype):
    nmax = max(lens)
    k = workloads.kv_numpy(w, 1, 0, nmax)
    v = workloads.kv_numpy(w, 2, 0, nmax)
    if all(n == nmax for n in lens):
        pair.append(k, v, dtype)
        return
    m = min(lens)
    pair.append(k[:, : nmax - m], v[:, : nmax - m], dtype)
    pair.append(k[:, nmax - m:], v[:, nmax - m:], dtype,
                lens=[nmax - m if n == nmax else 0 for n in lens])


ATTN_CASES = [
    # name, workload overrides (K/V formats, bias), lengths
    ("small", dict(k_bits=4, v_bits=4, km=True, vm=True, bias=2.0), [1000]),
    ("mid", dict(B=2, k_bits=5, v_bits=5, km=True, vm=True, bias=1.0), [700, 129]),     # q5_1
    ("long", dict(B=2, k_bits=8, v_bits=5, vm=True, tail=64, bias=1.0), [900, 300]),   # q8_0-q5_1
    ("long", dict(B=1, k_bits=5, v_bits=4, vm=True, tail=16, bias=3.0), [500]),        # q5_0-q4_1
    ("huge", dict(B=1, Hq=8, k_bits=4, v_bits=5, km=True, vm=True, bias=1.0), [600]),  # d256
    ("huge", dict(B=2, k_bits=5, v_bits=8, km=True), [300, 64]),                       # no bias
    ("small", dict(Hq=24, k_bits=4, v_bits=4, km=True, vm=True, bias=2.0), [513]),     # G = 3
    ("tiny", dict(B=2, k_bits=4, v_bits=4, km=True, vm=True, bias=4.0), [64, 1]),
]


def _attn_pair(w, lens, rot=True):
    return Pair(len(lens), w["Hkv"], w["d"], w["k_bits"], w["v_bits"], w["tail"],
                max(lens) + 5, rot, rot, k_min=w.get("km", False), v_min=w.get("vm", False))


@pytest.mark.parametrize("name,over,lens", ATTN_CASES,
                         ids=["%s-%d" % (c[0], i) for i, c in enumerate(ATTN_CASES)])
def test_min_decode_attention(name, over, lens):
    w = workloads.workload(name, **over)
    w["B"] = len(lens)
    pair = _attn_pair(w, lens)
    _fill(pair, w, lens, w["dtype"])
    q = workloads.q_numpy(w)
    got = pair.decode(q, w["dtype"])
    planes = gpu_planes(pair.cache, pair.cfg)
    errs = attention_errors(got, planes, to_values(q, w["dtype"]), lens, pair.cfg)
    worst = max(errs.values())
    say("worst rel L2 %.3e" % worst)
    assert worst <= TOL, sorted(errs.items(), key=lambda kv: -kv[1])[:3]


def test_min_decode_rotation_off():
    # without the rotation the per-channel bias stays in its channels: the
    # blocks are far from symmetric
    w = workloads.workload("small", B=1, k_bits=4, v_bits=5, km=True, vm=True, bias=3.0)
    pair = _attn_pair(w, [777], rot=False)
    _fill(pair, w, [777], "bf16")
    q = workloads.q_numpy(w)
    got = pair.decode(q, "bf16")
    errs = attention_errors(got, gpu_planes(pair.cache, pair.cfg), to_values(q, "bf16"),
                            [777], pair.cfg)
    assert max(errs.values()) <= TOL, max(errs.values())


PREFILL_CASES = [
    ("small", dict(k_bits=4, v_bits=4, km=True, vm=True, bias=2.0), [200], 40),
    ("long", dict(B=2, k_bits=8, v_bits=5, vm=True, tail=16, bias=1.0), [300, 0], 37),
    ("huge", dict(B=1, Hq=8, k_bits=5, v_bits=4, km=True, vm=True, bias=1.0), [150], 20),
]


@pytest.mark.parametrize("name,over,before,n_q", PREFILL_CASES,
                         ids=["%s-%d" % (c[0], i) for i, c in enumerate(PREFILL_CASES)])
def test_min_prefill_attention(name, over, before, n_q):
    import decode_attention_rotate_amd as kvq
    w = workloads.workload(name, **over)
    w["B"] = len(before)
    pair = Pair(w["B"], w["Hkv"], w["d"], w["k_bits"], w["v_bits"], w["tail"],
                max(before) + n_q + 5, k_min=w.get("km", False), v_min=w.get("vm", False))
    if max(before) > 0:
        _fill(pair, w, before, w["dtype"])
    pair.append(workloads.kv_numpy(w, 1, 20000, 20000 + n_q),
                workloads.kv_numpy(w, 2, 20000, 20000 + n_q), w["dtype"])
    lens = list(pair.lens)
    q = workloads.prefill_q_numpy(w, n_q)
    say("prefill", name, "n_q=%d" % n_q, "lens=%s" % lens)
    got = kvq.kvq_prefill_attention(pair.cfg, pair.cache, to_device(q, w["dtype"]), lens)
    got = got.cpu().numpy().astype(np.float64)
    ref = prefill_reference(gpu_planes(pair.cache, pair.cfg), to_values(q, w["dtype"]), lens,
                            w["Hkv"], w["d"], w["k_bits"], w["v_bits"], w["tail"],
                            k_min=w.get("km", False), v_min=w.get("vm", False))
    err = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    say("prefill worst rel L2 %.3e" % err.max())
    assert err.max() <= TOL, np.unravel_index(np.argmax(err), err.shape)
