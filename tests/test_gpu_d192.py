"""GPU parity at head_dim 192, a multiple of 64 that is not a power of two,
rotated block-diagonally by H_64 (velog.io post, section "application and
background": the rotation is on for every multiple of 64 from 64 up).
Planes and read-back bit-exact; decode and prefill attention within relative
L2 1e-3 of the float64 oracle on the device-produced cache."""

import numpy as np
import pytest

import workloads
from gpu_common import Pair, say, to_device, to_values, attention_errors, gpu_planes
from oracle import dequantize_reference, prefill_reference

pytestmark = pytest.mark.gpu

TOL = 1e-3
D = 192

APPEND_CASES = [
    # kb, vb, k_min, v_min, T, dtype, B, H, chunks, rotate, sign_seed
    (4, 4, False, False, 0, "bf16", 2, 2, [100, 1, 37], True, 0),
    (8, 5, False, False, 16, "f32", 1, 3, [90, 1, 1, 50], True, 0),
    (5, 6, False, False, 8, "bf16", 2, 2, [41, 3, 70], True, 7),
    (6, 8, False, False, 0, "bf16", 1, 2, [129], False, 0),
    (4, 5, True, True, 4, "bf16", 2, 2, [60, 1, 20], True, 0),
]


def _cid(c):
    kb, vb, km, vm, T, dt, B, H, ch, rot, seed = c
    return "k%d%s-v%d%s-T%d-%s-B%d-%s-s%d" % (kb, "m" if km else "", vb, "m" if vm else "", T, dt,
                                            B, "rot" if rot else "norot", seed)


@pytest.mark.parametrize("case", APPEND_CASES, ids=[_cid(c) for c in APPEND_CASES])
def test_d192_append_and_dequantize_bit_exact(case):
    import torch
    import decode_attention_rotate_amd as kvq
    kb, vb, km, vm, T, dtype, B, H, chunks, rot, seed = case
    n = sum(chunks)
    pair = Pair(B, H, D, kb, vb, T, n + 7, rot, rot, seed, k_min=km, v_min=vm)
    gen = workloads.shifted_numpy if (km or vm) else workloads.adversarial_numpy
    for i, c in enumerate(chunks):
        pair.append(gen(i + 1, (B, c, H, D), dtype), gen(1000 + i, (B, c, H, D), dtype), dtype)
    planes = pair.compare_planes()
    for which, bits, mf in ((0, kb, km), (1, vb, vm)):
        for space in (0, 1):
            b = B - 1
            say("dequantize d192", which, space)
            got = kvq.kvq_dequantize(pair.cfg, pair.cache, which, b, 0, n, pair.lens,
                                     space).cpu().numpy()
            torch.cuda.synchronize()
            want = dequantize_reference(planes, which, b, 0, n, n, H, D, bits, T, space,
                                        rotate=rot, sign_seed=seed, minf=mf)
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (which, space)


def test_d192_one_token_appends_bit_exact():
    pair = Pair(2, 2, D, 5, 4, 5, 100)
    pair.append(workloads.adversarial_numpy(1, (2, 9, 2, D)),
                workloads.adversarial_numpy(2, (2, 9, 2, D)), "bf16")
    for s in range(70):
        pair.append(workloads.adversarial_numpy(100 + s, (2, 1, 2, D)),
                    workloads.adversarial_numpy(300 + s, (2, 1, 2, D)), "bf16")
    pair.compare_planes()


def _fill(pair, w, lens):
    nmax = max(lens)
    k = workloads.kv_numpy(w, 1, 0, nmax)
    v = workloads.kv_numpy(w, 2, 0, nmax)
    if all(n == nmax for n in lens):
        pair.append(k, v, w["dtype"])
        return
    m = min(lens)
    pair.append(k[:, : nmax - m], v[:, : nmax - m], w["dtype"])
    pair.append(k[:, nmax - m:], v[:, nmax - m:], w["dtype"],
                lens=[nmax - m if n == nmax else 0 for n in lens])


ATTN_CASES = [
    # workload overrides, lengths, sign_seed
    (dict(k_bits=4, v_bits=4), [1000], 0),
    (dict(B=2, k_bits=8, v_bits=4, tail=64), [700, 130], 0),
    (dict(B=2, Hq=40, k_bits=5, v_bits=6, tail=16), [500, 500], 3),     # G = 5
    (dict(Hq=24, k_bits=6, v_bits=8), [300], 0),                          # G = 3
    (dict(k_bits=4, v_bits=5, km=True, vm=True, bias=2.0), [600], 0),     # q4_1 / q5_1
    (dict(B=2, Hq=64, k_bits=8, v_bits=5, vm=True, bias=1.0), [200, 65], 0),   # G = 8
]


@pytest.mark.parametrize("over,lens,seed", ATTN_CASES, ids=["case%d" % i for i in range(len(ATTN_CASES))])
def test_d192_decode_attention(over, lens, seed):
    w = workloads.workload("small", d=D, **over)
    w["B"] = len(lens)
    pair = Pair(w["B"], w["Hkv"], D, w["k_bits"], w["v_bits"], w["tail"], max(lens) + 5,
                sign_seed=seed, k_min=w.get("km", False), v_min=w.get("vm", False))
    _fill(pair, w, lens)
    q = workloads.q_numpy(w)
    got = pair.decode(q, w["dtype"])
    errs = attention_errors(got, gpu_planes(pair.cache, pair.cfg), to_values(q, w["dtype"]),
                            lens, pair.cfg)
    worst = max(errs.values())
    say("d192 worst rel L2 %.3e" % worst)
    assert worst <= TOL, sorted(errs.items(), key=lambda kv: -kv[1])[:3]


@pytest.mark.parametrize("over,before,n_q", [(dict(k_bits=8, v_bits=4, tail=16), [300], 40),
                                             (dict(B=2, k_bits=4, v_bits=5, km=True, vm=True,
                                                   bias=1.0), [100, 0], 21)],
                         ids=["k8v4-T16", "q4_1-q5_1"])
def test_d192_prefill_attention(over, before, n_q):
    import decode_attention_rotate_amd as kvq
    w = workloads.workload("small", d=D, **over)
    w["B"] = len(before)
    km, vm = w.get("km", False), w.get("vm", False)
    pair = Pair(w["B"], w["Hkv"], D, w["k_bits"], w["v_bits"], w["tail"], max(before) + n_q + 5,
                k_min=km, v_min=vm)
    if max(before) > 0:
        _fill(pair, w, before)
    pair.append(workloads.kv_numpy(w, 1, 20000, 20000 + n_q),
                workloads.kv_numpy(w, 2, 20000, 20000 + n_q), w["dtype"])
    lens = list(pair.lens)
    q = workloads.prefill_q_numpy(w, n_q)
    say("prefill d192", "n_q=%d" % n_q, "lens=%s" % lens)
    got = kvq.kvq_prefill_attention(pair.cfg, pair.cache, to_device(q, w["dtype"]), lens)
    got = got.cpu().numpy().astype(np.float64)
    ref = prefill_reference(gpu_planes(pair.cache, pair.cfg), to_values(q, w["dtype"]), lens,
                            w["Hkv"], D, w["k_bits"], w["v_bits"], w["tail"], k_min=km, v_min=vm)
    err = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    say("prefill d192 worst rel L2 %.3e" % err.max())
    assert err.max() <= TOL, np.unravel_index(np.argmax(err), err.shape)
