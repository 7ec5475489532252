"""GPU parity of the random-sign rotation R = H diag(s) (reading R21): the
appended codes, scales and tail rows bit-exact against the oracle, dequantized
values bit-exact in both spaces, and decode / prefill attention within 1e-3
relative L2 of the float64 oracle on the device cache."""

import numpy as np
import pytest

import workloads
from gpu_common import Pair, say, to_device, to_values, attention_errors, gpu_planes
from oracle import dequantize_reference, prefill_reference

pytestmark = pytest.mark.gpu

TOL = 1e-3

CASES = [
    # d, kb, vb, T, dtype, B, H, chunks, seed
    (64, 4, 4, 0, "f32", 1, 2, [100, 1, 1, 60], 1),
    (128, 8, 4, 16, "bf16", 2, 2, [70, 1, 1, 40], 0xDEADBEEF),
    (256, 5, 5, 8, "bf16", 1, 2, [65, 1, 9], 31337),
]


@pytest.mark.parametrize("case", CASES, ids=["d%d-k%d-v%d-T%d" % c[:4] for c in CASES])
def test_signed_append_dequantize_decode(case):
    import torch
    import decode_attention_rotate_amd as kvq
    d, kb, vb, T, dtype, B, H, chunks, seed = case
    n = sum(chunks)
    pair = Pair(B, H, d, kb, vb, T, n + 4, True, True, sign_seed=seed)
    for i, c in enumerate(chunks):
        pair.append(workloads.adversarial_numpy(10 + i, (B, c, H, d), dtype),
                    workloads.adversarial_numpy(50 + i, (B, c, H, d), dtype), dtype)
    planes = pair.compare_planes()
    for which, bits in ((0, kb), (1, vb)):
        for space in (0, 1):
            say("signed dequantize", which, space)
            got = kvq.kvq_dequantize(pair.cfg, pair.cache, which, 0, 0, n, pair.lens, space).cpu().numpy()
            torch.cuda.synchronize()
            want = dequantize_reference(planes, which, 0, 0, n, n, H, d, bits, T, space,
                                        sign_seed=seed)
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (which, space)
    # attention on workload-shaped data (adversarial rows include all-zero
    # blocks, whose exact attention output can be the zero vector)
    w = workloads.workload("small", B=B, Hkv=H, d=d, dtype=dtype)
    pair = Pair(B, H, d, kb, vb, T, n + 4, True, True, sign_seed=seed)
    pair.append(workloads.kv_numpy(w, 1, 0, n), workloads.kv_numpy(w, 2, 0, n), dtype)
    planes = pair.compare_planes()
    for hq in (H, 3 * H):
        w["Hq"] = hq
        q = workloads.q_numpy(w)
        got = pair.decode(q, dtype)
        errs = attention_errors(got, planes, to_values(q, dtype), list(pair.lens), pair.cfg)
        worst = max(errs.values())
        say("signed decode worst rel L2 %.3e" % worst)
        assert np.isfinite(worst) and worst <= TOL


def test_signed_rotation_flags_and_prefill():
    import decode_attention_rotate_amd as kvq
    w = workloads.workload("long", B=1, Hq=16, Hkv=4, tail=32)
    for rk, rv in ((True, False), (False, True)):
        pair = Pair(1, 4, 128, 8, 4, 32, 300, rk, rv, sign_seed=5)
        pair.append(workloads.kv_numpy(w, 1, 0, 250), workloads.kv_numpy(w, 2, 0, 250), "bf16")
        planes = pair.compare_planes()
        q = workloads.q_numpy(w)
        got = pair.decode(q, "bf16")
        errs = attention_errors(got, planes, to_values(q, "bf16"), list(pair.lens), pair.cfg)
        assert max(errs.values()) <= TOL, (rk, rv)
    pair = Pair(1, 4, 128, 8, 4, 32, 300, True, True, sign_seed=6)
    pair.append(workloads.kv_numpy(w, 1, 0, 250), workloads.kv_numpy(w, 2, 0, 250), "bf16")
    q = workloads.prefill_q_numpy(w, 40)
    got = kvq.kvq_prefill_attention(pair.cfg, pair.cache, to_device(q, "bf16"), list(pair.lens))
    ref = prefill_reference(gpu_planes(pair.cache, pair.cfg), to_values(q, "bf16"), list(pair.lens),
                            4, 128, 8, 4, 32, sign_seed=6)
    err = np.linalg.norm(got.cpu().numpy() - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    assert err.max() <= TOL, err.max()
