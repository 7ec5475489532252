"""GPU parity on caches of very small and very large magnitude.

Attention output is a weighted sum of V rows, so it scales with V; scores
scale with K (velog.io post "fix KV cache quantization outliers", section
"Hadamard rotation": the rotated scores and weighted sum are those of the
plain attention).  The HIP path keeps its fp16 P.V weights in fp16's normal
range whatever V's size, so its error against the float64 oracle must stay at
the same level when K and V are multiplied by 1e-2, 1e-3, 1e-4 (where plain
fp16 products p * scale_v would be subnormal), and when V alone is multiplied
by 1e3.  Two more cases sharpen the attention instead (K times 10: logits
with a spread of about 10, up to about 40): the query's 16-bit fixed point
perturbs it by about 2^-15 of its largest element, which moves the output
by about 1e-5 of the logits' spread.  Cases cover every V
width with absmax blocks, the scale-and-min blocks, a bf16 tail or none, the
one-wave head_dim 256 and 192 kernels, and chunked prefill."""

import numpy as np
import pytest

import workloads
from gpu_common import Pair, say, to_device, to_values, attention_errors, gpu_planes
from oracle import prefill_reference

pytestmark = pytest.mark.gpu

TOL = 1e-3

AMPS = (1e-2, 1e-3, 1e-4)
FORMATS = [
    # k_bits, v_bits, k_min, v_min
    (8, 4, False, False),
    (8, 5, False, False),
    (8, 6, False, False),
    (8, 8, False, False),
    (4, 4, True, True),     # q4_1
    (5, 5, True, True),     # q5_1
]

# amp_k, amp_v, format, tail
DECODE_CASES = [(amp, amp, f, T) for amp in AMPS for f in FORMATS for T in (0, 64)]
DECODE_CASES += [(1.0, 1e3, (8, 4, False, False), 64), (1.0, 1e3, (4, 4, True, True), 0),
                 (10.0, 1e-3, (8, 4, False, False), 64), (10.0, 1.0, (5, 5, True, True), 0)]


def _run_decode(w, lens, kb, vb, km, vm, T):
    w["B"] = len(lens)
    pair = Pair(w["B"], w["Hkv"], w["d"], kb, vb, T, max(lens) + 5, k_min=km, v_min=vm)
    k = workloads.kv_numpy(w, 1, 0, max(lens))
    v = workloads.kv_numpy(w, 2, 0, max(lens))
    pair.append(k, v, w["dtype"])
    q = workloads.q_numpy(w)
    got = pair.decode(q, w["dtype"], lens=lens)
    planes = gpu_planes(pair.cache, pair.cfg)
    errs = attention_errors(got, planes, to_values(q, w["dtype"]), lens, pair.cfg)
    return max(errs.values())


@pytest.mark.parametrize("amp_k,amp_v,fmt,T", DECODE_CASES,
                         ids=["k%g-v%g-k%dv%d%s-T%d" % (ak, av, f[0], f[1], "m" if f[2] else "", T)
                              for ak, av, f, T in DECODE_CASES])
def test_decode_scaled_cache(amp_k, amp_v, fmt, T):
    kb, vb, km, vm = fmt
    w = workloads.workload("long", amp_k=amp_k, amp_v=amp_v)
    say("decode amp K %g V %g" % (amp_k, amp_v), fmt, "T=%d" % T)
    worst = _run_decode(w, [900, 900], kb, vb, km, vm, T)
    say("worst rel L2 %.3e" % worst)
    assert worst <= TOL, worst


@pytest.mark.parametrize("name,over,fmt", [
    ("huge", dict(Hq=16, Hkv=4), (5, 4, False, False)),
    ("huge", dict(Hq=8, Hkv=2), (5, 5, True, True)),
    ("long", dict(d=192, Hq=10, Hkv=2), (8, 4, False, False)),
    ("long", dict(d=192, Hq=10, Hkv=2), (4, 4, True, True)),
])
def test_decode_scaled_cache_wide_heads(name, over, fmt):
    kb, vb, km, vm = fmt
    w = workloads.workload(name, amp_k=1e-3, amp_v=1e-4, **over)
    say("decode wide heads", name, over, fmt)
    worst = _run_decode(w, [700, 300], kb, vb, km, vm, 0)
    say("worst rel L2 %.3e" % worst)
    assert worst <= TOL, worst


@pytest.mark.parametrize("amp,fmt,T", [
    (1e-3, (8, 4, False, False), 64),
    (1e-4, (8, 8, False, False), 0),
    (1e-4, (4, 4, True, True), 16),
    (1e-2, (8, 6, False, False), 0),
])
def test_prefill_scaled_cache(amp, fmt, T):
    import decode_attention_rotate_amd as kvq
    kb, vb, km, vm = fmt
    w = workloads.workload("long", B=1, amp_k=amp, amp_v=amp)
    n_before, n_q = 400, 48
    pair = Pair(1, w["Hkv"], w["d"], kb, vb, T, n_before + n_q + 5, k_min=km, v_min=vm)
    pair.append(workloads.kv_numpy(w, 1, 0, n_before), workloads.kv_numpy(w, 2, 0, n_before), "bf16")
    pair.append(workloads.kv_numpy(w, 1, 20000, 20000 + n_q),
                workloads.kv_numpy(w, 2, 20000, 20000 + n_q), "bf16")
    lens = list(pair.lens)
    q = workloads.prefill_q_numpy(w, n_q)
    say("prefill amp %g" % amp, fmt, "T=%d" % T)
    got = kvq.kvq_prefill_attention(pair.cfg, pair.cache, to_device(q, "bf16"), lens)
    got = got.cpu().numpy().astype(np.float64)
    planes = gpu_planes(pair.cache, pair.cfg)
    ref = prefill_reference(planes, to_values(q, "bf16"), lens, w["Hkv"], w["d"], kb, vb, T,
                            k_min=km, v_min=vm)
    err = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    say("prefill worst rel L2 %.3e" % err.max())
    assert err.max() <= TOL, err.max()
