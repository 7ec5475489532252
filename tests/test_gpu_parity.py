"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

* Append: code, scale and tail planes byte-identical to the oracle's (the
  quantizer is an encoding, so bit-exactness is the bar).
* Dequantize: float32 output bit-identical to the oracle's on the device
  cache (rotated and original space).
* Decode attention: relative L2 error <= 1e-3 per (sequence, query head)
  against the float64 oracle evaluated on the device-produced cache.

Sizes span several 64-token tiles, several splits and ragged tails; the
workload shapes (head_dim, GQA ratio, bit widths, tail) follow workloads.py
with shorter contexts so the oracle finishes in seconds."""

import numpy as np
import pytest

import workloads
from gpu_common import Pair, say, to_device, to_values, attention_errors, gpu_planes
from oracle import dequantize_reference, prefill_reference

pytestmark = pytest.mark.gpu

TOL = 1e-3

APPEND_CASES = [
    # d, kb, vb, T, dtype, B, H, chunks, rotate
    (64, 4, 4, 0, "f32", 1, 1, [256], True),
    (128, 8, 8, 0, "bf16", 1, 8, [300, 1, 1, 211], True),
    (128, 4, 4, 0, "bf16", 2, 8, [130, 70], True),
    (128, 8, 4, 16, "bf16", 2, 8, [100, 1, 1, 40], True),
    (128, 8, 4, 64, "bf16", 1, 4, [10, 200, 1, 70], True),
    (256, 5, 4, 0, "bf16", 2, 4, [129, 63], True),
    (256, 8, 5, 8, "f32", 1, 2, [5, 90, 3], True),
    (64, 5, 8, 4, "bf16", 2, 2, [3, 3, 70], True),
    (128, 5, 5, 0, "f32", 1, 2, [65], True),
    (128, 4, 8, 0, "bf16", 1, 2, [80], False),
    (256, 4, 4, 32, "bf16", 1, 2, [40, 40], False),
    # q6_0
    (128, 6, 6, 0, "bf16", 2, 4, [130, 1, 61], True),
    (64, 6, 4, 8, "f32", 1, 2, [70, 1, 1], True),
    (256, 8, 6, 16, "bf16", 1, 2, [40, 1, 30], True),
]


def _case_id(c):
    d, kb, vb, T, dt, B, H, ch, rot = c
    return "d%d-k%d-v%d-T%d-%s-B%d-H%d-%s" % (d, kb, vb, T, dt, B, H, "rot" if rot else "norot")


@pytest.mark.parametrize("case", APPEND_CASES, ids=[_case_id(c) for c in APPEND_CASES])
def test_append_bit_exact(case):
    d, kb, vb, T, dtype, B, H, chunks, rot = case
    n = sum(chunks)
    pair = Pair(B, H, d, kb, vb, T, n + 7, rot, rot)
    seed = 0
    for c in chunks:
        seed += 1
        k = workloads.adversarial_numpy(seed, (B, c, H, d), dtype)
        v = workloads.adversarial_numpy(1000 + seed, (B, c, H, d), dtype)
        pair.append(k, v, dtype)
    pair.compare_planes()


ONE_TOKEN_CASES = [
    # d, kb, vb, T, dtype, B, H, rotate
    (64, 4, 8, 0, "f32", 2, 2, True),
    (128, 5, 4, 8, "bf16", 2, 2, True),
    (256, 8, 5, 3, "f32", 1, 2, True),
    (128, 4, 5, 0, "bf16", 1, 2, False),
    (128, 8, 4, 64, "bf16", 3, 1, True),
    (256, 4, 4, 1, "bf16", 1, 1, True),
    (128, 6, 6, 8, "bf16", 2, 2, True),
]


@pytest.mark.parametrize("case", ONE_TOKEN_CASES,
                         ids=[_case_id(c[:7] + ([1], c[7])) for c in ONE_TOKEN_CASES])
def test_one_token_appends_bit_exact(case):
    # decode-step appends, one token per sequence per call: 75 calls cross
    # 8-token V groups, a 64-token tile and every tail slot; then sequence 0
    # rolls back to an unaligned length and appends again, so codes merge
    # into V words that hold older codes
    d, kb, vb, T, dtype, B, H, rot = case
    pair = Pair(B, H, d, kb, vb, T, 120, rot, rot)
    pair.append(workloads.adversarial_numpy(1, (B, 13, H, d), dtype),
                workloads.adversarial_numpy(2, (B, 13, H, d), dtype), dtype)
    for s in range(75):
        pair.append(workloads.adversarial_numpy(100 + s, (B, 1, H, d), dtype),
                    workloads.adversarial_numpy(300 + s, (B, 1, H, d), dtype), dtype)
    pair.compare_planes()
    lens = list(pair.lens)
    lens[0] = 37
    pair.append(workloads.adversarial_numpy(500, (B, 1, H, d), dtype),
                workloads.adversarial_numpy(501, (B, 1, H, d), dtype), dtype, lens=lens)
    for s in range(5):
        pair.append(workloads.adversarial_numpy(510 + s, (B, 1, H, d), dtype),
                    workloads.adversarial_numpy(520 + s, (B, 1, H, d), dtype), dtype)
    pair.compare_planes()


DEQUANT_CASES = APPEND_CASES[:8] + APPEND_CASES[-3:]


@pytest.mark.parametrize("case", DEQUANT_CASES, ids=[_case_id(c) for c in DEQUANT_CASES])
def test_dequantize_bit_exact(case):
    import torch
    import decode_attention_rotate_amd as kvq
    d, kb, vb, T, dtype, B, H, chunks, rot = case
    n = sum(chunks)
    pair = Pair(B, H, d, kb, vb, T, n, rot, rot)
    k = workloads.adversarial_numpy(7, (B, n, H, d), dtype)
    v = workloads.adversarial_numpy(8, (B, n, H, d), dtype)
    pair.append(k, v, dtype)
    planes = gpu_planes(pair.cache, pair.cfg)
    for which, bits in ((0, kb), (1, vb)):
        for space in (0, 1):
            for b in range(B):
                for t0, t1 in ((0, n), (n // 3, n - 1)):
                    say("dequantize", which, b, t0, t1, space)
                    got = kvq.kvq_dequantize(pair.cfg, pair.cache, which, b, t0, t1,
                                             pair.lens, space).cpu().numpy()
                    torch.cuda.synchronize()
                    want = dequantize_reference(planes, which, b, t0, t1, n, H, d, bits, T,
                                                space, rotate=rot)
                    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
                        (which, space, b, t0, t1)


def _fill(pair, w, n_list, dtype, seed0=0):
    """Append workload tokens so sequence b ends with length n_list[b]:
    one append for everyone, then a second append that restarts the shorter
    sequences (a sequence given length 0 starts afresh)."""
    B = len(n_list)
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


ATTN_CASES = [
    # name, workload overrides, lengths
    ("tiny", dict(), [256]),
    ("small", dict(), [4096]),
    ("mid", dict(B=2), [1000, 333]),
    ("long", dict(B=2, tail=1024), [3000, 1500]),
    ("long", dict(B=2, tail=16), [700, 700]),
    ("long", dict(B=1, tail=64), [40]),
    ("huge", dict(B=2), [2000, 129]),
    ("small", dict(Hq=24), [513]),            # G = 3
    ("small", dict(Hq=48), [200]),            # G = 6
    ("small", dict(Hq=56), [130]),            # G = 7
    ("small", dict(Hq=96, B=2), [100, 64]),   # G = 12: two chunks of 6
    ("small", dict(Hq=8), [1]),               # G = 1, one token
    ("tiny", dict(B=2, k_bits=8, v_bits=5), [64, 63]),
    ("huge", dict(B=1, Hq=8, k_bits=4, v_bits=8, tail=100), [300]),
    ("mid", dict(B=2, k_bits=6, v_bits=6), [700, 129]),          # q6_0
    ("huge", dict(B=1, Hq=8, k_bits=6, v_bits=4), [300]),
    ("long", dict(B=1, k_bits=8, v_bits=6, tail=64), [500]),
]


@pytest.mark.parametrize("name,over,lens", ATTN_CASES,
                         ids=["%s-%d" % (c[0], i) for i, c in enumerate(ATTN_CASES)])
def test_decode_attention(name, over, lens):
    w = workloads.workload(name, **over)
    w["B"] = len(lens)
    d, dtype = w["d"], w["dtype"]
    pair = Pair(w["B"], w["Hkv"], d, w["k_bits"], w["v_bits"], w["tail"], max(lens) + 5)
    _fill(pair, w, lens, dtype)
    assert list(pair.lens) == lens
    q = workloads.q_numpy(w)
    got = pair.decode(q, dtype)
    planes = gpu_planes(pair.cache, pair.cfg)
    errs = attention_errors(got, planes, to_values(q, dtype), lens, pair.cfg)
    worst = max(errs.values())
    say("worst rel L2 %.3e" % worst)
    assert worst <= TOL, sorted(errs.items(), key=lambda kv: -kv[1])[:3]


def test_decode_rotation_flags_and_scale():
    w = workloads.workload("small", B=2, Hq=16)
    for rk, rv in ((False, True), (True, False), (False, False)):
        pair = Pair(2, 8, 128, 8, 4, 32, 600, rk, rv)
        _fill(pair, w, [520, 520], "bf16")
        q = workloads.q_numpy(w)
        got = pair.decode(q, "bf16", sm_scale=0.05)
        planes = gpu_planes(pair.cache, pair.cfg)
        errs = attention_errors(got, planes, to_values(q, "bf16"), [520, 520], pair.cfg,
                                sm_scale=0.05)
        assert max(errs.values()) <= TOL, (rk, rv)


def test_decode_fp32_query_and_repeat_calls():
    w = workloads.workload("mid", B=2, dtype="f32")
    pair = Pair(2, 8, 128, 4, 4, 0, 1100)
    _fill(pair, w, [1100, 1100], "f32")
    q = workloads.q_numpy(w)
    a = pair.decode(q, "f32")
    b = pair.decode(q, "f32")
    # the waves of a workgroup take tiles dynamically, so the float32
    # summation order and the running maximum each fp16 weight is rounded
    # against can change between calls: both calls must meet the bar, and
    # agree with each other to it
    rel = np.linalg.norm(a - b, axis=-1) / np.linalg.norm(a, axis=-1)
    say("repeat calls differ by rel L2 %.3e" % np.max(rel))
    assert np.max(rel) <= TOL, np.max(rel)
    planes = gpu_planes(pair.cache, pair.cfg)
    for out in (a, b):
        errs = attention_errors(out, planes, to_values(q, "f32"), [1100, 1100], pair.cfg)
        assert max(errs.values()) <= TOL


def test_decode_steps_with_single_token_appends():
    # the decode step as a serving loop runs it: append one token, attend
    w = workloads.workload("long", B=2, tail=32)
    pair = Pair(2, 8, 128, 8, 4, 32, 400)
    _fill(pair, w, [300, 300], "bf16")
    for step in range(3):
        k = workloads.new_tokens_numpy(w, 1, step)
        v = workloads.new_tokens_numpy(w, 2, step)
        pair.append(k, v, "bf16")
        q = workloads.q_numpy(w, step)
        got = pair.decode(q, "bf16")
        planes = pair.compare_planes()
        errs = attention_errors(got, planes, to_values(q, "bf16"), list(pair.lens), pair.cfg)
        assert max(errs.values()) <= TOL


def test_decode_reuses_one_workspace():
    # one caller-owned workspace serves calls of different head counts and
    # lengths: nothing in it may carry over from one call into the next
    import torch
    import decode_attention_rotate_amd as kvq
    w = workloads.workload("long", B=2, tail=64)
    pair = Pair(2, 8, 128, 8, 4, 64, 3000)
    _fill(pair, w, [2500, 900], "bf16")
    need = max(kvq.kvq_decode_workspace_bytes(pair.cfg, hq) for hq in (40, 16, 96))
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    planes = gpu_planes(pair.cache, pair.cfg)
    for call, hq in enumerate((40, 16, 96, 40)):
        q = workloads.q_numpy(dict(w, Hq=hq), call)
        qt = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to("cuda")
        say("decode with shared workspace", call, hq)
        got = kvq.kvq_decode_attention(pair.cfg, pair.cache, qt, list(pair.lens), workspace=ws)
        torch.cuda.synchronize()
        errs = attention_errors(got.cpu().numpy(), planes, to_values(q, "bf16"), list(pair.lens),
                                pair.cfg)
        assert max(errs.values()) <= TOL, (call, hq, max(errs.values()))


PREFILL_CASES = [
    # name, workload overrides, lengths before the chunk, n_q
    ("tiny", dict(), [0], 64),                          # from scratch: a full causal square
    ("long", dict(B=2, tail=1024), [700, 300], 40),     # the chunk stays in the bf16 tail
    ("long", dict(B=1, tail=16), [500], 50),            # tokens leave the tail during the chunk
    ("mid", dict(B=2), [300, 0], 37),                   # no tail, ragged, one from scratch
    ("huge", dict(B=1, Hq=8), [200], 70),               # d256, 5-bit K
    ("small", dict(Hq=24), [0], 129),                   # G = 3, several row blocks
    ("small", dict(Hq=56, dtype="f32"), [100], 10),     # G = 7, float32 queries
    ("tiny", dict(B=2, k_bits=8, v_bits=5, tail=8), [64, 1], 3),
    ("small", dict(k_bits=6, v_bits=6), [200], 30),
]


def _prefill_case(w, before, n_q, rot=True):
    B = len(before)
    w["B"] = B
    d, dtype = w["d"], w["dtype"]
    pair = Pair(B, w["Hkv"], d, w["k_bits"], w["v_bits"], w["tail"], max(before) + n_q + 5, rot, rot)
    if max(before) > 0:
        _fill(pair, w, before, dtype)
    k = workloads.kv_numpy(w, 1, 20000, 20000 + n_q)
    v = workloads.kv_numpy(w, 2, 20000, 20000 + n_q)
    pair.append(k, v, dtype)
    return pair


@pytest.mark.parametrize("name,over,before,n_q", PREFILL_CASES,
                         ids=["%s-%d" % (c[0], i) for i, c in enumerate(PREFILL_CASES)])
def test_prefill_attention(name, over, before, n_q):
    import decode_attention_rotate_amd as kvq
    w = workloads.workload(name, **over)
    pair = _prefill_case(w, before, n_q)
    lens = list(pair.lens)
    q = workloads.prefill_q_numpy(w, n_q)
    say("prefill", name, "n_q=%d" % n_q, "lens=%s" % lens)
    got = kvq.kvq_prefill_attention(pair.cfg, pair.cache, to_device(q, w["dtype"]), lens)
    got = got.cpu().numpy().astype(np.float64)
    planes = gpu_planes(pair.cache, pair.cfg)
    ref = prefill_reference(planes, to_values(q, w["dtype"]), lens, w["Hkv"], w["d"],
                            w["k_bits"], w["v_bits"], w["tail"])
    err = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    say("prefill worst rel L2 %.3e" % err.max())
    assert err.max() <= TOL, np.unravel_index(np.argmax(err), err.shape)


def test_prefill_one_query_and_rotation_off():
    # one query is a decode step; with rotation off the oracle skips both
    # rotations and so must the kernel
    import decode_attention_rotate_amd as kvq
    w = workloads.workload("long", B=2, tail=32)
    pair = _prefill_case(w, [400, 90], 1)
    q = workloads.prefill_q_numpy(w, 1)
    qd = to_device(q, "bf16")
    pre = kvq.kvq_prefill_attention(pair.cfg, pair.cache, qd, list(pair.lens)).cpu().numpy()
    dec = kvq.kvq_decode_attention(pair.cfg, pair.cache, qd[:, 0].contiguous(),
                                   list(pair.lens)).cpu().numpy()
    rel = np.linalg.norm(pre[:, 0] - dec, axis=-1) / np.linalg.norm(dec, axis=-1)
    assert rel.max() <= TOL, rel.max()
    w2 = workloads.workload("small", B=1, Hq=16)
    pair2 = _prefill_case(w2, [150], 33, rot=False)
    q2 = workloads.prefill_q_numpy(w2, 33)
    got = kvq.kvq_prefill_attention(pair2.cfg, pair2.cache, to_device(q2, "bf16"),
                                    list(pair2.lens)).cpu().numpy().astype(np.float64)
    ref = prefill_reference(gpu_planes(pair2.cache, pair2.cfg), to_values(q2, "bf16"),
                            list(pair2.lens), 8, 128, 8, 8, 0, rotate_k=False, rotate_v=False)
    err = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    assert err.max() <= TOL, err.max()


def test_decode_at_the_largest_batch():
    """KVQ_MAX_BATCH sequences of ragged lengths (1 .. 300) in one call: the
    length array and the grid at their largest; without a tail, positions
    past a sequence's length are never read."""
    import decode_attention_rotate_amd as kvq
    B = kvq.KVQ_MAX_BATCH
    w = workloads.workload("tiny", B=B, Hq=2, Hkv=1, dtype="bf16")
    lens = [1 + (37 * b) % 300 for b in range(B)]
    pair = Pair(B, 1, 64, 4, 4, 0, 320)
    pair.append(workloads.kv_numpy(w, 1, 0, max(lens)), workloads.kv_numpy(w, 2, 0, max(lens)),
                "bf16")
    q = workloads.q_numpy(w)
    got = pair.decode(q, "bf16", lens=lens)
    planes = gpu_planes(pair.cache, pair.cfg)
    errs = attention_errors(got, planes, to_values(q, "bf16"), lens, pair.cfg)
    worst = max(errs.values())
    say("largest batch worst rel L2 %.3e" % worst)
    assert worst <= TOL


def test_profiling_events_bound_to_the_kernels():
    """kvq_profile_decode_events makes the decode split kernel and the
    matrix-core prefill kernel launch with the two events bound to them; the
    results stay those of the plain launch (against the oracle) and the
    events give a positive elapsed time; switching them off restores plain
    launches."""
    import torch
    import decode_attention_rotate_amd as kvq
    w = workloads.workload("long", B=2, tail=64)
    pair = Pair(2, 8, 128, 8, 4, 64, 2100)
    _fill(pair, w, [2000, 700], "bf16")
    lens = list(pair.lens)
    q = workloads.q_numpy(w)
    qd = to_device(q, "bf16")
    planes = gpu_planes(pair.cache, pair.cfg)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    try:
        say("decode with profiling events")
        kvq.kvq_profile_decode_events(e0, e1)
        got = kvq.kvq_decode_attention(pair.cfg, pair.cache, qd, lens)
        torch.cuda.synchronize()
        ms = kvq.kernel_elapsed_ms(e0, e1)
        assert np.isfinite(ms) and ms > 0, ms
        errs = attention_errors(got.cpu().numpy().astype(np.float64), planes, to_values(q, "bf16"),
                                lens, pair.cfg)
        assert max(errs.values()) <= TOL, max(errs.values())
        say("prefill with profiling events")
        qp = workloads.prefill_q_numpy(w, 16)
        e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        kvq.kvq_profile_decode_events(e2, e3)
        pre = kvq.kvq_prefill_attention(pair.cfg, pair.cache, to_device(qp, "bf16"), lens)
        torch.cuda.synchronize()
        ms = kvq.kernel_elapsed_ms(e2, e3)
        assert np.isfinite(ms) and ms > 0, ms
        ref = prefill_reference(planes, to_values(qp, "bf16"), lens, 8, 128, 8, 4, 64)
        got = pre.cpu().numpy().astype(np.float64)
        err = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
        assert err.max() <= TOL, err.max()
    finally:
        kvq.kvq_profile_decode_events(None, None)
    say("decode after switching the events off")
    got = kvq.kvq_decode_attention(pair.cfg, pair.cache, qd, lens)
    torch.cuda.synchronize()
    errs = attention_errors(got.cpu().numpy().astype(np.float64), planes, to_values(q, "bf16"),
                            lens, pair.cfg)
    assert max(errs.values()) <= TOL, max(errs.values())
