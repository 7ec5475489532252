"""GPU parity of the fused decode step (kvq_decode_step): one call appends
one token per sequence and attends over the cache with it.

After every step the device cache must hold exactly the bytes the oracle's
append produces (the quantizer is an encoding: bit-exact), and the attention
output must be within 1e-3 relative L2 of the float64 oracle evaluated on
that post-append cache.  Steps run in sequence, so the cases cross the
points where the step's special positions change: a cache shorter than the
tail (nothing leaves it), the first position that leaves the tail, a tile
boundary, and no tail at all (the new token itself is quantized).  Sources:
velog.io post "fix KV cache quantization outliers", section "Hadamard
rotation" (rotate and store at append, rotated scores and weighted sum at
attention); aitrends.kr article 92204, glossary "Precision Tail"."""

import numpy as np
import pytest

import workloads
from gpu_common import Pair, say, to_device, to_values, attention_errors, fill_lengths

pytestmark = pytest.mark.gpu

TOL = 1e-3

CASES = [
    # name, overrides, d, kb, vb, km, vm, T, initial lengths, steps
    ("long-T64", dict(), 128, 8, 4, False, False, 64, [62, 200], 4),      # 62 -> 63, 64, 65: first graduation
    ("long-T64-tile", dict(), 128, 8, 4, False, False, 64, [126, 1], 4),   # tile edge; a one-token sequence
    ("mid-T0", dict(), 128, 4, 4, False, False, 0, [62, 300], 4),          # the new token is quantized
    ("small-T0-k8v8", dict(Hq=16), 128, 8, 8, False, False, 0, [0, 129], 3),   # from an empty cache
    ("tiny-d64", dict(Hq=2, Hkv=1), 64, 4, 4, False, False, 8, [7, 40], 3),
    ("huge-d256", dict(Hq=16, Hkv=4), 256, 5, 4, False, False, 0, [64, 300], 3),
    ("huge-d256-T", dict(Hq=8, Hkv=2), 256, 8, 5, False, False, 32, [31, 90], 3),
    ("d192", dict(d=192, Hq=10, Hkv=2), 192, 8, 4, False, False, 16, [15, 100], 3),
    ("q6", dict(), 128, 6, 6, False, False, 32, [31, 64], 3),
    ("q4_1-q5_1", dict(bias=0.5), 128, 4, 5, True, True, 16, [15, 300], 3),
    ("q5_1-T0", dict(bias=0.5), 128, 5, 4, True, False, 0, [63, 64], 3),
    ("G12-chunks", dict(Hq=96), 128, 8, 4, False, False, 16, [15, 77], 2),     # two head chunks per KV head
    ("f32-inputs", dict(dtype="f32"), 128, 8, 4, False, False, 64, [70, 10], 2),
]


def _ids(c):
    return c[0]


def _run(case, rotate=True, sign_seed=0, paged=False):
    import decode_attention_rotate_amd as kvq
    name, over, d, kb, vb, km, vm, T, lens0, steps = case
    base = "huge" if d == 256 else ("tiny" if d == 64 else "long")
    w = workloads.workload(base, B=len(lens0), **over)
    w["d"] = d
    dtype = w["dtype"]
    B, Hkv = len(lens0), w["Hkv"]
    max_ctx = max(lens0) + steps + 3
    table = None
    pool = 0
    if paged:
        tiles = (max_ctx + 63) // 64
        pool = B * tiles + 3
        table = np.random.default_rng(7).permutation(pool)[:B * tiles].astype(np.int32).reshape(B, tiles)
    pair = Pair(B, Hkv, d, kb, vb, T, max_ctx, rotate, rotate, sign_seed, km, vm, pool, table)
    if max(lens0) > 0:
        fill_lengths(pair, w, lens0, dtype)
    assert [int(x) for x in pair.lens] == lens0
    for step in range(steps):
        kn = workloads.new_tokens_numpy(w, 1, step)
        vn = workloads.new_tokens_numpy(w, 2, step)
        q = workloads.q_numpy(w, step)
        lens = [int(x) for x in pair.lens]
        say("decode step", name, "step %d" % step, "lens=%s" % lens, pair.cfg)
        out = kvq.kvq_decode_step(pair.cfg, pair.cache, to_device(kn, dtype), to_device(vn, dtype),
                                  to_device(q, dtype), lens)
        import torch
        torch.cuda.synchronize()
        out = out.cpu().numpy().astype(np.float64)
        pair.orc.append(kn, vn, np.asarray(lens, dtype=np.int64), dtype=dtype)
        pair.lens = pair.lens + 1
        planes = pair.compare_planes()
        errs = attention_errors(out, planes, to_values(q, dtype), list(pair.lens), pair.cfg)
        worst = max(errs.values())
        say("worst rel L2 %.3e" % worst)
        assert worst <= TOL, (step, sorted(errs.items(), key=lambda kv: -kv[1])[:3])


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_decode_step(case):
    _run(case)


def test_decode_step_rotation_off_and_signs():
    _run(CASES[0], rotate=False)
    _run(CASES[2], sign_seed=12345)


def test_decode_step_paged():
    _run(CASES[0], paged=True)
    _run(CASES[3], paged=True)
