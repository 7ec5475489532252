"""Seeded sweep over the supported configuration matrix (GPU against the
oracle): head_dim 64/128/192/256, K and V code widths 4/5/6/8 with absmax or
(4/5 bits) scale-and-min blocks, bf16 tail lengths, rotation flags and
random-sign rotations, query heads per KV head 1..8 and 12, bf16 and float32
inputs, ragged batches appended in two chunks (odd sequences restart at
position 0 for the second).  Each case checks:

* every code, scale and tail byte bit-exact against the oracle cache;
* decode attention of every (sequence, query head) within 1e-3 relative L2
  of the float64 oracle on the device planes;
* for absmax caches, chunked prefill of the last n_q positions within 1e-3.

The cases are drawn once from a fixed seed, so the sweep is the same on
every run; each case's inputs come from the workload generators with a
per-case stream index."""

import numpy as np
import pytest

import workloads
from gpu_common import Pair, say, to_device, to_values, attention_errors, gpu_planes
from oracle import prefill_reference

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _draw_cases(n=24, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128, 192, 256]))
        kb = int(rng.choice([4, 5, 6, 8]))
        vb = int(rng.choice([4, 5, 6, 8]))
        km = bool(kb <= 5 and rng.random() < 0.3)
        vm = bool(vb <= 5 and rng.random() < 0.3)
        T = int(rng.choice([0, 0, 16, 100]))
        G = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12]))
        H = int(rng.choice([1, 2]))
        B = int(rng.choice([1, 2, 3]))
        lens = sorted(int(x) for x in rng.integers(1, 700, size=2))
        first = lens[0]
        second = lens[1] - lens[0]
        rot = [(True, True), (True, True), (False, True), (True, False)][int(rng.integers(4))]
        sign_seed = int(rng.choice([0, 0, 7]))
        dtype = "bf16" if rng.random() < 0.75 else "f32"
        dist = "t3" if rng.random() < 0.3 else "normal"
        n_q = int(rng.integers(1, 40))
        cases.append(dict(i=i, d=d, kb=kb, vb=vb, km=km, vm=vm, T=T, G=G, H=H, B=B, first=first,
                          second=second, rot=rot, sign_seed=sign_seed, dtype=dtype, dist=dist, n_q=n_q))
    return cases


CASES = _draw_cases()
# Case 18 of the draw from seed 4242 (head_dim 64, K5 V4, bf16 tail 16, 6 query
# heads per KV head, bf16): its prefill rows came out 1.6e-3 off the oracle
# while the split kernel rounded each P.V weight to one fp16 value; kept as a
# regression case for the high + low weight parts those rows now carry.
CASES += [dict(c, tag="seed4242-") for c in _draw_cases(n=19, seed=4242)[18:19]]


def _case_id(c):
    fk = "%d%s" % (c["kb"], "_1" if c["km"] else "")
    fv = "%d%s" % (c["vb"], "_1" if c["vm"] else "")
    return "%s%d-d%d-K%s-V%s-T%d-G%d-%s" % (c.get("tag", ""), c["i"], c["d"], fk, fv, c["T"], c["G"],
                                            c["dtype"])


@pytest.mark.parametrize("c", CASES, ids=[_case_id(c) for c in CASES])
def test_sweep_case(c):
    import decode_attention_rotate_amd as kvq
    d, B, H = c["d"], c["B"], c["H"]
    w = workloads.workload("small", idx=100 + c["i"], B=B, Hkv=H, Hq=H * c["G"], d=d,
                           k_bits=c["kb"], v_bits=c["vb"], tail=c["T"], dtype=c["dtype"],
                           dist=c["dist"], outlier="per_head", count=3, factor=20.0)
    n = c["first"] + c["second"]
    rk, rv = c["rot"]
    pair = Pair(B, H, d, c["kb"], c["vb"], c["T"], n + 3, rk, rv, c["sign_seed"], c["km"], c["vm"])
    k = workloads.kv_numpy(w, 1, 0, n)
    v = workloads.kv_numpy(w, 2, 0, n)
    # the first chunk for every sequence, then the rest, with the odd
    # sequences restarting from position 0 (ragged lengths when B > 1)
    pair.append(k[:, :c["first"]], v[:, :c["first"]], c["dtype"])
    if c["second"] > 0:
        restart = [c["first"] if b % 2 == 0 else 0 for b in range(B)]
        pair.append(k[:, c["first"]:], v[:, c["first"]:], c["dtype"], lens=restart)
    say("sweep case", _case_id(c), "lens", list(pair.lens))
    planes = pair.compare_planes()
    lens = list(pair.lens)
    q = workloads.q_numpy(w)
    got = pair.decode(q, c["dtype"])
    errs = attention_errors(got, planes, to_values(q, c["dtype"]), lens, pair.cfg)
    worst = max(errs.values())
    say("decode worst rel L2 %.3e" % worst)
    assert worst <= TOL, sorted(errs.items(), key=lambda kv: -kv[1])[:3]
    if c["km"] or c["vm"]:
        return
    n_q = min(c["n_q"], min(lens))
    qp = workloads.prefill_q_numpy(w, n_q)
    say("prefill n_q=%d" % n_q)
    pre = kvq.kvq_prefill_attention(pair.cfg, pair.cache, to_device(qp, c["dtype"]), lens)
    pre = pre.cpu().numpy().astype(np.float64)
    ref = prefill_reference(planes, to_values(qp, c["dtype"]), lens, H, d, c["kb"], c["vb"], c["T"],
                            rotate_k=rk, rotate_v=rv, sign_seed=c["sign_seed"])
    err = np.linalg.norm(pre - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    say("prefill worst rel L2 %.3e" % err.max())
    assert err.max() <= TOL, np.unravel_index(np.argmax(err), err.shape)
