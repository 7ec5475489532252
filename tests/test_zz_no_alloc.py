"""The decode entry point for callers that cannot allocate device memory
(kvq_decode_attention_static, whose split partials live in the library's
static device workspace): through the C ABI its output matches
kvq_decode_attention's on the same inputs, and both match the float64
oracle, on two calls in a row where the second is smaller (fewer sequences'
worth of tokens and fewer query heads), so the second call must not depend
on what the first left in the shared workspace."""

import numpy as np
import pytest

import workloads
from gpu_common import Pair, say, to_device, to_values, attention_errors, gpu_planes

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _check(pair, w, lens, hq, step):
    import decode_attention_rotate_amd as kvq
    wq = dict(w, Hq=hq)
    q = workloads.q_numpy(wq, step)
    qd = to_device(q, "bf16")
    say("static-workspace decode", pair.cfg, "Hq=%d" % hq, "lens=%s" % lens)
    got = kvq.kvq_decode_attention_static(pair.cfg, pair.cache, qd, lens)
    ref_call = kvq.kvq_decode_attention(pair.cfg, pair.cache, qd, lens)
    import torch
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    ref_call = ref_call.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(got - ref_call, axis=-1) / np.linalg.norm(ref_call, axis=-1)
    say("static vs workspace call: rel L2 %.3e" % rel.max())
    assert rel.max() <= TOL, rel.max()
    planes = gpu_planes(pair.cache, pair.cfg)
    for out in (got, ref_call):
        errs = attention_errors(out, planes, to_values(q, "bf16"), lens, pair.cfg)
        assert max(errs.values()) <= TOL, max(errs.values())


def test_static_workspace_matches_workspace_call():
    w = workloads.workload("long", B=2, tail=64)
    pair = Pair(2, 8, 128, 8, 4, 64, 3000)
    pair.append(workloads.kv_numpy(w, 1, 0, 2500), workloads.kv_numpy(w, 2, 0, 2500), "bf16")
    _check(pair, w, [2500, 2500], 40, 0)
    # second call smaller: shorter lengths, fewer query heads
    _check(pair, w, [700, 300], 16, 1)
