"""GPU parity of the outlier-channel path (32 channels per plane and KV head
kept at 8 bits in the original space, the rest rotated and quantized; the
reading of the velog.io post "fix KV cache quantization outliers", section
"application and background", that the oracle's outlier module states).

The device cache must hold exactly the oracle's bytes in all six planes
(the rest's codes and scales, the outliers' codes and scales: an encoding,
bit-exact), after a chunked append and after single-token decode steps.
Attention is compared with the float64 split-form reference evaluated on
the device planes, within 1e-3 relative L2; read-back is bit-exact in both
spaces (space 1: the rest rotated back plus the outlier values at their
channels, one float32 add).  Channel lists are the workload's outlier
channels first, then seeded fill, in a shuffled order (list order matters:
it is the order of the outlier block)."""

import numpy as np
import pytest

import workloads
from gpu_common import DEV, say, to_device, to_values, rel_l2

pytestmark = pytest.mark.gpu

TOL = 1e-3


class OutPair:
    """A device cache with outlier channels and the oracle's OutlierCache fed
    the same appends."""

    def __init__(self, w, B, kb, vb, max_ctx, lists, rotate=True, sign_seed=0, page_pool=0,
                 table=None):
        import torch
        import decode_attention_rotate_amd as kvq
        from oracle.outliers import OutlierCache
        Hkv, d = w["Hkv"], w["d"]
        self.cfg = kvq.kvq_config(B, Hkv, d, max_ctx, kb, vb, 0, rotate, rotate, sign_seed,
                                  False, False, page_pool, outliers=32)
        self.table = None if table is None else np.asarray(table, np.int32)
        dev_table = None if table is None else torch.from_numpy(self.table).to(DEV)
        self.idx_dev = torch.from_numpy(np.ascontiguousarray(lists)).to(DEV)
        self.cache = kvq.KVCache(self.cfg, DEV, page_table=dev_table, outlier_idx=self.idx_dev)
        self.orc = OutlierCache(B, Hkv, d, kb, vb, max_ctx, lists[0], lists[1], rotate, rotate,
                                sign_seed)
        self.lists = lists
        self.lens = np.zeros(B, np.int64)

    def append(self, k, v, dtype, lens=None):
        import torch
        import decode_attention_rotate_amd as kvq
        lens = self.lens if lens is None else np.asarray(lens, np.int64)
        say("outlier append", self.cfg, "n_new=%d" % k.shape[1], "lens=%s" % list(lens))
        kvq.kvq_rotate_quantize_append(self.cfg, self.cache, to_device(k, dtype), to_device(v, dtype),
                                       lens)
        torch.cuda.synchronize()
        self.orc.append(k, v, lens, dtype=dtype)
        self.lens = lens + k.shape[1]

    def planes(self):
        """Device planes shaped like OutlierCache.physical()."""
        from gpu_common import gpu_planes
        from oracle import pages_to_contiguous
        cfg = self.cfg
        B, H = cfg.batch, cfg.n_kv_heads
        cap = (cfg.max_ctx + 63) // 64 * 64
        out = gpu_planes(self.cache, cfg, self.table)
        for p in ("k", "v"):
            codes = self.cache[p + "_out_codes"].cpu().numpy()
            scales = self.cache[p + "_out_scales"].cpu().numpy().view(np.uint16)
            if cfg.page_pool > 0:
                codes = pages_to_contiguous(codes, self.table, H, 64 * 32)
                scales = pages_to_contiguous(scales, self.table, H, 64)
            out[p + "_out_codes"] = codes.reshape(B, H, cap * 32)
            out[p + "_out_scales"] = scales.reshape(B, H, cap)
        return out

    def compare_planes(self):
        got, want = self.planes(), self.orc.physical()
        for key in want:
            a, b = got[key], want[key]
            assert a.shape == b.shape, (key, a.shape, b.shape)
            if not np.array_equal(a, b):
                bad = np.argwhere(a != b)
                raise AssertionError("%s differs at %d places, first %s: gpu %s oracle %s"
                                     % (key, len(bad), bad[0], a[tuple(bad[0])], b[tuple(bad[0])]))
        return got

    def errors(self, out, planes, qv, lens):
        from oracle.outliers import decode_reference_outliers
        cfg = self.cfg
        ref = decode_reference_outliers(planes, qv, lens, cfg.n_kv_heads, cfg.head_dim, cfg.k_bits,
                                        cfg.v_bits, self.lists[0], self.lists[1],
                                        rotate_k=bool(cfg.rotate_k), rotate_v=bool(cfg.rotate_v),
                                        sign_seed=cfg.sign_seed)
        B, Hq, _ = qv.shape
        return {(b, h): rel_l2(out[b, h], ref[b, h]) for b in range(B) for h in range(Hq)}


def fill(pair, w, lens, dtype, chunks=2):
    """Append workload tokens so sequence b has length lens[b] (at most two
    distinct lengths), the longer part in `chunks` appends."""
    nmax = max(lens)
    k = workloads.kv_numpy(w, 1, 0, nmax)
    v = workloads.kv_numpy(w, 2, 0, nmax)
    m = min(lens)
    assert all(x in (nmax, m) for x in lens)
    first = nmax - m if m < nmax else nmax   # what every sequence appends first
    cut = [0] + [first * (i + 1) // chunks for i in range(chunks)]
    for a, b in zip(cut[:-1], cut[1:]):
        if b > a:
            pair.append(k[:, a:b], v[:, a:b], dtype)
    if 0 < m < nmax:
        restart = [nmax - m if x == nmax else 0 for x in lens]
        pair.append(k[:, nmax - m:], v[:, nmax - m:], dtype, lens=restart)


CASES = [
    # name, workload, overrides, kb, vb, lengths
    ("long-k8v4", "long", dict(B=2, tail=0), 8, 4, [300, 129]),
    ("mid-k4v4", "mid", dict(B=2), 4, 4, [200, 64]),
    ("small-k8v8-G2", "small", dict(B=2), 8, 8, [190, 1]),
    ("k4v5", "mid", dict(B=2, Hq=8), 4, 5, [130, 130]),
    ("k6v6-G1", "small", dict(B=2, Hq=8), 6, 6, [97, 33]),
    ("k5v4-G12", "long", dict(B=2, Hq=96, tail=0), 5, 4, [150, 70]),
    # heavy-tailed (Student-t) inputs: large scores magnify the query's
    # fixed-point step, for the outlier channels' part as for the rest
    ("t3-k8v4", "long", dict(B=2, tail=0, dist="t3"), 8, 4, [700, 350]),
    ("t3-k4v4-G4", "mid", dict(B=2, dist="t3"), 4, 4, [600, 257]),
    ("t3-k8v8-G8", "small", dict(B=2, Hq=64, dist="t3"), 8, 8, [400, 400]),
    ("f32-k8v8", "small", dict(B=2, dtype="f32"), 8, 8, [100, 100]),
]


def _build(case, rotate=True, sign_seed=0, paged=False, extra=8):
    name, base, over, kb, vb, lens = case
    w = workloads.workload(base, **over)
    lists = workloads.outlier_lists(w)
    max_ctx = max(lens) + extra
    table, pool = None, 0
    B = len(lens)
    if paged:
        tiles = (max_ctx + 63) // 64
        pool = B * tiles + 2
        table = np.random.default_rng(5).permutation(pool)[:B * tiles].astype(np.int32).reshape(B, tiles)
    pair = OutPair(w, B, kb, vb, max_ctx, lists, rotate, sign_seed, pool, table)
    fill(pair, w, lens, w["dtype"])
    return w, pair


def _decode_check(w, pair, step=0):
    import torch
    import decode_attention_rotate_amd as kvq
    dtype = w["dtype"]
    planes = pair.compare_planes()
    q = workloads.q_numpy(w, step)
    lens = [int(x) for x in pair.lens]
    say("outlier decode", pair.cfg, "Hq=%d" % q.shape[1], "lens=%s" % lens)
    out = kvq.kvq_decode_attention(pair.cfg, pair.cache, to_device(q, dtype), lens)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    errs = pair.errors(out, planes, to_values(q, dtype), lens)
    worst = max(errs.values())
    say("worst rel L2 %.3e" % worst)
    assert worst <= TOL, sorted(errs.items(), key=lambda kv: -kv[1])[:3]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_outlier_append_and_decode(case):
    w, pair = _build(case)
    _decode_check(w, pair)


@pytest.mark.parametrize("case", CASES[:3], ids=[c[0] for c in CASES[:3]])
def test_outlier_decode_steps(case):
    """kvq_decode_step on a cache with outlier channels: one token appended
    and attended per call."""
    import torch
    import decode_attention_rotate_amd as kvq
    w, pair = _build(case)
    dtype = w["dtype"]
    for step in range(3):
        kn = workloads.new_tokens_numpy(w, 1, step)
        vn = workloads.new_tokens_numpy(w, 2, step)
        q = workloads.q_numpy(w, step + 1)
        lens = [int(x) for x in pair.lens]
        say("outlier decode step", case[0], "step %d" % step, "lens=%s" % lens)
        out = kvq.kvq_decode_step(pair.cfg, pair.cache, to_device(kn, dtype), to_device(vn, dtype),
                                  to_device(q, dtype), lens)
        torch.cuda.synchronize()
        out = out.cpu().numpy().astype(np.float64)
        pair.orc.append(kn, vn, np.asarray(lens, np.int64), dtype=dtype)
        pair.lens = pair.lens + 1
        planes = pair.compare_planes()
        errs = pair.errors(out, planes, to_values(q, dtype), [int(x) for x in pair.lens])
        worst = max(errs.values())
        say("worst rel L2 %.3e" % worst)
        assert worst <= TOL, (step, sorted(errs.items(), key=lambda kv: -kv[1])[:3])


def test_outlier_rotation_off_signs_and_paged():
    w, pair = _build(CASES[0], rotate=False)
    _decode_check(w, pair)
    w, pair = _build(CASES[1], sign_seed=777)
    _decode_check(w, pair)
    w, pair = _build(CASES[3], paged=True)
    _decode_check(w, pair)


@pytest.mark.parametrize("space", [0, 1])
@pytest.mark.parametrize("signs", [0, 4242])
def test_outlier_dequantize(space, signs):
    """Read-back: space 0 is the rotated rest, space 1 the reconstruction
    (the rest rotated back, the outliers added at their channels)."""
    import torch
    import decode_attention_rotate_amd as kvq
    from oracle import dequantize_reference
    from oracle.outliers import outlier_values
    w, pair = _build(CASES[3], sign_seed=signs)
    planes = pair.compare_planes()
    cfg = pair.cfg
    for which in (0, 1):
        for b, (t0, t1) in enumerate([(0, 130), (61, 129)]):
            say("outlier dequant", "which=%d b=%d [%d,%d) space=%d" % (which, b, t0, t1, space))
            got = kvq.kvq_dequantize(cfg, pair.cache, which, b, t0, t1, [int(x) for x in pair.lens],
                                     space).cpu().numpy()
            bits = cfg.k_bits if which == 0 else cfg.v_bits
            want = dequantize_reference(planes, which, b, t0, t1, int(pair.lens[b]), cfg.n_kv_heads,
                                        cfg.head_dim, bits, 0, space, rotate=True, sign_seed=signs)
            if space == 1:
                p = "k" if which == 0 else "v"
                for g in range(cfg.n_kv_heads):
                    o = outlier_values(planes, p, b, g, t1)[t0:t1]
                    ch = pair.lists[which, g]
                    want[:, g, ch] = (want[:, g, ch] + o).astype(np.float32)
            assert got.shape == want.shape
            assert np.array_equal(got, want), np.argwhere(got != want)[:3]
