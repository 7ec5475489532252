"""Seeded synthetic workloads shared by the tests, the benchmark and smoke().

This module only draws random numbers and describes shapes.  It holds none of
the method's arithmetic (no rotation, no quantization, no attention), so both
the CPU oracle and the HIP path can take their inputs from it.

Workloads (the pages measure on trained models and text corpora that are not
available here; these synthetic inputs stand in for them with the shapes and
value distributions of the cases below):

  tiny   1 sequence, 1 head, head_dim 64, 256 cached tokens, fp32 inputs
         N(0,1); channels 3 and 41 scaled x20 in K and V; K4 V4; no tail.
  small  B1, 16 query / 8 KV heads, head_dim 128, 4096 tokens, bf16 N(0,1);
         4 random channels per KV head x15 (K and V); K8 V8; no tail.
  mid    B16, 32 query / 8 KV heads, head_dim 128, 32768 tokens, bf16 N(0,1);
         1 % of (head, channel) pairs (10 of 1024) x20; K4 V4; no tail.
  long   B8, 40 query / 8 KV heads, head_dim 128, 65536 tokens, bf16 N(0,1);
         10 (head, channel) pairs x20; K8 V4; newest 1024 tokens bf16 tail.
  huge   B32, 16 query / 4 KV heads, head_dim 256, 131072 tokens, bf16
         Student-t (nu = 3); 2 channels per KV head x30; K5 V4; no tail.

Outlier channels are one fixed (head, channel) set per workload, the same for
every token and sequence, drawn independently for K and V.  q carries no
outliers.  An optional field bias = b adds a fixed per-(head, channel) offset
b * N(0, 1) to every K and V token (stream role 6; absent in the workloads
above), which makes blocks asymmetric about zero, the case scale-and-min
blocks are for.  Optional fields amp_k / amp_v multiply every K / V value
(outliers and bias included) by a constant, for caches of very small or very
large magnitude.  Random streams are keyed by (workload, role, chunk) so any token
range can be regenerated on its own: role 0 = outlier choice, 1 = K, 2 = V,
3 = Q, 4 = new decode tokens.
"""

import numpy as np

CHUNK_TOKENS = 1024

WORKLOADS = {
    "tiny": dict(idx=1, B=1, Hq=1, Hkv=1, d=64, n=256, k_bits=4, v_bits=4,
                 tail=0, dtype="f32", dist="normal", outlier="fixed",
                 channels=(3, 41), factor=20.0),
    "small": dict(idx=2, B=1, Hq=16, Hkv=8, d=128, n=4096, k_bits=8, v_bits=8,
                  tail=0, dtype="bf16", dist="normal", outlier="per_head",
                  count=4, factor=15.0),
    "mid": dict(idx=3, B=16, Hq=32, Hkv=8, d=128, n=32768, k_bits=4, v_bits=4,
                tail=0, dtype="bf16", dist="normal", outlier="pairs",
                count=10, factor=20.0),
    "long": dict(idx=4, B=8, Hq=40, Hkv=8, d=128, n=65536, k_bits=8, v_bits=4,
                 tail=1024, dtype="bf16", dist="normal", outlier="pairs",
                 count=10, factor=20.0),
    "huge": dict(idx=5, B=32, Hq=16, Hkv=4, d=256, n=131072, k_bits=5,
                 v_bits=4, tail=0, dtype="bf16", dist="t3", outlier="per_head",
                 count=2, factor=30.0),
}


def workload(name, **overrides):
    """Copy of a workload description, optionally with fields replaced
    (e.g. a shorter n for a test that must finish on the CPU)."""
    w = dict(WORKLOADS[name])
    w["name"] = name
    w.update(overrides)
    return w


def outlier_scale(w, role):
    """[Hkv][d] float32 multipliers (1 or the outlier factor) for K (role 1)
    or V (role 2)."""
    Hkv, d = w["Hkv"], w["d"]
    s = np.ones((Hkv, d), dtype=np.float32)
    f = np.float32(w["factor"])
    if w["outlier"] == "fixed":
        s[:, list(w["channels"])] = f
        return s
    rng = np.random.default_rng((w["idx"], 0, role))
    if w["outlier"] == "per_head":
        for g in range(Hkv):
            s[g, rng.choice(d, size=w["count"], replace=False)] = f
    elif w["outlier"] == "pairs":
        flat = rng.choice(Hkv * d, size=w["count"], replace=False)
        s.reshape(-1)[flat] = f
    return s


def outlier_lists(w, seed=11, m=32):
    """[2][Hkv][m] int32 channel lists for a cache with outlier channels
    (K's, then V's): per KV head the channels outlier_scale makes large, then
    seeded other channels, the list in a seeded order.  What a calibration
    pass would pick for these inputs."""
    Hkv, d = w["Hkv"], w["d"]
    rng = np.random.default_rng((w["idx"], 7, seed))
    out = np.zeros((2, Hkv, m), np.int32)
    for pl, role in ((0, 1), (1, 2)):
        big = outlier_scale(w, role) > 1
        for g in range(Hkv):
            must = [int(c) for c in np.flatnonzero(big[g])][:m]
            rest = [int(c) for c in rng.permutation(d) if c not in must]
            out[pl, g] = rng.permutation(np.array(must + rest[: m - len(must)], np.int32))
    return out


def amplitude(w, role):
    """Constant factor of K (role 1) or V (role 2) values: amp_k / amp_v, 1 if
    absent."""
    return float(w.get("amp_k" if role == 1 else "amp_v", 1.0))


def channel_bias(w, role):
    """[Hkv][d] float32 per-channel offsets of K (role 1) or V (role 2):
    zero unless the workload sets bias."""
    Hkv, d = w["Hkv"], w["d"]
    b = w.get("bias", 0.0)
    if not b:
        return np.zeros((Hkv, d), dtype=np.float32)
    rng = np.random.default_rng((w["idx"], 6, role))
    return (rng.standard_normal((Hkv, d)) * b).astype(np.float32)


def to_bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (input preparation)."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    b = b.astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _draw(rng, dist, shape):
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "t3":
        return rng.standard_t(3, size=shape).astype(np.float32)
    raise ValueError(dist)


def kv_numpy(w, role, t0, t1, batch=None):
    """K (role 1) or V (role 2) tokens [t0, t1) as [B][t1-t0][Hkv][d].

    Returns float32 values for fp32 workloads, bf16 bit patterns (uint16)
    for bf16 workloads.  batch: optional list of sequence indices."""
    bs = range(w["B"]) if batch is None else batch
    scale = outlier_scale(w, role)
    out = []
    for b in bs:
        parts = []
        c0, c1 = t0 // CHUNK_TOKENS, (t1 + CHUNK_TOKENS - 1) // CHUNK_TOKENS
        for c in range(c0, c1):
            rng = np.random.default_rng((w["idx"], role, b, c))
            x = _draw(rng, w["dist"], (CHUNK_TOKENS, w["Hkv"], w["d"]))
            lo, hi = max(t0, c * CHUNK_TOKENS), min(t1, (c + 1) * CHUNK_TOKENS)
            parts.append(x[lo - c * CHUNK_TOKENS: hi - c * CHUNK_TOKENS])
        x = np.concatenate(parts, axis=0) * scale[None]
        if w.get("bias"):
            x = x + channel_bias(w, role)[None]
        out.append(x * np.float32(amplitude(w, role)))
    x = np.stack(out).astype(np.float32)
    return to_bf16_bits(x) if w["dtype"] == "bf16" else x


def q_numpy(w, step=0):
    """Queries [B][Hq][d] for decode step `step` (float32 or bf16 bits)."""
    rng = np.random.default_rng((w["idx"], 3, step))
    x = _draw(rng, w["dist"], (w["B"], w["Hq"], w["d"]))
    return to_bf16_bits(x) if w["dtype"] == "bf16" else x


def prefill_q_numpy(w, n_q, step=0):
    """Queries [B][n_q][Hq][d] of a prompt chunk (float32 or bf16 bits)."""
    rng = np.random.default_rng((w["idx"], 5, step))
    x = _draw(rng, w["dist"], (w["B"], n_q, w["Hq"], w["d"]))
    return to_bf16_bits(x) if w["dtype"] == "bf16" else x


def new_tokens_numpy(w, role, step, n_new=1):
    """Tokens appended at decode step `step`: [B][n_new][Hkv][d]."""
    rng = np.random.default_rng((w["idx"], 4, role, step))
    x = _draw(rng, w["dist"], (w["B"], n_new, w["Hkv"], w["d"]))
    x = x * outlier_scale(w, role)[None, None]
    if w.get("bias"):
        x = x + channel_bias(w, role)[None, None]
    x = (x * np.float32(amplitude(w, role))).astype(np.float32)
    return to_bf16_bits(x) if w["dtype"] == "bf16" else x


# ---------------------------------------------------------------- torch side
def _torch_draw(torch, gen, dist, shape, device):
    if dist == "normal":
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if dist == "t3":
        z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        c = torch.randn((3,) + tuple(shape), generator=gen, device=device,
                        dtype=torch.float32).pow_(2).sum(0)
        return z / torch.sqrt(c / 3.0)
    raise ValueError(dist)


def kv_torch(w, role, t0, t1, device, torch):
    """Device-side generator for full-size workloads: K/V tokens [t0, t1) as
    a [B][t1-t0][Hkv][d] tensor (bf16, or fp32 for fp32 workloads).

    Uses torch's own generator, seeded per (workload, role, chunk); it is a
    different random stream from kv_numpy.  Tests that check these inputs on
    the CPU copy the same tensors to the host."""
    B, Hkv, d = w["B"], w["Hkv"], w["d"]
    scale = torch.from_numpy(outlier_scale(w, role)).to(device)
    parts = []
    c0, c1 = t0 // CHUNK_TOKENS, (t1 + CHUNK_TOKENS - 1) // CHUNK_TOKENS
    for c in range(c0, c1):
        gen = torch.Generator(device=device)
        gen.manual_seed(((w["idx"] * 8 + role) << 32) + c)
        x = _torch_draw(torch, gen, w["dist"], (B, CHUNK_TOKENS, Hkv, d), device)
        lo, hi = max(t0, c * CHUNK_TOKENS), min(t1, (c + 1) * CHUNK_TOKENS)
        parts.append(x[:, lo - c * CHUNK_TOKENS: hi - c * CHUNK_TOKENS])
    x = torch.cat(parts, dim=1) * scale
    if w.get("bias"):
        x = x + torch.from_numpy(channel_bias(w, role)).to(device)
    x = x * amplitude(w, role)
    dt = torch.bfloat16 if w["dtype"] == "bf16" else torch.float32
    return x.to(dt).contiguous()


def q_torch(w, step, device, torch):
    """Device-side queries [B][Hq][d] for decode step `step`."""
    gen = torch.Generator(device=device)
    gen.manual_seed(((w["idx"] * 8 + 3) << 32) + step)
    x = _torch_draw(torch, gen, w["dist"], (w["B"], w["Hq"], w["d"]), device)
    dt = torch.bfloat16 if w["dtype"] == "bf16" else torch.float32
    return x.to(dt).contiguous()


def prefill_q_torch(w, n_q, step, device, torch):
    """Device-side queries [B][n_q][Hq][d] of a prompt chunk."""
    gen = torch.Generator(device=device)
    gen.manual_seed(((w["idx"] * 8 + 5) << 32) + step)
    x = _torch_draw(torch, gen, w["dist"], (w["B"], n_q, w["Hq"], w["d"]), device)
    dt = torch.bfloat16 if w["dtype"] == "bf16" else torch.float32
    return x.to(dt).contiguous()


def new_tokens_torch(w, role, step, device, torch, n_new=1):
    """Device-side decode-step tokens [B][n_new][Hkv][d]."""
    gen = torch.Generator(device=device)
    gen.manual_seed(((w["idx"] * 8 + 4) << 32) + (role << 24) + step)
    x = _torch_draw(torch, gen, w["dist"], (w["B"], n_new, w["Hkv"], w["d"]), device)
    x = x * torch.from_numpy(outlier_scale(w, role)).to(device)
    if w.get("bias"):
        x = x + torch.from_numpy(channel_bias(w, role)).to(device)
    x = x * amplitude(w, role)
    dt = torch.bfloat16 if w["dtype"] == "bf16" else torch.float32
    return x.to(dt).contiguous()


def adversarial_numpy(seed, shape, dtype="bf16"):
    """Rows that stress the block quantizer: normal rows with outliers, all-zero
    rows, rows so small the fp16 scale underflows or is subnormal, rows large
    enough to saturate the fp16 scale, and rows with exact ties after scaling.
    shape = (B, n, H, d).  Returns bf16 bits or float32 like kv_numpy."""
    rng = np.random.default_rng((99, seed))
    x = rng.standard_normal(shape, dtype=np.float32)
    x[..., 3] *= 20.0
    flat = x.reshape(-1, shape[-1])
    kinds = rng.integers(0, 8, size=flat.shape[0])
    flat[kinds == 1] = 0.0
    flat[kinds == 2] *= np.float32(1e-30)
    flat[kinds == 3] *= np.float32(2.0 ** -18)
    flat[kinds == 4] *= np.float32(3e5)
    ints = rng.integers(-15, 16, size=flat.shape).astype(np.float32) * np.float32(0.5)
    flat[kinds == 5] = ints[kinds == 5]
    x = flat.reshape(shape)
    return to_bf16_bits(x) if dtype == "bf16" else x


def shifted_numpy(seed, shape, dtype="bf16"):
    """adversarial_numpy rows moved off zero: each row gets an offset of up to
    four times its largest magnitude, and one row in eight is constant (a
    block whose range is zero).  shape = (B, n, H, d)."""
    rng = np.random.default_rng((97, seed))
    x = adversarial_numpy(seed, shape, "f32").copy()
    flat = x.reshape(-1, shape[-1])
    spread = np.abs(flat).max(axis=1, keepdims=True)
    flat += rng.uniform(-4, 4, (flat.shape[0], 1)).astype(np.float32) * spread
    const = rng.integers(0, 8, size=flat.shape[0]) == 7
    flat[const] = flat[const, :1]
    x = flat.reshape(shape)
    return to_bf16_bits(x) if dtype == "bf16" else x
