"""Build libkvq.so (HIP for gfx950) in-tree, compiling translation units in
parallel.  Usage: python -m decode_attention_rotate_amd.build [--jobs N]."""

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvq.so")
# read-bandwidth probes for the benchmark (include/kvq_ceiling.h), a library
# of their own so the attention library holds only the attention path
CEILING_LIB = os.path.join(PKG, "libkvq_ceiling.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall",
    # bit-exact quantizer: IEEE float32, no contraction of a*b+c into fma
    "-ffp-contract=off",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]
DEVICE = [
    "--offload-arch=" + ARCH,
    # never emit packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# head_dim 256, and head_dim 192 with scale-and-min blocks or prefill rows,
# run one wave per SIMD with all 512 registers: left to itself the compiler
# puts the matrix products' results in AGPRs and moves every one to a VGPR
# (and the P.V accumulators back and forth each step), 89 of 693 vector
# instructions per step at head_dim 256.  Results kept in VGPRs measured about
# 5% faster at head_dim 256 (131k tokens) and 5-9% at head_dim 192 (64k
# tokens, q4_1 V / q5_1 K).  Kernels at two waves per SIMD use no AGPRs and
# compile the same either way.
VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form"]


def units():
    """(source, object, extra flags) for every translation unit."""
    out = []
    for name in ("append.hip", "dequant.hip", "decode_main.hip", "prefill_mfma.hip"):
        out.append((os.path.join(CSRC, name), name.replace(".hip", ".o"), DEVICE))
    # K formats: (bits, scale-and-min) for q4_0 q5_0 q6_0 q8_0 q4_1 q5_1
    # (head_dim 256 also builds its paged-layout kernels as units of their own)
    for d, paged in ((256, 0), (256, 1), (192, 0), (128, 0), (64, 0)):   # the slowest first
        for kb, km in ((4, 0), (5, 0), (6, 0), (8, 0), (4, 1), (5, 1)):
            out.append((os.path.join(CSRC, "decode_inst.hip"),
                        "decode_d%d_k%d_m%d%s.o" % (d, kb, km, "_paged" if paged else ""),
                        DEVICE + ["-DKVQ_INST_D=%d" % d, "-DKVQ_INST_KB=%d" % kb,
                                  "-DKVQ_INST_KM=%d" % km] + (["-DKVQ_INST_PAGED=1"] if paged else [])
                        + (VGPR_MFMA if d >= 192 else [])))
    out.append((os.path.join(CSRC, "kvq_host.cpp"), "kvq_host.o", DEVICE + ["-x", "hip"]))
    return out


def _sources_newer(obj_path):
    """True when any source or header of the library is newer than obj_path."""
    if not os.path.exists(obj_path):
        return True
    t = os.path.getmtime(obj_path)
    srcs = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(ROOT, "include", "kvq.h")]
    return any(os.path.getmtime(f) > t for f in srcs)


def _compile(job, incremental=False):
    src, obj, extra = job
    if incremental and not _sources_newer(os.path.join(BUILD, obj)):
        return obj, 0, "", []
    cmd = [HIPCC] + COMMON + extra + ["-c", src, "-o", os.path.join(BUILD, obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("unknown target feature", "packed-fp32-ops", "warning generated")
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if l.strip() and not any(n in l for n in noise))
    return obj, r.returncode, msgs, cmd


# Host-side sanitizer check of the C ABI (tests/asan/capi_check.cpp): the
# library's host code built with AddressSanitizer and UBSan, linked with the
# uninstrumented kernel objects; run by tests/test_capi_sanitizers.py.
SAN_BIN = os.path.join(BUILD, "kvq_capi_asan")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LINK = ["-fsanitize=address,undefined", "-fno-gpu-sanitize"]


def build_sanitizer_check(objs):
    """Compile the host file and the check program with the sanitizers and
    link them with the other objects into SAN_BIN."""
    host = os.path.join(BUILD, "kvq_host_asan.o")
    drv = os.path.join(BUILD, "capi_check_asan.o")
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    steps = [
        [HIPCC] + flags + DEVICE + SAN_HOST + ["-x", "hip", "-c", os.path.join(CSRC, "kvq_host.cpp"), "-o", host],
        [HIPCC] + flags + SAN_HOST + ["-c", os.path.join(ROOT, "tests", "asan", "capi_check.cpp"), "-o", drv],
        [HIPCC, "--offload-arch=" + ARCH] + SAN_LINK + ["-o", SAN_BIN, drv, host] + objs,
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("sanitizer check build failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    return SAN_BIN


def build(jobs=None, verbose=False, only=None, incremental=False):
    """Compile every unit and link libkvq.so; raises on any failure.
    only: compile just the units whose object name contains this string
    (the others must already be built); incremental: skip units whose
    object is newer than every source (development builds)."""
    if not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found at %s" % HIPCC)
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(16, os.cpu_count() or 4)
    failed = []
    todo = [u for u in units() if only is None or any(o in u[1] for o in only.split(","))]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for obj, rc, msgs, cmd in ex.map(lambda u: _compile(u, incremental), todo):
            if rc != 0:
                failed.append((obj, msgs, cmd))
            elif verbose and msgs:
                print("[%s]\n%s" % (obj, msgs))
    if failed:
        raise RuntimeError("\n\n".join("%s failed:\n%s\n%s" % (o, " ".join(c), m) for o, m, c in failed))
    objs = [os.path.join(BUILD, o) for _, o, _ in units()]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    shutil.move(tmp, LIB)
    tmp = CEILING_LIB + ".tmp"
    cmd = [HIPCC] + COMMON + DEVICE + ["-shared", os.path.join(CSRC, "ceiling.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("ceiling library failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    shutil.move(tmp, CEILING_LIB)
    build_sanitizer_check([o for o in objs if not o.endswith("kvq_host.o")])
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--only", default=None, help="compile only units whose object name contains one of these (comma-separated)")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose, only=args.only))


if __name__ == "__main__":
    sys.exit(main())
