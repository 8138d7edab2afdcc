"""Build libkvq.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc,
and libkvq_stream.so (the benchmark's streaming-bandwidth kernels).

    python -m kv_cache_quantization_quantize_amd.build

Every translation unit is compiled for gfx950 only, at -O3, with packed-FP32
instruction selection disabled (-packed-fp32-ops) and IEEE-conformant fp32
(no fast-math), then linked into kv_cache_quantization_quantize_amd/libkvq.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libkvq.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["kvq_int4.hip", "kvq_vq.hip", "kvq_attend.hip", "kvq_kmeans.hip", "kvq_api.cpp"]
# practical-bandwidth kernels of the benchmark, in a library of their own
STREAM_SOURCES = ["kvq_stream.hip"]
STREAM_OUT = os.path.join(HERE, "libkvq_stream.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-ffp-contract=fast",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-file extra flags.  The VQ search takes maxima of MFMA results; without
# -fno-honor-nans every fmaxf first canonicalises its (possibly signalling-NaN)
# inputs.  Non-finite inputs are outside the library's documented domain.
# The attention kernel rescales its MFMA accumulators on the VALU; keeping
# MFMA operands and results in VGPRs (rather than AGPRs) avoids copying the
# accumulators between the two register files every step.
EXTRA = {"kvq_vq.hip": ["-fno-honor-nans"],
         "kvq_attend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _up_to_date(src: str, obj: str) -> bool:
    """The object is newer than its source and every header it may include."""
    if not os.path.exists(obj):
        return False
    deps = [os.path.join(CSRC, src), os.path.join(ROOT, "include", "kvq.h")]
    deps += [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    t = os.path.getmtime(obj)
    return all(os.path.getmtime(d) < t for d in deps)


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    if incremental and _up_to_date(src, obj):
        return obj
    lang = ["-x", "hip"]
    cmd = [HIPCC, *lang, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on %s" % src)
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of %s failed" % os.path.basename(out))
    os.replace(tmp, out)


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (incremental: only those whose object is older
    than the source or a header), link libkvq.so, and link the benchmark's
    streaming-bandwidth kernels into libkvq_stream.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(STREAM_SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, incremental), SOURCES + STREAM_SOURCES))
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], STREAM_OUT)
    if verbose:
        print("built", OUT, "and", STREAM_OUT)
    return OUT


def asm(src: str = "kvq_int4.hip", out: str | None = None) -> str:
    """Device assembly of one source (for inspecting register use and ISA)."""
    out = out or os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".s")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = [HIPCC, "-x", "hip", *COMMON, *EXTRA.get(src, []), "--cuda-device-only", "-S", os.path.join(CSRC, src),
           "-o", out]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
