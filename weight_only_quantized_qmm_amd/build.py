"""Build libqmm.so (the C-ABI library of include/qmm.h) for gfx950 with hipcc.

Every library source under csrc/ is compiled for --offload-arch=gfx950 only,
with the packed-fp32 instruction feature switched off, and linked into one
shared library next to this file. The benchmark's measurement kernels
(csrc/qmm_calib.hip: dispatch floor, stream read/copy, MFMA rate) go into a
separate libqmm_calib.so that only bench.py loads. Run
``python -m weight_only_quantized_qmm_amd.build`` or call ``build()``.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libqmm.so")
CALIB_LIB = os.path.join(HERE, "libqmm_calib.so")
OBJDIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + INCLUDE, "-I" + CSRC, "-Wall"]

SOURCES = ["qmm_w4a16_skinny.hip", "qmm_w4a16_wide.hip", "qmm_gemv.hip", "qmm_reduce.hip", "qmm_dense.hip",
           "qmm_attn.hip", "qmm_noalloc.hip", "qmm_api.cpp"]
CALIB_SOURCES = ["qmm_calib.hip"]


def _compile(src, verbose):
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJDIR, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *lang, "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that note is harmless.
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    if out.strip() and verbose:
        print(out, flush=True)
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose=False):
    """Compile every kernel and the host ABI, link libqmm.so and libqmm_calib.so; returns libqmm.so's path."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in CALIB_SOURCES], CALIB_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
