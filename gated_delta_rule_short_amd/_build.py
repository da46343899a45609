"""Build libkda.so (HIP, gfx950) in-tree with hipcc.

Each .hip source is compiled to an object in parallel, then linked into
gated_delta_rule_short_amd/libkda.so.  Packed-fp32 instruction selection is
disabled for all device code (-packed-fp32-ops).  Matrix-core instructions are
kept in their VGPR form (-amdgpu-mfma-vgpr-form): on gfx950 a 16x16x32 bf16
result held in AGPRs needs about eight wait states before v_accvgpr_read sees
all of it, which is exactly the padding the compiler emits, and a read at that
distance returned stale rows behind an interleaved MFMA; the VGPR form is read
fresh after five.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.hip", "kda_conv.hip", "kda_decode.hip", "kda_gate_proj.hip", "kda_pool.hip",
           "kda_prefill.hip", "kda_prefill_split.hip"]
# measurement-only streaming kernels (include/kda_calib.h), a library of their own
CALIB_LIB = os.path.join(PKG, "libkda_calib.so")
CALIB_SOURCES = ["kda_calib.hip"]
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


# Sources whose matrix-core results must stay in VGPRs (see the module docstring).
# The one-pass prefill is left to the default heuristic: the compiler does not
# build it with the VGPR form forced.
VGPR_FORM = {"kda_prefill_split.hip"}


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    extra = ["-mllvm", "-amdgpu-mfma-vgpr-form"] if src in VGPR_FORM else []
    cmd = [hipcc()] + flags() + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag: drop that line
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
    return obj, err


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        results = dict(zip(srcs, ex.map(_compile, srcs)))
    for obj, err in results.values():
        if verbose and err.strip():
            print(err)
    _link([results[s][0] for s in SOURCES], LIB)
    _link([results[s][0] for s in CALIB_SOURCES], CALIB_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
