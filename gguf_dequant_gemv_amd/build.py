"""Build libqgemv.so (the HIP library) in-tree for gfx950.

    python -m gguf_dequant_gemv_amd.build

hipcc compiles for gfx950 only.  Packed-FP32 instruction selection is turned
off for the device code (-packed-fp32-ops); the host pass warns that it does
not know that feature, which is harmless.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqgemv.so")
SOURCES = [os.path.join(CSRC, f) for f in
           ["qg_abi.hip", "qg_route.hip", "qg_block.hip", "qg_gemm.hip", "qg_moe1.hip", "qg_kq1.hip", "qg_planes.hip", "qg_inst_dequant.hip", "qg_inst_mfma.hip"] +
           ["qg_inst_%s_t%d.hip" % (t, n) for t in ("q8_0", "q4_0", "q4_k", "q6_k") for n in (1, 2, 4, 8)]]
DEPS = SOURCES + [os.path.join(CSRC, f) for f in ("qg_device.h", "qg_kernels.h", "qg_inst.h", "qg_block.h", "qg_moe1.h", "qg_down1.h", "qg_kq1.h", "qg_planes.h")] + [
    os.path.join(os.path.dirname(HERE), "include", "qgemv.h")]
OBJDIR = os.path.join(HERE, "_build")


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Werror",
         "-Wno-unused-command-line-argument",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, msg


def build(verbose=False, jobs=None):
    """Compile each translation unit to an object in parallel, then link."""
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, os.path.basename(src) + ".o") for src in SOURCES]
    cmds = [[hipcc()] + FLAGS + ["-c", src, "-o", obj] for src, obj in zip(SOURCES, objs)]
    jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1), 16)
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, msg), src in zip(results, SOURCES):
        if rc != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, msg))
        if verbose and msg.strip():
            print(msg)
    tmp = LIB + ".tmp"
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(link), flush=True)
    rc, msg = _run(link)
    if rc != 0:
        raise RuntimeError("link failed:\n" + msg)
    os.replace(tmp, LIB)
    return LIB


def stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
