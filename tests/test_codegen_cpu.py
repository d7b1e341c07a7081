"""Code-generation checks on the gfx950 assembly (CPU only, needs hipcc):
every GEMV kernel runs without scratch memory, and no buffer load sits in a
waterfall loop (a descriptor the compiler cannot prove uniform is re-read lane
group by lane group, which multiplies the load count)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gguf_dequant_gemv_amd", "csrc")


def _asm(tu, tmp_path):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if not os.path.exists(hipcc) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path / (tu + ".s")
    cmd = [hipcc if os.path.exists(hipcc) else "hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Wno-unused-command-line-argument", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "--cuda-device-only", "-S", "-o", str(out), os.path.join(CSRC, tu)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernels(asm):
    return {m.group(1): m.group(2) for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", asm, re.S)}


def _bodies(asm):
    out, cur, name = {}, None, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            name, cur = m.group(1), []
            out[name] = cur
        elif cur is not None:
            if line.startswith(".Lfunc_end"):
                cur = None
            else:
                cur.append(line.strip())
    return out


@pytest.mark.parametrize("tu", ["qg_inst_q8_0_t1.hip", "qg_inst_q4_k_t1.hip", "qg_inst_q6_k_t1.hip", "qg_inst_mfma.hip",
                                "qg_gemm.hip", "qg_moe1.hip"])
def test_no_scratch_no_waterfall(tu, tmp_path):
    asm = _asm(tu, tmp_path)
    kern = _kernels(asm)
    assert kern, "no kernels found"
    for name, meta in kern.items():
        scratch = int(re.search(r"private_segment_fixed_size (\d+)", meta).group(1))
        assert scratch == 0, "%s uses %d bytes of scratch" % (name, scratch)
    for name, body in _bodies(asm).items():
        for i, ins in enumerate(body):
            if ins.startswith("buffer_load"):
                window = body[max(0, i - 4):i]
                assert not any(w.startswith("s_and_saveexec") for w in window) or \
                    not any("v_cmp_eq_u64" in w or "v_readfirstlane" in w for w in window), \
                    "%s: buffer load inside a waterfall loop:\n%s" % (name, "\n".join(window + [ins]))
