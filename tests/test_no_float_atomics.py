"""Audit of the library's own GPU code: every HIP source is compiled to gfx950 assembly (this
build, on this machine) and no floating-point atomic instruction may appear. The combine and
every reduction sum in a fixed order instead, which is what makes two runs bit-identical."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from mixture_experts_ffn_ids_amd import build as moe_build

FLOAT_ATOMIC = re.compile(r"\b(?:global|flat|buffer|ds)_(?:atomic_)?(?:pk_)?(?:add|sub|min|max)(?:_rtn)?_"
                          r"(?:f16|bf16|f32|f64)\b")
ANY_ATOMIC = re.compile(r"\b(?:global|flat|buffer)_atomic_\w+|\bds_(?:add|sub|inc|dec|min|max|and|or|xor|"
                        r"cmpst|wrxchg)\w*")


def _asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.splitext(os.path.basename(src))[0] + ".s")
    cmd = [moe_build.hipcc(), *moe_build.common_flags(), "--cuda-device-only", "-S", src, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_no_float_atomics_in_device_code():
    srcs = [os.path.join(moe_build.CSRC, s) for s in moe_build.SOURCES]
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(len(srcs)) as ex:
            outs = list(ex.map(lambda s: _asm(s, tmp), srcs))
        found, atomics = {}, {}
        for src, out in zip(srcs, outs):
            text = open(out).read()
            assert "v_mfma" in text or "gemm" not in src, f"{src}: no matrix ops compiled"
            hits = sorted(set(FLOAT_ATOMIC.findall(text)))
            if hits:
                found[os.path.basename(src)] = hits
            a = sorted(set(m.group(0) for m in ANY_ATOMIC.finditer(text)))
            if a:
                atomics[os.path.basename(src)] = a
        assert not found, f"floating-point atomics in device code: {found}"
        # the only atomics at all are integer ones in the dispatch (counting)
        assert set(atomics) <= {"dispatch.hip"}, atomics


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_the_audit_sees_planted_atomics():
    # a float atomic add in both of its compiled forms: the hardware instruction and the
    # compare-and-swap loop that plain atomicAdd on a float becomes
    src = ("#include <hip/hip_runtime.h>\n"
           "__global__ void k(float* p, float v) { unsafeAtomicAdd(p, v); atomicAdd(p + 1, v); }\n")
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "planted.hip")
        with open(path, "w") as f:
            f.write(src)
        text = open(_asm(path, tmp)).read()
    assert FLOAT_ATOMIC.search(text)
    assert ANY_ATOMIC.search(text)
