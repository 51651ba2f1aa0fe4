"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer: built into a temporary
folder with -fsanitize=address,undefined (no recovery) and driven from a child Python process
through every entry point on small inputs, including the error paths. Any invalid access or
undefined operation aborts the child."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

CHILD = r'''
import sys
sys.path.insert(0, ROOT)
import numpy as np
import oracle
oracle._LIB_PATH = LIB
from workloads import Config, make_routing, make_x_bits
from workloads.gen import make_block_inputs, make_experts_host, make_shared_host

cfg = Config("san", 24, 256, 128, 6, 2, "normal", "uniform", "softmax", True, seed=61)
x = make_x_bits(cfg)
ids, w = make_routing(cfg)
ex, sh = make_experts_host(cfg), make_shared_host(cfg)
h, g = make_block_inputs(cfg)
oracle.dispatch(ids, cfg.E)
assert oracle._load()._name == LIB, oracle._load()._name
oracle.moe_forward(x, ids, w, ex, sh, threads=1)
oracle.moe_forward(x, ids, w, ex, None, tokens=np.array([3, 0, 23]), threads=1, residual=h)
oracle.expert_rows(x, ex, np.array([1, 2]), np.array([0, 5]), threads=1)
oracle.rmsnorm_rows(h, g, 1e-6)
oracle.quant_rows_bf16(x)
oracle.e4m3_encode(np.linspace(-500, 500, 1001).astype(np.float32))
bad = ids.copy(); bad[0, 0] = cfg.E
for a in (bad, np.where(np.arange(ids.size).reshape(ids.shape) == 1, ids[0, 0], ids)):
    try:
        oracle.moe_forward(x, a, w, ex, threads=1)
    except oracle.OracleError:
        pass
    else:
        raise SystemExit("bad ids not rejected")
print("sanitized-ok")
'''


def _run_sanitized(src_text: str):
    """Build the given oracle source with ASan + UBSan and run the child on it."""
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan runtime not found")
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "moe_oracle.c")
        with open(src, "w") as f:
            f.write(src_text)
        lib = os.path.join(tmp, "liboracle_san.so")
        subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-std=c11", "-shared", "-fPIC",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                        src, "-o", lib, "-lm"], check=True)
        env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")
        code = f"ROOT = {ROOT!r}\nLIB = {lib!r}\n" + CHILD
        return subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan():
    r = _run_sanitized(open(SRC).read())
    assert r.returncode == 0 and "sanitized-ok" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_the_sanitized_run_catches_a_planted_overrun():
    # the harness itself: one element past each quantisation group is read, and the run aborts
    text = open(SRC).read()
    planted = text.replace("for (int i = 0; i < n; ++i) {\n        float a = fabsf(v[i]);",
                           "for (int i = 0; i <= n; ++i) {\n        float a = fabsf(v[i]);", 1)
    assert planted != text
    r = _run_sanitized(planted)
    assert r.returncode != 0 and "sanitized-ok" not in r.stdout
