"""The GPU parity suites against the LDS-poisoning debug build of the
library (``libgqa_ldspoison.so``, built by ``build()`` with GQA_LDS_POISON:
every kernel first fills its LDS arrays with all-ones bits, a NaN as fp32 and
as bf16, before any load lands).  A kernel that reads LDS that nothing in its
workgroup wrote then turns the affected outputs into NaN, which the
element-wise comparisons with the oracle reject.  The suites run in a child
process that loads the debug library through GQA_LIB (the binding loads one
library per process)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
POISON = os.path.join(ROOT, "transformer_attention_layer_amd", "libgqa_ldspoison.so")
SUITES = ["tests/test_gpu_parity.py", "tests/test_gpu_fp8.py", "tests/test_gpu_backward.py"]


@pytest.mark.gpu
def test_parity_suites_with_poisoned_lds():
    assert os.path.exists(POISON), "build() makes libgqa_ldspoison.so next to libgqa.so"
    env = dict(os.environ, GQA_LIB=POISON)
    # the child's binding loads the debug build (it alone exports the marker)
    probe = ("import transformer_attention_layer_amd as T; "
             "assert T.lib().gqa_lds_poison_build() == 1; print(T.LIB_PATH)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and POISON in r.stdout, r.stderr[-2000:]
    cmd = [sys.executable, "-u", "-m", "pytest", *SUITES, "-m", "gpu", "-x", "-q",
           "-p", "no:cacheprovider", "--timeout", "300", "--timeout-method", "thread"]
    print("[lds poison] " + " ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    print(r.stdout[-4000:])
    print(r.stderr[-2000:])
    assert r.returncode == 0, "a parity suite failed on the LDS-poisoning build"
