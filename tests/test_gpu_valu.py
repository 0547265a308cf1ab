"""GPU parity of the vector-ALU decode partition kernel (PKV_DECODE_MATH=valu),
the measured alternative to the matrix-core kernels for FP8 decode with
per-tensor scales and groups of at most eight query heads.

The cases run in a child process (tests/valu_cases.py), since the library
picks its kernels once per process.  Each output must be within the FP8
tolerance of the oracle (max abs error 1e-2, fp16 2e-3), and must differ from
the matrix-core kernels' output on the same inputs where the variant applies
(proof that it ran) or equal it bit for bit where it does not (groups of 16
heads, fp16 caches: those keep the matrix cores).
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import valu_cases  # noqa: E402
from gpu_common import TOL  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def _child(tmp_path, which, timeout):
    env = dict(os.environ, PKV_DECODE_MATH="valu")
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "valu_cases.py"), str(tmp_path),
                        which], env=env, capture_output=True, text=True, timeout=timeout)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stderr[-4000:]
    with open(tmp_path / (which + ".json")) as f:
        return json.load(f)


def _check(tmp_path, cases, errs):
    for name, fn in cases:
        valu = np.load(tmp_path / (name + ".npy"))
        fp8 = not name.startswith("fp16")
        assert errs[name] <= TOL[fp8], (name, errs[name])
        mfma, err = fn()   # this process: the matrix-core kernels
        assert err <= TOL[fp8], (name, err)
        applies = fp8 and "hq16_hkv1" not in name
        same = np.array_equal(valu.view(np.uint32), mfma.view(np.uint32))
        print(f"[valu] {name}: valu err {errs[name]:.3e}, mfma err {err:.3e}, "
              f"bit-identical {same}", flush=True)
        assert same != applies, name


@pytest.mark.timeout(300)
def test_valu_decode_small(tmp_path):
    errs = _child(tmp_path, "small", 280)
    _check(tmp_path, valu_cases.small_cases(), errs)


@pytest.mark.timeout(300)
def test_valu_decode_llama70b_fp8_full(tmp_path):
    errs = _child(tmp_path, "full", 280)
    _check(tmp_path, valu_cases.full_cases(), errs)
