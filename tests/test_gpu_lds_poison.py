"""The LDS-poisoning debug build against the release build, bit for bit.

libgdr_poison.so is the library built with -DGDR_LDS_POISON: every kernel fills its LDS with
0xFF bytes (a NaN in bfloat16 and float32) at entry, the scans refill it between chunk steps,
and the chunk kernels poison each LDS region at the point where its contents die.  A kernel
that reads LDS it never wrote (or dead contents) would get NaN there, where the release build
gets whatever the CU's previous workgroup left behind.  Every case in tests/_poison_cases.py
(all variants, both I/O types, packed sequences with an empty one, gate logits, q/k
normalisation, residual outputs, decode, 32-row scan tiles, forced segments, the time-split
backward) runs forward and backward through both builds: the debug build in a child process (a
process loads one build), the release build here.  The results must be finite and identical.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

from gated_delta_rule_73_amd import build as gbuild
from tests import _poison_cases as PC

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def poisoned(tmp_path_factory):
    lib = gbuild.POISON_LIB
    assert os.path.exists(lib), f"{lib} is missing: build it with `python -m gated_delta_rule_73_amd.build`"
    out = str(tmp_path_factory.mktemp("poison") / "poisoned.npz")
    env = dict(os.environ)
    env["GDR_LIBRARY"] = lib
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    for k in ("GDR_SCAN_BV", "GDR_SEG_CHUNKS", "GDR_PIPELINE", "GDR_TSPLIT_CHUNKS"):
        env.pop(k, None)
    r = subprocess.run([sys.executable, "-m", "tests._poison_cases", out], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    with np.load(out) as z:
        return {k: z[k] for k in z.files}


@pytest.mark.parametrize("case", PC.CASES, ids=[c["name"] for c in PC.CASES])
def test_poisoned_build_matches_release(poisoned, case):
    got = PC.run_case(case)
    assert got, case["name"]
    for name, rel in got.items():
        key = f"{case['name']}/{name}"
        assert key in poisoned, key
        dbg = poisoned[key]
        assert np.isfinite(dbg).all(), f"{key}: the LDS-poisoned build returned NaN or Inf"
        assert np.isfinite(rel).all(), f"{key}: the release build returned NaN or Inf"
        assert dbg.shape == rel.shape, key
        bad = np.flatnonzero(dbg.view(np.uint32) != rel.view(np.uint32)) if dbg.dtype == np.float32 else \
            np.flatnonzero(dbg != rel)
        assert bad.size == 0, f"{key}: {bad.size} elements differ from the release build (first {bad[:8]})"
