"""The compile-time variants of the HIP sources (4-wave tile, ping-pong stage
schedule, ring of four 32-k stages, the 32x32x16 MFMA tile) still type-check for gfx950: a device-side
syntax pass instantiates every kernel template, so a static assertion or a
template error in a variant's path fails here (about a second each)."""
import os
import subprocess

import pytest

from sync_protocols_amd import build as B


@pytest.mark.parametrize("define", ["-DFG_WAVES=4", "-DFG_PINGPONG=1", "-DFG_BK=32", "-DFG_MFMA16=0"])
def test_variant_type_checks(define):
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc is not available")
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    r = subprocess.run([B.HIPCC, *flags, define, "--cuda-device-only", "-fsyntax-only", *B.SOURCES],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
