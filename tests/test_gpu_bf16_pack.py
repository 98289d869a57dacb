"""The Newton-Schulz B X kernel packs X' to bf16 with gfx950's
v_cvt_pk_bf16_f32.  A helper program (tests/helpers/bf16_cvt_check.hip, built
by __graft_entry__.build()) runs that instruction on every fp32 bit pattern
and compares it with the integer round-to-nearest-even of the write-back
kernels: no difference on any non-NaN input, and NaN stays NaN."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "helpers", "_build",
                   "bf16_cvt_check")


def test_hardware_bf16_pack_is_round_to_nearest_even():
    assert os.path.exists(EXE), "run __graft_entry__.build() first"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("non-NaN differences 0 "), r.stdout
