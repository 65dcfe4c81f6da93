"""The library's constant SiLU / SiLU' tables (written at build time by
csrc/gen_act_tab.cpp) equal the oracle's correctly rounded values, bit for bit,
for every bf16 value the tables cover (|u| in [2**-16, 2**8)); runs on the CPU."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import formats as fmt
from oracle import silu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEN = os.path.join(ROOT, "precision_moe_numerics_quant_amd", "csrc", "gen_act_tab.cpp")


def test_generated_tables_match_oracle(tmp_path):
    cxx = shutil.which(os.environ.get("CXX", "g++"))
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "gen")
    subprocess.run([cxx, "-O2", "-std=c++17", "-o", exe, GEN], check=True)
    text = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    vals = [float.fromhex(tok.strip()[:-1]) for line in text.splitlines() if not line.startswith("/*")
            for tok in line.split(",") if tok.strip()]
    n = 6144
    assert len(vals) == 2 * n
    got = np.array(vals, dtype=np.float64).astype(np.float32).reshape(2, n)
    assert np.array_equal(got.astype(np.float64), np.array(vals).reshape(2, n))   # literals are float32 values
    # index i: sign i // 3072; in the half, binade (i % 3072) >> 7 above 2**-16 and mantissa i & 127
    i = np.arange(n, dtype=np.uint32)
    bits = (((i // 3072) << 15) | ((((i % 3072) >> 7) + 111) << 7) | (i & 127)).astype(np.uint16)
    u = fmt.bf16_to_f32(bits)
    assert np.all((np.abs(u) >= 2.0 ** -16) & (np.abs(u) < 2.0 ** 8))
    # every bf16 magnitude in range once per sign
    assert len(np.unique(bits)) == n and np.count_nonzero(bits >> 15) == n // 2
    assert np.array_equal(got[0].view(np.uint32), silu.silu_f32(bits).view(np.uint32))
    assert np.array_equal(got[1].view(np.uint32), silu.dsilu_f32(bits).view(np.uint32))
