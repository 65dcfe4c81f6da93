"""The library's constant SiLU / SiLU' tables (written at build time by
csrc/gen_act_tab.cpp) equal the oracle's correctly rounded values, bit for bit,
for every bf16 value the tables cover (|u| in [2**-8, 2**8)); runs on the CPU."""
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
    assert len(vals) == 2 * 4096
    got = np.array(vals, dtype=np.float64).astype(np.float32).reshape(2, 4096)
    assert np.array_equal(got.astype(np.float64), np.array(vals).reshape(2, 4096))   # literals are float32 values
    # index i: sign bit i >> 11, binade (i >> 7) & 15 above 2**-8, mantissa i & 127
    i = np.arange(4096, dtype=np.uint32)
    bits = (((i >> 11) << 15) | ((((i >> 7) & 15) + 119) << 7) | (i & 127)).astype(np.uint16)
    u = fmt.bf16_to_f32(bits)
    assert np.all((np.abs(u) >= 2.0 ** -8) & (np.abs(u) < 2.0 ** 8))
    assert np.array_equal(got[0].view(np.uint32), silu.silu_f32(bits).view(np.uint32))
    assert np.array_equal(got[1].view(np.uint32), silu.dsilu_f32(bits).view(np.uint32))
