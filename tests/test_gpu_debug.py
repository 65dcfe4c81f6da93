"""Device-side error reports and capture-safety of the library (GPU).

* The bounded wait between workgroups of the fused weight quantisation is made
  to give up from the host (the test hook makes every wait look for a count
  that never arrives, with a tiny spin limit, so every kernel still exits);
  moe4_debug_check must then report it, clear it, and the next call must be
  correct again.
* A routed row index outside its range is clamped by the kernels (no fault)
  and reported the same way.
* The library's first call in a fresh process may be made inside a stream
  capture: its SiLU tables are constant data, so nothing is filled or waited
  for at run time.
"""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest
import torch

from gpu_helpers import assert_bytes_equal, cuda_i32, to_np
from oracle import mxfp8 as mx
from oracle import nvfp4 as nv

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import precision_moe_numerics_quant_amd as m4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_debug_check_clean():
    m4.moe4_debug_check()


# (6, 64, 512) takes the ticketed weight-quantisation kernel, (6, 128, 2048)
# the single-read one; both have a bounded wait
@pytest.mark.parametrize("G,Rg,C", [(6, 64, 512), (6, 128, 2048)])
def test_forced_wait_timeout_is_reported_then_cleared(G, Rg, C):
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((G * Rg, C)) * 0.02).astype(np.float32)
    wt = torch.from_numpy(w).cuda()
    m4.moe4_debug_check()
    m4.moe4_debug_force_wait_timeout(True)
    try:
        print("forced wait timeout: launch", flush=True)
        m4.nvfp4_quant_requant_T(wt, G, seed=3, stream_id=2)
        with pytest.raises(m4.Moe4DeviceError, match="gave up"):
            m4.moe4_debug_check()
    finally:
        m4.moe4_debug_force_wait_timeout(False)
    m4.moe4_debug_check()                      # the report was cleared
    off = np.arange(G + 1) * Rg
    q = nv.nvfp4_quantize(w, nv.MODE_6, off)
    mc_ref, ms_ref = mx.requant_sr_t(q["codes"], q["sf"], q["ts"], off, True, seed=3, stream_id=2)
    codes, sf, ts, mc, ms = m4.nvfp4_quant_requant_T(wt, G, seed=3, stream_id=2)
    assert_bytes_equal(to_np(codes), q["codes"], "codes")
    assert_bytes_equal(to_np(ts).view(np.uint32), np.asarray(q["ts"], np.float32).view(np.uint32), "ts")
    assert_bytes_equal(to_np(mc), mc_ref, "mx codes")
    assert_bytes_equal(to_np(ms), ms_ref, "mx scales")
    m4.moe4_debug_check()


def test_clamped_index_is_reported():
    T, k, d = 16, 2, 64
    codes = torch.zeros((T, d // 2), dtype=torch.uint8, device="cuda")
    sf = torch.zeros((T, d // 16), dtype=torch.uint8, device="cuda")
    perm = np.arange(T * k, dtype=np.int32)
    m4.moe4_debug_check()
    m4.moe_gather_rows(codes, sf, cuda_i32(perm), k)
    m4.moe4_debug_check()                      # in range: no report
    perm[5] = T * k + 40                       # past the source rows: clamped to the last row
    m4.moe_gather_rows(codes, sf, cuda_i32(perm), k)
    with pytest.raises(m4.Moe4DeviceError, match="clamped"):
        m4.moe4_debug_check()
    yp = torch.ones((T * k, d), dtype=torch.float32, device="cuda")
    gates = torch.full((T, k), 0.5, dtype=torch.float32, device="cuda")
    inv = np.arange(T * k, dtype=np.int32)
    inv[3] = -7
    y = m4.moe_combine(yp, gates, cuda_i32(inv))
    with pytest.raises(m4.Moe4DeviceError, match="clamped"):
        m4.moe4_debug_check()
    assert torch.all(y.float() == 1.0)         # clamped to row 0, whose values are the same
    m4.moe4_debug_check()


_FIRST_CALL_CAPTURED = textwrap.dedent("""
    import sys
    sys.path.insert(0, {root!r})
    import numpy as np
    import torch
    import precision_moe_numerics_quant_amd as m4
    torch.cuda.set_device(0)
    g = torch.Generator(device="cuda").manual_seed(5)
    u = (torch.randn((256, 512), generator=g, device="cuda") * 3).to(torch.bfloat16)
    off = torch.tensor([0, 100, 100, 256], dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            # the first library call of this process, inside the capture
            codes, sf, ts = m4.nvfp4_quant_46(u, m4.NVFP4_4OVER6, off, m4.PRE_SILU)
            sv, dv = m4.moe_silu_eval(u)
    outs = []
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (codes, sf, ts, sv, dv)])
        m4.nvfp4_quant_46(u * 2, m4.NVFP4_4OVER6, off, m4.PRE_SILU)   # eager work between replays
        torch.cuda.synchronize()
    ref = list(m4.nvfp4_quant_46(u, m4.NVFP4_4OVER6, off, m4.PRE_SILU)) + list(m4.moe_silu_eval(u))
    torch.cuda.synchronize()
    for o in outs:
        for a, b in zip(o, ref):
            assert torch.equal(a, b)
    m4.moe4_debug_check()
    print("FIRST_CALL_CAPTURED_OK")
""")


def test_first_library_call_inside_graph_capture():
    """In a fresh process, the library's first call is captured; three replays
    (eager calls and syncs between them) equal the eager results byte for byte."""
    print("subprocess: first library call under capture", flush=True)
    r = subprocess.run([sys.executable, "-c", _FIRST_CALL_CAPTURED.format(root=ROOT)], capture_output=True,
                       text=True, timeout=100)
    assert r.returncode == 0 and "FIRST_CALL_CAPTURED_OK" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
