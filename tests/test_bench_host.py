"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the traffic
summary of two counter passes and its guard on the kernel's source, and the
algorithmic work of the calls."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def _csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, v in rows:
            f.write(f'"{name}",{counter},{v}\n')


def test_pmc_summary_scales_by_the_copy(tmp_path):
    # the copy reads and writes 1 GiB; its counters read half / all of it, so
    # the kernel's readings scale by 2 (fetch) and 1 (write)
    kib = (1 << 30) / 1024
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    # (the run's three calibration copies are its largest copy dispatches; a
    # small copy elsewhere in the run does not count)
    # (the two tiny dispatches stand for the tiny layer's launches of the same
    # kernel, which the summary leaves out)
    _csv(f, "FETCH_SIZE", [("k_wgrad_ws256(args)", 1000.0), ("k_wgrad_ws256(args)", 3000.0),
                           ("k_wgrad_ws256(args)", 2.0),
                           ("__amd_rocclr_copyBuffer", 10.0)] + [("__amd_rocclr_copyBuffer", kib / 2)] * 3)
    _csv(w, "WRITE_SIZE", [("k_wgrad_ws256(args)", 4000.0), ("k_wgrad_ws256(args)", 4000.0),
                           ("k_wgrad_ws256(args)", 3.0),
                           ("__amd_rocclr_copyBuffer", 20.0)] + [("__amd_rocclr_copyBuffer", kib)] * 3)
    out = bench.pmc_summary(str(f), str(w), "k_wgrad_ws256")
    vals = dict(line[2:].split(" = ", 1) for line in out.strip().splitlines())
    assert float(vals["copy_fetch_factor"]) == 0.5 and float(vals["copy_write_factor"]) == 1.0
    fetch = float(vals["hbm_fetch_bytes_per_launch"])
    write = float(vals["hbm_write_bytes_per_launch"])
    assert abs(fetch - 2000.0 * 1024 / 0.5) / fetch < 1e-3
    assert abs(write - 4000.0 * 1024) / write < 1e-3


def test_traffic_only_for_the_profiled_source(monkeypatch):
    kernel = "k_wgrad_ws256"
    prof, src = bench.PMC_PROFILE[kernel]
    assert os.path.exists(os.path.join(ROOT, prof)) and os.path.exists(os.path.join(ROOT, src))
    real = bench.source_sha256
    monkeypatch.setattr(bench, "source_sha256", lambda rel: "0" * 64)
    assert bench.pmc_traffic(kernel) is None          # a changed kernel: no figure
    monkeypatch.setattr(bench, "source_sha256", real)
    assert bench.pmc_traffic("not_profiled") is None


def test_work_table_matches_the_formulas():
    c = synth.CONFIGS[4]
    E, T, k, d, F = c["E"], c["T"], c["k"], c["d"], c["F"]
    rng = np.random.default_rng(0)
    counts = rng.multinomial(T * k, np.ones(E) / E)
    off = np.concatenate([[0], np.cumsum(counts)])
    off_pad = np.concatenate([[0], np.cumsum((counts + 31) // 32 * 32)])
    t = bench.work_table(c, off, off_pad)
    gemm = 2.0 * T * k * d * F
    for name in ("F6 up GEMM (NVFP4)", "F8 down GEMM (NVFP4)", "B3 down dgrad (MXFP8)", "B8 up dgrad (MXFP8)"):
        assert t[name][1] == gemm
    P = off_pad[-1]
    wg = E * d * F * 4 + (d + F) * P * 33 / 32
    assert abs(t["B5 down wgrad (MXFP8)"][2] - wg) / wg < 1e-12
    assert abs(t["B10 up wgrad (MXFP8)"][2] - wg) / wg < 1e-12
    assert t["F9 combine"][1] == T * k * d * 4 + T * d * 2 + T * k * 8   # Yp rows, y, gates + indices


def test_wgrad_work_counts_only_active_experts():
    """The weight gradients of experts without tokens are not written: the
    wgrad's algorithmic bytes count the active experts' dW only."""
    c = synth.CONFIGS[4]
    E, d, F = c["E"], c["d"], c["F"]
    counts = np.zeros(E, dtype=np.int64)
    counts[:100] = c["T"] * c["k"] // 100
    counts[0] += c["T"] * c["k"] - counts.sum()
    off = np.concatenate([[0], np.cumsum(counts)])
    off_pad = np.concatenate([[0], np.cumsum((counts + 31) // 32 * 32)])
    t = bench.work_table(c, off, off_pad)
    wg = 100 * d * F * 4 + (d + F) * off_pad[-1] * 33 / 32
    assert abs(t["B5 down wgrad (MXFP8)"][2] - wg) / wg < 1e-12


def test_trace_summary_keeps_the_layer_shape_launches(tmp_path):
    p = tmp_path / "kt.csv"
    with open(p, "w") as f:
        f.write("Kind,Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for dur_ns in (4_000_000, 4_200_000, 7_000, 6_000):           # two layer launches, two tiny ones
            f.write(f'KERNEL_DISPATCH,"moe4::k_encode_requant_T(float const*)",1000,{1000 + dur_ns}\n')
        f.write('KERNEL_DISPATCH,"moe4::k_wgrad_ws256(unsigned char const*)",0,2000000\n')
    out = bench.trace_summary(str(p))
    row = [line for line in out.splitlines() if "k_encode_requant_T" in line][0]
    cells = [x.strip() for x in row.strip("|").split("|")]
    assert cells[1] == "4" and cells[2] == "2" and abs(float(cells[3]) - 4100.0) < 1e-6
    assert abs(float(cells[4]) - 4100.0) < 1e-6                              # median of the two
