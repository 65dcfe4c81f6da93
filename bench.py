"""Benchmark of the NVFP4-forward / MXFP8-backward MoE expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch: NVFP4 weight
quantisation of the fp32 masters (with, in the same pass, the weights' SR
transposed MXFP8 copies for the backward), routing and permutation, X
quantisation (4/6), dispatch gather, up GEMM, SiLU + H quantisation (4/6),
down GEMM, combine; then the backward: gradient MXFP8 quantisation (row-wise
and transposed), the SR requantisations of H and X, dgrad and wgrad grouped
GEMMs for both projections, dU quantisation with SiLU', un-permuting sum,
gate gradient and the router backward into the logits.  Workload: T = 16384 tokens,
d = 4096, F = 1536, 384 experts, top-8 routing from N(0,1) logits with a
Zipf(1.1) expert bias; upstream gradient N(0, 1e-3); synthetic seeded inputs
resident in HBM before the timed region.

The same layer with an MXFP8 forward (the pages' higher-precision layers,
and their full-MXFP8 baseline) is timed on the same inputs afterwards and
reported under `mxfp8_forward_variant`.

Printed: one JSON line.  `value` is the step's grouped-GEMM work (6 GEMMs,
2*M*N*K each, padding excluded) divided by the whole step time; the
per-call breakdown (HIP events recorded on the stream the library launches
on) gives every GEMM's TFLOP/s and every quantiser's GB/s with the fraction
of MI355X's peak; `roofline` is the dominant call's.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_F16 = 2.5e15          # dense FP16/BF16 MFMA, FLOP/s
PEAK_FP8 = 5.0e15
PEAK_FP4 = 10.1e15
CFG_ID = 4                 # layer forward + backward at T=16384, d=4096, F=1536, E=384, k=8


def work_table(c, off, off_pad):
    """Algorithmic work of every step call: (kind, amount, peak, extra)."""
    T, d, F, E, k = c["T"], c["d"], c["F"], c["E"], c["k"]
    A = T * k
    Ptot = int(off_pad[-1])
    nv = 9.0 / 16.0            # NVFP4 bytes per element (codes + E4M3 scales)
    mxb = 33.0 / 32.0          # MXFP8 bytes per element (codes + E8M0 scales)
    gem = 2.0 * A * d * F
    # wgrad: the active experts' float32 dW (experts without tokens are not
    # written: the step skips their zero-fill by contract) + both operands
    E_act = int((np.diff(np.asarray(off)) > 0).sum())
    wg_bytes = lambda n1, n2: E_act * n1 * n2 * 4.0 + (n1 + n2) * Ptot * mxb
    return {
        # one fp32 read (each expert matrix stays in registers from its amax to
        # its encode), the NVFP4 write and the backward's MXFP8 copy
        "F1 W_up quant (+ requant)": ("hbm", E * F * d * (4.0 + nv + mxb)),
        "F1 W_down quant (+ requant)": ("hbm", E * F * d * (4.0 + nv + mxb)),
        "F2-F3 route + permutation": ("hbm", T * E * 4.0 + A * 16.0),
        "F4 X quant (NVFP4 4/6)": ("hbm", T * d * (4.0 + nv)),
        "F5 dispatch gather": ("hbm", 2.0 * A * d * nv),
        "F6 up GEMM (NVFP4)": ("f16", gem),
        # (the per-expert SiLU amax is folded into F6's epilogue: one read of U here)
        "F7 SiLU + H quant (NVFP4 4/6)": ("hbm", A * F * (2.0 + nv)),
        "F8 down GEMM (NVFP4)": ("f16", gem),
        "F9 combine": ("hbm", A * d * 4.0 + T * d * 2.0 + A * 8.0),
        "B1 dY quant row-wise + transposed (MXFP8)": ("hbm", T * d * 2.0 + A * 8.0 + A * d * mxb + d * Ptot * mxb),
        "B2 W_down requant SR-T": ("hbm", E * d * F * (nv + mxb)),
        "B3 down dgrad (MXFP8)": ("fp8", gem),
        "B4 H requant SR-T": ("hbm", A * F * nv + F * Ptot * mxb),
        "B5 down wgrad (MXFP8)": ("fp8", gem, wg_bytes(d, F)),
        "B6 SiLU' + dU quant row-wise + transposed": ("hbm", A * F * (4.0 + 2.0 + mxb) + F * Ptot * mxb),
        "B7 W_up requant SR-T": ("hbm", E * d * F * (nv + mxb)),
        "B8 up dgrad (MXFP8)": ("fp8", gem),
        "B9 X requant SR-T": ("hbm", A * d * nv + d * Ptot * mxb),
        "B10 up wgrad (MXFP8)": ("fp8", gem, wg_bytes(F, d)),
        "B11 un-permute sum": ("hbm", A * d * 4.0 + T * d * 2.0),
        "B12 gate gradient": ("hbm", A * d * 4.0 + T * d * 2.0 + A * 8.0),
        "B13 router backward": ("hbm", T * E * 4.0 + A * 12.0),
    }


# the library kernel behind each call (several calls may launch one kernel)
KERNEL_OF = {
    "F1 W_up quant (+ requant)": "k_wq_resident",
    "F1 W_down quant (+ requant)": "k_wq_resident",
    "F2-F3 route + permutation": "route", "F4 X quant (NVFP4 4/6)": "nvfp4 quant 4/6 bf16",
    "F5 dispatch gather": "k_gather_rows", "F6 up GEMM (NVFP4)": "k_gemm_fwd_ws (bf16)",
    "F8 down GEMM (NVFP4)": "k_gemm_fwd_ws (f32)",
    "F7 SiLU + H quant (NVFP4 4/6)": "nvfp4 quant 4/6 silu", "F9 combine": "k_combine",
    "B1 dY quant row-wise + transposed (MXFP8)": "k_mx_T (rows + T, gather)",
    "B2 W_down requant SR-T": "k_requant_T", "B7 W_up requant SR-T": "k_requant_T",
    "B4 H requant SR-T": "k_requant_T (H)", "B9 X requant SR-T": "k_requant_T (X)",
    "B3 down dgrad (MXFP8)": "k_dgrad_ws", "B8 up dgrad (MXFP8)": "k_dgrad_ws",
    "B5 down wgrad (MXFP8)": "k_wgrad_ws256", "B10 up wgrad (MXFP8)": "k_wgrad_ws256",
    "B6 SiLU' + dU quant row-wise + transposed": "k_mx_T (rows + T, dsilu)",
    "B11 un-permute sum": "k_combine (unpermute)", "B12 gate gradient": "k_dgates",
    "B13 router backward": "k_route_backward",
}

# calls that launch several kernels of comparable length (zero, amax, scale,
# encode; route's four): not candidates for the single dominant kernel.  (The
# weight quantisation F1 is one persistent kernel after a workspace clear of a
# few microseconds: it is a candidate.)
MULTI_KERNEL_CALLS = {"F2-F3 route + permutation", "F4 X quant (NVFP4 4/6)", "F7 SiLU + H quant (NVFP4 4/6)"}

# the quantisers (float -> NVFP4 / MXFP8 codes) and the data-movement calls
# (gather, combine, un-permute, gate gradient), pooled separately
QUANTIZER_CALLS = {"F1 W_up quant (+ requant)", "F1 W_down quant (+ requant)", "F4 X quant (NVFP4 4/6)",
                   "F7 SiLU + H quant (NVFP4 4/6)", "B1 dY quant row-wise + transposed (MXFP8)", "B4 H requant SR-T",
                   "B6 SiLU' + dU quant row-wise + transposed", "B9 X requant SR-T"}
MOVEMENT_CALLS = {"F5 dispatch gather", "F9 combine", "B11 un-permute sum", "B12 gate gradient"}

# rocprofv3 --pmc summaries (FETCH_SIZE and WRITE_SIZE passes, scaled by a
# plain copy of known size) of a kernel, with the hash of its source file:
# the HBM bytes per launch are reported only while that source is unchanged.
PMC_PROFILE = {"k_wgrad_ws256": ("profiles/k_wgrad_ws256_T16384_E384_pmc.md",
                                 "precision_moe_numerics_quant_amd/csrc/gemm_bwd.hip"),
               "k_wq_resident": ("profiles/k_wq_resident_E384_4096x1536_pmc.md",
                                 "precision_moe_numerics_quant_amd/csrc/nvfp4_quant.hip")}


def source_sha256(rel):
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def pmc_traffic(kernel):
    if kernel not in PMC_PROFILE:
        return None
    prof, src = PMC_PROFILE[kernel]
    path = os.path.join(ROOT, prof)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and " = " in line:
                k, v = line[2:].split(" = ", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != source_sha256(src):
        return None                      # the kernel changed since the counters were taken
    return float(vals["hbm_bytes_per_launch"])


def pmc_summary(fetch_csv, write_csv, kernel_pat, copy_bytes=1 << 30):
    """Markdown summary of two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE;
    KiB per dispatch): the kernel's average per launch, scaled by the factor
    the same counter shows for the calibration copy (copy_bytes read and
    written by torch's copy kernel)."""
    import csv

    def per_kernel(path, counter):
        rows = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                rows.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return rows

    fe, wr = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    pick = lambda d, pat: [v for k, vs in d.items() if pat in k for v in vs]
    # the layer's launches: the run also launches the kernel for the tiny
    # layer, whose counters are orders of magnitude smaller
    big = lambda vs: [v for v in vs if v >= 0.1 * max(vs)]
    kf, kw = big(pick(fe, kernel_pat)), big(pick(wr, kernel_pat))
    # the calibration copies are the run's last and largest copy dispatches
    cf = sorted(pick(fe, "copyBuffer") or pick(fe, "copy_kernel"))[-3:]
    cw = sorted(pick(wr, "copyBuffer") or pick(wr, "copy_kernel"))[-3:]
    ref_kib = copy_bytes / 1024.0
    f_fetch = float(np.median(cf)) / ref_kib
    f_write = float(np.median(cw)) / ref_kib
    fetch_b = float(np.mean(kf)) * 1024.0 / f_fetch
    write_b = float(np.mean(kw)) * 1024.0 / f_write
    return (f"- kernel = `{kernel_pat}` ({len(kf)} FETCH / {len(kw)} WRITE dispatches)\n"
            f"- fetch_kib_per_launch = {np.mean(kf):.1f}\n- write_kib_per_launch = {np.mean(kw):.1f}\n"
            f"- copy_fetch_factor = {f_fetch:.4f}\n- copy_write_factor = {f_write:.4f}\n"
            f"- hbm_fetch_bytes_per_launch = {fetch_b:.4e}\n- hbm_write_bytes_per_launch = {write_b:.4e}\n"
            f"- hbm_bytes_per_launch = {fetch_b + write_b:.4e}\n")


def trace_summary(trace_csv, min_frac=0.1):
    """Markdown table of a rocprofv3 --kernel-trace csv: per kernel name, the
    launches at the layer's shape (at least min_frac of that name's longest
    launch: the run also launches the same kernels for the small workloads)
    with their count and average duration, and all launches' total."""
    import csv
    durs = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            durs.setdefault(name, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    total = sum(sum(v) for v in durs.values())
    rows = []
    for name, v in durs.items():
        big = [x for x in v if x >= min_frac * max(v)]
        rows.append((sum(v), name, len(v), len(big), float(np.mean(big)), float(np.median(big))))
    rows.sort(reverse=True)
    out = ["| kernel | launches | at layer shape | avg us at layer shape | median us at layer shape | total ms (all) "
           "| % of GPU time |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    for tot, name, n, nb, avg, med in rows[:30]:
        short = name.split("(")[0] if "<" not in name.split("(")[0] else name.split(")")[0].split("(")[0]
        out.append(f"| `{short[:90]}` | {n} | {nb} | {avg:.1f} | {med:.1f} | {tot / 1000.0:.2f} "
                   f"| {100.0 * tot / total:.2f} |")
    return "\n".join(out) + "\n"


def busy_summary(pmc_csv, kernels, n_simd=1024, n_cu=256, n_xcd=8, min_frac=0.1):
    """MFMA and VALU utilisation per kernel from one rocprofv3 --pmc pass of
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_ACTIVE_INST_VALU, SQ_INSTS_VALU,
    SQ_INSTS_MFMA and GRBM_GUI_ACTIVE: over the kernel's launches at the
    layer's shape (GRBM_GUI_ACTIVE at least min_frac of its largest),
    MfmaUtil = MFMA busy cycles / (active cycles x SIMDs) and VALUBusy =
    VALU-active cycles / (active cycles x CUs), as rocprofv3's derived
    metrics define them.  The GRBM_GUI_ACTIVE a dispatch reports is the sum
    over the chip's 8 XCDs (about 8x the kernel's cycles), so the active
    cycles are that sum / n_xcd."""
    import csv
    vals = {}
    with open(pmc_csv) as f:
        for r in csv.DictReader(f):
            key = (r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id", "")))
            vals.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    out = ["| kernel | launches | MfmaUtil % | VALUBusy % | VALU insts per launch | MFMA insts per launch |",
           "|---|---:|---:|---:|---:|---:|"]
    for pat in kernels:
        rows = [v for (name, _), v in vals.items() if pat in name and "GRBM_GUI_ACTIVE" in v]
        if not rows:
            continue
        top = max(v["GRBM_GUI_ACTIVE"] for v in rows)
        rows = [v for v in rows if v["GRBM_GUI_ACTIVE"] >= min_frac * top]
        act = sum(v["GRBM_GUI_ACTIVE"] for v in rows) / n_xcd
        mfma = 100.0 * sum(v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for v in rows) / (act * n_simd)
        valu = 100.0 * sum(v.get("SQ_ACTIVE_INST_VALU", 0.0) for v in rows) / (act * n_cu)
        iv = np.mean([v.get("SQ_INSTS_VALU", 0.0) for v in rows])
        im = np.mean([v.get("SQ_INSTS_MFMA", 0.0) for v in rows])
        out.append(f"| `{pat}` | {len(rows)} | {mfma:.1f} | {valu:.1f} | {iv:.3e} | {im:.3e} |")
    return "\n".join(out) + "\n"


def gpu_run(steps, warmup, layer_only=False):
    import precision_moe_numerics_quant_amd as m4
    from precision_moe_numerics_quant_amd import layer

    m4.lib()
    c = synth.CONFIGS[CFG_ID]
    inp = synth.config_inputs(CFG_ID, device="cuda", seed=0)
    torch.cuda.synchronize()
    k = c["k"]

    events = []            # (name, event) in stream order

    def timer(name):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        events.append((name, ev))

    def step(t=None):
        fw = layer.forward(inp["x"], inp["w_up"], inp["w_down"], inp["logits"], k, inp["bias"], timer=t,
                           seed=synth.SR_SEED)
        bw = layer.backward(fw, inp["dy"], seed=synth.SR_SEED, timer=t, skip_empty_dw=True)
        return fw, bw

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    # plain timed region (no per-call events)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fw, bw = step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / steps
    # device-side reports of the timed steps (a bounded wait that gave up, a
    # clamped index): a step that had one did not compute what it should
    try:
        m4.moe4_debug_check()
        device_error = None
    except m4.Moe4DeviceError as exc:
        device_error = str(exc)
        print(f"bench: device-side error in the timed steps: {exc}", file=sys.stderr)
    ref_outputs = None if layer_only else _fingerprint(fw, bw)
    # per-call breakdown over the same number of steps (events between calls)
    events.clear()
    torch.cuda.synchronize()
    for _ in range(steps):
        fw, bw = step(timer)
    torch.cuda.synchronize()
    per = {}
    prev = None
    for name, ev in events:
        if prev is not None and name is not None:
            per.setdefault(name, []).append(prev.elapsed_time(ev))
        prev = ev
    off = fw["route"]["off"].cpu().numpy()
    off_pad = fw["route"]["off_pad"].cpu().numpy()
    if layer_only:          # (profiling runs: the layer's launches only)
        return c, ms_step, wall, per, off, off_pad, None, None, None, None, device_error, None
    zero_fill = wgrad_zero_fill_bench(fw, bw, c, off)
    router_r = router_bench(inp, fw, bw, c)
    payload = combine_payload_bench(fw, c)
    small = small_configs_bench(inp, fw["wq"])
    del fw, bw
    # the MXFP8-forward variant of the same layer on the same inputs
    def step_mx(t=None):
        fw = layer.forward_mx(inp["x"], inp["w_up"], inp["w_down"], inp["logits"], k, inp["bias"], timer=t,
                              seed=synth.SR_SEED)
        layer.backward_mx(fw, inp["dy"], seed=synth.SR_SEED, timer=t, skip_empty_dw=True)
    for _ in range(warmup):
        step_mx()
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        step_mx()
    end.record()
    torch.cuda.synchronize()
    ms_mx = start.elapsed_time(end) / steps
    events.clear()
    step_mx(timer)
    torch.cuda.synchronize()
    per_mx = {}
    prev = None
    for name, ev in events:
        if prev is not None and name is not None:
            per_mx[name] = round(prev.elapsed_time(ev), 4)
        prev = ev
    # last, since its memory pool makes the caching allocator's later large
    # allocations slow: the step replayed from one HIP graph
    graph_run = graph_steps(step, steps, ref_outputs)
    return (c, ms_step, wall, per, off, off_pad, (ms_mx, per_mx), payload, (small, router_r), zero_fill,
            device_error, graph_run)


def _median_ms(fn, reps):
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts))


def router_bench(inp, fw, bw, c, reps=20):
    """The BF16 router in front of the layer (not part of the step, whose
    logits are an input): its GEMM on the step's x with [384, 4096] bf16
    weights, the un-permuting sum with the router's input gradient against the
    plain one, and the router's weight gradient, on the step's dXp, dlogits
    and routing (median of reps each)."""
    import precision_moe_numerics_quant_amd as m4
    T, d, E, k = c["T"], c["d"], c["E"], c["k"]
    g = torch.Generator(device="cuda").manual_seed(7)
    w = (torch.randn((E, d), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    r = fw["route"]
    x, dXp, dl = inp["x"], bw["dXp"], bw["dlogits"]
    t_g = _median_ms(lambda: m4.moe_router_logits(x, w), reps)
    t_u = _median_ms(lambda: m4.moe_unpermute_sum(dXp, r["inv_perm"], T, k), reps)
    t_ur = _median_ms(lambda: m4.moe_unpermute_sum_router(dXp, r["inv_perm"], T, k, dl, r["idx"], w), reps)
    t_w = _median_ms(lambda: m4.moe_router_wgrad(x, dl, r["perm"], r["off"], k), reps)
    fl = 2.0 * T * E * d
    wbytes = T * k * d * 2.0 + E * d * 4.0 + T * k * 8.0       # routed x rows, dW_r, perm + dz
    return {"workload": f"x [{T}, {d}] bf16, W_r [{E}, {d}] bf16, top-{k}",
            "gemm": {"ms": round(t_g, 4), "TFLOPs": round(fl / t_g / 1e9, 1),
                     "frac_peak": round(fl / t_g / 1e9 / (PEAK_F16 / 1e12), 4)},
            "unpermute_plus_router_dx_ms": round(t_ur, 4), "unpermute_ms": round(t_u, 4),
            "wgrad": {"ms": round(t_w, 4), "GBps": round(wbytes / t_w / 1e6, 1),
                      "frac_hbm": round(wbytes / t_w / 1e6 / (PEAK_HBM / 1e9), 4)}}


def wgrad_zero_fill_bench(fw, bw, c, off, reps=10):
    """The step's weight gradients leave the experts without tokens unwritten
    (their gradient is zero, and the route's offsets say which they are).
    This times both wgrad calls on the step's operands with and without the
    zero-fill of those experts' dW (median of reps each)."""
    import precision_moe_numerics_quant_amd as m4
    d, F, E = c["d"], c["F"], c["E"]
    op = fw["route"]["off_pad"]
    dWd, dWu = torch.empty_like(bw["dW_down"]), torch.empty_like(bw["dW_up"])

    def both(skip):
        m4.moe_grouped_gemm_bwd_wgrad(bw["dy_col"][0], bw["dy_col"][1], bw["hT"][0], bw["hT"][1], op, d, F, dw=dWd,
                                      skip_empty=skip)
        m4.moe_grouped_gemm_bwd_wgrad(bw["du_col"][0], bw["du_col"][1], bw["xT"][0], bw["xT"][1], op, F, d, dw=dWu,
                                      skip_empty=skip)
    both(False)
    t_fill = _median_ms(lambda: both(False), reps)
    t_skip = _median_ms(lambda: both(True), reps)
    empty = int((np.diff(off) == 0).sum())
    return {"empty_experts": empty, "zero_fill_bytes": empty * 2.0 * d * F * 4.0,
            "ms_both_wgrad_skip": round(t_skip, 4), "ms_both_wgrad_zero_fill": round(t_fill, 4),
            "ms_zero_fill": round(t_fill - t_skip, 4)}


def _fingerprint(fw, bw):
    """Copies of a step's outputs to compare bit for bit: y, dx, dg and the
    weight gradients of the first four experts that received tokens."""
    off = fw["route"]["off"]
    act = torch.nonzero(off[1:] > off[:-1]).flatten()[:4]
    return [fw["y"].clone(), bw["dx"].clone(), bw["dg"].clone(), bw["dW_up"][act].clone(), bw["dW_down"][act].clone()]


def graph_steps(step, steps, ref):
    """The layer step captured once in a HIP graph (through torch.cuda.CUDAGraph,
    the second stream's fork and join included) and replayed: every kernel of
    the step runs on every replay, without the per-call launch and binding work
    on the host.  The first replay must equal the eager step (ref) bit for bit;
    then `steps` replays are timed.  Returns dict(bit_identical, ms_per_step)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # (warm-up on the capturing stream, as torch asks)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gfw, gbw = step()
    graph.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in zip(ref, _fingerprint(gfw, gbw)))
    ms = None
    if same:
        graph.replay()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            graph.replay()
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
    del gfw, gbw, graph
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"bit_identical": same, "ms_per_step": ms}


def small_configs_bench(inp4, wq, reps=20):
    """The two small workloads, median of reps calls each (HIP events):
    the RL-shaped forward (512 tokens, unbiased routing, the weights already
    quantised, as they are between optimizer steps), bound by streaming the
    NVFP4 weights, and the tiny layer's whole step (256 tokens, 8 experts),
    bound by launches."""
    from precision_moe_numerics_quant_amd import layer
    c5 = synth.CONFIGS[5]
    T5, d, F, E, k = c5["T"], c5["d"], c5["F"], c5["E"], c5["k"]
    x5 = synth.activations(T5, d, "cuda", 0)
    lg5 = synth.randn((T5, E), 1.0, "cuda", 0, "logits")
    fwd5 = lambda: layer.forward(x5, inp4["w_up"], inp4["w_down"], lg5, k, None, wq=wq)
    o = fwd5()
    active = int((o["route"]["off"][1:] - o["route"]["off"][:-1] > 0).sum().item())
    t5 = _median_ms(fwd5, reps)
    w_active = active * 2.0 * F * d * 9.0 / 16.0       # NVFP4 codes + scales of both matrices
    c1 = synth.CONFIGS[1]
    inp1 = synth.config_inputs(1, device="cuda")
    calls = []
    step1 = lambda t=None: layer.backward(layer.forward(inp1["x"], inp1["w_up"], inp1["w_down"], inp1["logits"],
                                                        c1["k"], timer=t, seed=synth.SR_SEED),
                                          inp1["dy"], seed=synth.SR_SEED, timer=t)
    step1(lambda name: calls.append(name) if name is not None else None)
    torch.cuda.synchronize()
    t1 = _median_ms(step1, reps)
    # the same step captured once in a graph and replayed (no per-call launch
    # and binding overhead)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step1()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step1()
    t1g = _median_ms(graph.replay, reps)
    del graph
    return {
        "rl_forward_T512": {"workload": "forward, 512 tokens, top-8 of 384 experts, unbiased logits, d=4096, F=1536, "
                                        "weights quantised beforehand", "ms": round(t5, 4), "active_experts": active,
                            "weight_bytes": w_active, "GBps_weights": round(w_active / t5 / 1e6, 1),
                            "frac_hbm": round(w_active / t5 / 1e6 / (PEAK_HBM / 1e9), 4)},
        "tiny_layer_T256": {"workload": "forward + backward, 256 tokens, top-2 of 8 experts, d=256, F=512",
                            "us_per_step": round(t1 * 1000.0, 1), "library_calls_per_step": len(calls),
                            "us_per_call": round(t1 * 1000.0 / max(len(calls), 1), 1),
                            "us_per_step_graph_replay": round(t1g * 1000.0, 1)},
    }


def combine_payload_bench(fw, c, reps=20):
    """The combine with the expert outputs sent as the 8.25-bit payload (32-point
    Hadamard + 8-bit fixed point, E8M0 scale per 32) on this step's Yp and
    routing: the sender's quantiser and the receiver's decode + combine, each
    the median of reps runs timed with HIP events on the library's stream,
    against the float32 combine of the same rows."""
    import precision_moe_numerics_quant_amd as m4
    Yp, r = fw["Yp"], fw["route"]
    T, k, d = c["T"], c["k"], c["d"]
    A = T * k
    codes, sf = m4.moe_hmx8_quant(Yp)
    torch.cuda.synchronize()

    def timed(fn):
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    t_q = timed(lambda: m4.moe_hmx8_quant(Yp))
    t_c = timed(lambda: m4.moe_combine_hmx8(codes, sf, r["gates"], r["inv_perm"]))
    t_f = timed(lambda: m4.moe_combine(Yp, r["gates"], r["inv_perm"]))
    # the down GEMM alone and with the payload written by its epilogue
    hq, (wd_c, wd_s, wd_t) = fw["hq"], fw["wq"]["wd"]
    E, F = c["E"], c["F"]
    dargs = (hq[0], hq[1], hq[2], wd_c.view(E, d, F // 2), wd_s.view(E, d, F // 16), wd_t, r["off"])
    t_g = timed(lambda: m4.moe_grouped_gemm_fwd(*dargs, torch.float32, a_ts_per_group=True))
    try:
        t_gh = timed(lambda: m4.moe_grouped_gemm_fwd_hmx8(*dargs, a_ts_per_group=True))
    except m4.Moe4Unsupported:
        t_gh = None
    pay = A * d * (1 + 1 / 32)
    b_q = A * d * 4 + pay
    b_c = pay + A * 8 + T * d * 2
    b_f = A * d * 4 + A * 8 + T * d * 2

    def rate(b, t):
        return {"ms": round(t, 4), "GBps": round(b / t / 1e6, 1), "frac_hbm": round(b / t / 1e6 / (PEAK_HBM / 1e9), 4)}

    return {"bits_per_value": 8.0 * pay / (A * d), "payload_bytes": int(pay), "float32_bytes": A * d * 4,
            "bf16_bytes": A * d * 2, "quant": rate(b_q, t_q), "combine_from_payload": rate(b_c, t_c),
            "float32_combine": rate(b_f, t_f), "down_gemm_ms": round(t_g, 4),
            "down_gemm_with_payload_ms": None if t_gh is None else round(t_gh, 4),
            "payload_in_epilogue_extra_ms": None if t_gh is None else round(t_gh - t_g, 4)}


def quantizer_microbench(reps=20):
    """16384 x 7168 bf16 (1% of rows x50): NVFP4 4/6 quantisation (one group)
    and the dequant -> transpose -> MXFP8 SR requantisation of its result.
    Median of reps runs, each timed with HIP events on the library's stream."""
    import precision_moe_numerics_quant_amd as m4
    cfg = synth.CONFIGS[2]
    R, C = cfg["R"], cfg["C"]
    x = synth.config_inputs(2, device="cuda")["x"]
    off = torch.tensor([0, R], dtype=torch.int32, device="cuda")
    q = m4.nvfp4_quant_46(x, m4.NVFP4_4OVER6)
    m4.mxfp8_requant_sr_T(q[0], q[1], q[2], off, off, False, synth.SR_SEED, 0)
    torch.cuda.synchronize()

    def timed(fn):
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    # cold: before each timed call, a 1 GiB buffer is written, which evicts
    # the 4 MB L2s and the 256 MB Infinity Cache
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def cold(fn):
        ts = []
        for _ in range(reps):
            flush.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    fq = lambda: m4.nvfp4_quant_46(x, m4.NVFP4_4OVER6)
    fr = lambda: m4.mxfp8_requant_sr_T(q[0], q[1], q[2], off, off, False, synth.SR_SEED, 0)
    t_q, t_r = timed(fq), timed(fr)
    c_q, c_r = cold(fq), cold(fr)
    del flush
    n = R * C
    bytes_q = n * 2 * 2 + n * 9 / 16          # two bf16 reads (amax, encode) + codes and scales
    bytes_q1 = n * 2 + n * 9 / 16             # one-read basis
    bytes_r = n * 9 / 16 + n * 33 / 32        # NVFP4 in, MXFP8 out

    def rate(b, t):
        return {"ms": round(t, 4), "GBps": round(b / t / 1e6, 1), "frac_hbm": round(b / t / 1e6 / (PEAK_HBM / 1e9), 4)}
    return {"workload": f"bf16 {R}x{C}, 1% of rows x50 (median of {reps}; cold: a 1 GiB buffer written before "
                        f"each call, evicting the L2s and the 256 MB Infinity Cache; warm: back to back)",
            "nvfp4_46_quant": {"basis": "two bf16 reads + codes and scales", "cold": rate(bytes_q, c_q),
                               "warm": rate(bytes_q, t_q),
                               "cold_GBps_one_read_basis": round(bytes_q1 / c_q / 1e6, 1)},
            "mxfp8_requant_sr_T": {"basis": "NVFP4 read + MXFP8 write", "cold": rate(bytes_r, c_r),
                                   "warm": rate(bytes_r, t_r)}}


def copy_calibration(n_bytes=1 << 30, reps=3):
    """A plain device copy of known size (for scaling rocprofv3 FETCH_SIZE /
    WRITE_SIZE readings to bytes)."""
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


def cpu_baseline():
    """The oracle on a bounded sample of the same workload: the expert layer's
    forward + backward for the first 1536 tokens routed top-2 among the first 2
    experts (d = 4096, F = 1536 full size), timed on this host's cores (about
    10-15 s of CPU work)."""
    from oracle import layer as olayer
    c = synth.CONFIGS[CFG_ID]
    Ts, Es, ks = 1536, 2, 2
    full = synth.layer_inputs(Ts, c["d"], c["F"], Es, ks, device="cpu", seed=0, zipf=c["zipf"])
    x = synth.bf16_bits(full["x"])
    wu, wd = synth.f32_np(full["w_up"]), synth.f32_np(full["w_down"])
    lg, bias = synth.f32_np(full["logits"]), synth.f32_np(full["bias"])
    dy = synth.bf16_bits(full["dy"])
    t0 = time.perf_counter()
    fw = olayer.forward(x, wu, wd, lg, ks, bias)
    olayer.backward(fw, dy, seed=synth.SR_SEED)
    dt = time.perf_counter() - t0
    flops = 6 * 2.0 * Ts * ks * c["d"] * c["F"]
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle forward+backward of the expert layer on {Ts} tokens, top-{ks} of {Es} experts, "
                      f"d={c['d']}, F={c['F']} ({flops / 1e9:.1f} GFLOP of GEMM work in {dt:.1f} s; "
                      f"float64 GEMMs via NumPy BLAS, quantisers single-threaded NumPy; host os.cpu_count()="
                      f"{os.cpu_count()})"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="print the per-call table to stderr")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with a 1 GiB device copy (reference kernel for rocprofv3 byte counters)")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "KERNEL"),
                    help="print the traffic summary of two rocprofv3 --pmc csv files and exit (no GPU)")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="print the per-kernel table of a rocprofv3 --kernel-trace csv and exit (no GPU)")
    ap.add_argument("--busy-summary", nargs="+", metavar="ARG",
                    help="PMC_CSV KERNEL...: print MFMA / VALU utilisation per kernel and exit (no GPU)")
    ap.add_argument("--layer-only", action="store_true",
                    help="time the layer step only and print its line (for profiler runs: no other workloads)")
    args = ap.parse_args()
    if args.trace_summary:
        print(trace_summary(args.trace_summary), end="")
        return
    if args.busy_summary:
        print(busy_summary(args.busy_summary[0], args.busy_summary[1:]), end="")
        return
    if args.pmc_summary:
        print(pmc_summary(*args.pmc_summary), end="")
        if args.pmc_summary[2] in PMC_PROFILE:
            print(f"- source_sha256 = {source_sha256(PMC_PROFILE[args.pmc_summary[2]][1])}")
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    c, ms_step, wall, per, off, off_pad, mxv, payload, small, zero_fill, device_error, graph_run = gpu_run(args.steps, args.warmup,
                                                                                  args.layer_only)
    table = work_table(c, off, off_pad)
    peaks = {"hbm": PEAK_HBM, "f16": PEAK_F16, "fp8": PEAK_FP8}
    calls = {}
    gemm_flops = 0.0
    gemm_ms = 0.0
    pool = {"q": [0.0, 0.0], "m": [0.0, 0.0]}
    for name, times in per.items():
        kind, amount = table[name][0], table[name][1]
        ms = float(np.mean(times))
        rate = amount / (ms * 1e-3)
        entry = {"ms": round(ms, 4)}
        if kind == "hbm":
            entry.update(GBps=round(rate / 1e9, 1), frac_hbm=round(rate / PEAK_HBM, 4))
            key = "q" if name in QUANTIZER_CALLS else ("m" if name in MOVEMENT_CALLS else None)
            if key:
                pool[key][0] += amount
                pool[key][1] += ms
        else:
            entry.update(TFLOPs=round(rate / 1e12, 1), frac_peak=round(rate / peaks[kind], 4))
            if kind == "f16":
                entry["frac_fp4_peak"] = round(rate / PEAK_FP4, 4)
            if len(table[name]) > 2:
                bw = table[name][2] / (ms * 1e-3)
                entry["GBps"] = round(bw / 1e9, 1)
                entry["frac_hbm"] = round(bw / PEAK_HBM, 4)
            gemm_flops += amount
            gemm_ms += ms
        calls[name] = entry
    # dominant kernel: the one with the largest share of the step (calls that
    # launch the same kernel are pooled: e.g. both wgrad projections)
    fam = {}
    for name in per:
        if name not in MULTI_KERNEL_CALLS:
            fam.setdefault(KERNEL_OF[name], []).append(name)
    dom_k = max(fam, key=lambda k: sum(np.mean(per[n]) for n in fam[k]))
    names = fam[dom_k]
    ms_dom = float(np.mean([t for n in names for t in per[n]]))
    kind = table[names[0]][0]
    if kind == "hbm" or len(table[names[0]]) > 2:   # wgrad: fp32 dW writes bound it (HBM floor > MFMA floor)
        work = float(np.mean([table[n][2] if len(table[n]) > 2 else table[n][1] for n in names]))
        roof = {"bound": "hbm", "achieved": work / (ms_dom * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    else:
        work = float(np.mean([table[n][1] for n in names]))
        roof = {"bound": "mfma", "achieved": work / (ms_dom * 1e-3) / 1e12, "peak": peaks[kind] / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["achieved"] = round(roof["achieved"], 2)
    roof["kernel"] = dom_k
    roof["calls"] = names
    roof["ms_per_launch"] = round(ms_dom, 4)
    roof["algorithmic_bytes_per_launch" if roof["bound"] == "hbm" else "algorithmic_flop_per_launch"] = work
    roof["traffic"] = pmc_traffic(dom_k)
    step_gemm_flops = 6 * 2.0 * c["T"] * c["k"] * c["d"] * c["F"]
    out = {
        "metric": "expert grouped-GEMM TFLOPS (NVFP4 fwd, MXFP8 bwd) + quantizer GB/s, % of peak",
        "value": round(step_gemm_flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 mfma (fwd, exact nvfp4 dequant) / fp8 mfma (bwd), fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": "moe_expert_layer_fwd_bwd", "tokens": c["T"], "d_model": c["d"], "d_expert": c["F"],
                   "experts": c["E"], "top_k": c["k"], "router_bias": "zipf1.1", "active_experts": int((np.diff(off) > 0).sum()),
                   "max_rows_per_expert": int(np.diff(off).max())},
        "gemm_tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 2),
        # pooled over the step's quantiser calls (F1, F4, F7, B1, B4, B6, B9), and
        # over its data-movement calls (F5, F9, B11, B12): bytes / time
        "quantizer_gbps": round(pool["q"][0] / (pool["q"][1] * 1e-3) / 1e9, 1),
        "data_movement_gbps": round(pool["m"][0] / (pool["m"][1] * 1e-3) / 1e9, 1),
        "breakdown": calls,
        "roofline": roof,
        # a device-side report during the timed steps (null: none)
        "device_error": device_error,
    }
    if graph_run is not None:
        # the same step captured once in a HIP graph and replayed (every kernel
        # runs on every replay; the first replay equals the eager step bit for bit)
        out["graph_replay"] = {"bit_identical": graph_run["bit_identical"],
                               "ms_per_step": None if graph_run["ms_per_step"] is None
                               else round(graph_run["ms_per_step"], 3)}
    if not args.layer_only:
        ms_mx, per_mx = mxv
        out.update({
            "wgrad_zero_fill": zero_fill,
            "quantizer_microbench": quantizer_microbench(),
            # the same layer with an MXFP8 forward (the pages' higher-precision
            # layers, and their full-MXFP8 baseline): whole step, and per call (ms)
            "mxfp8_forward_variant": {
                "ms_per_step": round(ms_mx, 3),
                "value": round(step_gemm_flops / (ms_mx * 1e-3) / 1e12, 2),
                "fwd_gemm_tflops": {n: round(2.0 * c["T"] * c["k"] * c["d"] * c["F"] / (per_mx[n] * 1e-3) / 1e12, 1)
                                    for n in ("F6 up GEMM (MXFP8)", "F8 down GEMM (MXFP8)") if n in per_mx},
                "breakdown_ms": per_mx,
            },
            # the combine fed by the 8.25-bit payload the pages send back between GPUs
            "combine_payload_8p25": payload,
            # the small workloads: weight streaming (RL-shaped forward) and launch latency (tiny layer)
            **small[0],
            "router_bf16": small[1],
        })
    if args.copy_calibration:
        copy_calibration()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    if args.breakdown:
        for n, e in calls.items():
            print(f"{n:40s} {e}", file=sys.stderr)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
