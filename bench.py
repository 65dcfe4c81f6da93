"""Benchmark of the NVFP4-forward / MXFP8-backward MoE expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch: NVFP4 weight
quantisation of the fp32 masters, routing and permutation, X quantisation
(4/6), dispatch gather, up GEMM, SiLU + H quantisation (4/6), down GEMM,
combine; then the backward: gradient MXFP8 quantisation (row-wise and
transposed), the three SR requantisations of weights and activations (four
with both weights), dgrad and wgrad grouped GEMMs for both projections, dU
quantisation with SiLU', un-permuting sum.  Workload: T = 16384 tokens,
d = 4096, F = 1536, 384 experts, top-8 routing from N(0,1) logits with a
Zipf(1.1) expert bias; upstream gradient N(0, 1e-3); synthetic seeded inputs
resident in HBM before the timed region.

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
    wg_bytes = lambda n1, n2: E * n1 * n2 * 4.0 + (n1 + n2) * Ptot * mxb
    return {
        "F1 W_up quant": ("hbm", E * F * d * (8.0 + nv)),
        "F1 W_down quant": ("hbm", E * F * d * (8.0 + nv)),
        "F2-F3 route + permutation": ("hbm", T * E * 4.0 + A * 16.0),
        "F4 X quant (NVFP4 4/6)": ("hbm", T * d * (4.0 + nv)),
        "F5 dispatch gather": ("hbm", 2.0 * A * d * nv),
        "F6 up GEMM (NVFP4)": ("f16", gem),
        "F7 SiLU + H quant (NVFP4 4/6)": ("hbm", A * F * (4.0 + nv)),
        "F8 down GEMM (NVFP4)": ("f16", gem),
        "F9 combine": ("hbm", A * d * 4.0 + T * d * 2.0 + A * 8.0),
        "B1 dY quant row-wise (MXFP8)": ("hbm", T * d * 2.0 + A * 8.0 + A * d * mxb),
        "B1 dY quant transposed (MXFP8)": ("hbm", T * d * 2.0 + A * 8.0 + d * Ptot * mxb),
        "B2 W_down requant SR-T": ("hbm", E * d * F * (nv + mxb)),
        "B3 down dgrad (MXFP8)": ("fp8", gem),
        "B4 H requant SR-T": ("hbm", A * F * nv + F * Ptot * mxb),
        "B5 down wgrad (MXFP8)": ("fp8", gem, wg_bytes(d, F)),
        "B6 SiLU' + dU quant row-wise": ("hbm", A * F * (4.0 + 2.0 + mxb)),
        "B6 SiLU' + dU quant transposed": ("hbm", A * F * 6.0 + F * Ptot * mxb),
        "B7 W_up requant SR-T": ("hbm", E * d * F * (nv + mxb)),
        "B8 up dgrad (MXFP8)": ("fp8", gem),
        "B9 X requant SR-T": ("hbm", A * d * nv + d * Ptot * mxb),
        "B10 up wgrad (MXFP8)": ("fp8", gem, wg_bytes(F, d)),
        "B11 un-permute sum": ("hbm", A * d * 4.0 + T * d * 2.0),
    }


def gpu_run(steps, warmup):
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
        fw = layer.forward(inp["x"], inp["w_up"], inp["w_down"], inp["logits"], k, inp["bias"], timer=t)
        bw = layer.backward(fw, inp["dy"], seed=synth.SR_SEED, timer=t)
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
    return c, ms_step, wall, per, off, off_pad


def cpu_baseline():
    """The oracle on a bounded sample of the same workload: the expert layer's
    forward + backward for the first 256 tokens routed top-2 among the first 2
    experts (d = 4096, F = 1536 full size), timed on this host's cores."""
    from oracle import layer as olayer
    c = synth.CONFIGS[CFG_ID]
    Ts, Es, ks = 256, 2, 2
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
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    c, ms_step, wall, per, off, off_pad = gpu_run(args.steps, args.warmup)
    table = work_table(c, off, off_pad)
    peaks = {"hbm": PEAK_HBM, "f16": PEAK_F16, "fp8": PEAK_FP8}
    calls = {}
    gemm_flops = 0.0
    gemm_ms = 0.0
    q_bytes = 0.0
    q_ms = 0.0
    for name, times in per.items():
        kind, amount = table[name][0], table[name][1]
        ms = float(np.mean(times))
        rate = amount / (ms * 1e-3)
        entry = {"ms": round(ms, 4)}
        if kind == "hbm":
            entry.update(GBps=round(rate / 1e9, 1), frac_hbm=round(rate / PEAK_HBM, 4))
            if "route" not in name:
                q_bytes += amount
                q_ms += ms
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
    dom = max(per, key=lambda n: np.mean(per[n]))
    kind = table[dom][0]
    ms_dom = float(np.mean(per[dom]))
    if kind == "hbm":
        roof = {"bound": "hbm", "achieved": table[dom][1] / (ms_dom * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": table[dom][1] / (ms_dom * 1e-3) / 1e12, "peak": peaks[kind] / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["achieved"] = round(roof["achieved"], 2)
    roof["frac"] = round(roof["frac"], 4)
    roof["kernel"] = dom
    roof["traffic"] = None
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
        "dtype": "nvfp4-fwd/mxfp8-bwd (f16 and fp8 MFMA, fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": "moe_expert_layer_fwd_bwd", "tokens": c["T"], "d_model": c["d"], "d_expert": c["F"],
                   "experts": c["E"], "top_k": c["k"], "router_bias": "zipf1.1", "active_experts": int((np.diff(off) > 0).sum()),
                   "max_rows_per_expert": int(np.diff(off).max())},
        "gemm_tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 2),
        "quantizer_gbps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
        "breakdown": calls,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    if args.breakdown:
        for n, e in calls.items():
            print(f"{n:40s} {e}", file=sys.stderr)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
