"""Seeded synthetic inputs for the MoE expert-layer workloads.

This module holds only random-number generation and the input recipes; none of
the quantisation, routing or GEMM arithmetic.  Both the HIP path's tests and
benchmark and the CPU oracle take their inputs from here.

Recipes (the workloads the pages describe: a mixture-of-experts layer routing
each token to 8 of 384 experts, fourweekmba.com page, "Update"; bf16
activations and fp32 master weights, lhc.media page, paragraph on the
precisions that remain):

* activations x: bf16, drawn N(0, 1) in float32 then rounded to bf16; "outliers"
  multiply the float32 draw before the rounding.
* weights W_up [E, F, d], W_down [E, d, F]: float32 N(0, 0.02) (std 0.02).
* router logits [T, E]: float32 N(0, 1); a Zipf(s) expert bias
  b_e = -s * ln(e + 1) makes softmax(bias) Zipf(s) over expert rank e + 1.
* upstream gradient dy [T, d]: bf16 N(0, 1e-3).

Every tensor has its own generator, seeded by (config seed, tensor id), so any
tensor can be regenerated alone.  Draws use torch's generator on the device
asked for; CPU and GPU generators give different (but each deterministic)
streams, so a test generates once and hands the same tensor to both sides.
"""
import math

import numpy as np
import torch

TENSOR_IDS = {"x": 1, "w_up": 2, "w_down": 3, "logits": 4, "dy": 5, "rows": 6, "outlier": 7,
              "u": 8, "dh": 9, "misc": 10, "yp": 11}


def generator(device, seed, tensor):
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1000003 + TENSOR_IDS[tensor] * 7919) & 0x7FFFFFFFFFFFFFFF)
    return g


def randn(shape, std, device, seed, tensor, dtype=torch.float32):
    g = generator(device, seed, tensor)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def activations(T, d, device, seed, outlier_p=0.0, outlier_mul=1.0, row_frac=0.0, row_mul=1.0):
    """bf16 [T, d]: N(0,1); each element x outlier_mul w.p. outlier_p; round(row_frac*T) rows x row_mul."""
    x = randn((T, d), 1.0, device, seed, "x")
    if outlier_p > 0:
        g = generator(device, seed, "outlier")
        mask = torch.rand((T, d), generator=g, device=device) < outlier_p
        x = torch.where(mask, x * outlier_mul, x)
    if row_frac > 0:
        n = int(round(row_frac * T))
        g = generator(device, seed, "rows")
        rows = torch.randperm(T, generator=g, device=device)[:n]
        x[rows] *= row_mul
    return x.to(torch.bfloat16)


def zipf_bias(E, s, device):
    return torch.tensor([-s * math.log(e + 1) for e in range(E)], dtype=torch.float32, device=device)


def layer_inputs(T, d, F, E, k, device="cpu", seed=0, outlier_p=0.0, outlier_mul=1.0,
                 zipf=None, dy_std=1e-3, with_dy=True, w_std=0.02):
    """Inputs of one expert layer (forward and, if asked, backward)."""
    out = dict(
        T=T, d=d, F=F, E=E, k=k,
        x=activations(T, d, device, seed, outlier_p, outlier_mul),
        w_up=randn((E, F, d), w_std, device, seed, "w_up"),
        w_down=randn((E, d, F), w_std, device, seed, "w_down"),
        logits=randn((T, E), 1.0, device, seed, "logits"),
        bias=None if zipf is None else zipf_bias(E, zipf, device),
    )
    if with_dy:
        out["dy"] = randn((T, d), dy_std, device, seed, "dy", torch.bfloat16)
    return out


# The five workloads.  Sizes: tokens T, model dim d, expert hidden F, experts E, top-k.
CONFIGS = {
    1: dict(name="tiny_layer_fwd_bwd", T=256, d=256, F=512, E=8, k=2,
            outlier_p=0.001, outlier_mul=20.0, zipf=None, dy_std=1e-3),
    2: dict(name="quantizer_microbench", R=16384, C=7168, row_frac=0.01, row_mul=50.0),
    3: dict(name="layer_fwd", T=16384, d=4096, F=1536, E=384, k=8, zipf=1.1),
    4: dict(name="layer_fwd_bwd", T=16384, d=4096, F=1536, E=384, k=8, zipf=1.1, dy_std=1e-3),
    5: dict(name="rl_rollout_fwd", T=512, d=4096, F=1536, E=384, k=8, zipf=None),
}

SR_SEED = 1


def config_inputs(cfg_id, device="cpu", seed=0):
    c = CONFIGS[cfg_id]
    if cfg_id == 2:
        return dict(x=activations(c["R"], c["C"], device, seed, row_frac=c["row_frac"], row_mul=c["row_mul"]))
    return layer_inputs(c["T"], c["d"], c["F"], c["E"], c["k"], device=device, seed=seed,
                        outlier_p=c.get("outlier_p", 0.0), outlier_mul=c.get("outlier_mul", 1.0),
                        zipf=c.get("zipf"), dy_std=c.get("dy_std", 1e-3), with_dy=cfg_id in (1, 4))


def bf16_bits(t):
    """numpy uint16 bit patterns of a bf16 tensor (any device)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def f32_np(t):
    return t.detach().to("cpu").contiguous().numpy().astype(np.float32)
