"""Shared helpers of the GPU parity tests (tensor <-> numpy, tolerances)."""
import numpy as np
import torch

from oracle import formats as fmt


def to_np(t):
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_from_bits(bits, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def cuda_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def cuda_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def cuda_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def assert_bytes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
    assert bad.size == 0, f"{what}: {bad.size} of {got.size} differ; first at {bad[:5]}: got {got.reshape(-1)[bad[:5]]} want {want.reshape(-1)[bad[:5]]}"


def gemm_tol_check(got, exact, absbound, what, out_bf16=False, rel=1e-3):
    """Per element: |got - exact| <= rel * sum|a*b| + half an ulp of the output
    dtype, the ulp taken at |exact| + rel * sum|a*b| (the float32 accumulation
    stays within the first term, the output rounding within the second, also
    when the accumulated value crosses into the next binade)."""
    got = np.asarray(got, dtype=np.float64)
    slack = rel * np.asarray(absbound, dtype=np.float64)
    a = np.abs(exact) + slack
    mant = 7 if out_bf16 else 23
    ulp = np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - mant)
    err = np.abs(got - exact)
    lim = slack + 0.5 * ulp
    bad = np.nonzero(err > lim)
    assert bad[0].size == 0, f"{what}: {bad[0].size} elements out of tolerance; worst ratio {np.max(err / np.maximum(lim, 1e-300)):.3g}"
    # normwise: against the exact result rounded to the output dtype, so that the
    # output rounding itself (up to 2**-9 relative for bf16) is not counted
    ref = fmt.bf16_to_f32(fmt.f64_to_bf16(exact)).astype(np.float64) if out_bf16 else exact
    nrm = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    assert nrm <= rel, f"{what}: normwise error {nrm:.3g}"
    return nrm
