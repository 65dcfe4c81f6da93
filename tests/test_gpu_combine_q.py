"""GPU parity of the combine-path quantiser (block Hadamard + 8-bit fixed-point
MX, 8.25 bits per value) and of the combine from its payload, against the
oracle: codes, scales, decoded values and the bf16 combine bit for bit."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import assert_bytes_equal, cuda_i32, to_np
from oracle import combine_q as cq
from oracle import route

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import precision_moe_numerics_quant_amd as m4


def _values(R, C, seed):
    """Expert-output-like rows: N(0,1) with per-row scale spread, 0.1% outliers
    x50, an all-zero block, a row of tiny (subnormal-range) values and a row
    near the top of the allowed range."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, C)) * np.exp(rng.uniform(-6, 6, (R, 1)))
    out = rng.random((R, C)) < 0.001
    x[out] *= 50.0
    x = x.astype(np.float32)
    if R > 3:
        x[1, :32] = 0.0
        x[2] = (rng.standard_normal(C) * 2.0 ** -135).astype(np.float32)
        x[3] = (rng.standard_normal(C) * 2.0 ** 110).astype(np.float32)
    return x


@pytest.mark.parametrize("R,C,seed", [(1, 32, 0), (7, 96, 1), (300, 512, 2), (129, 4096, 3), (64, 7168, 4)])
def test_hmx8_quant_bit_exact(R, C, seed):
    x = _values(R, C, seed)
    codes, sf = m4.moe_hmx8_quant(torch.from_numpy(x).cuda())
    c_want, s_want = cq.quantize(x)
    assert_bytes_equal(to_np(sf), s_want, "scales")
    assert_bytes_equal(to_np(codes), c_want, "codes")


def test_hmx8_quant_ties_and_clamp():
    # values whose scaled transform lands on .5 ties and just below 128
    # (rounds to 128, clamped to 127): built on the transformed side, then
    # mapped back with the exact inverse (H / 32) so the sender sees them.
    rng = np.random.default_rng(11)
    R = 64
    y = rng.integers(-126, 127, size=(R, 32)).astype(np.float64) + 0.5   # ties
    y[:, 0] = 127.75                                                      # clamp
    y = y * 2.0 ** -6                                                     # e = 0 blocks
    H = cq.hadamard_matrix(32).astype(np.float64)
    x = (y @ H / 32).astype(np.float32)
    codes, sf = m4.moe_hmx8_quant(torch.from_numpy(x).cuda())
    c_want, s_want = cq.quantize(x)
    assert_bytes_equal(to_np(sf), s_want, "scales")
    assert_bytes_equal(to_np(codes), c_want, "codes")


def test_hmx8_dequant_every_code_and_scale():
    rng = np.random.default_rng(12)
    R, C = 255, 256
    codes = rng.integers(-127, 128, size=(R, C)).astype(np.int8)
    codes[0, :254] = np.arange(-127, 127)
    sf = np.repeat(np.arange(255, dtype=np.uint8)[:, None], C // 32, axis=1)   # every scale byte 0..254
    got = m4.moe_hmx8_dequant(torch.from_numpy(codes).cuda(), torch.from_numpy(sf).cuda())
    assert_bytes_equal(to_np(got).view(np.uint32), cq.dequantize(codes, sf).view(np.uint32), "decoded values")


@pytest.mark.parametrize("T,k,d,E,seed", [(200, 3, 128, 6, 0), (61, 1, 32, 4, 1), (300, 8, 4096, 40, 2),
                                          (33, 16, 96, 20, 3)])
def test_combine_hmx8_bit_exact(T, k, d, E, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    P = route.permutation(idx, E)
    yp = _values(T * k, d, seed + 100)
    gates = rng.random((T, k)).astype(np.float32)
    codes, sf = m4.moe_hmx8_quant(torch.from_numpy(yp).cuda())
    y = m4.moe_combine_hmx8(codes, sf, torch.from_numpy(gates).cuda(), cuda_i32(P["inv_perm"]))
    c_np, s_np = cq.quantize(yp)
    assert_bytes_equal(to_np(codes), c_np, "codes")
    want = cq.combine_payload(c_np, s_np, gates, P["inv_perm"], k)
    assert_bytes_equal(to_np(y), want, "combine from the payload")


def test_combine_hmx8_full_size_sampled():
    """The layer's shape (16384 tokens, top-8, d = 4096, 384 experts, Zipf 1.1
    routing bias) in the launch configuration the benchmark times: the whole
    payload on the GPU, the oracle on sampled tokens and their rows."""
    c = synth.CONFIGS[4]
    T, k, d, E = c["T"], c["k"], c["d"], c["E"]
    inp = synth.config_inputs(4, device="cuda", seed=0)
    r = m4.moe_route_topk(inp["logits"], k, inp["bias"])
    yp = synth.randn((T * k, d), 0.05, "cuda", 5, "yp")
    codes, sf = m4.moe_hmx8_quant(yp)
    y = m4.moe_combine_hmx8(codes, sf, r["gates"], r["inv_perm"])
    torch.cuda.synchronize()
    inv = to_np(r["inv_perm"]).astype(np.int64)
    gates = to_np(r["gates"])
    rng = np.random.default_rng(9)
    toks = np.concatenate([[0, T - 1], rng.choice(T, 30, replace=False)])
    rows = inv.reshape(T, k)[toks].reshape(-1)
    yp_rows = to_np(yp[torch.from_numpy(rows).cuda()])
    c_want, s_want = cq.quantize(yp_rows)
    assert_bytes_equal(to_np(codes[torch.from_numpy(rows).cuda()]), c_want, "sampled codes")
    assert_bytes_equal(to_np(sf[torch.from_numpy(rows).cuda()]), s_want, "sampled scales")
    want = cq.combine_payload(c_want, s_want, gates[toks], np.arange(len(toks) * k), k)
    assert_bytes_equal(to_np(y)[toks], want, "sampled combine")


def test_hmx8_edge_cases():
    z = torch.zeros((0, 64), dtype=torch.float32, device="cuda")
    codes, sf = m4.moe_hmx8_quant(z)
    assert codes.shape == (0, 64) and sf.shape == (0, 2)
    with pytest.raises(m4.Moe4Error):
        m4.moe_hmx8_quant(torch.zeros((4, 48), dtype=torch.float32, device="cuda"))
    c8 = torch.zeros((17 * 4, 64), dtype=torch.int8, device="cuda")
    s8 = torch.zeros((17 * 4, 2), dtype=torch.uint8, device="cuda")
    with pytest.raises(m4.Moe4Error):   # k = 17 > 16
        m4.moe_combine_hmx8(c8[:68], s8[:68], torch.zeros((4, 17), device="cuda"),
                            torch.arange(68, dtype=torch.int32, device="cuda"))
    y = m4.moe_combine_hmx8(c8[:0], s8[:0], torch.zeros((0, 2), device="cuda"),
                            torch.zeros(0, dtype=torch.int32, device="cuda"))
    assert y.shape == (0, 64)
