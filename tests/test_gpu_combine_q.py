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


# ------------------------------------- the payload from the down GEMM's epilogue

def _small_code_operands(M_list, N, K, seed):
    """NVFP4 operands with codes in {0, +-0.5, +-1, +-2}, power-of-two block
    and tensor scales: every partial sum of the GEMM and of the Hadamard
    transform is exact in float32, so C and its payload have one right answer."""
    from oracle import nvfp4 as nv
    rng = np.random.default_rng(seed)
    E = len(M_list)
    off = np.concatenate([[0], np.cumsum(M_list)]).astype(np.int64)
    M = int(off[-1])
    small = np.array([0, 1, 2, 4, 8, 9, 10, 12])
    ca = nv.pack_codes(rng.choice(small, (M, K)))
    cb = nv.pack_codes(rng.choice(small, (E * N, K)))
    sa = rng.choice([0x38, 0x30, 0x40], (M, K // 16)).astype(np.uint8)
    sb = rng.choice([0x38, 0x30, 0x40], (E * N, K // 16)).astype(np.uint8)
    ta = rng.choice([0.25, 0.5, 1.0], E).astype(np.float32)      # per expert, as the down GEMM's H
    tb = rng.choice([0.5, 1.0, 2.0, 4.0], E).astype(np.float32)
    return off, ca, sa, ta, cb, sb, tb


def _dev_args(off, ca, sa, ta, cb, sb, tb, N, K):
    E = len(off) - 1
    return (torch.from_numpy(ca).cuda(), torch.from_numpy(sa).cuda(), torch.from_numpy(ta).cuda(),
            torch.from_numpy(cb).cuda().view(E, N, K // 2), torch.from_numpy(sb).cuda().view(E, N, K // 16),
            torch.from_numpy(tb).cuda(), cuda_i32(off))


# N % 256 == 0 takes the 128 x 256 warp-specialised kernel, N = 384 the
# 128 x 128 one; ragged experts (0 rows, tails of 1 .. 127 rows)
@pytest.mark.parametrize("M_list,N,K", [([50, 0, 90], 256, 256), ([70, 33, 0, 129], 384, 512),
                                        ([300, 1, 0, 37, 200], 512, 256)])
def test_down_gemm_payload_exact_special_case(M_list, N, K):
    """moe_grouped_gemm_fwd_hmx8 on exactly representable operands: C equals
    the exact product and the payload equals the oracle's quantisation of it,
    byte for byte."""
    from oracle import gemm as og
    from oracle import nvfp4 as nv
    off, ca, sa, ta, cb, sb, tb = _small_code_operands(M_list, N, K, N + K)
    E = len(M_list)
    c, codes, sf = m4.moe_grouped_gemm_fwd_hmx8(*_dev_args(off, ca, sa, ta, cb, sb, tb, N, K), a_ts_per_group=True)
    exact = og.grouped_nt(nv.nvfp4_exact_f64(ca, sa, ta, off),
                          nv.nvfp4_exact_f64(cb, sb, tb, np.arange(E + 1) * N).reshape(E, N, K), off)
    assert np.array_equal(to_np(c).astype(np.float64), exact)
    c_want, s_want = cq.quantize(exact.astype(np.float32))
    assert_bytes_equal(to_np(sf), s_want, "scales")
    assert_bytes_equal(to_np(codes), c_want, "codes")


@pytest.mark.parametrize("M_list,N,K", [([0, 37, 130, 1, 300], 384, 512), ([5, 300, 0, 129], 512, 1024)])
def test_down_gemm_payload_matches_plain_gemm_and_quantiser(M_list, N, K):
    """General operands: C is byte for byte that of moe_grouped_gemm_fwd (same
    kernel, same summation) and the payload is the oracle's quantisation of
    that C (the quantiser's decisions taken on the same float32 values);
    moe_hmx8_quant of C gives the same bytes."""
    from oracle import nvfp4 as nv
    E = len(M_list)
    off = np.concatenate([[0], np.cumsum(M_list)]).astype(np.int64)
    xb = synth.bf16_bits(synth.activations(int(off[-1]), K, "cpu", K, outlier_p=0.001, outlier_mul=20.0))
    qa = nv.nvfp4_quantize(xb, 46, off)
    w = synth.randn((E, N, K), 0.02, "cpu", N, "w_down").numpy()
    qb = nv.nvfp4_quantize(w.reshape(E * N, K), 6, np.arange(E + 1) * N)
    args = _dev_args(off, qa["codes"], qa["sf"], qa["ts"], qb["codes"], qb["sf"], qb["ts"], N, K)
    c, codes, sf = m4.moe_grouped_gemm_fwd_hmx8(*args, a_ts_per_group=True)
    c2 = m4.moe_grouped_gemm_fwd(*args, torch.float32, a_ts_per_group=True)
    assert torch.equal(c.view(torch.int32), c2.view(torch.int32))
    c_want, s_want = cq.quantize(to_np(c))
    assert_bytes_equal(to_np(sf), s_want, "scales")
    assert_bytes_equal(to_np(codes), c_want, "codes")
    codes2, sf2 = m4.moe_hmx8_quant(c2)
    assert torch.equal(codes, codes2) and torch.equal(sf, sf2)


def test_down_gemm_payload_unsupported_and_empty():
    from oracle import nvfp4 as nv
    # few rows per expert (the weight-streaming kernel) and K % 256 != 0
    for M_list, N, K in (([3, 12, 0, 40, 1, 19], 256, 512), ([40, 24], 128, 320)):
        off, ca, sa, ta, cb, sb, tb = _small_code_operands(M_list, N, K, 1)
        with pytest.raises(m4.Moe4Unsupported):
            m4.moe_grouped_gemm_fwd_hmx8(*_dev_args(off, ca, sa, ta, cb, sb, tb, N, K), a_ts_per_group=True)
    off, ca, sa, ta, cb, sb, tb = _small_code_operands([0, 0], 256, 256, 2)
    c, codes, sf = m4.moe_grouped_gemm_fwd_hmx8(*_dev_args(off, ca, sa, ta, cb, sb, tb, 256, 256),
                                                a_ts_per_group=True)
    assert c.shape == (0, 256) and codes.shape == (0, 256) and sf.shape == (0, 8)


def test_down_gemm_payload_full_size_sampled():
    """The down GEMM at the layer's shape (131072 routed rows, N = d = 4096,
    K = F = 1536, 384 experts, Zipf 1.1 routing): C byte for byte that of
    moe_grouped_gemm_fwd; the payload of sampled rows equal to the oracle's
    quantisation of those rows of C."""
    c = synth.CONFIGS[4]
    T, k, d, F, E = c["T"], c["k"], c["d"], c["F"], c["E"]
    inp = synth.config_inputs(4, device="cuda", seed=0)
    r = m4.moe_route_topk(inp["logits"], k, inp["bias"])
    A = T * k
    h = synth.randn((A, F), 1.0, "cuda", 3, "u").to(torch.bfloat16)
    hq = m4.nvfp4_quant_46(h, m4.NVFP4_4OVER6, r["off"])
    wd = synth.randn((E * d, F), 0.02, "cuda", 4, "w_down").to(torch.bfloat16)
    wq = m4.nvfp4_quant_46(wd, 6, torch.arange(E + 1, dtype=torch.int32, device="cuda") * d)
    del h, wd
    args = (hq[0], hq[1], hq[2], wq[0].view(E, d, F // 2), wq[1].view(E, d, F // 16), wq[2], r["off"])
    y, codes, sf = m4.moe_grouped_gemm_fwd_hmx8(*args, a_ts_per_group=True)
    y2 = m4.moe_grouped_gemm_fwd(*args, torch.float32, a_ts_per_group=True)
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    del y2
    off = to_np(r["off"]).astype(np.int64)
    rng = np.random.default_rng(7)
    last = off[1:][np.diff(off) > 0] - 1                     # each non-empty expert's last row
    rows = np.unique(np.r_[0, A - 1, rng.choice(last, 32, replace=False), rng.choice(A, 64, replace=False)])
    sel = torch.from_numpy(rows).cuda()
    c_want, s_want = cq.quantize(to_np(y[sel]))
    assert_bytes_equal(to_np(codes[sel]), c_want, "sampled codes")
    assert_bytes_equal(to_np(sf[sel]), s_want, "sampled scales")
