"""GPU parity of routing, data movement and the grouped GEMMs against the oracle."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import assert_bytes_equal, bf16_from_bits, cuda_i32, gemm_tol_check, to_np
from oracle import formats as fmt
from oracle import gemm as og
from oracle import layer as olayer
from oracle import mxfp8 as mx
from oracle import nvfp4 as nv
from oracle import route

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import precision_moe_numerics_quant_amd as m4


# ---------------------------------------------------------------------- routing

@pytest.mark.parametrize("T,E,k,zipf", [(256, 8, 2, None), (1000, 384, 8, 1.1), (77, 40, 5, None), (64, 1024, 16, None)])
def test_route_bit_exact(T, E, k, zipf):
    logits = synth.randn((T, E), 1.0, "cpu", T + E, "logits").numpy()
    if T == 77:
        logits = np.round(logits * 2) / 2          # many exact ties
    bias = None if zipf is None else (-zipf * np.log(np.arange(E) + 1)).astype(np.float32)
    r = m4.moe_route_topk(torch.from_numpy(logits).cuda(), k, None if bias is None else torch.from_numpy(bias).cuda())
    idx, gates = route.topk_gates(logits, k, bias)
    P = route.permutation(idx, E)
    assert_bytes_equal(to_np(r["idx"]), idx, "topk idx")
    assert_bytes_equal(to_np(r["gates"]).view(np.uint32), gates.view(np.uint32), "gates")
    for key in ("off", "off_pad", "perm", "inv_perm"):
        assert_bytes_equal(to_np(r[key]), P[key], key)


def test_route_empty_tokens():
    r = m4.moe_route_topk(torch.zeros((0, 16), dtype=torch.float32, device="cuda"), 2)
    assert (to_np(r["off"]) == 0).all() and (to_np(r["off_pad"]) == 0).all()


def test_gather_combine_unpermute_bit_exact():
    T, d, k, E = 200, 128, 3, 6
    rng = np.random.default_rng(0)
    xb = synth.bf16_bits(synth.activations(T, d, "cpu", 1))
    xq = nv.nvfp4_quantize(xb, 46)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    P = route.permutation(idx, E)
    oc, os_ = m4.moe_gather_rows(torch.from_numpy(xq["codes"]).cuda(), torch.from_numpy(xq["sf"]).cuda(),
                                 cuda_i32(P["perm"]), k)
    src = P["perm"] // k
    assert_bytes_equal(to_np(oc), xq["codes"][src], "gather codes")
    assert_bytes_equal(to_np(os_), xq["sf"][src], "gather scales")
    yp = rng.standard_normal((T * k, d)).astype(np.float32)
    gates = rng.random((T, k)).astype(np.float32)
    y = m4.moe_combine(torch.from_numpy(yp).cuda(), torch.from_numpy(gates).cuda(), cuda_i32(P["inv_perm"]))
    assert_bytes_equal(to_np(y), olayer.combine(yp, gates, P["inv_perm"], k), "combine")
    dx = m4.moe_unpermute_sum(torch.from_numpy(yp).cuda(), cuda_i32(P["inv_perm"]), T, k)
    assert_bytes_equal(to_np(dx), olayer.unpermute_sum(yp, P["inv_perm"], T, k), "unpermute")


# ------------------------------------------------------------------------ GEMMs

def _fwd_operands(M_list, N, K, seed, ts_per_group=False):
    E = len(M_list)
    off = np.concatenate([[0], np.cumsum(M_list)]).astype(np.int64)
    M = int(off[-1])
    xb = synth.bf16_bits(synth.activations(max(M, 1), K, "cpu", seed, outlier_p=0.001, outlier_mul=20.0))[:M]
    qa = nv.nvfp4_quantize(xb, 46, off if ts_per_group else None)
    w = synth.randn((E, N, K), 0.02, "cpu", seed, "w_up").numpy()
    qb = nv.nvfp4_quantize(w.reshape(E * N, K), 6, np.arange(E + 1) * N)
    return off, qa, qb


# Few rows per expert (at most 32 on average) take the weight-streaming kernel:
# ragged experts of 0 .. 33 rows and one of 70 (three 32-token passes)
_FEW = [0, 1, 2, 3, 5, 9, 10, 13, 16, 17, 31, 32, 33, 70, 0, 4, 8, 12, 1, 0]


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
# (N, K) pick the kernels: 192 x 320 and 64 x 64 the register-staged one,
# 160 x 256 the 128 x 128 direct-to-LDS one, 384 x 512 the warp-specialised
# 128 x 128 one, 512 x 1024 the warp-specialised 128 x 256 one
@pytest.mark.parametrize("M_list,N,K", [([0, 37, 130, 1, 300], 192, 320), ([64], 64, 64), ([5, 0, 0, 257], 512, 1024),
                                        ([5, 300, 0, 129], 160, 256), ([0, 37, 130, 1, 300], 384, 512),
                                        (_FEW, 192, 512), ([3, 12, 0, 40, 1, 19], 1536, 1024), ([1], 64, 256)])
def test_grouped_gemm_fwd_tolerance(M_list, N, K, out_dtype):
    E = len(M_list)
    per_group = out_dtype == "f32"
    off, qa, qb = _fwd_operands(M_list, N, K, seed=N + K, ts_per_group=per_group)
    tdt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    c = m4.moe_grouped_gemm_fwd(torch.from_numpy(qa["codes"]).cuda(), torch.from_numpy(qa["sf"]).cuda(),
                                torch.from_numpy(qa["ts"]).cuda(), torch.from_numpy(qb["codes"]).cuda().view(E, N, K // 2),
                                torch.from_numpy(qb["sf"]).cuda().view(E, N, K // 16), torch.from_numpy(qb["ts"]).cuda(),
                                cuda_i32(off), tdt, a_ts_per_group=per_group)
    A64 = nv.nvfp4_exact_f64(qa["codes"], qa["sf"], qa["ts"], off if per_group else None)
    B64 = nv.nvfp4_exact_f64(qb["codes"], qb["sf"], qb["ts"], np.arange(E + 1) * N).reshape(E, N, K)
    exact = og.grouped_nt(A64, B64, off)
    bound = og.abs_bound_nt(A64, B64, off)
    got = to_np(c)
    got = fmt.bf16_to_f32(got).astype(np.float64) if out_dtype == "bf16" else got.astype(np.float64)
    gemm_tol_check(got, exact, bound, "fwd", out_bf16=out_dtype == "bf16")


@pytest.mark.parametrize("E,N,K,M_list", [(3, 64, 128, [50, 0, 90]), (4, 128, 256, [7, 0, 20, 33])])
def test_grouped_gemm_fwd_exact_special_case(E, N, K, M_list):
    """Codes in {0, +-0.5, +-1, +-2} with power-of-two scales and small K keep
    every partial sum exact in float32: the GPU result equals the exact one
    (the second case takes the few-rows-per-expert kernel)."""
    rng = np.random.default_rng(3)
    off = np.concatenate([[0], np.cumsum(M_list)])
    M = off[-1]
    small = np.array([0, 1, 2, 4, 8, 9, 10, 12])     # codes of 0, .5, 1, 2, -0, -.5, -1, -2
    qa = rng.choice(small, (M, K)); qb = rng.choice(small, (E * N, K))
    sa = rng.choice([0x38, 0x30, 0x40], (M, K // 16)).astype(np.uint8)         # 1, .5, 2
    sb = rng.choice([0x38, 0x30, 0x40], (E * N, K // 16)).astype(np.uint8)
    ta = np.float32([0.25]); tb = np.float32([1.0, 2.0, 0.5, 4.0][:E])
    ca, cb = nv.pack_codes(qa), nv.pack_codes(qb)
    c = m4.moe_grouped_gemm_fwd(torch.from_numpy(ca).cuda(), torch.from_numpy(sa).cuda(), torch.from_numpy(ta).cuda(),
                                torch.from_numpy(cb).cuda().view(E, N, K // 2), torch.from_numpy(sb).cuda().view(E, N, K // 16),
                                torch.from_numpy(tb).cuda(), cuda_i32(off), torch.float32)
    exact = og.grouped_nt(nv.nvfp4_exact_f64(ca, sa, ta), nv.nvfp4_exact_f64(cb, sb, tb, np.arange(E + 1) * N).reshape(E, N, K), off)
    assert np.array_equal(to_np(c).astype(np.float64), exact)


def _mx_rows(M, K, seed, scale=1.0):
    x = (synth.randn((M, K), scale, "cpu", seed, "dh").numpy())
    return mx.quantize_rowwise(x, mx.RNE)


# 192 x 320 and 96 x 96: register-staged kernel; 128 x 256: warp-specialised
# 128 x 128; 256 x 384: warp-specialised 128 x 256 (three slabs).  The last
# two cover the warp-specialised kernel's per-XCD tile rectangles over more
# than one band of m-tiles: N = 1280 (5 n-tiles in rectangles of 3: a
# rectangle column past the last n-tile) and N = 4096 (16 n-tiles, 2 per XCD)
@pytest.mark.parametrize("M_list,N,K", [([0, 37, 130, 1, 300], 192, 320), ([256], 128, 4096 // 16), ([3, 200], 96, 96),
                                        ([0, 37, 130, 1, 300], 256, 384), ([2100, 3000, 1, 0, 900], 1280, 256),
                                        ([700, 1500, 3], 4096, 128)])
def test_grouped_gemm_dgrad_tolerance(M_list, N, K):
    E = len(M_list)
    off = np.concatenate([[0], np.cumsum(M_list)]).astype(np.int64)
    M = int(off[-1])
    ac, as_ = _mx_rows(max(M, 1), K, seed=1, scale=1e-3)
    ac, as_ = ac[:M], as_[:M]
    bc, bs = _mx_rows(E * N, K, seed=2, scale=0.02)
    c = m4.moe_grouped_gemm_bwd_dgrad(torch.from_numpy(ac).cuda(), torch.from_numpy(as_).cuda(),
                                      torch.from_numpy(bc).cuda(), torch.from_numpy(bs).cuda(), cuda_i32(off))
    A64 = mx.dequant_rowwise(ac, as_)
    B64 = mx.dequant_rowwise(bc, bs).reshape(E, N, K)
    exact = og.grouped_nt(A64, B64, off)
    gemm_tol_check(to_np(c).astype(np.float64), exact, og.abs_bound_nt(A64, B64, off), "dgrad")


@pytest.mark.parametrize("beta", [0.0, 1.0])
def test_grouped_gemm_wgrad_tolerance(beta):
    N1, N2 = 160, 96
    M_list = [0, 37, 130, 1, 64, 300]
    E = len(M_list)
    off = np.concatenate([[0], np.cumsum(M_list)]).astype(np.int64)
    offp = mx.padded_offsets(off)
    M = int(off[-1])
    a = synth.randn((M, N1), 1e-3, "cpu", 3, "dh").numpy()
    b = synth.randn((M, N2), 1.0, "cpu", 4, "dh").numpy()
    ac, as_ = mx.quantize_transposed(a, off, mx.RNE, sf_layout=mx.SF_BLOCKS)
    bc, bs = mx.quantize_transposed(b, off, mx.SR, 1, 1, sf_layout=mx.SF_BLOCKS)
    dw0 = np.random.default_rng(5).standard_normal((E, N1, N2)).astype(np.float32)
    dw = torch.from_numpy(dw0.copy()).cuda()
    m4.moe_grouped_gemm_bwd_wgrad(torch.from_numpy(ac).cuda(), torch.from_numpy(as_).cuda(), torch.from_numpy(bc).cuda(),
                                  torch.from_numpy(bs).cuda(), cuda_i32(offp), N1, N2, dw=dw, beta=beta)
    Al = mx.dequant_transposed(ac, as_, off, N1, mx.SF_BLOCKS)
    Bl = mx.dequant_transposed(bc, bs, off, N2, mx.SF_BLOCKS)
    exact = og.wgrad(Al, Bl)
    bound = og.wgrad([np.abs(x) for x in Al], [np.abs(x) for x in Bl])
    got = to_np(dw).astype(np.float64)
    if beta == 1.0:
        got = got - dw0.astype(np.float64)
        bound = bound + np.abs(dw0) * 1e3 * 2.0 ** -24     # the one float32 addition
    else:
        assert not got[0].any()                            # empty expert -> zeros
    gemm_tol_check(got, exact, bound, f"wgrad beta={beta}")


@pytest.mark.parametrize("beta", [0.0, 1.0])
def test_grouped_gemm_wgrad_many_experts(beta):
    """More tiles than resident workgroups: each workgroup walks several tiles,
    including empty experts, one-slab experts and multi-slab experts in a row."""
    N1, N2, E = 256, 192, 300
    rng = np.random.default_rng(11)
    M_list = rng.choice([0, 0, 0, 1, 31, 32, 33, 64, 100, 200, 257], E)
    off = np.concatenate([[0], np.cumsum(M_list)]).astype(np.int64)
    offp = mx.padded_offsets(off)
    M = int(off[-1])
    a = synth.randn((M, N1), 1.0, "cpu", 6, "dh").numpy()
    b = synth.randn((M, N2), 1e-2, "cpu", 7, "dh").numpy()
    ac, as_ = mx.quantize_transposed(a, off, mx.RNE, sf_layout=mx.SF_BLOCKS)
    bc, bs = mx.quantize_transposed(b, off, mx.RNE, sf_layout=mx.SF_BLOCKS)
    dw0 = np.random.default_rng(8).standard_normal((E, N1, N2)).astype(np.float32)
    dw = torch.from_numpy(dw0.copy()).cuda()
    m4.moe_grouped_gemm_bwd_wgrad(torch.from_numpy(ac).cuda(), torch.from_numpy(as_).cuda(), torch.from_numpy(bc).cuda(),
                                  torch.from_numpy(bs).cuda(), cuda_i32(offp), N1, N2, dw=dw, beta=beta)
    Al = mx.dequant_transposed(ac, as_, off, N1, mx.SF_BLOCKS)
    Bl = mx.dequant_transposed(bc, bs, off, N2, mx.SF_BLOCKS)
    exact = og.wgrad(Al, Bl)
    bound = og.wgrad([np.abs(x) for x in Al], [np.abs(x) for x in Bl])
    got = to_np(dw).astype(np.float64)
    if beta == 1.0:
        got = got - dw0.astype(np.float64)
        bound = bound + np.abs(dw0) * 1e3 * 2.0 ** -24
    else:
        assert not got[M_list == 0].any()
    gemm_tol_check(got, exact, bound, f"wgrad many experts beta={beta}")


@pytest.mark.parametrize("M_list,N1,N2", [
    ([0] * 5 + [2000] + [0] * 6 + [1, 0, 33, 0], 128, 128),   # 16 tiles: two workgroups per XCD, most ranges empty
    ([700], 512, 512),                                         # one expert cut into several XCD ranges
    ([3, 0, 1500, 64, 0, 0, 31, 900] * 3, 256, 128),          # 48 tiles, heavy experts next to empty ones
    ([50, 0, 700, 5], 288, 160),                               # a 256-row tile with 32 valid rows
])
def test_grouped_gemm_wgrad_skewed_xcd_ranges(M_list, N1, N2):
    """Tile counts that are multiples of 8 but below the resident grid, with
    token counts skewed so that the cost-balanced per-XCD ranges cut inside
    experts, or hold only empty experts."""
    M_list = np.array(M_list)
    E = len(M_list)
    off = np.concatenate([[0], np.cumsum(M_list)]).astype(np.int64)
    offp = mx.padded_offsets(off)
    M = int(off[-1])
    a = synth.randn((M, N1), 1.0, "cpu", 9, "dh").numpy()
    b = synth.randn((M, N2), 1.0, "cpu", 10, "dh").numpy()
    ac, as_ = mx.quantize_transposed(a, off, mx.RNE, sf_layout=mx.SF_BLOCKS)
    bc, bs = mx.quantize_transposed(b, off, mx.RNE, sf_layout=mx.SF_BLOCKS)
    dw = torch.full((E, N1, N2), float("nan"), dtype=torch.float32, device="cuda")
    m4.moe_grouped_gemm_bwd_wgrad(torch.from_numpy(ac).cuda(), torch.from_numpy(as_).cuda(), torch.from_numpy(bc).cuda(),
                                  torch.from_numpy(bs).cuda(), cuda_i32(offp), N1, N2, dw=dw, beta=0.0)
    Al = mx.dequant_transposed(ac, as_, off, N1, mx.SF_BLOCKS)
    Bl = mx.dequant_transposed(bc, bs, off, N2, mx.SF_BLOCKS)
    exact = og.wgrad(Al, Bl)
    bound = og.wgrad([np.abs(x) for x in Al], [np.abs(x) for x in Bl])
    got = to_np(dw).astype(np.float64)
    assert np.isfinite(got).all()                          # every tile written
    assert not got[M_list == 0].any()
    gemm_tol_check(got, exact, bound, "wgrad skewed")


@pytest.mark.parametrize("N1,N2,E", [(256, 192, 300), (64, 32, 2100)])
def test_grouped_gemm_wgrad_skip_empty(N1, N2, E):
    """MOE4_WGRAD_SKIP_EMPTY: experts without rows keep what dw held (a NaN
    sentinel here), the others are byte for byte the beta = 0 result; both the
    warp-specialized kernel and (E > 2048) the register-staged one."""
    rng = np.random.default_rng(12)
    M_list = rng.choice([0, 0, 0, 1, 31, 32, 33, 64, 100, 200, 257], E) if E < 1000 else rng.choice([0, 0, 1, 5], E)
    off = np.concatenate([[0], np.cumsum(M_list)]).astype(np.int64)
    offp = mx.padded_offsets(off)
    M = int(off[-1])
    a = synth.randn((M, N1), 1.0, "cpu", 6, "dh").numpy()
    b = synth.randn((M, N2), 1e-2, "cpu", 7, "dh").numpy()
    ac, as_ = mx.quantize_transposed(a, off, mx.RNE, sf_layout=mx.SF_BLOCKS)
    bc, bs = mx.quantize_transposed(b, off, mx.RNE, sf_layout=mx.SF_BLOCKS)
    args = [torch.from_numpy(t).cuda() for t in (ac, as_, bc, bs)] + [cuda_i32(offp), N1, N2]
    full = m4.moe_grouped_gemm_bwd_wgrad(*args, beta=0.0)
    dw = torch.full((E, N1, N2), float("nan"), dtype=torch.float32, device="cuda")
    m4.moe_grouped_gemm_bwd_wgrad(*args, dw=dw, beta=0.0, skip_empty=True)
    got = to_np(dw)
    empty = M_list == 0
    assert empty.any() and np.isnan(got[empty]).all()
    assert_bytes_equal(got[~empty].view(np.uint32), to_np(full)[~empty].view(np.uint32), "skip-empty wgrad")


def test_grouped_gemm_wgrad_more_experts_than_offset_staging():
    """More experts than the warp-specialized kernel stages offsets for: the
    register-staged persistent kernel takes over, same results."""
    N1, N2, E = 64, 32, 2100
    rng = np.random.default_rng(21)
    M_list = rng.choice([0, 0, 0, 0, 1, 5, 32, 40], E)
    off = np.concatenate([[0], np.cumsum(M_list)]).astype(np.int64)
    offp = mx.padded_offsets(off)
    M = int(off[-1])
    a = synth.randn((M, N1), 1.0, "cpu", 12, "dh").numpy()
    b = synth.randn((M, N2), 1.0, "cpu", 13, "dh").numpy()
    ac, as_ = mx.quantize_transposed(a, off, mx.RNE, sf_layout=mx.SF_BLOCKS)
    bc, bs = mx.quantize_transposed(b, off, mx.RNE, sf_layout=mx.SF_BLOCKS)
    dw = torch.full((E, N1, N2), float("nan"), dtype=torch.float32, device="cuda")
    m4.moe_grouped_gemm_bwd_wgrad(torch.from_numpy(ac).cuda(), torch.from_numpy(as_).cuda(), torch.from_numpy(bc).cuda(),
                                  torch.from_numpy(bs).cuda(), cuda_i32(offp), N1, N2, dw=dw, beta=0.0)
    Al = mx.dequant_transposed(ac, as_, off, N1, mx.SF_BLOCKS)
    Bl = mx.dequant_transposed(bc, bs, off, N2, mx.SF_BLOCKS)
    exact = og.wgrad(Al, Bl)
    bound = og.wgrad([np.abs(x) for x in Al], [np.abs(x) for x in Bl])
    got = to_np(dw).astype(np.float64)
    assert np.isfinite(got).all()
    assert not got[M_list == 0].any()
    gemm_tol_check(got, exact, bound, "wgrad fallback")


@pytest.mark.parametrize("T,k,d", [(37, 3, 200), (4, 1, 8), (130, 8, 4096)])
def test_dgates_tolerance(T, k, d):
    """dg[t, j] = <dy[t], Yp[inv[t*k + j]]> against the oracle's exact sums."""
    rng = np.random.default_rng(T + d)
    inv = rng.permutation(T * k).astype(np.int32)
    yp = rng.standard_normal((T * k, d)).astype(np.float32)
    dy_t = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    dy = synth.bf16_bits(dy_t)
    dg = to_np(m4.moe_dgates(dy_t.cuda(), torch.from_numpy(yp).cuda(), cuda_i32(inv), k)).astype(np.float64)
    exact = olayer.dgates(dy, yp, inv, k)
    bound = olayer.dgates(dy & 0x7FFF, np.abs(yp), inv, k)
    gemm_tol_check(dg, exact, bound, f"dgates T={T} k={k} d={d}")


@pytest.mark.parametrize("T,E,k", [(300, 384, 8), (5, 4, 1), (64, 1024, 16), (77, 40, 5)])
def test_route_backward_bit_exact(T, E, k):
    """Softmax backward into the logits: the library's float32 steps equal the
    oracle's, bit for bit, on the forward's own gates and indices."""
    rng = np.random.default_rng(T * 7 + E)
    logits = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32))
    r = m4.moe_route_topk(logits.cuda(), k)
    dg = torch.from_numpy(rng.standard_normal((T, k)).astype(np.float32))
    got = to_np(m4.moe_route_backward(dg.cuda(), r["gates"], r["idx"], E))
    want = route.route_backward(dg.numpy(), to_np(r["gates"]), to_np(r["idx"]), E)
    assert_bytes_equal(got.view(np.uint32), want.view(np.uint32), "dlogits")


# warp-specialised kernels for N = 128 (128 x 128) and N = 512 (128 x 256)
@pytest.mark.parametrize("M_list,N,K", [([0, 37, 130, 1, 300], 192, 256), ([256], 128, 1024), ([3, 200], 96, 128),
                                        ([0, 37, 130, 1, 300], 512, 256)])
def test_grouped_gemm_mx_bf16_and_f32(M_list, N, K):
    """The MXFP8 forward GEMM: bf16 output within tolerance of the exact
    product; float32 output identical to the dgrad call."""
    E = len(M_list)
    off = np.concatenate([[0], np.cumsum(M_list)]).astype(np.int64)
    M = int(off[-1])
    a = synth.randn((M, K), 1.0, "cpu", 15, "dh").numpy()
    b = synth.randn((E * N, K), 0.05, "cpu", 16, "dh").numpy()
    ac, as_ = mx.quantize_rowwise(a, mx.RNE)
    bc, bs = mx.quantize_rowwise(b, mx.RNE)
    args = (torch.from_numpy(ac).cuda(), torch.from_numpy(as_).cuda(), torch.from_numpy(bc).cuda().view(E, N, K),
            torch.from_numpy(bs).cuda().view(E, N, K // 32), cuda_i32(off))
    c16 = m4.moe_grouped_gemm_mx(*args, torch.bfloat16)
    c32 = m4.moe_grouped_gemm_mx(*args, torch.float32)
    cdg = m4.moe_grouped_gemm_bwd_dgrad(*args)
    assert torch.equal(c32, cdg)
    A64 = mx.dequant_rowwise(ac, as_)
    B64 = mx.dequant_rowwise(bc, bs).reshape(E, N, K)
    exact = og.grouped_nt(A64, B64, off)
    got = fmt.bf16_to_f32(to_np(c16.view(torch.int16)).view(np.uint16)).astype(np.float64)
    gemm_tol_check(got, exact, og.abs_bound_nt(A64, B64, off), "mx gemm bf16", out_bf16=True)


@pytest.mark.parametrize("M_list,N,K", [([300, 0, 37, 1, 129], 256, 512), ([5, 64, 200], 384, 256),
                                        ([1000, 3], 1536, 1024), ([3, 12, 0, 40, 1, 19], 256, 512),
                                        (_FEW, 192, 512)])
def test_fwd_silu_amax_epilogue_matches_separate_pass(M_list, N, K):
    """moe_grouped_gemm_fwd_silu_amax (SiLU amax per expert folded into the up
    GEMM's epilogue) gives the same U, and nvfp4_quant_46 with PRE_SILU_AMAX on
    its workspace the same H (codes, scales, tensor scales) byte for byte as
    the plain GEMM followed by nvfp4_quant_46 with PRE_SILU (whose amax pass is
    pinned to the oracle elsewhere)."""
    E = len(M_list)
    off, qa, qb = _fwd_operands(M_list, N, K, seed=N + K + 7)
    args = (torch.from_numpy(qa["codes"]).cuda(), torch.from_numpy(qa["sf"]).cuda(), torch.from_numpy(qa["ts"]).cuda(),
            torch.from_numpy(qb["codes"]).cuda().view(E, N, K // 2), torch.from_numpy(qb["sf"]).cuda().view(E, N, K // 16),
            torch.from_numpy(qb["ts"]).cuda(), cuda_i32(off))
    u1, ws = m4.moe_grouped_gemm_fwd_silu_amax(*args)
    u2 = m4.moe_grouped_gemm_fwd(*args, torch.bfloat16)
    assert torch.equal(u1.view(torch.int16), u2.view(torch.int16))
    h1 = m4.nvfp4_quant_46(u1, m4.NVFP4_4OVER6, cuda_i32(off), m4.PRE_SILU_AMAX, ws=ws)
    h2 = m4.nvfp4_quant_46(u2, m4.NVFP4_4OVER6, cuda_i32(off), m4.PRE_SILU)
    for a, b, what in zip(h1, h2, ("codes", "scales", "tensor scales")):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), what


def test_fwd_silu_amax_unsupported_shape():
    # K % 256 != 0: neither the warp-specialised nor the few-rows kernels
    off, qa, qb = _fwd_operands([40, 24], 96, 320, seed=5)
    with pytest.raises(m4.Moe4Unsupported):
        m4.moe_grouped_gemm_fwd_silu_amax(
            torch.from_numpy(qa["codes"]).cuda(), torch.from_numpy(qa["sf"]).cuda(), torch.from_numpy(qa["ts"]).cuda(),
            torch.from_numpy(qb["codes"]).cuda().view(2, 96, 160), torch.from_numpy(qb["sf"]).cuda().view(2, 96, 20),
            torch.from_numpy(qb["ts"]).cuda(), cuda_i32(off))
