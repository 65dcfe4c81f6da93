"""GPU parity of the quantisers against the oracle: bit-exact codes and scales."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import assert_bytes_equal, bf16_from_bits, cuda_i32, to_np
from oracle import formats as fmt
from oracle import mxfp8 as mx
from oracle import nvfp4 as nv
from oracle import silu as osilu

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import precision_moe_numerics_quant_amd as m4

SF_ROWS, SF_BLOCKS = 0, 1                                   # the library's scale-arrangement codes
LAYOUTS = {SF_ROWS: mx.SF_ROWS, SF_BLOCKS: mx.SF_BLOCKS}    # ... and the oracle's names for them


def _bf16_input(R, C, seed, outliers=True):
    x = synth.activations(R, C, "cpu", seed, outlier_p=0.001 if outliers else 0.0, outlier_mul=20.0)
    return synth.bf16_bits(x)


# ------------------------------------------------------------------ SiLU tables

def test_silu_tables_exhaustive():
    bits, s_ref, d_ref = osilu.tables()
    u = bf16_from_bits(bits)
    s, d = m4.moe_silu_eval(u)
    assert_bytes_equal(to_np(s).view(np.uint32), s_ref.view(np.uint32), "silu")
    assert_bytes_equal(to_np(d).view(np.uint32), d_ref.view(np.uint32), "dsilu")


# ------------------------------------------------------------------------ NVFP4

@pytest.mark.parametrize("mode", [m4_mode for m4_mode in (6, 46)])
@pytest.mark.parametrize("R,C", [(1, 16), (7, 48), (256, 256), (333, 1536)])
def test_nvfp4_bf16_one_group(R, C, mode):
    xb = _bf16_input(R, C, seed=R * 7 + C)
    codes, sf, ts = m4.nvfp4_quant_46(bf16_from_bits(xb), mode)
    ref = nv.nvfp4_quantize(xb, mode)
    assert_bytes_equal(to_np(ts).view(np.uint32), ref["ts"].view(np.uint32), "ts")
    assert_bytes_equal(to_np(sf), ref["sf"], "sf")
    assert_bytes_equal(to_np(codes), ref["codes"], "codes")


def test_nvfp4_f32_weights_grouped_mode6():
    E, F, d = 5, 96, 160
    w = synth.randn((E, F, d), 0.02, "cpu", 3, "w_up").numpy()
    off = np.arange(E + 1) * F
    codes, sf, ts = m4.nvfp4_quant_46(torch.from_numpy(w).cuda().view(E * F, d), 6, cuda_i32(off))
    ref = nv.nvfp4_quantize(w.reshape(E * F, d), 6, off)
    assert_bytes_equal(to_np(ts).view(np.uint32), ref["ts"].view(np.uint32), "ts")
    assert_bytes_equal(to_np(sf), ref["sf"], "sf")
    assert_bytes_equal(to_np(codes), ref["codes"], "codes")


def test_nvfp4_f32_weights_grouped_mode6_many_chunks():
    """More 1024-element chunks than resident waves: each wave walks several
    chunks and crosses expert boundaries (per-expert amax and scale)."""
    E, F, d = 16, 512, 2048
    w = synth.randn((E, F, d), 0.02, "cpu", 9, "w_up").numpy()
    w[3] *= 40.0                                   # one expert with a much larger range
    w[7] = 0.0                                     # one all-zero expert (S = 1)
    off = np.arange(E + 1) * F
    codes, sf, ts = m4.nvfp4_quant_46(torch.from_numpy(w).cuda().view(E * F, d), 6, cuda_i32(off))
    ref = nv.nvfp4_quantize(w.reshape(E * F, d), 6, off)
    assert_bytes_equal(to_np(ts).view(np.uint32), ref["ts"].view(np.uint32), "ts")
    assert_bytes_equal(to_np(sf), ref["sf"], "sf")
    assert_bytes_equal(to_np(codes), ref["codes"], "codes")


def test_nvfp4_bf16_46_many_chunks_ragged_groups():
    R, C = 8192, 1024
    off = np.array([0, 100, 100, 4000, 8192])
    xb = synth.bf16_bits(synth.activations(R, C, "cpu", 3, outlier_p=0.001, outlier_mul=20.0))
    codes, sf, ts = m4.nvfp4_quant_46(bf16_from_bits(xb), 46, cuda_i32(off))
    ref = nv.nvfp4_quantize(xb, 46, off)
    assert_bytes_equal(to_np(ts).view(np.uint32), ref["ts"].view(np.uint32), "ts")
    assert_bytes_equal(to_np(sf), ref["sf"], "sf")
    assert_bytes_equal(to_np(codes), ref["codes"], "codes")


def test_nvfp4_ragged_groups_silu():
    # empty groups, single-row groups and a group larger than one workgroup's rows
    R, C = 400, 512
    off = np.array([0, 0, 1, 1, 90, 91, 300, 400, 400])
    u = synth.randn((R, C), 1.5, "cpu", 11, "u", torch.bfloat16)
    ub = synth.bf16_bits(u)
    codes, sf, ts = m4.nvfp4_quant_46(u.cuda(), 46, cuda_i32(off), m4.PRE_SILU)
    ref = nv.nvfp4_quantize(osilu.silu_f32(ub), 46, off)
    assert_bytes_equal(to_np(ts).view(np.uint32), ref["ts"].view(np.uint32), "ts")
    assert_bytes_equal(to_np(sf), ref["sf"], "sf")
    assert_bytes_equal(to_np(codes), ref["codes"], "codes")


def test_nvfp4_special_values():
    # zeros, -0, tiny and huge magnitudes, exact grid points, ties
    C = 64
    rows = [np.zeros(C), -np.zeros(C), np.full(C, 1e-38), np.linspace(-6, 6, C), np.full(C, 3e38),
            np.r_[np.full(C // 2, 0.25), np.full(C // 2, -0.75)], np.float32(2.0) ** np.arange(-32, 32)]
    x = np.stack(rows).astype(np.float32)
    for mode in (6, 46):
        for groups in (None, np.arange(len(rows) + 1)):
            off_t = None if groups is None else cuda_i32(groups)
            codes, sf, ts = m4.nvfp4_quant_46(torch.from_numpy(x).cuda(), mode, off_t)
            ref = nv.nvfp4_quantize(x, mode, groups)
            assert_bytes_equal(to_np(ts).view(np.uint32), ref["ts"].view(np.uint32), "ts")
            assert_bytes_equal(to_np(sf), ref["sf"], "sf")
            assert_bytes_equal(to_np(codes), ref["codes"], "codes")


def test_nvfp4_power_of_two_equivariance_gpu():
    xb = _bf16_input(64, 256, seed=5)
    x = bf16_from_bits(xb)
    base = m4.nvfp4_quant_46(x, 46)
    for j in (-9, 4):
        y = (x.float() * 2.0 ** j).to(torch.bfloat16)
        q = m4.nvfp4_quant_46(y, 46)
        assert torch.equal(q[0], base[0]) and torch.equal(q[1], base[1])
        assert q[2].item() == base[2].item() * 2.0 ** j


@pytest.mark.parametrize("pre", ["none", "silu"])
def test_nvfp4_group_split_invariance_gpu(pre):
    """Quantising ragged groups in one launch or each group in a launch of its
    own (other grids, other ticket orders) gives the same bytes."""
    xb = _bf16_input(600, 512, seed=8)
    x = bf16_from_bits(xb)
    off = np.array([0, 100, 100, 357, 361, 600])
    op = m4.PRE_SILU if pre == "silu" else m4.PRE_NONE
    whole = m4.nvfp4_quant_46(x, 46, cuda_i32(off), op)
    for g in range(len(off) - 1):
        r0, r1 = int(off[g]), int(off[g + 1])
        if r1 == r0:
            continue
        part = m4.nvfp4_quant_46(x[r0:r1].contiguous(), 46, cuda_i32(np.array([0, r1 - r0])), op)
        assert torch.equal(part[0], whole[0][r0:r1]) and torch.equal(part[1], whole[1][r0:r1]), g
        assert part[2].view(torch.int32)[0].item() == whole[2].view(torch.int32)[g].item(), g


def test_nvfp4_dequant_matches_oracle():
    xb = _bf16_input(96, 128, seed=6)
    codes, sf, ts = m4.nvfp4_quant_46(bf16_from_bits(xb), 46)
    out = m4.nvfp4_dequant(codes, sf, ts)
    ref = nv.nvfp4_dequantize(to_np(codes), to_np(sf), to_np(ts))
    assert_bytes_equal(to_np(out).view(np.uint32), ref.view(np.uint32), "dequant")


def test_nvfp4_config2_full_size_sampled_rows():
    """16384 x 7168 bf16 with 1% of rows x50, in the launch the benchmark times;
    rows sampled (including outlier rows) are compared with the oracle, which
    takes the GPU-independent tensor amax from the full input."""
    cfg = synth.CONFIGS[2]
    x = synth.config_inputs(2, device="cuda")["x"]
    codes, sf, ts = m4.nvfp4_quant_46(x, 46)
    xs = x.float().abs().max().item()
    S_ref = np.float32(np.float32(xs) / np.float32(1792.0))
    assert to_np(ts)[0] == S_ref
    rng = np.random.default_rng(0)
    rows = np.unique(np.r_[rng.choice(cfg["R"], 48, replace=False), 0, cfg["R"] - 1])
    big = torch.nonzero(x[:, :64].float().abs().amax(1) > 30).flatten().cpu().numpy()[:8]
    rows = np.unique(np.r_[rows, big])
    xb = synth.bf16_bits(x[torch.from_numpy(rows).cuda()])
    q, sc, _ = nv.quantize_blocks(fmt.bf16_to_f32(xb), np.full(len(rows), S_ref, np.float32), 46)
    assert_bytes_equal(to_np(sf[torch.from_numpy(rows).cuda()]), sc.astype(np.uint8), "sf")
    assert_bytes_equal(to_np(codes[torch.from_numpy(rows).cuda()]), nv.pack_codes(q), "codes")


# ------------------------------------------------------------------------ MXFP8

def _nvfp4_operand(R, C, seed, groups=None, per_group=True):
    xb = _bf16_input(R, C, seed)
    ref = nv.nvfp4_quantize(xb, 46, groups if per_group else None)
    return ref


@pytest.mark.parametrize("R,C,groups", [
    (64, 128, None),
    (100, 96, [0, 0, 33, 33, 34, 100]),
    (517, 256, [0, 200, 201, 480, 517]),
    (300, 1056, [0, 7, 7, 299, 300]),
])
@pytest.mark.parametrize("lay", [SF_ROWS, SF_BLOCKS])
def test_requant_sr_t_bit_exact(R, C, groups, lay):
    off = np.array([0, R]) if groups is None else np.array(groups)
    ref_q = _nvfp4_operand(R, C, R + C, off)
    offp = mx.padded_offsets(off)
    c_ref, s_ref = mx.requant_sr_t(ref_q["codes"], ref_q["sf"], ref_q["ts"], off, True, seed=1, stream_id=3,
                                   sf_layout=LAYOUTS[lay])
    oc, os_ = m4.mxfp8_requant_sr_T(torch.from_numpy(ref_q["codes"]).cuda(), torch.from_numpy(ref_q["sf"]).cuda(),
                                    torch.from_numpy(ref_q["ts"]).cuda(), cuda_i32(off), cuda_i32(offp), True, 1, 3,
                                    sf_layout=lay)
    n = C * offp[-1]
    assert_bytes_equal(to_np(os_)[: n // 32], s_ref, "requant scales")
    assert_bytes_equal(to_np(oc)[:n], c_ref, "requant codes")


def test_requant_single_tensor_scale_and_seeds():
    R, C = 96, 64
    off = np.array([0, 10, 96])
    xb = _bf16_input(R, C, 9)
    ref_q = nv.nvfp4_quantize(xb, 46)
    offp = mx.padded_offsets(off)
    for seed, sid in ((1, 0), (7, 1), (1 << 40, 17)):
        c_ref, s_ref = mx.requant_sr_t(ref_q["codes"], ref_q["sf"], ref_q["ts"], off, False, seed, sid)
        oc, os_ = m4.mxfp8_requant_sr_T(torch.from_numpy(ref_q["codes"]).cuda(), torch.from_numpy(ref_q["sf"]).cuda(),
                                        torch.from_numpy(ref_q["ts"]).cuda(), cuda_i32(off), cuda_i32(offp), False,
                                        seed, sid)
        n = C * offp[-1]
        assert_bytes_equal(to_np(oc)[:n], c_ref, f"codes seed {seed}")
        assert_bytes_equal(to_np(os_)[: n // 32], s_ref, f"scales seed {seed}")


def test_sr_conversion_all_random_words():
    """Every 16-bit random word against the oracle's rounding rule, for values
    across the E4M3 range (normal, subnormal, negative, grid points)."""
    vals = np.float32([1.03125, 1.0 + 2 ** -20, 7.77, 300.1, 447.9, 0.0005, 0.0123, -2.3, -0.004, 3.0, 2 ** -7 + 2 ** -20])
    # one MX block per value: the value at column 0 plus 448 * 2**e-pinning companion so e = 0
    R = 65536
    C = 32
    x = np.zeros((len(vals), R, C), dtype=np.float32)
    # transposed mode quantises along rows: put the value in every row of column 0 and
    # make the block amax 448 with a companion row so that e = 0 -> w = v
    for i, v in enumerate(vals):
        x[i, :, 0] = v
    # rows are blocks of 32 along the token dimension: force amax 448 in row 0 of each block
    x[:, ::32, 0] = 448.0
    for i in range(len(vals)):
        off = np.array([0, R])
        c_ref, s_ref = mx.quantize_transposed(x[i], off, mx.SR, seed=1, stream_id=5)
        oc, os_ = m4.mxfp8_quant(torch.from_numpy(x[i]).cuda(), transpose=True, group_row_off=cuda_i32(off),
                                 group_off_pad=cuda_i32(off), max_pr=R, rnd=m4.SR, seed=1, stream_id=5)
        assert_bytes_equal(to_np(oc), c_ref, f"SR codes value {vals[i]}")
        assert_bytes_equal(to_np(os_), s_ref, f"SR scales value {vals[i]}")


@pytest.mark.parametrize("rnd", [0, 1])
@pytest.mark.parametrize("transpose", [False, "rows", "blocks"])
def test_mxfp8_grad_quant_gated_rows(rnd, transpose):
    T, d, k, E = 130, 96, 3, 7
    rng = np.random.default_rng(1)
    dy = synth.randn((T, d), 1e-3, "cpu", 2, "dy", torch.bfloat16)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    from oracle import route
    P = route.permutation(idx, E)
    gates = rng.random((T, k)).astype(np.float32)
    dyp = (gates.reshape(-1)[P["perm"]][:, None] * fmt.bf16_to_f32(synth.bf16_bits(dy))[P["perm"] // k]).astype(np.float32)
    A = T * k
    args = dict(rows=A, row_map=cuda_i32(P["perm"]), map_div=k, row_scale=torch.from_numpy(gates.reshape(-1)).cuda(),
                rnd=rnd, seed=3, stream_id=4)
    if transpose:
        lay = SF_ROWS if transpose == "rows" else SF_BLOCKS
        oc, os_ = m4.mxfp8_quant(dy.cuda(), transpose=True, group_row_off=cuda_i32(P["off"]),
                                 group_off_pad=cuda_i32(P["off_pad"]), sf_layout=lay, **args)
        c_ref, s_ref = mx.quantize_transposed(dyp, P["off"], rnd, 3, 4, sf_layout=LAYOUTS[lay])
        n = d * P["off_pad"][-1]
        assert_bytes_equal(to_np(oc)[:n], c_ref, "codes")
        assert_bytes_equal(to_np(os_)[: n // 32], s_ref, "scales")
    else:
        oc, os_ = m4.mxfp8_quant(dy.cuda(), **args)
        c_ref, s_ref = mx.quantize_rowwise(dyp, rnd, 3, 4)
        assert_bytes_equal(to_np(oc), c_ref, "codes")
        assert_bytes_equal(to_np(os_), s_ref, "scales")


@pytest.mark.parametrize("lay", [SF_ROWS, SF_BLOCKS])
@pytest.mark.parametrize("rnd", [0, 1])                          # RNE, SR
def test_mxfp8_quant_rows_T_gated_against_oracle(rnd, lay):
    """Both copies of the gated, gathered dY from one read, against the
    oracle's row-wise and transposed quantisations (ragged groups, an empty
    expert, a column count past one 128-column tile)."""
    T, d, k, E = 130, 160, 3, 7
    rng = np.random.default_rng(11)
    dy = synth.randn((T, d), 1e-3, "cpu", 12, "dy", torch.bfloat16)
    idx = np.stack([rng.permutation(E - 1)[:k] for _ in range(T)])        # expert E - 1 gets no tokens
    from oracle import route
    P = route.permutation(idx, E)
    gates = rng.random((T, k)).astype(np.float32)
    dyp = (gates.reshape(-1)[P["perm"]][:, None] * fmt.bf16_to_f32(synth.bf16_bits(dy))[P["perm"] // k]).astype(np.float32)
    A = T * k
    rc_, rs_, tc, ts = m4.mxfp8_quant_rows_T(dy.cuda(), cuda_i32(P["off"]), cuda_i32(P["off_pad"]), rows=A,
                                             row_map=cuda_i32(P["perm"]), map_div=k,
                                             row_scale=torch.from_numpy(gates.reshape(-1)).cuda(), rnd=rnd, seed=3,
                                             stream_id=4, sf_layout=lay)
    c_ref, s_ref = mx.quantize_rowwise(dyp, rnd, 3, 4)
    assert_bytes_equal(to_np(rc_), c_ref, "row codes")
    assert_bytes_equal(to_np(rs_), s_ref, "row scales")
    c_ref, s_ref = mx.quantize_transposed(dyp, P["off"], rnd, 3, 4, sf_layout=LAYOUTS[lay])
    n = d * P["off_pad"][-1]
    assert_bytes_equal(to_np(tc)[:n], c_ref, "transposed codes")
    assert_bytes_equal(to_np(ts)[: n // 32], s_ref, "transposed scales")


@pytest.mark.parametrize("rnd", [0, 1])                          # RNE, SR
def test_mxfp8_quant_rows_T_dsilu_matches_separate_calls(rnd):
    """SiLU'-scaled float32 gradient: the fused call equals the two separate
    calls byte for byte (each pinned to the oracle above)."""
    R, F = 300, 256
    off = np.array([0, 40, 40, 170, 300])
    dh = torch.from_numpy(synth.randn((R, F), 1e-3, "cpu", 14, "dh").numpy()).cuda()
    u = synth.randn((R, F), 2.0, "cpu", 15, "u", torch.bfloat16).cuda()
    offp = mx.padded_offsets(off)
    kw = dict(dsilu_src=u, rnd=rnd, seed=9, stream_id=2)
    rc_, rs_, tc, ts = m4.mxfp8_quant_rows_T(dh, cuda_i32(off), cuda_i32(offp), sf_layout=SF_BLOCKS, **kw)
    oc, os_ = m4.mxfp8_quant(dh, **kw)
    tc2, ts2 = m4.mxfp8_quant(dh, transpose=True, group_row_off=cuda_i32(off), group_off_pad=cuda_i32(offp),
                              sf_layout=SF_BLOCKS, **kw)
    assert torch.equal(rc_, oc) and torch.equal(rs_, os_)
    n = F * offp[-1]
    assert torch.equal(tc[:n], tc2[:n]) and torch.equal(ts[: n // 32], ts2[: n // 32])


@pytest.mark.parametrize("transpose", [False, "rows", "blocks"])
def test_mxfp8_grad_quant_dsilu(transpose):
    R, F = 150, 128
    off = np.array([0, 40, 40, 150])
    dh = synth.randn((R, F), 1e-3, "cpu", 4, "dh").numpy()
    u = synth.randn((R, F), 2.0, "cpu", 5, "u", torch.bfloat16)
    du = (dh * osilu.dsilu_f32(synth.bf16_bits(u))).astype(np.float32)
    if transpose:
        offp = mx.padded_offsets(off)
        lay = SF_ROWS if transpose == "rows" else SF_BLOCKS
        oc, os_ = m4.mxfp8_quant(torch.from_numpy(dh).cuda(), transpose=True, dsilu_src=u.cuda(),
                                 group_row_off=cuda_i32(off), group_off_pad=cuda_i32(offp), sf_layout=lay)
        c_ref, s_ref = mx.quantize_transposed(du, off, mx.RNE, sf_layout=LAYOUTS[lay])
        n = F * offp[-1]
        assert_bytes_equal(to_np(oc)[:n], c_ref, "codes")
        assert_bytes_equal(to_np(os_)[: n // 32], s_ref, "scales")
    else:
        oc, os_ = m4.mxfp8_quant(torch.from_numpy(dh).cuda(), dsilu_src=u.cuda())
        c_ref, s_ref = mx.quantize_rowwise(du, mx.RNE)
        assert_bytes_equal(to_np(oc), c_ref, "codes")
        assert_bytes_equal(to_np(os_), s_ref, "scales")


@pytest.mark.parametrize("lay", [SF_ROWS, SF_BLOCKS])
def test_requant_config2_full_size_sampled_columns(lay):
    """16384 x 7168 requant in the benchmark's launch; output rows (source
    columns) sampled and compared with the oracle on the same NVFP4 input."""
    x = synth.config_inputs(2, device="cuda")["x"]
    codes, sf, ts = m4.nvfp4_quant_46(x, 46)
    R, C = x.shape
    off = cuda_i32([0, R])
    oc, os_ = m4.mxfp8_requant_sr_T(codes, sf, ts, off, off, True, 1, 0, max_pr=R, sf_layout=lay)
    rng = np.random.default_rng(1)
    cols = np.unique(np.r_[rng.choice(C // 16, 6, replace=False) * 16, C - 16])   # whole NVFP4 blocks
    for c0 in cols:
        blk = slice(c0 // 2, c0 // 2 + 8)
        sub_codes = to_np(codes[:, blk])
        sub_sf = to_np(sf[:, c0 // 16: c0 // 16 + 1])
        q = nv.unpack_codes(sub_codes)
        v = nv.dequant_values(q, np.repeat(sub_sf.astype(np.int64), 16, axis=1), to_np(ts)[0])
        # element (r, c0 + j) has source index r * C + c0 + j: quantise with that index map
        got_c = to_np(oc).reshape(C, R)[c0:c0 + 16]
        got_s = (to_np(os_).reshape(C, R // 32) if lay == SF_ROWS else to_np(os_).reshape(R // 32, C).T)[c0:c0 + 16]
        vt = v.T.astype(np.float64)
        nb = R // 32
        idx = (np.arange(R, dtype=np.uint64)[None, :] * np.uint64(C) + (np.uint64(c0) + np.arange(16, dtype=np.uint64))[:, None])
        cc, ss = mx.quantize_blocks_rows(v.T.reshape(16 * nb, 32), mx.SR, 1, 0, idx.reshape(16 * nb, 32))
        assert_bytes_equal(got_c, cc.reshape(16, R), f"codes cols {c0}")
        assert_bytes_equal(got_s, ss.reshape(16, nb), f"scales cols {c0}")


def test_run_twice_deterministic():
    xb = _bf16_input(300, 512, 12)
    x = bf16_from_bits(xb)
    a = m4.nvfp4_quant_46(x, 46)
    b = m4.nvfp4_quant_46(x, 46)
    assert all(torch.equal(p, q) for p, q in zip(a, b))
    off = cuda_i32([0, 300])
    r1 = m4.mxfp8_requant_sr_T(a[0], a[1], a[2], off, cuda_i32([0, 320]), True, 1, 0)
    r2 = m4.mxfp8_requant_sr_T(a[0], a[1], a[2], off, cuda_i32([0, 320]), True, 1, 0)
    n = 512 * 320      # the written extent; the buffers are sized by the padded upper bound
    assert torch.equal(r1[0][:n], r2[0][:n]) and torch.equal(r1[1][:n // 32], r2[1][:n // 32])


# The first six take the ticketed kernel; (320, 32, 512) and (200, 96, 1056)
# have more tiles than the launch has workgroups (two per CU), so workgroups
# take many amax and encode tickets each.  The rest take the single-read
# kernel (groups of a multiple of 128 rows and 256 columns, a multiple of 32
# tiles of 128 x 64): one round or a few, 33 groups (rounds in threes and a
# tail), 128 tiles per group, and groups whose tensor scales fall outside the
# range where the MX factor folds into one multiply (tiny and huge values).
@pytest.mark.parametrize("G,Rg,C", [(1, 32, 32), (3, 64, 1056), (2, 160, 512), (5, 96, 96), (320, 32, 512),
                                    (200, 96, 1056), (1, 128, 8192), (2, 512, 512), (3, 256, 1024),
                                    (7, 128, 2048), (33, 256, 2048), (5, 1024, 512)])
def test_fused_weight_quant_requant_bit_exact(G, Rg, C):
    """nvfp4_quant_requant_T equals nvfp4_quant_46 (mode 6, G equal groups)
    followed by mxfp8_requant_sr_T (row-major scales), byte for byte, against
    the oracle's two steps."""
    R = G * Rg
    rng = np.random.default_rng(G * 1000 + C)
    w = (rng.standard_normal((R, C)) * 0.02).astype(np.float32)
    w[rng.random((R, C)) < 0.002] *= 40.0                       # outliers
    w[Rg:2 * Rg] *= 0.0 if G > 2 else 1.0                        # an all-zero group
    if G > 4:
        w[3 * Rg:4 * Rg] *= np.float32(2.0 ** -110)              # tensor scale near 2^-120
        w[4 * Rg:5 * Rg] *= np.float32(2.0 ** 20)                # tensor scale near 2^10
    off = np.arange(G + 1) * Rg
    q = nv.nvfp4_quantize(w, nv.MODE_6, off)
    mc_ref, ms_ref = mx.requant_sr_t(q["codes"], q["sf"], q["ts"], off, True, seed=7, stream_id=19)
    codes, sf, ts, mc, ms = m4.nvfp4_quant_requant_T(torch.from_numpy(w).cuda(), G, seed=7, stream_id=19)
    assert_bytes_equal(to_np(codes), q["codes"], "codes")
    assert_bytes_equal(to_np(sf), q["sf"], "scales")
    assert_bytes_equal(to_np(ts).view(np.uint32), np.asarray(q["ts"], dtype=np.float32).view(np.uint32), "ts")
    assert_bytes_equal(to_np(mc), mc_ref, "mx codes")
    assert_bytes_equal(to_np(ms), ms_ref, "mx scales")


def test_fused_weight_quant_midpoint_scales():
    """The single-read weight kernel where its shortcuts must step aside:
    group 0 has the tensor scale S = 2^-8 exactly (amax 2688 * 2^-8) and
    16-blocks whose amax / (6 S) is exactly a midpoint between two E4M3
    values, so the product with the rounded reciprocal 1 / (6 S) cannot decide
    the scale byte and the division must (ties to even); group 1 is so small
    (about 2^-127, float32 subnormals) that 6 S is subnormal and every scale
    byte comes from the division; group 2 is ordinary.  Byte for byte against
    the oracle."""
    G, Rg, C = 3, 256, 1024                                      # 8 x 4 = 32 tiles of 32 x 256 per group
    rng = np.random.default_rng(77)
    w = (rng.standard_normal((G * Rg, C)) * 0.004).astype(np.float32)
    w[0, 0] = np.float32(2688.0 * 2.0 ** -8)                     # group 0's amax: S = 2^-8
    mids = [(2 * n + 1) / 16.0 * 2.0 ** e for n in range(8, 16) for e in range(-4, 3)]
    blocks = rng.choice(Rg * (C // 16) - 1, size=len(mids), replace=False) + 1
    for m, b in zip(mids, blocks):                               # block amax 6 m 2^-8, the rest below it
        r, c = divmod(int(b), C // 16)
        blk = (rng.random(16) * 2 - 1) * (6.0 * m * 2.0 ** -8) * 0.9
        blk[rng.integers(16)] = 6.0 * m * 2.0 ** -8 * (1 if rng.random() < 0.5 else -1)
        w[r, 16 * c:16 * c + 16] = blk.astype(np.float32)
    w[Rg:2 * Rg] *= np.float32(2.0 ** -120)
    w[Rg:2 * Rg] *= np.float32(2.0 ** -7)                        # (two steps: the factor itself is normal)
    assert np.float32(np.abs(w[Rg:2 * Rg]).max()) / np.float32(2688.0) * 6 < 2.0 ** -126
    off = np.arange(G + 1) * Rg
    q = nv.nvfp4_quantize(w, nv.MODE_6, off)
    assert np.asarray(q["ts"], dtype=np.float32)[0] == np.float32(2.0 ** -8)
    mc_ref, ms_ref = mx.requant_sr_t(q["codes"], q["sf"], q["ts"], off, True, seed=5, stream_id=3)
    codes, sf, ts, mc, ms = m4.nvfp4_quant_requant_T(torch.from_numpy(w).cuda(), G, seed=5, stream_id=3)
    assert_bytes_equal(to_np(ts).view(np.uint32), np.asarray(q["ts"], dtype=np.float32).view(np.uint32), "ts")
    assert_bytes_equal(to_np(sf), q["sf"], "scales")
    assert_bytes_equal(to_np(codes), q["codes"], "codes")
    assert_bytes_equal(to_np(mc), mc_ref, "mx codes")
    assert_bytes_equal(to_np(ms), ms_ref, "mx scales")


@pytest.mark.parametrize("G,Rg,C", [(1, 32, 32), (3, 64, 1056), (2, 160, 512), (5, 96, 96), (320, 32, 512)])
def test_fused_mx_weight_quant_requant_bit_exact(G, Rg, C):
    """mxfp8_quant_requant_T (the MXFP8-forward weights) equals MXFP8 RNE
    row-wise quantisation followed by the transposed SR requantisation of its
    result (G equal groups, row-major scales), byte for byte, against the
    oracle's two steps; rows of tiny (float32-subnormal after scaling) and huge
    values included."""
    R = G * Rg
    rng = np.random.default_rng(G * 1000 + C + 1)
    w = (rng.standard_normal((R, C)) * 0.02).astype(np.float32)
    w[rng.random((R, C)) < 0.002] *= 40.0                       # outliers
    w[Rg:2 * Rg] *= 0.0 if G > 2 else 1.0                        # an all-zero group
    w[0] = (rng.standard_normal(C) * 2.0 ** -130).astype(np.float32)
    w[1] = (rng.standard_normal(C) * 2.0 ** 100).astype(np.float32)
    off = np.arange(G + 1) * Rg
    c_ref, s_ref = mx.quantize_rowwise(w, mx.RNE)
    tc_ref, ts_ref = mx.requant_mx_sr_t(c_ref, s_ref, off, seed=7, stream_id=19, sf_layout=mx.SF_ROWS)
    codes, sf, tc, ts = m4.mxfp8_quant_requant_T(torch.from_numpy(w).cuda(), G, seed=7, stream_id=19)
    assert_bytes_equal(to_np(codes), c_ref, "row codes")
    assert_bytes_equal(to_np(sf), s_ref, "row scales")
    assert_bytes_equal(to_np(tc), tc_ref, "transposed codes")
    assert_bytes_equal(to_np(ts), ts_ref, "transposed scales")
    with pytest.raises(m4.Moe4Error):
        m4.mxfp8_quant_requant_T(torch.zeros(96, 64, device="cuda"), 2)   # groups of 48 rows


def test_fused_weight_quant_rejects_bad_shapes():
    w = torch.zeros(64, 48, device="cuda")
    with pytest.raises(m4.Moe4Error):
        m4.nvfp4_quant_requant_T(w, 2)                               # cols % 32 != 0
    w = torch.zeros(96, 64, device="cuda")
    with pytest.raises(m4.Moe4Error):
        m4.nvfp4_quant_requant_T(w, 2)                               # groups of 48 rows


# bf16 patterns at and around the ends of the SiLU tables: +-0, +-subnormal,
# +-2**-20, just under 2**-16 and 2**-16 (the first entry), either side of
# 2**-8, the last entry (255) and 256, 300 (past the table: per-value rules)
_SILU_EDGES = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x3580, 0xB580, 0x377F, 0xB77F, 0x3780, 0xB780,
                        0x3B7F, 0xBB7F, 0x3B80, 0xBB80, 0x437F, 0xC37F, 0x4380, 0xC380, 0x4396, 0xC396],
                       dtype=np.uint16)


def _planted_u(R, C, seed, rate=1.0 / 700):
    """bf16 bits of N(0, 1.5**2) with about `rate` of the entries replaced by
    _SILU_EDGES: waves that meet one take the per-value path of the SiLU
    evaluation, the others the table-only path."""
    ub = synth.bf16_bits(synth.randn((R, C), 1.5, "cpu", seed, "u", torch.bfloat16)).copy()
    rng = np.random.default_rng(seed)
    hit = rng.random((R, C)) < rate
    ub[hit] = rng.choice(_SILU_EDGES, size=int(hit.sum()))
    return ub


@pytest.mark.parametrize("kind", ["nvfp4", "silu_rows", "silu_T", "dsilu_rows", "dsilu_T", "dsilu_rows_T"])
def test_silu_table_and_per_value_paths(kind):
    """Every quantiser that evaluates SiLU or SiLU' from bf16 U, on U with
    table-end patterns planted among normal values, bit-exact to the oracle."""
    R, C = 520, 256
    off = np.array([0, 7, 7, 300, 520])
    offp = mx.padded_offsets(off)
    n = C * offp[-1]
    ub = _planted_u(R, C, 31)
    assert np.isin(_SILU_EDGES, ub).all()
    u = bf16_from_bits(ub)
    if kind == "nvfp4":
        codes, sf, ts = m4.nvfp4_quant_46(u, 46, cuda_i32(off), m4.PRE_SILU)
        ref = nv.nvfp4_quantize(osilu.silu_f32(ub), 46, off)
        assert_bytes_equal(to_np(ts).view(np.uint32), ref["ts"].view(np.uint32), "ts")
        assert_bytes_equal(to_np(sf), ref["sf"], "sf")
        assert_bytes_equal(to_np(codes), ref["codes"], "codes")
        return
    if kind.startswith("silu"):
        src, ref, kw = u, osilu.silu_f32(ub), dict(pre_op=m4.PRE_SILU)
    else:
        dh = synth.randn((R, C), 1e-3, "cpu", 32, "dh").numpy()
        src, ref, kw = torch.from_numpy(dh).cuda(), (dh * osilu.dsilu_f32(ub)).astype(np.float32), dict(dsilu_src=u)
    if kind.endswith("rows_T"):
        rc_, rs_, tc, ts = m4.mxfp8_quant_rows_T(src, cuda_i32(off), cuda_i32(offp), sf_layout=SF_BLOCKS, **kw)
        c_ref, s_ref = mx.quantize_rowwise(ref, mx.RNE)
        assert_bytes_equal(to_np(rc_), c_ref, "row codes")
        assert_bytes_equal(to_np(rs_), s_ref, "row scales")
        c_ref, s_ref = mx.quantize_transposed(ref, off, mx.RNE, sf_layout=mx.SF_BLOCKS)
        assert_bytes_equal(to_np(tc)[:n], c_ref, "transposed codes")
        assert_bytes_equal(to_np(ts)[: n // 32], s_ref, "transposed scales")
    elif kind.endswith("_T"):
        oc, os_ = m4.mxfp8_quant(src, transpose=True, group_row_off=cuda_i32(off), group_off_pad=cuda_i32(offp), **kw)
        c_ref, s_ref = mx.quantize_transposed(ref, off, mx.RNE)
        assert_bytes_equal(to_np(oc)[:n], c_ref, "codes")
        assert_bytes_equal(to_np(os_)[: n // 32], s_ref, "scales")
    else:
        oc, os_ = m4.mxfp8_quant(src, **kw)
        c_ref, s_ref = mx.quantize_rowwise(ref, mx.RNE)
        assert_bytes_equal(to_np(oc), c_ref, "codes")
        assert_bytes_equal(to_np(os_), s_ref, "scales")


@pytest.mark.parametrize("transpose", [False, True])
def test_mxfp8_quant_silu_pre_op(transpose):
    """MXFP8 of silu(U) for bf16 U (the MXFP8 forward's H), bit-exact."""
    R, F = 150, 128
    u = synth.randn((R, F), 2.0, "cpu", 14, "u", torch.bfloat16)
    h = osilu.silu_f32(synth.bf16_bits(u))
    if transpose:
        off = np.array([0, 40, 40, 150])
        offp = mx.padded_offsets(off)
        oc, os_ = m4.mxfp8_quant(u.cuda(), transpose=True, pre_op=m4.PRE_SILU, group_row_off=cuda_i32(off),
                                 group_off_pad=cuda_i32(offp))
        c_ref, s_ref = mx.quantize_transposed(h, off, mx.RNE)
        n = F * offp[-1]
        assert_bytes_equal(to_np(oc)[:n], c_ref, "codes")
        assert_bytes_equal(to_np(os_)[: n // 32], s_ref, "scales")
    else:
        oc, os_ = m4.mxfp8_quant(u.cuda(), pre_op=m4.PRE_SILU)
        c_ref, s_ref = mx.quantize_rowwise(h, mx.RNE)
        assert_bytes_equal(to_np(oc), c_ref, "codes")
        assert_bytes_equal(to_np(os_), s_ref, "scales")


@pytest.mark.parametrize("R,C,groups", [(64, 128, None), (100, 96, [0, 0, 33, 33, 34, 100]),
                                        (517, 1056, [0, 200, 201, 480, 517])])
@pytest.mark.parametrize("lay", [SF_ROWS, SF_BLOCKS])
def test_requant_mx_sr_t_bit_exact(R, C, groups, lay):
    """MXFP8 row-wise -> MXFP8 SR transposed (the MXFP8 forward's operands)."""
    off = np.array([0, R]) if groups is None else np.array(groups)
    offp = mx.padded_offsets(off)
    rng = np.random.default_rng(R + C)
    x = (rng.standard_normal((R, C)) * np.exp2(rng.integers(-8, 8, (R, 1)))).astype(np.float32)
    x[rng.random((R, C)) < 0.002] *= 50.0
    c, s = mx.quantize_rowwise(x, mx.RNE)
    c_ref, s_ref = mx.requant_mx_sr_t(c, s, off, seed=5, stream_id=33, sf_layout=LAYOUTS[lay])
    oc, os_ = m4.mxfp8_requant_mx_sr_T(torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda(), cuda_i32(off),
                                       cuda_i32(offp), 5, 33, sf_layout=lay)
    n = C * offp[-1]
    assert_bytes_equal(to_np(oc)[:n], c_ref, "codes")
    assert_bytes_equal(to_np(os_)[: n // 32], s_ref, "scales")
