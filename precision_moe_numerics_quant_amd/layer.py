"""The NVFP4-forward / MXFP8-backward MoE expert layer, chained from the C-ABI calls.

The recipe is the one the pages report for Inkling 2 Small's expert layers
(agihunt.info page, "Confirmed": NVFP4 forward with a dedicated kernel, MXFP8
backward with requantisation and stochastic rounding, 4/6 activation
quantisation; lhc.media page: FP32 master weights, BF16 activations, NVFP4
dispatch, the dequantise -> transpose -> requantise step).  Every arithmetic
step runs in the HIP kernels of libmoe4; this module only sequences the calls
and holds the tensors between them.

Forward:  weights -> NVFP4 (mode 6, per-expert tensor scale); route; x ->
NVFP4 4/6 (one tensor scale, quantised once before dispatch); gather rows into
expert order; up GEMM -> U (bf16); silu + NVFP4 4/6 per expert -> Hq; down GEMM
-> Yp (fp32); gate-weighted combine -> y (bf16).

Backward: g * dy gathered into expert order -> MXFP8 (RNE) row-wise and
transposed per expert; forward NVFP4 operands -> MXFP8 by the stochastic-
rounding transposed requantisation (stream 16*layer + role: 0 X, 1 H, 2 W_up,
3 W_down); dgrad/wgrad grouped GEMMs on native block-scaled MFMA; dU = dH *
silu'(U) -> MXFP8; un-permuting sum -> dx (bf16); gate gradient
dg[t, j] = <dy[t], Yp[row(t, j)]> (float32) and its softmax backward into the
router logits.
"""
import torch

from . import (NVFP4_4OVER6, PRE_SILU, PRE_SILU_AMAX, SF_BLOCKS, SF_ROWS, Moe4Unsupported, max_padded_rows,
               moe_combine, moe_combine_hmx8, moe_dgates, moe_gather_rows, moe_grouped_gemm_bwd_dgrad,
               moe_grouped_gemm_bwd_wgrad, moe_grouped_gemm_fwd, moe_grouped_gemm_fwd_hmx8,
               moe_grouped_gemm_fwd_silu_amax, moe_grouped_gemm_mx,
               moe_hmx8_quant, moe_route_backward, moe_route_topk, moe_router_logits, moe_router_wgrad,
               moe_unpermute_sum, moe_unpermute_sum_router, mxfp8_quant, mxfp8_quant_requant_T, mxfp8_quant_rows_T,
               mxfp8_requant_mx_sr_T, mxfp8_requant_sr_T, nvfp4_quant_46, nvfp4_quant_requant_T)

ROLE_X, ROLE_H, ROLE_WUP, ROLE_WDOWN = 0, 1, 2, 3

_SIDE = {}  # device index -> the backward's second stream (default priority)
# smallest T * k * d whose untimed backward uses the second stream (below it
# the stream handoffs cost more than the overlap gains)
SIDE_STREAM_MIN_ELEMS = 1 << 26


def _side_stream(device):
    s = _SIDE.get(device.index)
    if s is None:
        s = _SIDE[device.index] = torch.cuda.Stream(device=device)
    return s


def _tick(timer, name):
    if timer is not None:
        timer(name)


def quantize_weights(w_up, w_down, timer=None, seed=1, layer=0):
    """NVFP4 (mode 6) of the fp32 masters, one tensor scale per expert matrix,
    and in the same pass the backward's transposed MXFP8 SR copies (wuT, wdT;
    SR stream 16*layer + role, as the backward would requantise them).

    ``timer``, if given, is called with a step name after each library call
    (the benchmark records a HIP event there)."""
    E, F, d = w_up.shape
    dev = w_up.device
    off_f = torch.arange(E + 1, dtype=torch.int32, device=dev) * F
    off_d = torch.arange(E + 1, dtype=torch.int32, device=dev) * d
    _tick(timer, None)
    u = nvfp4_quant_requant_T(w_up.view(E * F, d), E, seed, 16 * layer + ROLE_WUP)
    _tick(timer, "F1 W_up quant (+ requant)")
    dn = nvfp4_quant_requant_T(w_down.view(E * d, F), E, seed, 16 * layer + ROLE_WDOWN)
    _tick(timer, "F1 W_down quant (+ requant)")
    return dict(wu=u[:3], wd=dn[:3], wuT=u[3:], wdT=dn[3:], sr=(seed, layer), off_f=off_f, off_d=off_d,
                shape=(E, F, d))


def forward(x, w_up, w_down, logits, k, bias=None, wq=None, timer=None, seed=1, layer=0, combine_payload=False,
            router_w=None):
    """x [T, d] bf16, w_up [E, F, d] / w_down [E, d, F] fp32, logits [T, E] fp32.
    (seed, layer): the SR key of the weights' backward copies made here.
    combine_payload: send the expert outputs to the combine as the 8.25-bit
    payload (32-point Hadamard + 8-bit fixed point with an E8M0 scale per 32,
    lhc.media page, paragraph on communication) instead of float32; the
    backward treats that quantisation as the identity.
    router_w: [E, d] bf16 router weights; when given, the logits are made here
    by the BF16 router GEMM (logits may be None) and the backward adds the
    router's input gradient to dx and returns its weight gradient."""
    T, d = x.shape
    E, F, _ = w_up.shape
    if wq is None:
        wq = quantize_weights(w_up, w_down, timer, seed, layer)
    if router_w is not None:
        _tick(timer, None)
        logits = moe_router_logits(x, router_w)
        _tick(timer, "F0 router GEMM (BF16)")
    _tick(timer, None)
    if timer is None and x.is_cuda and T * k * d >= SIDE_STREAM_MIN_ELEMS:
        # routing on the second stream beside X's quantisation (independent)
        main = torch.cuda.current_stream(x.device)
        side = _side_stream(x.device)
        side.wait_stream(main)
        with torch.cuda.stream(side):
            r = moe_route_topk(logits, k, bias)
        xq = nvfp4_quant_46(x, NVFP4_4OVER6)
        main.wait_stream(side)
    else:
        r = moe_route_topk(logits, k, bias)
        _tick(timer, "F2-F3 route + permutation")
        xq = nvfp4_quant_46(x, NVFP4_4OVER6)
        _tick(timer, "F4 X quant (NVFP4 4/6)")
    xq_perm = moe_gather_rows(xq[0], xq[1], r["perm"], k)
    _tick(timer, "F5 dispatch gather")
    wu_c, wu_s, wu_t = wq["wu"]
    wd_c, wd_s, wd_t = wq["wd"]
    # F6 with the per-expert SiLU amax of F7 folded into its epilogue (when
    # the shape takes the warp-specialised kernels), so F7 only encodes
    try:
        U, amax_ws = moe_grouped_gemm_fwd_silu_amax(xq_perm[0], xq_perm[1], xq[2], wu_c.view(E, F, d // 2),
                                                    wu_s.view(E, F, d // 16), wu_t, r["off"])
    except Moe4Unsupported:
        U, amax_ws = moe_grouped_gemm_fwd(xq_perm[0], xq_perm[1], xq[2], wu_c.view(E, F, d // 2),
                                          wu_s.view(E, F, d // 16), wu_t, r["off"], torch.bfloat16), None
    _tick(timer, "F6 up GEMM (NVFP4)")
    if amax_ws is None:
        hq = nvfp4_quant_46(U, NVFP4_4OVER6, r["off"], PRE_SILU)
    else:
        hq = nvfp4_quant_46(U, NVFP4_4OVER6, r["off"], PRE_SILU_AMAX, ws=amax_ws)
    _tick(timer, "F7 SiLU + H quant (NVFP4 4/6)")
    payload = None
    if combine_payload:
        # the payload from F8's epilogue when the shape takes the
        # warp-specialised kernels, else from a pass of its own
        try:
            Yp, h_codes, h_sf = moe_grouped_gemm_fwd_hmx8(hq[0], hq[1], hq[2], wd_c.view(E, d, F // 2),
                                                          wd_s.view(E, d, F // 16), wd_t, r["off"],
                                                          a_ts_per_group=True)
            payload = (h_codes, h_sf)
            _tick(timer, "F8+F9a down GEMM (NVFP4) + 8.25-bit payload")
        except Moe4Unsupported:
            Yp = moe_grouped_gemm_fwd(hq[0], hq[1], hq[2], wd_c.view(E, d, F // 2), wd_s.view(E, d, F // 16), wd_t,
                                      r["off"], torch.float32, a_ts_per_group=True)
            _tick(timer, "F8 down GEMM (NVFP4)")
            payload = moe_hmx8_quant(Yp)
            _tick(timer, "F9a Yp -> 8.25-bit payload (Hadamard + 8-bit)")
        y = moe_combine_hmx8(payload[0], payload[1], r["gates"], r["inv_perm"])
        _tick(timer, "F9b combine from the payload")
    else:
        Yp = moe_grouped_gemm_fwd(hq[0], hq[1], hq[2], wd_c.view(E, d, F // 2), wd_s.view(E, d, F // 16), wd_t,
                                  r["off"], torch.float32, a_ts_per_group=True)
        _tick(timer, "F8 down GEMM (NVFP4)")
        y = moe_combine(Yp, r["gates"], r["inv_perm"])
        _tick(timer, "F9 combine")
    return dict(y=y, route=r, xq=xq, xq_perm=xq_perm, U=U, hq=hq, Yp=Yp, wq=wq, dims=(T, d, F, E, k),
                payload=payload, x=x, router_w=router_w, logits=logits)


def backward(fw, dy, seed=1, layer=0, timer=None, skip_empty_dw=False):
    """dy [T, d] bf16 -> dict(dx [T, d] bf16, dW_up [E, F, d] fp32, dW_down [E, d, F] fp32, dg, dlogits, ...).
    skip_empty_dw: the weight gradients of experts that received no token are
    left unwritten (their gradient is zero; dW[e] holds a value iff
    route off[e + 1] > off[e]) instead of being filled with zeros."""
    T, d, F, E, k = fw["dims"]
    r = fw["route"]
    mpr = max_padded_rows(T * k, E)
    sid = lambda role: 16 * layer + role
    wq = fw["wq"]
    pre = wq.get("sr") == (seed, layer)  # the weights were requantised with their forward quantisation

    def wreq(name, w, goff, role, rows):
        if pre:
            return wq[name], None
        return mxfp8_requant_sr_T(*w, goff, goff, True, seed, sid(role), max_pr=rows), True
    hq, xp = fw["hq"], fw["xq_perm"]
    return _backward_chain(fw, dy, timer, skip_empty_dw, dict(
        wdT=lambda: wreq("wdT", wq["wd"], wq["off_d"], ROLE_WDOWN, E * d),
        hT=lambda: (mxfp8_requant_sr_T(*hq, r["off"], r["off_pad"], True, seed, sid(ROLE_H), max_pr=mpr,
                                       sf_layout=SF_BLOCKS), True),
        wuT=lambda: wreq("wuT", wq["wu"], wq["off_f"], ROLE_WUP, E * F),
        xT=lambda: (mxfp8_requant_sr_T(xp[0], xp[1], fw["xq"][2], r["off"], r["off_pad"], False, seed, sid(ROLE_X),
                                       max_pr=mpr, sf_layout=SF_BLOCKS), True)))


def _backward_chain(fw, dy, timer, skip_empty_dw, req):
    """The backward calls in order; req[name]() gives the transposed MXFP8
    operand 'wdT', 'hT', 'wuT' or 'xT' and whether a library call made it
    (for the timer).

    Without a timer (and for T k d >= SIDE_STREAM_MIN_ELEMS), the calls that
    only read tensors the chain does not write run on a second stream beside
    it: the gate gradient and the router
    backward (B12, B13: dy, Yp and the routing) beside B1 (HBM-bound reads
    beside a VALU-bound quantiser), and the un-permuting sum (B11, from dXp)
    beside B9 and B10.  The chain's stream waits for the second stream before
    returning.  Every tensor the second stream reads outlives the call, and
    the second stream waits for the chain's stream before each of its turns,
    so no block either stream frees is reused while the other still reads
    it.  With a timer every call runs in order on one stream, so that each
    one's time can be read."""
    T, d, F, E, k = fw["dims"]
    r = fw["route"]
    A = T * k
    mpr = max_padded_rows(A, E)
    g_flat = r["gates"].view(-1)
    rw = fw.get("router_w")
    side = None
    if timer is None and dy.is_cuda and A * d >= SIDE_STREAM_MIN_ELEMS:
        main = torch.cuda.current_stream(dy.device)
        side = _side_stream(dy.device)
        side.wait_stream(main)
        with torch.cuda.stream(side):
            dg = moe_dgates(dy, fw["Yp"], r["inv_perm"], k)
            dlogits = moe_route_backward(dg, r["gates"], r["idx"], E)

    def get(name, label):
        out, called = req[name]()
        if called:
            _tick(timer, label)
        return out
    _tick(timer, None)
    # B1: both MXFP8 copies of the gated, gathered dY from one read
    q = mxfp8_quant_rows_T(dy, r["off"], r["off_pad"], rows=A, row_map=r["perm"], map_div=k, row_scale=g_flat,
                           max_pr=mpr, sf_layout=SF_BLOCKS)
    dy_row, dy_col = q[:2], q[2:]
    _tick(timer, "B1 dY quant row-wise + transposed (MXFP8)")
    wdT = get("wdT", "B2 W_down requant SR-T")
    dH = moe_grouped_gemm_bwd_dgrad(dy_row[0], dy_row[1], wdT[0], wdT[1], r["off"])
    _tick(timer, "B3 down dgrad (MXFP8)")
    hT = get("hT", "B4 H requant SR-T")
    dW_down = moe_grouped_gemm_bwd_wgrad(dy_col[0], dy_col[1], hT[0], hT[1], r["off_pad"], d, F,
                                         skip_empty=skip_empty_dw)
    _tick(timer, "B5 down wgrad (MXFP8)")
    # B6: both MXFP8 copies of dU = dH * silu'(U) from one read
    q = mxfp8_quant_rows_T(dH, r["off"], r["off_pad"], dsilu_src=fw["U"], max_pr=mpr, sf_layout=SF_BLOCKS)
    du_row, du_col = q[:2], q[2:]
    _tick(timer, "B6 SiLU' + dU quant row-wise + transposed")
    wuT = get("wuT", "B7 W_up requant SR-T")
    dXp = moe_grouped_gemm_bwd_dgrad(du_row[0], du_row[1], wuT[0], wuT[1], r["off"])
    _tick(timer, "B8 up dgrad (MXFP8)")
    if side is not None and rw is None:
        side.wait_stream(main)
        with torch.cuda.stream(side):
            dx = moe_unpermute_sum(dXp, r["inv_perm"], T, k)
    xT = get("xT", "B9 X requant SR-T")
    dW_up = moe_grouped_gemm_bwd_wgrad(du_col[0], du_col[1], xT[0], xT[1], r["off_pad"], F, d,
                                       skip_empty=skip_empty_dw)
    _tick(timer, "B10 up wgrad (MXFP8)")
    dW_router = None
    if side is not None:
        main.wait_stream(side)
    else:
        if rw is None:
            dx = moe_unpermute_sum(dXp, r["inv_perm"], T, k)
            _tick(timer, "B11 un-permute sum")
        dg = moe_dgates(dy, fw["Yp"], r["inv_perm"], k)
        _tick(timer, "B12 gate gradient")
        dlogits = moe_route_backward(dg, r["gates"], r["idx"], E)
        _tick(timer, "B13 router backward")
    if rw is not None:
        # the router's input gradient joins the un-permuting sum; then its weight gradient
        dx = moe_unpermute_sum_router(dXp, r["inv_perm"], T, k, dlogits, r["idx"], rw)
        _tick(timer, "B11 un-permute sum (+ router input gradient)")
        dW_router = moe_router_wgrad(fw["x"], dlogits, r["perm"], r["off"], k)
        _tick(timer, "B14 router weight gradient")
    return dict(dx=dx, dg=dg, dlogits=dlogits, dW_up=dW_up, dW_down=dW_down, dH=dH, dXp=dXp, dy_row=dy_row,
                dy_col=dy_col, wdT=wdT, hT=hT, du_row=du_row, du_col=du_col, wuT=wuT, xT=xT, dW_router=dW_router)


# ------------------------------------------------ MXFP8-forward variant
#
# The layers kept at higher precision (the last sixth) run their forward in
# MXFP8 on the native block-scaled FP8 MFMA: x (gathered into expert order),
# the weights and H = silu(U) are quantised to MXFP8 (RNE, blocks along the
# forward contraction, no tensor scale); U is stored in bf16.  The backward
# is the same chain as above with the transposed SR requantisations reading
# the MXFP8 forward operands.

def quantize_weights_mx(w_up, w_down, timer=None, seed=1, layer=0):
    """MXFP8 (RNE) of the fp32 masters and, in the same pass, the backward's
    transposed MXFP8 SR copies (SR stream 16*layer + role, as backward_mx
    would requantise them)."""
    E, F, d = w_up.shape
    dev = w_up.device
    off_f = torch.arange(E + 1, dtype=torch.int32, device=dev) * F
    off_d = torch.arange(E + 1, dtype=torch.int32, device=dev) * d
    _tick(timer, None)
    u = mxfp8_quant_requant_T(w_up.view(E * F, d), E, seed, 16 * layer + ROLE_WUP)
    _tick(timer, "F1 W_up quant (+ requant, MXFP8)")
    dn = mxfp8_quant_requant_T(w_down.view(E * d, F), E, seed, 16 * layer + ROLE_WDOWN)
    _tick(timer, "F1 W_down quant (+ requant, MXFP8)")
    return dict(wu=u[:2], wd=dn[:2], wuT=u[2:], wdT=dn[2:], sr=(seed, layer), off_f=off_f, off_d=off_d,
                shape=(E, F, d))


def forward_mx(x, w_up, w_down, logits, k, bias=None, wq=None, timer=None, seed=1, layer=0):
    T, d = x.shape
    E, F, _ = w_up.shape
    if wq is None:
        wq = quantize_weights_mx(w_up, w_down, timer, seed, layer)
    _tick(timer, None)
    r = moe_route_topk(logits, k, bias)
    _tick(timer, "F2-F3 route + permutation")
    A = T * k
    xq_perm = mxfp8_quant(x, rows=A, row_map=r["perm"], map_div=k)
    _tick(timer, "F4-F5 X quant + gather (MXFP8)")
    wu_c, wu_s = wq["wu"]
    wd_c, wd_s = wq["wd"]
    U = moe_grouped_gemm_mx(xq_perm[0], xq_perm[1], wu_c.view(E, F, d), wu_s.view(E, F, d // 32), r["off"],
                            torch.bfloat16)
    _tick(timer, "F6 up GEMM (MXFP8)")
    hq = mxfp8_quant(U, pre_op=PRE_SILU)
    _tick(timer, "F7 SiLU + H quant (MXFP8)")
    Yp = moe_grouped_gemm_mx(hq[0], hq[1], wd_c.view(E, d, F), wd_s.view(E, d, F // 32), r["off"])
    _tick(timer, "F8 down GEMM (MXFP8)")
    y = moe_combine(Yp, r["gates"], r["inv_perm"])
    _tick(timer, "F9 combine")
    return dict(y=y, route=r, xq_perm=xq_perm, U=U, hq=hq, Yp=Yp, wq=wq, dims=(T, d, F, E, k), mx=True)


def backward_mx(fw, dy, seed=1, layer=0, timer=None, skip_empty_dw=False):
    """The backward of forward_mx: the requantisations read MXFP8 operands."""
    T, d, F, E, k = fw["dims"]
    r = fw["route"]
    A = T * k
    mpr = max_padded_rows(A, E)
    sid = lambda role: 16 * layer + role
    wq = fw["wq"]

    pre = wq.get("sr") == (seed, layer)  # the weights were requantised with their forward quantisation

    def req(q, goff, goff_pad, role, layout, max_pr):
        return mxfp8_requant_mx_sr_T(q[0], q[1], goff, goff_pad, seed, sid(role), max_pr=max_pr,
                                     sf_layout=layout), True

    def wreq(name, q, goff, role, rows):
        if pre:
            return wq[name], None
        return req(q, goff, goff, role, SF_ROWS, rows)
    return _backward_chain(fw, dy, timer, skip_empty_dw, dict(
        wdT=lambda: wreq("wdT", wq["wd"], wq["off_d"], ROLE_WDOWN, E * d),
        hT=lambda: req(fw["hq"], r["off"], r["off_pad"], ROLE_H, SF_BLOCKS, mpr),
        wuT=lambda: wreq("wuT", wq["wu"], wq["off_f"], ROLE_WUP, E * F),
        xT=lambda: req(fw["xq_perm"], r["off"], r["off_pad"], ROLE_X, SF_BLOCKS, mpr)))
