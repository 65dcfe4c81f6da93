"""MI355X-native NVFP4-forward / MXFP8-backward MoE expert layer.

Thin Python binding of ``libmoe4.so`` (C ABI in ``include/moe4.h``): each
function checks tensor devices, dtypes and shapes, allocates outputs with
torch, passes raw device pointers and torch's current HIP stream, and raises
on a non-zero return code.  Every step of the computation runs in the HIP
kernels; there is no CPU or PyTorch fallback: if the library is missing the
functions raise.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe4.so")

BF16, F32 = 0, 1
NVFP4_6, NVFP4_4OVER6 = 6, 46
PRE_NONE, PRE_SILU, PRE_SILU_AMAX = 0, 1, 2
EUNSUPPORTED = -5
EDEVICE = -6
RNE, SR = 0, 1
SF_ROWS, SF_BLOCKS = 0, 1   # group-major scale arrangement: [C][P_g/32] or [P_g/32][C]

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_int = ctypes.c_int
_u64 = ctypes.c_uint64
_u32 = ctypes.c_uint32
_f32 = ctypes.c_float
_size = ctypes.c_size_t

_SIGS = {
    "moe4_last_error": (ctypes.c_char_p, []),
    "moe4_version": (ctypes.c_char_p, []),
    "nvfp4_quant_46": (_int, [_c_void_p, _int, _i64, _i64, _c_void_p, _i32, _int, _int, _c_void_p, _c_void_p,
                              _c_void_p, _c_void_p, _size, _c_void_p]),
    "nvfp4_quant_46_ws_bytes": (_size, [_i32]),
    "nvfp4_quant_46_noalloc": (_int, [_c_void_p, _int, _i64, _i64, _c_void_p, _i32, _int, _int, _c_void_p,
                                      _c_void_p, _c_void_p, _c_void_p]),
    "nvfp4_quant_requant_T": (_int, [_c_void_p, _i64, _i64, _i32, _c_void_p, _c_void_p, _c_void_p, _u64, _u32,
                                     _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
    "nvfp4_quant_requant_T_ws_bytes": (_size, [_i32]),
    "nvfp4_dequant": (_int, [_c_void_p, _c_void_p, _c_void_p, _int, _c_void_p, _i32, _i64, _i64, _c_void_p,
                             _c_void_p]),
    "mxfp8_requant_sr_T": (_int, [_c_void_p, _c_void_p, _c_void_p, _int, _i64, _i64, _c_void_p, _c_void_p, _i32,
                                  _i64, _u64, _u32, _int, _c_void_p, _c_void_p, _c_void_p]),
    "mxfp8_requant_mx_sr_T": (_int, [_c_void_p, _c_void_p, _i64, _i64, _c_void_p, _c_void_p, _i32, _i64, _u64,
                                     _u32, _int, _c_void_p, _c_void_p, _c_void_p]),
    "moe_grouped_gemm_mx": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64, _i64, _i64,
                                   _c_void_p, _int, _c_void_p]),
    "mxfp8_quant": (_int, [_c_void_p, _int, _i64, _i64, _c_void_p, _i32, _c_void_p, _c_void_p, _int, _int,
                           _c_void_p, _c_void_p, _i32, _i64, _int, _u64, _u32, _c_void_p, _c_void_p, _c_void_p]),
    "mxfp8_quant_rows_T": (_int, [_c_void_p, _int, _i64, _i64, _c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p,
                                  _c_void_p, _i32, _i64, _int, _u64, _u32, _int, _c_void_p, _c_void_p, _c_void_p,
                                  _c_void_p, _c_void_p]),
    "moe_route_backward": (_int, [_c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32, _c_void_p, _c_void_p]),
    "moe_dgates": (_int, [_c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i64, _c_void_p, _c_void_p]),
    "moe4_debug_check": (_int, [_c_void_p]),
    "moe4_debug_force_wait_timeout": (_int, [_int]),
    "moe_route_topk": (_int, [_c_void_p, _c_void_p, _i64, _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                              _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
    "moe_route_topk_ws_bytes": (_size, [_i64, _i32, _i32]),
    "moe_gather_rows": (_int, [_c_void_p, _c_void_p, _i64, _i64, _c_void_p, _i32, _i64, _c_void_p, _c_void_p,
                               _c_void_p]),
    "moe_grouped_gemm_fwd": (_int, [_c_void_p, _c_void_p, _c_void_p, _int, _c_void_p, _c_void_p, _c_void_p,
                                    _c_void_p, _i32, _i64, _i64, _i64, _c_void_p, _int, _c_void_p]),
    "moe_grouped_gemm_bwd_dgrad": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64, _i64,
                                          _i64, _c_void_p, _c_void_p]),
    "moe_grouped_gemm_bwd_wgrad": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64, _i64,
                                          _c_void_p, _f32, _int, _c_void_p]),
    "moe_grouped_gemm_bwd": (_int, [_c_void_p] * 10 + [_i32, _i64, _i64, _i64, _c_void_p, _c_void_p, _f32, _int,
                                                       _c_void_p]),
    "moe_combine": (_int, [_c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i64, _c_void_p, _c_void_p]),
    "moe_unpermute_sum": (_int, [_c_void_p, _c_void_p, _i64, _i32, _i64, _c_void_p, _c_void_p]),
    "moe_silu_eval": (_int, [_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p]),
    "moe_router_logits": (_int, [_c_void_p, _c_void_p, _i64, _i32, _i64, _c_void_p, _c_void_p]),
    "moe_unpermute_sum_router": (_int, [_c_void_p, _c_void_p, _i64, _i32, _i64, _c_void_p, _c_void_p, _i32, _c_void_p,
                                        _c_void_p, _c_void_p]),
    "moe_router_wgrad": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32, _i64, _c_void_p,
                                _c_void_p, _size, _c_void_p]),
    "moe_router_wgrad_ws_bytes": (_size, [_i64, _i32, _i32, _i64]),
    "mxfp8_quant_requant_T": (_int, [_c_void_p, _i64, _i64, _i32, _u64, _u32, _c_void_p, _c_void_p, _c_void_p,
                                     _c_void_p, _c_void_p]),
    "moe_grouped_gemm_fwd_silu_amax": (_int, [_c_void_p, _c_void_p, _c_void_p, _int, _c_void_p, _c_void_p, _c_void_p,
                                              _c_void_p, _i32, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p]),
    "moe_hmx8_quant": (_int, [_c_void_p, _i64, _i64, _c_void_p, _c_void_p, _c_void_p]),
    "moe_hmx8_dequant": (_int, [_c_void_p, _c_void_p, _i64, _i64, _c_void_p, _c_void_p]),
    "moe_combine_hmx8": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i64, _c_void_p,
                                _c_void_p]),
    "moe_grouped_gemm_fwd_hmx8": (_int, [_c_void_p, _c_void_p, _c_void_p, _int, _c_void_p, _c_void_p, _c_void_p,
                                         _c_void_p, _i32, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                         _c_void_p]),
}

EXPORTS = tuple(_SIGS)
_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m precision_moe_numerics_quant_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class Moe4Error(RuntimeError):
    pass


class Moe4Unsupported(Moe4Error):
    """The call does not support this shape or kernel choice (nothing was launched)."""


class Moe4DeviceError(Moe4Error):
    """moe4_debug_check found a device-side error report (a clamped index or a
    bounded wait that gave up)."""


def _check(rc, name):
    if rc != 0:
        msg = lib().moe4_last_error().decode(errors="replace")
        cls = {EUNSUPPORTED: Moe4Unsupported, EDEVICE: Moe4DeviceError}.get(rc, Moe4Error)
        raise cls(f"{name} failed ({rc}): {msg}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    if not (t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError(f"{name}: expected a contiguous {dtype} tensor on the GPU, got {t.dtype} on {t.device}")
    return t


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def _ws(nbytes, like):
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=like.device)


def pad32(n):
    return (int(n) + 31) // 32 * 32


def max_padded_rows(rows, n_groups):
    """Upper bound of the padded row count of a grouped transposed layout."""
    return pad32(rows + 31 * n_groups)


# --------------------------------------------------------------------- NVFP4

def nvfp4_quant_46(x, mode=NVFP4_4OVER6, group_row_off=None, pre_op=PRE_NONE, ws=None):
    """NVFP4 of x [R, C] (bf16 or float32) -> (codes [R, C/2] u8, sf [R, C/16] u8, ts [G] f32).
    ws: the workspace (uint8 tensor); with PRE_SILU_AMAX it must hold the group amax
    words written by moe_grouped_gemm_fwd_silu_amax."""
    dt = {torch.bfloat16: BF16, torch.float32: F32}.get(x.dtype)
    if dt is None:
        raise ValueError("nvfp4_quant_46: x must be bf16 or float32")
    _dev(x, x.dtype, "x")
    R, C = x.shape
    G = 1 if group_row_off is None else group_row_off.numel() - 1
    if group_row_off is not None:
        _dev(group_row_off, torch.int32, "group_row_off")
    codes = _empty((R, C // 2), torch.uint8, x)
    sf = _empty((R, C // 16), torch.uint8, x)
    ts = _empty((G,), torch.float32, x)
    if ws is None:
        ws = _ws(lib().nvfp4_quant_46_ws_bytes(G), x)
    rc = lib().nvfp4_quant_46(_p(x), dt, R, C, _p(group_row_off), G, mode, pre_op, _p(codes), _p(sf), _p(ts),
                              _p(ws), ws.numel(), _stream())
    _check(rc, "nvfp4_quant_46")
    return codes, sf, ts


def nvfp4_quant_46_noalloc(x, mode=NVFP4_4OVER6, group_row_off=None, pre_op=PRE_NONE, out=None):
    """nvfp4_quant_46 with the library's static scratch instead of a workspace.
    out: optional (codes, sf, ts) tensors to write into (nothing is allocated
    then); otherwise they are allocated here, outside the library call."""
    dt = {torch.bfloat16: BF16, torch.float32: F32}.get(x.dtype)
    if dt is None:
        raise ValueError("nvfp4_quant_46_noalloc: x must be bf16 or float32")
    _dev(x, x.dtype, "x")
    R, C = x.shape
    G = 1 if group_row_off is None else group_row_off.numel() - 1
    if group_row_off is not None:
        _dev(group_row_off, torch.int32, "group_row_off")
    if out is None:
        out = (_empty((R, C // 2), torch.uint8, x), _empty((R, C // 16), torch.uint8, x),
               _empty((G,), torch.float32, x))
    codes, sf, ts = out
    rc = lib().nvfp4_quant_46_noalloc(_p(x), dt, R, C, _p(group_row_off), G, mode, pre_op, _p(codes), _p(sf),
                                      _p(ts), _stream())
    _check(rc, "nvfp4_quant_46_noalloc")
    return codes, sf, ts


def nvfp4_quant_requant_T(x, n_groups, seed=1, stream_id=0):
    """Weights [G*R_g, C] float32 -> NVFP4 mode 6 (codes, sf, ts per group) and
    its transposed MXFP8 SR copy (mx_codes [C*rows], mx_sf [C*rows/32]) in one pass."""
    _dev(x, torch.float32, "x")
    R, C = x.shape
    codes = _empty((R, C // 2), torch.uint8, x)
    sf = _empty((R, C // 16), torch.uint8, x)
    ts = _empty((n_groups,), torch.float32, x)
    mc = _empty((C * R,), torch.uint8, x)
    ms = _empty((C * R // 32,), torch.uint8, x)
    ws = _ws(lib().nvfp4_quant_requant_T_ws_bytes(n_groups), x)
    rc = lib().nvfp4_quant_requant_T(_p(x), R, C, n_groups, _p(codes), _p(sf), _p(ts), seed, stream_id, _p(mc),
                                     _p(ms), _p(ws), ws.numel(), _stream())
    _check(rc, "nvfp4_quant_requant_T")
    return codes, sf, ts, mc, ms


def mxfp8_quant_requant_T(x, n_groups, seed=1, stream_id=0):
    """Weights [G*R_g, C] float32 -> MXFP8 RNE row-wise (codes [R, C], sf [R, C/32])
    and its transposed MXFP8 SR copy (t_codes [C*R], t_sf [C*R/32]) in one pass."""
    _dev(x, torch.float32, "x")
    R, C = x.shape
    codes = _empty((R, C), torch.uint8, x)
    sf = _empty((R, C // 32), torch.uint8, x)
    tc = _empty((C * R,), torch.uint8, x)
    ts = _empty((C * R // 32,), torch.uint8, x)
    rc = lib().mxfp8_quant_requant_T(_p(x), R, C, n_groups, seed, stream_id, _p(codes), _p(sf), _p(tc), _p(ts),
                                     _stream())
    _check(rc, "mxfp8_quant_requant_T")
    return codes, sf, tc, ts


def nvfp4_dequant(codes, sf, ts, group_row_off=None, ts_per_group=False):
    R, H = codes.shape
    G = 1 if group_row_off is None else group_row_off.numel() - 1
    out = _empty((R, 2 * H), torch.float32, codes)
    rc = lib().nvfp4_dequant(_p(codes), _p(sf), _p(ts), int(ts_per_group), _p(group_row_off), G, R, 2 * H, _p(out),
                             _stream())
    _check(rc, "nvfp4_dequant")
    return out


# --------------------------------------------------------------------- MXFP8

def mxfp8_requant_sr_T(codes, sf, ts, group_row_off, group_off_pad, ts_per_group=True, seed=1, stream_id=0,
                       max_pr=None, sf_layout=SF_ROWS):
    """NVFP4 [R, C] -> MXFP8 SR, group-major padded: (codes [C*P], sf [C*P/32]) with P = max_pr;
    scales row-major per group (SF_ROWS) or block-major (SF_BLOCKS)."""
    R, H = codes.shape
    C = 2 * H
    G = group_row_off.numel() - 1
    _dev(group_row_off, torch.int32, "group_row_off")
    _dev(group_off_pad, torch.int32, "group_off_pad")
    if max_pr is None:
        max_pr = max_padded_rows(R, G)
    oc = _empty((C * max_pr,), torch.uint8, codes)
    os_ = _empty((C * max_pr // 32,), torch.uint8, codes)
    rc = lib().mxfp8_requant_sr_T(_p(codes), _p(sf), _p(ts), int(ts_per_group), R, C, _p(group_row_off),
                                  _p(group_off_pad), G, max_pr, seed, stream_id, int(sf_layout), _p(oc), _p(os_),
                                  _stream())
    _check(rc, "mxfp8_requant_sr_T")
    return oc, os_


def mxfp8_requant_mx_sr_T(codes, sf, group_row_off, group_off_pad, seed=1, stream_id=0, max_pr=None,
                          sf_layout=SF_ROWS):
    """MXFP8 row-wise [R, C] -> MXFP8 SR transposed, group-major padded: (codes [C*P], sf [C*P/32])."""
    R, C = codes.shape
    G = group_row_off.numel() - 1
    _dev(group_row_off, torch.int32, "group_row_off")
    _dev(group_off_pad, torch.int32, "group_off_pad")
    if max_pr is None:
        max_pr = max_padded_rows(R, G)
    oc = _empty((C * max_pr,), torch.uint8, codes)
    os_ = _empty((C * max_pr // 32,), torch.uint8, codes)
    rc = lib().mxfp8_requant_mx_sr_T(_p(codes), _p(sf), R, C, _p(group_row_off), _p(group_off_pad), G, max_pr, seed,
                                     stream_id, int(sf_layout), _p(oc), _p(os_), _stream())
    _check(rc, "mxfp8_requant_mx_sr_T")
    return oc, os_


def mxfp8_quant(x, rows=None, transpose=False, row_map=None, map_div=1, row_scale=None, dsilu_src=None,
                group_row_off=None, group_off_pad=None, max_pr=None, rnd=RNE, seed=0, stream_id=0,
                sf_layout=SF_ROWS, pre_op=PRE_NONE):
    """MXFP8 of a gradient (see moe4.h).  Row mode -> ([rows, C], [rows, C/32]);
    transposed -> (codes [C*max_pr], sf [C*max_pr/32]), scales per group
    row-major (SF_ROWS) or block-major (SF_BLOCKS)."""
    dt = {torch.bfloat16: BF16, torch.float32: F32}.get(x.dtype)
    if dt is None:
        raise ValueError("mxfp8_quant: x must be bf16 or float32")
    _dev(x, x.dtype, "x")
    C = x.shape[1]
    R = (row_map.numel() if row_map is not None else x.shape[0]) if rows is None else rows
    if row_map is not None:
        _dev(row_map, torch.int32, "row_map")
    if row_scale is not None:
        _dev(row_scale, torch.float32, "row_scale")
    if dsilu_src is not None:
        _dev(dsilu_src, torch.bfloat16, "dsilu_src")
    if transpose:
        G = group_row_off.numel() - 1
        if max_pr is None:
            max_pr = max_padded_rows(R, G)
        oc = _empty((C * max_pr,), torch.uint8, x)
        os_ = _empty((C * max_pr // 32,), torch.uint8, x)
    else:
        G = 0
        max_pr = 0
        oc = _empty((R, C), torch.uint8, x)
        os_ = _empty((R, C // 32), torch.uint8, x)
    mode = 0 if not transpose else (2 if sf_layout == SF_BLOCKS else 1)
    rc = lib().mxfp8_quant(_p(x), dt, R, C, _p(row_map), map_div, _p(row_scale), _p(dsilu_src), pre_op, mode,
                           _p(group_row_off), _p(group_off_pad), G, max_pr, rnd, seed, stream_id, _p(oc), _p(os_),
                           _stream())
    _check(rc, "mxfp8_quant")
    return oc, os_


def mxfp8_quant_rows_T(x, group_row_off, group_off_pad, rows=None, row_map=None, map_div=1, row_scale=None,
                       dsilu_src=None, max_pr=None, rnd=RNE, seed=0, stream_id=0, sf_layout=SF_ROWS):
    """Both MXFP8 copies of a gradient from one read (see moe4.h): returns
    (row_codes [rows, C], row_sf [rows, C/32], t_codes [C*max_pr], t_sf [C*max_pr/32])."""
    dt = {torch.bfloat16: BF16, torch.float32: F32}.get(x.dtype)
    if dt is None:
        raise ValueError("mxfp8_quant_rows_T: x must be bf16 or float32")
    _dev(x, x.dtype, "x")
    C = x.shape[1]
    R = (row_map.numel() if row_map is not None else x.shape[0]) if rows is None else rows
    if row_map is not None:
        _dev(row_map, torch.int32, "row_map")
    if row_scale is not None:
        _dev(row_scale, torch.float32, "row_scale")
    if dsilu_src is not None:
        _dev(dsilu_src, torch.bfloat16, "dsilu_src")
    _dev(group_row_off, torch.int32, "group_row_off")
    _dev(group_off_pad, torch.int32, "group_off_pad")
    G = group_row_off.numel() - 1
    if max_pr is None:
        max_pr = max_padded_rows(R, G)
    rc_ = _empty((R, C), torch.uint8, x)
    rs_ = _empty((R, C // 32), torch.uint8, x)
    tc = _empty((C * max_pr,), torch.uint8, x)
    ts = _empty((C * max_pr // 32,), torch.uint8, x)
    rc = lib().mxfp8_quant_rows_T(_p(x), dt, R, C, _p(row_map), map_div, _p(row_scale), _p(dsilu_src),
                                  _p(group_row_off), _p(group_off_pad), G, max_pr, rnd, seed, stream_id, sf_layout,
                                  _p(rc_), _p(rs_), _p(tc), _p(ts), _stream())
    _check(rc, "mxfp8_quant_rows_T")
    return rc_, rs_, tc, ts


# ------------------------------------------------------------------- routing

def moe_route_topk(logits, k, bias=None):
    """Top-k routing + stable permutation.  Returns dict(idx, gates, off, off_pad, perm, inv_perm)."""
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    if bias is not None:
        _dev(bias, torch.float32, "bias")
    idx = _empty((T, k), torch.int32, logits)
    gates = _empty((T, k), torch.float32, logits)
    off = _empty((E + 1,), torch.int32, logits)
    off_pad = _empty((E + 1,), torch.int32, logits)
    perm = _empty((T * k,), torch.int32, logits)
    inv = _empty((T * k,), torch.int32, logits)
    ws = _ws(lib().moe_route_topk_ws_bytes(T, E, k), logits)
    rc = lib().moe_route_topk(_p(logits), _p(bias), T, E, k, _p(idx), _p(gates), _p(off), _p(off_pad), _p(perm),
                              _p(inv), _p(ws), ws.numel(), _stream())
    _check(rc, "moe_route_topk")
    return dict(idx=idx, gates=gates, off=off, off_pad=off_pad, perm=perm, inv_perm=inv)


def moe_gather_rows(codes, sf, perm, k):
    n_in, H = codes.shape
    A = perm.numel()
    oc = _empty((A, H), torch.uint8, codes)
    os_ = _empty((A, sf.shape[1]), torch.uint8, codes)
    rc = lib().moe_gather_rows(_p(codes), _p(sf), n_in, 2 * H, _p(perm), k, A, _p(oc), _p(os_), _stream())
    _check(rc, "moe_gather_rows")
    return oc, os_


# --------------------------------------------------------------------- GEMMs

def moe_grouped_gemm_fwd(a_codes, a_sf, a_ts, b_codes, b_sf, b_ts, expert_off, out_dtype=torch.bfloat16,
                         a_ts_per_group=False):
    """NVFP4 A [M, K] x NVFP4 B [E, N, K] grouped by expert_off -> C [M, N] (bf16 or float32)."""
    M, Kh = a_codes.shape
    E, N, _ = b_codes.shape
    c = _empty((M, N), out_dtype, a_codes)
    cd = BF16 if out_dtype == torch.bfloat16 else F32
    rc = lib().moe_grouped_gemm_fwd(_p(a_codes), _p(a_sf), _p(a_ts), int(a_ts_per_group), _p(b_codes), _p(b_sf),
                                    _p(b_ts), _p(expert_off), E, M, N, 2 * Kh, _p(c), cd, _stream())
    _check(rc, "moe_grouped_gemm_fwd")
    return c


def moe_grouped_gemm_fwd_silu_amax(a_codes, a_sf, a_ts, b_codes, b_sf, b_ts, expert_off, a_ts_per_group=False):
    """moe_grouped_gemm_fwd with bf16 U, plus each expert's max |silu(U)| as float bits
    in a workspace that nvfp4_quant_46(U, ..., PRE_SILU_AMAX, ws=...) takes.
    Raises Moe4Unsupported when the shape selects other kernels.  -> (U, ws)"""
    M, Kh = a_codes.shape
    E, N, _ = b_codes.shape
    c = _empty((M, N), torch.bfloat16, a_codes)
    ws = _ws(lib().nvfp4_quant_46_ws_bytes(E), a_codes)
    rc = lib().moe_grouped_gemm_fwd_silu_amax(_p(a_codes), _p(a_sf), _p(a_ts), int(a_ts_per_group), _p(b_codes),
                                              _p(b_sf), _p(b_ts), _p(expert_off), E, M, N, 2 * Kh, _p(c), _p(ws),
                                              _stream())
    _check(rc, "moe_grouped_gemm_fwd_silu_amax")
    return c, ws


def moe_grouped_gemm_fwd_hmx8(a_codes, a_sf, a_ts, b_codes, b_sf, b_ts, expert_off, a_ts_per_group=False):
    """moe_grouped_gemm_fwd with float32 C, plus C's combine-path payload written by the
    same epilogue.  Raises Moe4Unsupported when the shape selects other kernels.
    -> (C, codes int8 [M, N], scales uint8 [M, N/32])"""
    M, Kh = a_codes.shape
    E, N, _ = b_codes.shape
    c = _empty((M, N), torch.float32, a_codes)
    codes = _empty((M, N), torch.int8, a_codes)
    sf = _empty((M, N // 32), torch.uint8, a_codes)
    rc = lib().moe_grouped_gemm_fwd_hmx8(_p(a_codes), _p(a_sf), _p(a_ts), int(a_ts_per_group), _p(b_codes),
                                         _p(b_sf), _p(b_ts), _p(expert_off), E, M, N, 2 * Kh, _p(c), _p(codes),
                                         _p(sf), _stream())
    _check(rc, "moe_grouped_gemm_fwd_hmx8")
    return c, codes, sf


def moe_grouped_gemm_bwd_dgrad(a_codes, a_sf, b_codes, b_sf, expert_off):
    """MXFP8 A [M, K] x MXFP8 B [E, N, K] grouped by expert_off -> float32 C [M, N]."""
    M, K = a_codes.shape
    E = expert_off.numel() - 1
    N = b_codes.numel() // (E * K)
    c = _empty((M, N), torch.float32, a_codes)
    rc = lib().moe_grouped_gemm_bwd_dgrad(_p(a_codes), _p(a_sf), _p(b_codes), _p(b_sf), _p(expert_off), E, M, N, K,
                                          _p(c), _stream())
    _check(rc, "moe_grouped_gemm_bwd_dgrad")
    return c


def moe_grouped_gemm_mx(a_codes, a_sf, b_codes, b_sf, expert_off, out_dtype=torch.float32):
    """MXFP8 A [M, K] x MXFP8 B [E, N, K] per expert -> C [M, N] (float32 or bf16)."""
    M, K = a_codes.shape
    E = expert_off.numel() - 1
    N = b_codes.numel() // (E * K)
    cd = {torch.float32: F32, torch.bfloat16: BF16}[out_dtype]
    c = _empty((M, N), out_dtype, a_codes)
    rc = lib().moe_grouped_gemm_mx(_p(a_codes), _p(a_sf), _p(b_codes), _p(b_sf), _p(expert_off), E, M, N, K, _p(c),
                                   cd, _stream())
    _check(rc, "moe_grouped_gemm_mx")
    return c


WGRAD_SKIP_EMPTY = 1


def moe_grouped_gemm_bwd_wgrad(a_codes, a_sf, b_codes, b_sf, expert_off_pad, N1, N2, dw=None, beta=0.0,
                               skip_empty=False):
    """Group-major padded MXFP8 A [N1][P_e], B [N2][P_e] per expert -> dw [E, N1, N2] float32.
    skip_empty: experts without rows keep whatever dw holds (see moe4.h)."""
    E = expert_off_pad.numel() - 1
    if dw is None:
        dw = _empty((E, N1, N2), torch.float32, a_codes)
    rc = lib().moe_grouped_gemm_bwd_wgrad(_p(a_codes), _p(a_sf), _p(b_codes), _p(b_sf), _p(expert_off_pad), E, N1,
                                          N2, _p(dw), beta, WGRAD_SKIP_EMPTY if skip_empty else 0, _stream())
    _check(rc, "moe_grouped_gemm_bwd_wgrad")
    return dw


def moe_grouped_gemm_bwd(dy_codes, dy_sf, wT_codes, wT_sf, dyT_codes, dyT_sf, xT_codes, xT_sf, expert_off,
                         expert_off_pad, Nin, Nout, dw=None, beta=0.0, skip_empty=False):
    """dgrad and wgrad of one expert linear in one call: returns (dx float32
    [M, Nin], dw float32 [E, Nout, Nin]).  dy row-wise [M, Nout], W^T requantised
    [E][Nin][Nout], dy and x transposed group-major [Nout][P_e] / [Nin][P_e]
    with block-major scales."""
    M = dy_codes.shape[0]
    E = expert_off.numel() - 1
    dx = _empty((M, Nin), torch.float32, dy_codes)
    if dw is None:
        dw = _empty((E, Nout, Nin), torch.float32, dy_codes)
    rc = lib().moe_grouped_gemm_bwd(_p(dy_codes), _p(dy_sf), _p(wT_codes), _p(wT_sf), _p(dyT_codes), _p(dyT_sf),
                                    _p(xT_codes), _p(xT_sf), _p(expert_off), _p(expert_off_pad), E, M, Nin, Nout,
                                    _p(dx), _p(dw), beta, WGRAD_SKIP_EMPTY if skip_empty else 0, _stream())
    _check(rc, "moe_grouped_gemm_bwd")
    return dx, dw


# ----------------------------------------------------------- combine / misc

def moe_combine(yp, gates, inv_perm):
    T, k = gates.shape
    d = yp.shape[1]
    y = _empty((T, d), torch.bfloat16, yp)
    rc = lib().moe_combine(_p(yp), _p(gates), _p(inv_perm), T, k, d, _p(y), _stream())
    _check(rc, "moe_combine")
    return y


def moe_hmx8_quant(x):
    """Combine-path payload of x [rows, cols] float32: (codes int8, scales uint8 [rows, cols/32])."""
    _dev(x, torch.float32, "moe_hmx8_quant")
    rows, cols = x.shape
    codes = _empty((rows, cols), torch.int8, x)
    sf = _empty((rows, cols // 32), torch.uint8, x)
    rc = lib().moe_hmx8_quant(_p(x), rows, cols, _p(codes), _p(sf), _stream())
    _check(rc, "moe_hmx8_quant")
    return codes, sf


def moe_hmx8_dequant(codes, sf):
    rows, cols = codes.shape
    out = _empty((rows, cols), torch.float32, codes)
    rc = lib().moe_hmx8_dequant(_p(codes), _p(sf), rows, cols, _p(out), _stream())
    _check(rc, "moe_hmx8_dequant")
    return out


def moe_combine_hmx8(codes, sf, gates, inv_perm):
    T, k = gates.shape
    d = codes.shape[1]
    y = _empty((T, d), torch.bfloat16, codes)
    rc = lib().moe_combine_hmx8(_p(codes), _p(sf), _p(gates), _p(inv_perm), T, k, d, _p(y), _stream())
    _check(rc, "moe_combine_hmx8")
    return y


def moe_unpermute_sum(dxp, inv_perm, T, k):
    d = dxp.shape[1]
    dx = _empty((T, d), torch.bfloat16, dxp)
    rc = lib().moe_unpermute_sum(_p(dxp), _p(inv_perm), T, k, d, _p(dx), _stream())
    _check(rc, "moe_unpermute_sum")
    return dx


def moe_dgates(dy, yp, inv_perm, k):
    """Gate gradient dg [T, k] float32: dg[t, j] = <dy[t], yp[inv_perm[t*k + j]]>."""
    _dev(dy, torch.bfloat16, "dy")
    _dev(yp, torch.float32, "yp")
    _dev(inv_perm, torch.int32, "inv_perm")
    T, d = dy.shape
    dg = _empty((T, k), torch.float32, dy)
    rc = lib().moe_dgates(_p(dy), _p(yp), _p(inv_perm), T, k, d, _p(dg), _stream())
    _check(rc, "moe_dgates")
    return dg


def moe_route_backward(dg, gates, topk_idx, E):
    """dlogits [T, E] float32: softmax backward over each token's selected experts."""
    _dev(dg, torch.float32, "dg")
    _dev(gates, torch.float32, "gates")
    _dev(topk_idx, torch.int32, "topk_idx")
    T, k = gates.shape
    out = _empty((T, E), torch.float32, gates)
    rc = lib().moe_route_backward(_p(dg), _p(gates), _p(topk_idx), T, E, k, _p(out), _stream())
    _check(rc, "moe_route_backward")
    return out


# -------------------------------------------------------------------- router

def moe_router_logits(x, w):
    """BF16 router GEMM: x [T, d] bf16, w [E, d] bf16 -> logits [T, E] float32."""
    _dev(x, torch.bfloat16, "x")
    _dev(w, torch.bfloat16, "w")
    T, d = x.shape
    E = w.shape[0]
    out = _empty((T, E), torch.float32, x)
    rc = lib().moe_router_logits(_p(x), _p(w), T, E, d, _p(out), _stream())
    _check(rc, "moe_router_logits")
    return out


def moe_unpermute_sum_router(dxp, inv_perm, T, k, dlogits, topk_idx, w):
    """dx [T, d] bf16: the un-permuting sum of dxp plus the router's input
    gradient sum_j dlogits[t, e_j] * w[e_j] (see moe4.h for the order)."""
    _dev(dxp, torch.float32, "dxp")
    _dev(dlogits, torch.float32, "dlogits")
    _dev(topk_idx, torch.int32, "topk_idx")
    _dev(w, torch.bfloat16, "w")
    d = dxp.shape[1]
    E = w.shape[0]
    dx = _empty((T, d), torch.bfloat16, dxp)
    rc = lib().moe_unpermute_sum_router(_p(dxp), _p(inv_perm), T, k, d, _p(dlogits), _p(topk_idx), E, _p(w), _p(dx),
                                        _stream())
    _check(rc, "moe_unpermute_sum_router")
    return dx


def moe_router_wgrad(x, dlogits, perm, expert_off, k):
    """dW_r [E, d] float32 = sum over the tokens routed to e of dlogits[t, e] * x[t]."""
    _dev(x, torch.bfloat16, "x")
    _dev(dlogits, torch.float32, "dlogits")
    T, d = x.shape
    E = dlogits.shape[1]
    dw = _empty((E, d), torch.float32, x)
    ws = _ws(lib().moe_router_wgrad_ws_bytes(T, E, k, d), x)
    rc = lib().moe_router_wgrad(_p(x), _p(dlogits), _p(perm), _p(expert_off), T, E, k, d, _p(dw), _p(ws), ws.numel(),
                                _stream())
    _check(rc, "moe_router_wgrad")
    return dw


def moe4_debug_check():
    """Synchronise the current stream; raise Moe4Error on a failed launch and
    Moe4DeviceError on a device-side error report (which this clears)."""
    _check(lib().moe4_debug_check(_stream()), "moe4_debug_check")


def moe4_debug_force_wait_timeout(on):
    """Test hook: make nvfp4_quant_requant_T's bounded waits give up (see moe4.h)."""
    _check(lib().moe4_debug_force_wait_timeout(int(bool(on))), "moe4_debug_force_wait_timeout")


def moe_silu_eval(u):
    _dev(u, torch.bfloat16, "u")
    s = _empty(u.shape, torch.float32, u)
    d = _empty(u.shape, torch.float32, u)
    rc = lib().moe_silu_eval(_p(u), u.numel(), _p(s), _p(d), _stream())
    _check(rc, "moe_silu_eval")
    return s, d
