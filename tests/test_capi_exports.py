"""The C-ABI library loads and exports every function include/moe4.h declares
(no compute calls: this runs without a GPU), and host-side argument checks
reject bad calls before anything is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe4.h")
LIB = os.path.join(ROOT, "precision_moe_numerics_quant_amd", "libmoe4.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|void)\s*\**\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def _lib():
    if not os.path.exists(LIB):
        pytest.skip("libmoe4.so not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_named_calls():
    names = declared_functions()
    for n in ("nvfp4_quant_46", "nvfp4_quant_requant_T", "mxfp8_requant_sr_T", "moe_grouped_gemm_fwd", "moe_grouped_gemm_bwd",
              "moe_grouped_gemm_bwd_dgrad", "moe_grouped_gemm_bwd_wgrad", "moe_route_topk", "mxfp8_quant",
              "moe_dgates", "moe_route_backward", "moe4_debug_check"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    import precision_moe_numerics_quant_amd as m4
    assert sorted(set(m4.EXPORTS) - {"nvfp4_quant_46_ws_bytes", "moe_route_topk_ws_bytes"}) == \
        sorted(set(declared_functions()) - {"nvfp4_quant_46_ws_bytes", "moe_route_topk_ws_bytes"})


def test_validation_errors_without_gpu():
    """Argument checks run on the host and return before any HIP call."""
    L = _lib()
    L.nvfp4_quant_46.restype = ctypes.c_int
    L.moe4_last_error.restype = ctypes.c_char_p
    v = ctypes.c_void_p
    # cols not a multiple of 16
    rc = L.nvfp4_quant_46(v(16), 0, ctypes.c_int64(4), ctypes.c_int64(20), v(0), 1, 46, 0, v(16), v(16), v(16),
                          v(16), ctypes.c_size_t(64), v(0))
    assert rc == -1 and b"multiple of 16" in L.moe4_last_error()
    # bad mode
    rc = L.nvfp4_quant_46(v(16), 0, ctypes.c_int64(4), ctypes.c_int64(32), v(0), 1, 5, 0, v(16), v(16), v(16),
                          v(16), ctypes.c_size_t(64), v(0))
    assert rc == -1
    # workspace too small
    rc = L.nvfp4_quant_46(v(16), 0, ctypes.c_int64(4), ctypes.c_int64(32), v(16), 8, 46, 0, v(16), v(16), v(16),
                          v(16), ctypes.c_size_t(4), v(0))
    assert rc == -3
    # misaligned
    rc = L.nvfp4_quant_46(v(17), 0, ctypes.c_int64(4), ctypes.c_int64(32), v(0), 1, 46, 0, v(16), v(16), v(16),
                          v(16), ctypes.c_size_t(64), v(0))
    assert rc == -2
    L.moe_route_topk.restype = ctypes.c_int
    rc = L.moe_route_topk(v(16), v(0), ctypes.c_int64(4), 8, 9, v(16), v(16), v(16), v(16), v(16), v(16), v(16),
                          ctypes.c_size_t(1 << 20), v(0))
    assert rc == -1                                   # k > E
    L.mxfp8_quant.restype = ctypes.c_int
    rc = L.mxfp8_quant(v(16), 1, ctypes.c_int64(4), ctypes.c_int64(48), v(0), 1, v(0), v(0), 0, 0, v(0), v(0), 0,
                       ctypes.c_int64(0), 0, ctypes.c_uint64(0), ctypes.c_uint32(0), v(16), v(16), v(0))
    assert rc == -1                                   # cols % 32
    L.moe_grouped_gemm_fwd.restype = ctypes.c_int
    rc = L.moe_grouped_gemm_fwd(v(16), v(16), v(16), 0, v(16), v(16), v(16), v(16), 2, ctypes.c_int64(8),
                                ctypes.c_int64(64), ctypes.c_int64(100), v(16), 0, v(0))
    assert rc == -1                                   # K % 64
