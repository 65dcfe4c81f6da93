"""The allocation-free entry point nvfp4_quant_46_noalloc (the library's static
scratch in place of a workspace) gives the bytes nvfp4_quant_46 gives, on two
calls in a row with the second smaller, and rejects what its scratch cannot
hold with nothing enqueued."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import cuda_i32

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import precision_moe_numerics_quant_amd as m4


def _same(a, b, what):
    for i, (p, q) in enumerate(zip(a, b)):
        assert torch.equal(p, q), f"{what}: output {i} differs"


def _groups(R, G, seed):
    rng = np.random.default_rng(seed)
    cut = np.sort(rng.integers(0, R + 1, G - 1))
    return cuda_i32(np.concatenate([[0], cut, [R]]))


@pytest.mark.parametrize("pre_op", ["none", "silu"])
def test_noalloc_matches_workspace_call_twice_smaller_second(pre_op):
    pre = m4.PRE_SILU if pre_op == "silu" else m4.PRE_NONE
    # first call: 3000 ragged groups (some empty) of a 4096 x 512 bf16 tensor
    x1 = synth.activations(4096, 512, "cuda", 21, outlier_p=0.001, outlier_mul=30.0)
    off1 = _groups(4096, 3000, 1)
    print(f"noalloc call 1 ({pre_op}): 4096 x 512, 3000 groups", flush=True)
    a = m4.nvfp4_quant_46_noalloc(x1, m4.NVFP4_4OVER6, off1, pre)
    b = m4.nvfp4_quant_46(x1, m4.NVFP4_4OVER6, off1, pre)
    torch.cuda.synchronize()
    _same(a, b, "first call")
    # second call, smaller: 700 x 256, 7 groups; the scratch keeps the first
    # call's amax words beyond these, and the call must not see them
    x2 = synth.activations(700, 256, "cuda", 22) * 0.01
    off2 = _groups(700, 7, 2)
    print(f"noalloc call 2 ({pre_op}): 700 x 256, 7 groups", flush=True)
    a = m4.nvfp4_quant_46_noalloc(x2, m4.NVFP4_4OVER6, off2, pre)
    b = m4.nvfp4_quant_46(x2, m4.NVFP4_4OVER6, off2, pre)
    torch.cuda.synchronize()
    _same(a, b, "second call")
    # one group, float32, mode 6, written into caller-given outputs
    x3 = torch.randn((96, 64), device="cuda") * 0.02
    out = (torch.empty((96, 32), dtype=torch.uint8, device="cuda"),
           torch.empty((96, 4), dtype=torch.uint8, device="cuda"), torch.empty((1,), device="cuda"))
    a = m4.nvfp4_quant_46_noalloc(x3, m4.NVFP4_6, out=out)
    b = m4.nvfp4_quant_46(x3, m4.NVFP4_6)
    torch.cuda.synchronize()
    _same(a, b, "third call")
    m4.moe4_debug_check()


def test_noalloc_rejects_what_the_scratch_cannot_hold():
    x = torch.zeros((8, 32), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m4.Moe4Error, match="4096"):
        m4.nvfp4_quant_46_noalloc(x, m4.NVFP4_4OVER6, cuda_i32(np.zeros(4098, dtype=np.int32)))
    with pytest.raises(m4.Moe4Error, match="pre_op"):
        m4.nvfp4_quant_46_noalloc(x, m4.NVFP4_4OVER6, None, m4.PRE_SILU_AMAX)
