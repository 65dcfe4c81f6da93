"""CPU oracle for the NVFP4-forward / MXFP8-backward MoE expert layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never imports, calls or
links it, and this package imports nothing from the product path.

What this package computes is the method described on the pages about
Thinking Machines Lab's "End-to-End 4-Bit Training" post:

* NVFP4 forward quantisation of expert-layer operands (lhc.media page,
  paragraph on NVFP4 "four-bit values with a scale factor shared across
  sixteen values"; agihunt.info page, "Confirmed", for the Four Over Six
  choice between two scaling factors);
* the backward path's dequantise -> transpose at high precision -> MXFP8
  requantise with stochastic rounding (lhc.media page, the two paragraphs on
  transposition and stochastic rounding);
* the expert-grouped GEMMs and the routing glue around them.

Every function is plain and slow on purpose: float32 arithmetic is written as
one NumPy float32 operation per IEEE operation (NumPy never contracts a*b+c
into a fused multiply-add), sums are explicit loops in the stated order, and
GEMMs are float64 products of exactly dequantised operands.

Modules
-------
formats   E2M1 / E4M3 / E8M0 / BF16 codecs and roundings
srhash    the counter-based random words used by stochastic rounding
nvfp4     two-level NVFP4 quantisation with the Four-Over-Six choice
mxfp8     MX scale rule, RNE and stochastic rounding, transposed requantisation
route     top-k routing, gates and the stable expert permutation
silu      correctly rounded SiLU and SiLU' tables over all bf16 inputs
gemm      float64 grouped GEMMs on exactly dequantised operands
layer     the whole expert layer, forward and backward
combine_q the combine-path quantiser (block Hadamard + 8-bit fixed-point MX)

Parity pins: every function here is pinned in ``tests/test_oracle_*.py``
against closed forms, brute force, library routines or invariants; the pages
print no worked example for any step, so no pin comes from printed values.
"""
