"""CPU oracle for FP4 block-scaled quantization and the GEMMs that consume it.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``fp4_block_scaled_x16_amd/``) and never imports it.

Everything here is plain NumPy, written to be checked by eye against the
pages it follows:

* "Pretraining Large Language Models with NVFP4" (arXiv:2509.25149):
  §3 (background: E2M1, MXFP4, NVFP4), §4.2 (RHT), §4.3 (2D scaling),
  §4.4 (stochastic rounding), App. B.1-B.4 (Eqs. 1-5), App. C (Hadamard).
* The UE5M3 block-scale FP4 pretraining abstract (arXiv 2609.02846):
  unsigned E5M3 block scales, target T, periodic (stale) tensor amax.
* The 2D-block FP4 training abstract (arXiv 2607.24953): transposition-
  invariant scaling, truncation-free scaling, stochastic rounding on 2D
  blocks.

Floating-point decisions that pick an integer code are taken in fp32, the
precision the NVFP4 paper fixes for the tensor scale (App. B.1) and that its
"high precision" encode-scale inversion (App. B.2) is read to mean.  GEMM
sums are taken in fp64.

Modules:
  formats  - E2M1 / E4M3 / UE5M3 / UE8M0 tables; round-to-nearest-even and
             rounded-up scale encoders
  philox   - Philox4x32-10 counter-based generator (Salmon et al., SC'11)
  rht      - randomized Hadamard transform, 16-point and N = 4 ... 128
  quantize - tensor amax, two-level scales, 1D/2D/colwise quantize,
             stochastic rounding, counters, dequantize
  gemm     - block-scaled GEMM reference in fp64 and its error bound
"""
