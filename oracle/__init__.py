"""CPU oracle for the 4-bit fused-MoE expert path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product library uses this package: only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import it.  It shares
no code, tables or constants with the HIP library and never imports it.

The oracle is the plain definition of what the path computes, written from the
project pages (cited per function):

* ``nf4``   — NF4 blockwise quantise / pack / dequantise (block 64, fp32 absmax).
* ``mxfp4`` — MXFP4 quantise / pack / dequantise (e2m1 elements, e8m0 scale per 32).
* ``route`` — top-k routing with softmax weights, per-expert counts, offsets, and the
  expert-major stable slot order.
* ``moe``   — the MoE layer forward in float64: per-expert gate_up matmul, SwiGLU, down
  matmul, top-k weighted combine; plus the output tolerance.

Pins (tests/test_oracle_pins.py) tie each part to something other than itself: the
published NF4 codebook and its closed-form construction, the figures the pages print
(pack shapes, ~28% size, NF4 MAE/RMSE, round-trip errors), OCP e2m1 bit-field values,
exact round trips, power-of-two invariance, brute-force routing and brute-force matmul.
Whole-layer output values are not printed by any page: beyond those pins the forward is
"parity unpinned" and stands as the definition.
"""
