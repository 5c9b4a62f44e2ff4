"""CPU oracle for the FP8 (E4M3) P-cast attention forward.

TEST INFRASTRUCTURE ONLY. Plain, slow fp64 numpy code written from the P-Cast pages
(see each module's header for the passages it follows). Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import it. The HIP library
and its Python binding never import it, and it imports nothing from them.

Modules
  e4m3        OCP E4M3FN and bf16 codecs (round-to-nearest-even).
  attention   the block-wise online softmax with the P·S cast, forward or reverse KV
              order (also the sink-last reverse walk and the quantized row-sum
              denominator); its closed-form restatement; exact attention; the collapse
              counter; the rounding-boundary allowance; split-KV decode (split ranges,
              per-split states, their exact merge).
  theory      F(Δ,S), δ_k, Δ_c, d_p(S), the reverse-order bound, fp32 round trips.
  mfma_model  the FP8 matrix core's accumulation, used only to bound which casts the
              device may round the other way (its arithmetic also in csrc/mfma_model.c).

Pins: every function is checked in tests/test_oracle_*.py against values the pages
fix, closed forms, textbook routines or brute force. The absolute MSE values of the
pages' experiments are not printed on the pages (only ratios), so absolute MSE is
parity unpinned; the oracle's own value is the authority there.
"""
