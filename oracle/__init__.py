"""CPU oracle for the weight-quantized GEMM (test infrastructure only).

Only the test suite, the smoke check and the bench's CPU-baseline leg may
import this package; the product path never does.
"""
