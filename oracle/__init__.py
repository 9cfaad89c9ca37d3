"""CPU oracle for the K-grouped weight-gradient GEMM (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU product path never imports it.
"""
