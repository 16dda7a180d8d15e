"""CPU oracle for the quantized attention forward.

Test infrastructure only: the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import it; the GPU path never does.
"""
