"""fp64 CPU oracle for stable softmax cross-entropy.

Test infrastructure only: imported by the test suite, the package smoke
check and the benchmark's CPU-baseline leg, never by the HIP product path.
"""
