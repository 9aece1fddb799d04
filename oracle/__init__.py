"""CPU oracle for the DashAttention forward pass (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import this package.
"""
