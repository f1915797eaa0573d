"""TEST INFRASTRUCTURE ONLY: the CPU oracle for MX block-32 FP4 quantization.

Importable by tests, the smoke check and the benchmark's CPU-baseline leg;
never by the library itself.
"""
