"""MX block-32 FP4 quantization with block-Hadamard rotation, and the
block-scaled FP4 weight-gradient GEMM, on AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libmxq.so`` (hand-written HIP
kernels); ``mxq`` is its thin ctypes binding.  ``synth`` makes the seeded
synthetic inputs.
"""
