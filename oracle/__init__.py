"""CPU oracle (float64) for Fourier-approximated KV-cache decode.

TEST INFRASTRUCTURE: importable only by the test suite, the smoke check and
the benchmark's CPU-baseline leg.  The GPU library does not import it and it
imports nothing from the GPU library.
"""
from . import fourier_attention, batch  # noqa: F401
