"""Seeded synthetic inputs shared by the CPU oracle's tests, the GPU tests,
the smoke check and the benchmark.

This package builds inputs only (lengths, flat page tables, page pools,
query rows).  It holds none of the attention arithmetic, and neither the
library nor the oracle imports it.
"""
