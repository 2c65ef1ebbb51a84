"""Seeded synthetic workloads shared by the tests, the smoke check and the
benchmark.  This package draws random numbers and casts them to the input
types (BF16 bit patterns, int8 weights with FP16 scales); it holds none of
the method's arithmetic and imports neither the oracle nor the HIP path."""

from . import workloads  # noqa: F401
