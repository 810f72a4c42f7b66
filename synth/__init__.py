"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

Holds random-number generation, storage-format encoders and workload recipes
only; none of the attention method's arithmetic lives here.
"""
from . import configs, formats, rng  # noqa: F401
