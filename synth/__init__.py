"""Seeded synthetic inputs for the CSA layer (shared by the tests, the bench and the smoke check).

This package draws random numbers and encodes them into the storage formats the layer consumes
(fp32, bf16 bit patterns, MXFP4 codes with e8m0 scales). It holds none of the layer's arithmetic:
no pooling, scoring, selection or attention happens here.
"""
from .workloads import WORKLOADS, Workload, get  # noqa: F401
from .gen import make_inputs  # noqa: F401
