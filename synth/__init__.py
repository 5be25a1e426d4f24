"""Seeded synthetic workloads for block-sparse attention.

This module only draws random inputs and rounds them to the storage dtype.
It holds none of the attention method's arithmetic (no pooling, scores,
masks or softmax), so that both the fp64 oracle and the HIP path can take
their inputs from it without sharing any of the method's code.
"""
from .workloads import (  # noqa: F401
    Workload,
    WORKLOADS,
    make_workload,
    round_to_bf16,
    field_qk,
    lm_qk,
    centroid_qk,
)
