"""Seeded synthetic inputs for the MoE experts path.

This package is shared by the CPU oracle's tests and by the HIP path's
tests and benchmark. It only draws random numbers and lays them out; it
holds none of the experts computation (no grouping, no GEMM, no activation,
no combine). The router that turns logits into top-k ids and weights lives
here because routing happens before the experts path begins.
"""
from .moe_inputs import *  # noqa: F401,F403
