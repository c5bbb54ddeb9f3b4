"""Seeded synthetic inputs for the MoE experts path.

This package is shared by the CPU oracle's tests and by the HIP path's
tests and benchmark. It only draws random numbers and lays them out; it
holds none of the experts computation (no grouping, no GEMM, no activation,
no combine). make_routing draws the experts workloads' top-k ids and weights
(an input of the experts step, so both sides see identical ids); the router
kernel is checked against oracle.moe_router, never against make_routing, and
gets its logits from make_logits.
"""
from .moe_inputs import *  # noqa: F401,F403
