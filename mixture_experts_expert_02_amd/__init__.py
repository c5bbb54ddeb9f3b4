"""MoE experts step for MI355X (gfx950): HIP kernels behind a C ABI.

`binding` marshals torch tensors into the C ABI of libmoe_experts.so
(include/moe_experts.h); all computation happens in the HIP library.
"""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    MoeError, align, experts_forward, experts_forward_grouped, moe_align, moe_align_workspace_bytes,
    moe_device_error, moe_experts_forward, moe_experts_forward_grouped, moe_experts_forward_timed,
    moe_experts_grouped_workspace_bytes, moe_experts_workspace_bytes, moe_experts_workspace_layout,
    moe_route, moe_strerror, problem, route, route_problem,
)
