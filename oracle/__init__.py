"""CPU oracle for the MoE experts path — test infrastructure only.

Plain, slow, obviously correct float64 numpy code. Only the tests, the
package's smoke check and the benchmark's CPU-baseline leg may import it; the
HIP library never calls it and shares no code with it.
"""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_router  # noqa: F401,E402
from .moe_router import route, route_deepseek_v3, route_renormalize  # noqa: F401,E402
