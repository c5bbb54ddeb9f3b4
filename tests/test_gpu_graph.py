"""The experts step captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay equals the eager result bit for bit, with eager work
and synchronisations between replays. Covers the bf16 prefill path with
cold segments (the second stream forks from and joins the captured stream),
the MXFP4 x MXFP8 prefill path with packed weights (persistent workgroups),
and the decode path, each also on the kernels' packed weight layouts where
they have one. The first call runs eagerly before capture: it sets kernel
attributes and creates the second stream."""
import numpy as np
import pytest
import torch

from mixture_experts_expert_02_amd import binding as B
from test_gpu_forward import ACT_PARAMS, make_problem

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")

CASES = [
    # name, shape, weights, act, routing extras, activation format, packed weight layout
    ("bf16_cold_segments", (600, 192, 320, 24, 2), "bf16", "swiglu_oai", {"skew": 1.3}, "bf16", False),
    ("bf16_cold_segments_packed", (600, 192, 320, 24, 2), "bf16", "swiglu_oai", {"skew": 1.3}, "bf16", True),
    ("mxfp4_prefill_packed", (600, 320, 192, 3, 2), "mxfp4", "swiglu_oai", {}, "mxfp8", True),
    ("decode_mxfp4", (13, 192, 128, 5, 2), "mxfp4", "silu", {}, "bf16", False),
    ("decode_mxfp4_packed", (13, 192, 128, 5, 2), "mxfp4", "silu", {}, "bf16", True),
]


@pytest.mark.parametrize("name,shape,wfmt,act,extra,afmt,pack", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager(name, shape, wfmt, act, extra, afmt, pack):
    T, H, I, E, k = shape
    print(f"[graph] {name} T={T} H={H} I={I} E={E} k={k} {wfmt} {afmt}", flush=True)
    x, ids, w, W, S = make_problem(41, T, H, I, E, k, wfmt, **extra)
    xd, idd, wd = x.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    Wd = [t.to(DEV) for t in W]
    Sd = None if S is None else [t.to(DEV) for t in S]
    p = B.problem(T, H, I, E, k, wfmt, act, **ACT_PARAMS[act], act_fmt=afmt)
    packed = None
    if pack and wfmt == "mxfp4":
        packed = B.mx_pack_weights(p, *Wd, *Sd)
        p.mx_packed = packed.data_ptr()
    elif pack:
        packed = B.bf16_pack_weights(p, *Wd)
        p.bf16_packed = packed.data_ptr()
    ws = B.alloc_workspace(B.moe_experts_workspace_bytes(p), DEV)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    sg, su, sd = Sd if Sd is not None else (None, None, None)

    def fwd():
        rc = B.moe_experts_forward(p, xd, idd, wd, *Wd, sg, su, sd, out, ws)
        assert rc == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()  # eager, outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    for i in range(4):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=DEV).sum()  # the program's own eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager result"
        assert torch.isfinite(junk)
