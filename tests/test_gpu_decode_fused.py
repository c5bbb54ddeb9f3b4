"""The single-launch decode step (align prologue, then GEMM1, GEMM2 and the
combine in one persistent launch; flashinfer_moe_ep page, module docstring:
dispatch, compute and combine in one launch) against the separate launches
(MOE_EXPERTS_FUSED_DECODE=0) bit for bit, and against the oracle. Both paths
run the same tile code and the same fixed combine order, so any difference
is a hand-over error between workgroups (a stale or unwritten row). The
workspace is poisoned before every call, so the counters the single launch
needs zeroed must be zeroed by its own prologue, and no wait may give up."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL, Guarded, rel_err, to_np, wl_act_kw
from mixture_experts_expert_02_amd import binding as B
from test_gpu_forward import ACT_PARAMS, make_problem

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def run(p, x, ids, w, W, S, ws, monkeypatch, fused, **kw):
    monkeypatch.setenv("MOE_EXPERTS_FUSED_DECODE", "1" if fused else "0")
    ws.poison()
    out = torch.full((x.shape[0], x.shape[1]), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.experts_forward(x, ids, w, *W, scales=S, out=out, workspace=ws.body, **kw)
    torch.cuda.synchronize()
    ws.check_bands()
    assert B.moe_device_error(ws.body) >= 0  # raises on a timed-out wait
    assert B.moe_experts_workspace_layout(p).single_launch == (1 if fused else 0)
    return out


CASES = [
    ("mxfp4_swiglu", (9, 256, 320, 6, 3), "mxfp4", "swiglu_oai", "bf16", {}),
    ("mxfp4_mxfp8", (13, 192, 128, 5, 2), "mxfp4", "silu", "mxfp8", {}),
    ("mxfp4_ktail_masked_bad", (40, 2880, 192, 6, 3), "mxfp4", "swiglu_oai", "bf16", {"masked": 0.3, "bad": 0.1}),
    ("mxfp4_many_rows", (150, 128, 256, 3, 2), "mxfp4", "silu", "bf16", {}),
    ("mxfp4_one_token", (1, 256, 320, 6, 3), "mxfp4", "situ", "bf16", {}),
    ("bf16_silu", (20, 256, 192, 16, 2), "bf16", "silu", "bf16", {}),
    ("bf16_swiglu_masked", (9, 128, 320, 12, 4), "bf16", "swiglu_oai", "bf16", {"masked": 0.2}),
    ("mxfp4_4096", (6, 4096, 4096, 4, 2), "mxfp4", "swiglu_oai", "mxfp8", {}),
]


@pytest.mark.parametrize("name,shape,wfmt,act,afmt,extra", CASES, ids=[c[0] for c in CASES])
def test_single_launch_equals_separate_launches(name, shape, wfmt, act, afmt, extra, monkeypatch):
    T, H, I, E, k = shape
    print(f"[fused-decode] {name} T={T} H={H} I={I} E={E} k={k} {wfmt} {act} {afmt}", flush=True)
    x, ids, w, W, S = make_problem(zlib.crc32(name.encode()) % 1000, T, H, I, E, k, wfmt, **extra)
    kw = dict(act=act, act_fmt=afmt, **ACT_PARAMS[act])
    p = B.problem(T, H, I, E, k, wfmt, act, act_fmt=afmt, **ACT_PARAMS[act])
    ws = Guarded(B.moe_experts_workspace_bytes(p), DEV)
    args = (x.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), [t.to(DEV) for t in W],
            None if S is None else [t.to(DEV) for t in S])
    fused = run(p, *args, ws, monkeypatch, True, **kw)
    sep = run(p, *args, ws, monkeypatch, False, **kw)
    again = run(p, *args, ws, monkeypatch, True, **kw)
    assert torch.equal(fused, sep), "single launch differs from the separate launches"
    assert torch.equal(fused, again)
    Wn = [to_np(t) for t in W] if S is None else [(c.numpy(), s.numpy()) for c, s in zip(W, S)]
    ref = oracle.experts_forward(to_np(x), ids, w, *Wn, **kw)
    err = rel_err(to_np(fused), ref)
    print(f"[fused-decode] {name} rel err {err:.2e}", flush=True)
    assert err <= TOL


def test_single_launch_decode_workload_and_smaller_call_on_same_workspace(monkeypatch):
    wl = synth.workload("mxfp4_decode")
    ids, w = synth.make_routing(wl)
    x = synth.make_x(wl, device=DEV)
    (cg, sg), (cu, su), (cd, sd) = synth.make_mxfp4_weights(wl, device=DEV)
    kw = wl_act_kw(wl)
    p = B.problem(wl.T, wl.H, wl.I, wl.E, wl.k, "mxfp4", **kw)
    ws = Guarded(B.moe_experts_workspace_bytes(p), DEV)
    W, S = (cg, cu, cd), (sg, su, sd)
    ids_d, w_d = torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    for afmt in ("bf16", "mxfp8"):
        print(f"[fused-decode] decode workload, {afmt} activations", flush=True)
        f = run(p, x, ids_d, w_d, W, S, ws, monkeypatch, True, act_fmt=afmt, **kw)
        s_ = run(p, x, ids_d, w_d, W, S, ws, monkeypatch, False, act_fmt=afmt, **kw)
        assert torch.equal(f, s_)
    # a smaller problem on the same workspace, then the full one again
    Ts = 5
    f_small = run(p, x[:Ts], ids_d[:Ts].contiguous(), w_d[:Ts].contiguous(), W, S, ws, monkeypatch, True, **kw)
    ref_small = oracle.experts_forward(to_np(x[:Ts]), ids[:Ts], w[:Ts],
                                       *[(c.cpu().numpy(), s.cpu().numpy()) for c, s in zip(W, S)], **kw)
    assert rel_err(to_np(f_small), ref_small) <= TOL
    f2 = run(p, x, ids_d, w_d, W, S, ws, monkeypatch, True, **kw)
    s2 = run(p, x, ids_d, w_d, W, S, ws, monkeypatch, False, **kw)
    assert torch.equal(f2, s2)
