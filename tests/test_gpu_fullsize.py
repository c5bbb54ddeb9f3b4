"""The five workloads at full size, in the launch configuration the benchmark
times, compared with the oracle on every output row.

The oracle runs expert-outer (one float64 GEMM per expert over its rows, the
grouped form of moonep_grouped_gemm on the moonep_experts page), so the whole
output of even the fine-grained layer is checked in well under a minute on
the host. Before each call the output and the workspace are filled with bf16
NaN, and both sit between canary bands: a row or tile the kernels never write
shows up as NaN, and a write outside either buffer changes a band."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL, Guarded, LazyExperts, rel_err, to_np, wl_act_kw
from mixture_experts_expert_02_amd import binding as B

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def device_inputs(wl, seed=0):
    ids, w = synth.make_routing(wl, seed=seed)
    x = synth.make_x(wl, device=DEV, seed=seed)
    if wl.wfmt == "mxfp4":
        (cg, sg), (cu_, su), (cd, sd) = synth.make_mxfp4_weights(wl, device=DEV, seed=seed)
        W, S = (cg, cu_, cd), (sg, su, sd)
    else:
        W, S = synth.make_bf16_weights(wl, device=DEV, seed=seed), None
    return x, ids, w, W, S


def row_tiles_covered(counts, bm):
    """(segment, row tile) pairs of a grouping; with every row compared they
    are all checked."""
    return sum((int(c) + bm - 1) // bm for c in counts)


@pytest.mark.parametrize("name", ["tiny", "mixtral_prefill", "fine_grained_prefill", "mxfp4_decode"])
def test_token_major_workload_full_tensor(name):
    wl = synth.workload(name)
    print(f"[fullsize] {name}: T={wl.T} H={wl.H} I={wl.I} E={wl.E} k={wl.k} {wl.wfmt} {wl.act}", flush=True)
    x, ids, w, W, S = device_inputs(wl)
    ids_d, w_d = torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    kw = wl_act_kw(wl)
    p = B.problem(wl.T, wl.H, wl.I, wl.E, wl.k, wl.wfmt, **kw)
    ws = Guarded(B.moe_experts_workspace_bytes(p), DEV)
    out = Guarded(wl.T * wl.H * 2, DEV)
    outs = []
    for rep in range(2):
        ws.poison()
        out.poison()
        B.experts_forward(x, ids_d, w_d, *W, scales=S, out=out.view_bf16(wl.T, wl.H), workspace=ws.body, **kw)
        torch.cuda.synchronize()
        ws.check_bands()
        out.check_bands()
        outs.append(out.view_bf16(wl.T, wl.H).clone())
    assert B.moe_device_error(ws.body) == 0
    assert torch.equal(outs[0], outs[1]), "run-to-run results differ"
    got = outs[0].float()
    assert bool(torch.isfinite(got).all()), f"{int((~torch.isfinite(got)).sum())} output values not written"
    mx = wl.wfmt == "mxfp4"
    E = wl.E
    if mx:
        Wo = [(LazyExperts(W[i], range(E)), LazyExperts(S[i], range(E))) for i in range(3)]
    else:
        Wo = [LazyExperts(W[i], range(E)) for i in range(3)]
    ref = oracle.experts_forward(to_np(x), ids, w, *Wo, **kw)
    err = rel_err(to_np(outs[0]), ref)
    counts = np.bincount(ids[(ids >= 0) & (ids < E)].ravel(), minlength=E)
    tiles = row_tiles_covered(counts, 16 if mx or wl.T * wl.k <= 32 * E else 256)
    print(f"[fullsize] {name}: all {wl.T} tokens ({int(counts.sum())} routed rows, {tiles} row tiles), "
          f"max|err|/max|ref| {err:.2e}", flush=True)
    assert err <= TOL


def test_pregrouped_workload_full_tensor():
    wl = synth.workload("pregrouped")
    print(f"[fullsize] pregrouped: NvS={wl.T} H={wl.H} I={wl.I} segments={wl.E}", flush=True)
    lengths, source = synth.make_pregrouped_layout(wl)
    cu = np.cumsum(lengths).astype(np.int32)
    x = synth.make_x(wl, device=DEV)
    W = synth.make_bf16_weights(wl, device=DEV, source=source)
    rw = synth.make_route_weights_nvs(wl)
    cu_d = torch.from_numpy(cu).to(DEV)
    rw_d = torch.from_numpy(rw).to(DEV)
    p = B.problem(wl.T, wl.H, wl.I, wl.E, 1)
    ws = Guarded(B.moe_experts_grouped_workspace_bytes(p), DEV)
    out = Guarded(wl.T * wl.H * 2, DEV)
    outs = []
    for rep in range(2):
        ws.poison()
        out.poison()
        B.experts_forward_grouped(x, cu_d, rw_d, *W, out=out.view_bf16(wl.T, wl.H), workspace=ws.body)
        torch.cuda.synchronize()
        ws.check_bands()
        out.check_bands()
        outs.append(out.view_bf16(wl.T, wl.H).clone())
    assert B.moe_device_error(ws.body) == 0
    assert torch.equal(outs[0], outs[1])
    got = outs[0].float()
    assert bool(torch.isfinite(got).all()), f"{int((~torch.isfinite(got)).sum())} output values not written"
    Wl = [LazyExperts(t, range(wl.E)) for t in W]
    ref = oracle.pregrouped_forward(to_np(x), cu, rw, *Wl)
    err = rel_err(to_np(outs[0]), ref)
    print(f"[fullsize] pregrouped: all {wl.T} rows over {int(np.sum(lengths > 0))} non-empty segments "
          f"({row_tiles_covered(lengths, 256)} row tiles), max|err|/max|ref| {err:.2e}", flush=True)
    assert err <= TOL
