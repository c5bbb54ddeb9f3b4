"""The five workloads at full size, in the launch configuration the benchmark
times, compared with the oracle on every output row.

The oracle runs expert-outer (one float64 GEMM per expert over its rows, the
grouped form of moonep_grouped_gemm on the moonep_experts page), so the whole
output of even the fine-grained layer is checked in well under a minute on
the host. Before each call the output and the workspace are filled with bf16
NaN, and both sit between canary bands: a row or tile the kernels never write
shows up as NaN, and a write outside either buffer changes a band. The
weights run as the benchmark runs them, in the kernels' layouts
(moe_bf16_pack_weights, moe_mx_pack_weights), after one call on the
canonical layout that must give the same bits."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (TOL, Guarded, LazyExperts, check_mxfp8_output, mxfp8_activation_bounds, mxfp8_code_range,
                     mxfp8_reference_with_envelope, rel_err, to_np, wl_act_kw)
from test_gpu_mxfp8 import check_split
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
    packed = B.bf16_pack_weights(p, *W) if wl.wfmt == "bf16" else B.mx_pack_weights(p, *W, *S)
    pk = "bf16_packed" if wl.wfmt == "bf16" else "mx_packed"
    outs = []
    for rep in range(3):
        ws.poison()
        out.poison()
        B.experts_forward(x, ids_d, w_d, *W, scales=S, out=out.view_bf16(wl.T, wl.H), workspace=ws.body,
                          **{pk: packed if rep > 0 else None}, **kw)
        torch.cuda.synchronize()
        ws.check_bands()
        out.check_bands()
        outs.append(out.view_bf16(wl.T, wl.H).clone())
    assert B.moe_device_error(ws.body) == 0
    assert torch.equal(outs[-2], outs[-1]), "run-to-run results differ"
    assert torch.equal(outs[0], outs[1]), "the packed weights change the result"
    del packed
    got = outs[-1].float()
    assert bool(torch.isfinite(got).all()), f"{int((~torch.isfinite(got)).sum())} output values not written"
    mx = wl.wfmt == "mxfp4"
    E = wl.E
    if mx:
        Wo = [(LazyExperts(W[i], range(E)), LazyExperts(S[i], range(E))) for i in range(3)]
    else:
        Wo = [LazyExperts(W[i], range(E)) for i in range(3)]
    ref = oracle.experts_forward(to_np(x), ids, w, *Wo, **kw)
    err = rel_err(to_np(outs[-1]), ref)
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
    packed = B.bf16_pack_weights(p, *W)
    outs = []
    for rep in range(3):
        ws.poison()
        out.poison()
        B.experts_forward_grouped(x, cu_d, rw_d, *W, out=out.view_bf16(wl.T, wl.H), workspace=ws.body,
                                  bf16_packed=packed if rep > 0 else None)
        torch.cuda.synchronize()
        ws.check_bands()
        out.check_bands()
        outs.append(out.view_bf16(wl.T, wl.H).clone())
    assert B.moe_device_error(ws.body) == 0
    assert torch.equal(outs[1], outs[2])
    assert torch.equal(outs[0], outs[1]), "operand-block weights change the result"
    del packed
    got = outs[-1].float()
    assert bool(torch.isfinite(got).all()), f"{int((~torch.isfinite(got)).sum())} output values not written"
    Wl = [LazyExperts(t, range(wl.E)) for t in W]
    ref = oracle.pregrouped_forward(to_np(x), cu, rw, *Wl)
    err = rel_err(to_np(outs[-1]), ref)
    print(f"[fullsize] pregrouped: all {wl.T} rows over {int(np.sum(lengths > 0))} non-empty segments "
          f"({row_tiles_covered(lengths, 256)} row tiles), max|err|/max|ref| {err:.2e}", flush=True)
    assert err <= TOL


def test_mxfp4_prefill_workload_full_size():
    """MXFP4 weights with MXFP8 activations at 8192 tokens (the LDS-tiled
    block-scaled kernels). Every token: outputs written (NaN-poisoned
    buffers), canary bands intact, run-to-run bit equality, the quantized
    token rows bit for bit against the oracle's quantizer. The first 1024
    tokens (4096 activation rows, every expert): each activation code and
    scale GEMM1's epilogue wrote lies in the range the kernels' fp32 error
    bound allows, and the outputs are within the tolerance beyond the
    envelope of those decisions (helpers.mxfp8_reference_with_envelope; at
    K = 2880 the worst-case bound leaves a wide envelope, so the plain error
    is printed beside it)."""
    wl = synth.workload("mxfp4_prefill")
    print(f"[fullsize] mxfp4_prefill: T={wl.T} H={wl.H} I={wl.I} E={wl.E} k={wl.k} {wl.act} {wl.act_fmt}", flush=True)
    x, ids, w, W, S = device_inputs(wl)
    ids_d, w_d = torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    kw = wl_act_kw(wl)
    p = B.problem(wl.T, wl.H, wl.I, wl.E, wl.k, wl.wfmt, **kw)
    lay = B.moe_experts_workspace_layout(p)
    assert lay.mx_tiled == 1 and lay.xq_rows == wl.T
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
    check_split(ws.body, lay.xq, wl.T, wl.H, to_np(x), wl.T)

    n = 1024
    Wc, Sc = [t.cpu() for t in W], [t.cpu() for t in S]
    kw8 = dict(kw)
    sub = (x[:n].cpu(), ids[:n], w[:n], Wc, Sc, kw8)
    # the sample's activation rows inside the full problem's sorted order
    al_full = oracle.align(ids, wl.E)
    al_sub, a64, d64, _ = mxfp8_activation_bounds(*sub)
    full_rows = al_full["inv_perm"].reshape(wl.T, wl.k)[:n].reshape(-1)[al_sub["perm"]]
    check_activation_codes(ws.body, lay, wl, al_full, full_rows, a64, d64)
    ref, envl, n_amb = mxfp8_reference_with_envelope(*sub)
    err, beyond, used = check_mxfp8_output(to_np(outs[0][:n]), ref, envl)
    print(f"[fullsize] mxfp4_prefill: first {n} tokens max|err|/max|ref| {err:.2e}, beyond the decision envelope "
          f"{beyond:.2e} ({used} outputs inside it, {n_amb} activation elements with an open decision)", flush=True)
    assert beyond <= TOL


def check_activation_codes(ws, lay, wl, al, rows, a64, d64):
    """GEMM1's e4m3 activation codes and e8m0 scales (per-tile blocks) for
    sorted rows `rows` of the full problem, against the oracle's values a64
    and bounds d64 of those rows (in the same order)."""
    I, M = wl.I, wl.T * wl.k
    NTc = (I + 127) // 128
    # tile and row-in-tile of every sorted row: 256-row tiles of each segment
    cu = al["cu_seqlens"]
    starts = np.concatenate([[0], cu[:-1]])
    seg = np.searchsorted(cu, rows, side="right")
    local = rows - starts[seg]
    tiles_before = np.concatenate([[0], np.cumsum((np.diff(np.concatenate([[0], cu])) + 255) // 256)[:-1]])
    tile = tiles_before[seg] + local // 256
    in_tile = local % 256
    blocks = ws[lay.aq_sc: lay.aq_sc + int(tile.max() + 1) * NTc * 1024].cpu().numpy()
    KB = I // 32
    sc = np.zeros((len(rows), KB), dtype=np.int64)
    for cb in range(KB):
        g, b = cb // 4, cb % 4
        sc[:, cb] = blocks[(tile * NTc + g) * 1024 + in_tile * 4 + (((b & 1) << 1) | (b >> 1))]
    codes = ws[lay.aq: lay.aq + M * I].view(M, I)[torch.as_tensor(rows, device=ws.device)]
    got = codes.view(torch.float8_e4m3fn).to(torch.float64).cpu().numpy().reshape(len(rows), KB, 32)
    c_lo, c_hi = mxfp8_code_range(a64, d64)
    assert not ((sc < c_lo) | (sc > c_hi)).any(), "scale codes outside the range the kernels' precision allows"
    X = np.ldexp(1.0, (sc - 127).astype(np.int32))[..., None]
    lo = oracle.e4m3_round((a64 - d64).reshape(len(rows), KB, 32) / X)
    hi = oracle.e4m3_round((a64 + d64).reshape(len(rows), KB, 32) / X)
    far = (got < lo) | (got > hi)
    if far.any():
        detail = [f"row {int(rows[r])} (tile {int(tile[r])} row {int(in_tile[r])}) col {32 * b + i}: exact "
                  f"{a64[r, 32 * b + i]!r} bound {d64[r, 32 * b + i]!r} scale code {int(sc[r, b])} gpu "
                  f"{got[r, b, i]!r} allowed [{lo[r, b, i]!r}, {hi[r, b, i]!r}]" for r, b, i in np.argwhere(far)[:6]]
        raise AssertionError(f"{int(far.sum())} activation codes outside their allowed range: {detail}")
    _, elem, want = oracle.mxfp8_quantize(a64)
    print(f"[fullsize] activation codes of {len(rows)} rows: {int((sc != want).sum())} scale codes and "
          f"{int((got.reshape(elem.shape) != elem).sum())} elements differ from the oracle's own decisions, all "
          f"within the kernels' fp32 error bound", flush=True)
