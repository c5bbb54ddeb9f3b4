"""MXFP4 weights with MXFP8 activations at prefill sizes: the LDS-tiled
block-scaled kernels (gemm_mx.hpp) against the oracle's MXFP8 mode.

Covered: 256 rows per expert and more, K and N that are not multiples of 128
(half stages in both GEMMs, a half column tile in GEMM1), skewed routing with
empty experts, masked and bad ids, the route weight on the input, SiTu, GEMM2
with and without its K split, the quantized token rows bit for bit, GEMM1's
epilogue quantization (codes and the per-tile scale blocks) against the
oracle's exact activation, and the same problems on the weight-streaming
kernels (MOE_EXPERTS_MX_PREFILL=0) for comparison.

Outputs are held to 1e-2 of the largest reference value beyond the envelope
of the quantization decisions that the kernels' fp32 GEMM1 may take either
way (helpers.mxfp8_reference_with_envelope): an e4m3 step is up to 1/8 of
an activation value, so one activation element within the fp32 error of a
rounding midpoint moves its output row by up to that step times the down
weights, in the kernels and in the float64 oracle alike."""
import os
import zlib

import numpy as np
import pytest
import torch

import oracle
from helpers import (TOL, check_mxfp8_output, mxfp8_activation_bounds, mxfp8_code_range,
                     mxfp8_reference_with_envelope, rel_err, to_np)
from mixture_experts_expert_02_amd import binding as B
from test_gpu_forward import ACT_PARAMS, make_problem, oracle_out, run_gpu
from test_gpu_mxfp8 import check_split, e4m3_bytes_to_f64, edge_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")

CASES = [
    # name, (T, H, I, E, k), act, extras
    ("rows256", (512, 256, 256, 4, 2), "silu", {}),
    ("half_stages", (600, 320, 192, 3, 2), "swiglu_oai", {}),
    ("skew_ragged", (1500, 384, 512, 5, 2), "silu", {"skew": 1.0}),
    ("skew_empty_masked_bad", (800, 256, 384, 8, 2), "silu", {"skew": 2.0, "masked": 0.1, "bad": 0.05}),
    ("weight_on_input", (700, 256, 256, 4, 1), "silu", {"on_input": True}),
    ("situ", (500, 192, 320, 3, 2), "situ", {}),
    ("k2880", (300, 2880, 256, 2, 2), "swiglu_oai", {}),
]


class env:
    """Set environment variables for the duration of a block."""

    def __init__(self, **kv):
        self.kv = kv

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kv}
        os.environ.update({k: str(v) for k, v in self.kv.items()})

    def __exit__(self, *a):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def problem_for(name, shape, act, extra):
    T, H, I, E, k = shape
    extra = dict(extra)
    on_input = extra.pop("on_input", False)
    x, ids, w, W, S = make_problem(zlib.crc32(name.encode()) % 1000, T, H, I, E, k, "mxfp4", **extra)
    act_kw = dict(act=act, **ACT_PARAMS[act], act_fmt="mxfp8")
    if on_input:
        act_kw["weight_on_input"] = True
    return x, ids, w, W, S, act_kw


def layout_for(shape, act_kw):
    T, H, I, E, k = shape
    kw = {kk: v for kk, v in act_kw.items() if kk in ("act", "alpha", "beta", "limit", "act_fmt", "weight_on_input")}
    return B.moe_experts_workspace_layout(B.problem(T, H, I, E, k, "mxfp4", **kw))


@pytest.mark.parametrize("name,shape,act,extra", CASES, ids=[c[0] for c in CASES])
def test_mx_prefill_matches_oracle(name, shape, act, extra):
    T, H, I, E, k = shape
    print(f"[mx_prefill] {name} T={T} H={H} I={I} E={E} k={k} {act}", flush=True)
    x, ids, w, W, S, act_kw = problem_for(name, shape, act, extra)
    assert layout_for(shape, act_kw).mx_tiled == 1
    out = run_gpu(x, ids, w, W, S, act_kw)
    ref, envl, n_amb = mxfp8_reference_with_envelope(x, ids, w, W, S, act_kw)
    got = to_np(out)
    assert np.all(np.isfinite(got))
    err, beyond, used = check_mxfp8_output(got, ref, envl)
    exact = oracle_out(x, ids, w, W, S, {kk: v for kk, v in act_kw.items() if kk != "act_fmt"})
    print(f"[mx_prefill] {name} rel err {err:.2e}, beyond the decision envelope {beyond:.2e} ({used} outputs "
          f"inside it, {n_amb} activation elements with an open decision; MXFP8 vs exact activations in the "
          f"oracle: {rel_err(ref, exact):.2e})", flush=True)
    assert beyond <= TOL
    again = run_gpu(x, ids, w, W, S, act_kw)
    assert torch.equal(out, again), "run-to-run results differ"
    dead = np.all((ids < 0) | (ids >= E), axis=1)
    assert np.all(got[dead] == 0)
    # the weight-streaming kernels on the same problem
    with env(MOE_EXPERTS_MX_PREFILL=0):
        assert layout_for(shape, act_kw).mx_tiled == 0
        other = to_np(run_gpu(x, ids, w, W, S, act_kw))
    err_o, beyond_o, _ = check_mxfp8_output(other, ref, envl)
    print(f"[mx_prefill] {name} weight-streaming kernels: rel err {err_o:.2e} (beyond the envelope "
          f"{beyond_o:.2e}), tiled vs streaming {rel_err(got, other):.2e}", flush=True)
    assert beyond_o <= TOL


@pytest.mark.parametrize("split", [1, 4])
def test_mx_prefill_down_split(split):
    """GEMM2's K split into ranges (partial outputs summed by the combine)
    and unsplit give outputs within the tolerance of the oracle."""
    name, shape, act = "split", (640, 256, 640, 4, 2), "swiglu_oai"
    print(f"[mx_prefill] down projection with at most {split} K ranges", flush=True)
    x, ids, w, W, S, act_kw = problem_for(name, shape, act, {})
    with env(MOE_EXPERTS_MAX_SPLIT_K=split):
        out = to_np(run_gpu(x, ids, w, W, S, act_kw))
    ref, envl, _ = mxfp8_reference_with_envelope(x, ids, w, W, S, act_kw)
    err, beyond, used = check_mxfp8_output(out, ref, envl)
    print(f"[mx_prefill] split {split}: rel err {err:.2e}, beyond the decision envelope {beyond:.2e}", flush=True)
    assert beyond <= TOL


@pytest.mark.parametrize("shape", [(300, 320, 192, 3, 2), (520, 256, 384, 4, 2)])
def test_mx_prefill_quantized_rows(shape):
    """x's rows (token order) bit for bit against the oracle's quantizer; the
    activation rows GEMM1's epilogue writes (codes in sorted order, scales in
    the per-tile blocks) against the oracle's activation a and the bound d on
    the kernels' fp32 error (helpers.mxfp8_activation_bounds): each scale
    code lies between the codes of the block taken at magnitudes |a| - d and
    |a| + d, and each element, with the kernels' scale, between the e4m3
    roundings of a - d and a + d (rounding is monotone). Printed: how many codes and
    elements differ from the oracle's own decisions."""
    T, H, I, E, k = shape
    print(f"[mx_prefill] quantized rows T={T} H={H} I={I} E={E} k={k}", flush=True)
    x, ids, w, W, S = make_problem(31 + T, T, H, I, E, k, "mxfp4")
    x = edge_rows(x)
    act_kw = dict(act="swiglu_oai", **ACT_PARAMS["swiglu_oai"], act_fmt="mxfp8")
    kw = {kk: v for kk, v in act_kw.items() if kk != "act_fmt"}
    p = B.problem(T, H, I, E, k, "mxfp4", act_fmt="mxfp8", **kw)
    lay = B.moe_experts_workspace_layout(p)
    assert lay.mx_tiled == 1 and lay.xq_rows == T
    ws = B.alloc_workspace(B.moe_experts_workspace_bytes(p), DEV)
    B.experts_forward(x.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                      *[t.to(DEV) for t in W], scales=[t.to(DEV) for t in S], workspace=ws, **act_kw)
    torch.cuda.synchronize()
    check_split(ws, lay.xq, T, H, to_np(x), T)

    M = T * k
    al, a64, d64, _ = mxfp8_activation_bounds(x, ids, w, W, S, act_kw)
    n_valid = a64.shape[0]
    codes_ws = ws[lay.aq: lay.aq + M * I].view(M, I)[:n_valid]
    # scale codes from the per-tile blocks: the align's 256-row tiles of each
    # segment, in segment order
    NTc = (I + 127) // 128
    blocks = ws[lay.aq_sc:].cpu().numpy()
    sc = np.zeros((n_valid, I // 32), dtype=np.int64)
    t = 0
    start = 0
    for e in range(E):
        end = int(al["cu_seqlens"][e])
        for r0 in range(start, end, 256):
            for r in range(r0, min(r0 + 256, end)):
                for g in range(NTc):
                    at = (t * NTc + g) * 1024 + (r - r0) * 4
                    for b in range(4):
                        if 4 * g + b < I // 32:
                            sc[r, 4 * g + b] = blocks[at + (((b & 1) << 1) | (b >> 1))]
            t += 1
        start = end
    _, elem, want = oracle.mxfp8_quantize(a64)
    c_lo, c_hi = mxfp8_code_range(a64, d64)
    bad = (sc < c_lo) | (sc > c_hi)
    assert not bad.any(), f"{int(bad.sum())} scale codes outside the range the kernels' precision allows"
    X = np.ldexp(1.0, (sc - 127).astype(np.int32))[..., None]
    got = e4m3_bytes_to_f64(codes_ws).reshape(n_valid, I // 32, 32)
    lo = oracle.e4m3_round((a64 - d64).reshape(n_valid, I // 32, 32) / X)
    hi = oracle.e4m3_round((a64 + d64).reshape(n_valid, I // 32, 32) / X)
    far = (got < lo) | (got > hi)
    if far.any():
        where = np.argwhere(far)[:6]
        detail = [f"row {r} col {32 * b + i}: exact {a64[r, 32 * b + i]!r} bound {d64[r, 32 * b + i]!r} code {int(sc[r, b])} "
                  f"gpu {got[r, b, i]!r} allowed [{lo[r, b, i]!r}, {hi[r, b, i]!r}]" for r, b, i in where]
        raise AssertionError(f"{int(far.sum())} elements outside their allowed range: {detail}")
    same = (sc == want)[..., None] & np.ones((1, 1, 32), dtype=bool)
    diff = (got != elem.reshape(n_valid, I // 32, 32)) & same
    print(f"[mx_prefill] epilogue quantization: {int((sc != want).sum())} of {sc.size} scale codes and "
          f"{int(diff.sum())} of {diff.size} elements differ from the oracle's own decisions (all within the "
          f"kernels' fp32 error bound)", flush=True)


# ------------------------------------------------------------------ packed weights
def host_pack(W, S, H, I):
    """The packed layout of moe_mx_pack_weights, written out on the host from
    the header's description (test infrastructure, not the oracle)."""
    E = W[0].shape[0]
    out = []
    for g1, N, K in ((True, I, H), (False, H, I)):
        KT = -(-K // 128)
        NTc = -(-N // 128) if g1 else -(-N // 256)
        mats = [(W[0].numpy(), S[0].numpy()), (W[1].numpy(), S[1].numpy())] if g1 else [(W[2].numpy(), S[2].numpy())]
        for e in range(E):
            for nt in range(NTc):
                for u in range(KT):
                    blk = np.zeros(17408, dtype=np.uint8)
                    for r in range(256):
                        c_mat, s_mat = mats[r // 128] if g1 else mats[0]
                        n = nt * 128 + (r & 127) if g1 else nt * 256 + r
                        for c in range(4):
                            kb = u * 64 + c * 16
                            if n < N and kb < K // 2:
                                slot = c ^ ((r >> 2) & 3)
                                blk[r * 64 + 16 * slot: r * 64 + 16 * slot + 16] = c_mat[e, n, kb:kb + 16]
                        srow = s_mat[e, min(n, N - 1)]
                        v = [srow[4 * u + t] if 4 * u + t < K // 32 else 0 for t in range(4)]
                        blk[16384 + r * 4: 16384 + r * 4 + 4] = [v[0], v[2], v[1], v[3]]
                    out.append(blk)
    return np.concatenate(out)


def test_mx_pack_layout_matches_host_packer():
    """moe_mx_pack_weights byte for byte against the layout the header
    describes: K with a half stage (H = 320), N with a half column tile
    (I = 192: rows past N are zero), two experts."""
    T, H, I, E, k = 64, 320, 192, 2, 2
    _, _, _, W, S = make_problem(77, T, H, I, E, k, "mxfp4")
    p = B.problem(T, H, I, E, k, "mxfp4", "swiglu_oai", act_fmt="mxfp8")
    packed = B.mx_pack_weights(p, *[t.to(DEV) for t in W], *[t.to(DEV) for t in S])
    torch.cuda.synchronize()
    want = host_pack(W, S, H, I)
    assert packed.numel() == want.size == B.moe_mx_packed_bytes(p)
    got = packed.cpu().numpy()
    assert np.array_equal(got, want), f"{int((got != want).sum())} bytes differ"


@pytest.mark.parametrize("name,shape,act,extra", [CASES[0], CASES[1], CASES[3], CASES[6]],
                         ids=[CASES[i][0] for i in (0, 1, 3, 6)])
def test_mx_prefill_packed_weights_bitwise(name, shape, act, extra):
    """With the packed weights the GEMMs read the same bytes in the same
    order: outputs bit for bit equal to the unpacked path."""
    T, H, I, E, k = shape
    print(f"[mx_prefill] packed weights {name} T={T} H={H} I={I} E={E} k={k}", flush=True)
    x, ids, w, W, S, act_kw = problem_for(name, shape, act, extra)
    Wd, Sd = [t.to(DEV) for t in W], [t.to(DEV) for t in S]
    kw = {kk: v for kk, v in act_kw.items() if kk in ("act", "alpha", "beta", "limit", "weight_on_input")}
    p = B.problem(T, H, I, E, k, "mxfp4", act_fmt="mxfp8", **kw)
    packed = B.mx_pack_weights(p, *Wd, *Sd)
    xd, idd, wd = x.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    a = B.experts_forward(xd, idd, wd, *Wd, scales=Sd, **act_kw)
    b = B.experts_forward(xd, idd, wd, *Wd, scales=Sd, mx_packed=packed, **act_kw)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------------ decode kernels on packed codes
DECODE_PK_CASES = [
    # name, (T, H, I, E, k), act, activation format
    ("silu", (13, 192, 128, 5, 2), "silu", "bf16"),
    ("swiglu_col_tail", (9, 256, 320, 6, 3), "swiglu_oai", "bf16"),  # I = 320: half a column tile, 2.5 K stages
    ("ktail", (6, 2880, 192, 4, 2), "swiglu_oai", "bf16"),           # H = 2880: 22.5 K stages in GEMM1
    ("many_rows", (150, 128, 256, 3, 2), "silu", "bf16"),            # several 16-row tiles per expert
    ("mxfp8", (9, 256, 320, 6, 3), "swiglu_oai", "mxfp8"),
    ("mxfp8_ktail", (6, 2880, 192, 4, 2), "situ", "mxfp8"),
]


@pytest.mark.parametrize("name,shape,act,afmt", DECODE_PK_CASES, ids=[c[0] for c in DECODE_PK_CASES])
def test_decode_packed_codes_bitwise(name, shape, act, afmt):
    """The weight-streaming kernels reading their codes from the packed layout
    (moe_problem.mx_packed) give outputs bit for bit equal to the canonical
    codes': the same codes meet the same activations in the same order, and
    K past the end meets zero activations either way."""
    T, H, I, E, k = shape
    print(f"[mx_packed] decode {name} T={T} H={H} I={I} E={E} k={k} {act} {afmt}", flush=True)
    x, ids, w, W, S = make_problem(21, T, H, I, E, k, "mxfp4")
    kw = dict(act=act, **ACT_PARAMS[act])
    p = B.problem(T, H, I, E, k, "mxfp4", act_fmt=afmt, **kw)
    assert not B.moe_experts_workspace_layout(p).mx_tiled
    Wd, Sd = [t.to(DEV) for t in W], [t.to(DEV) for t in S]
    packed = B.mx_pack_weights(p, *Wd, *Sd)
    xd, idd, wd = x.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    a = B.experts_forward(xd, idd, wd, *Wd, scales=Sd, act_fmt=afmt, **kw)
    b = B.experts_forward(xd, idd, wd, *Wd, scales=Sd, act_fmt=afmt, mx_packed=packed, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_decode_packed_codes_grouped_bitwise():
    """Pre-grouped entry with MXFP4 weights (weight-streaming kernels): packed
    codes against canonical ones, segments of 0, 2, 17 and 40 rows, K = 320."""
    H, I = 320, 256
    lengths = np.array([2, 0, 17, 40], dtype=np.int64)
    G, NvS = len(lengths), int(lengths.sum())
    print(f"[mx_packed] grouped decode NvS={NvS} H={H} I={I} G={G}", flush=True)
    x, _, _, W, S = make_problem(23, NvS, H, I, G, 1, "mxfp4")
    rw = np.random.default_rng(4).random(NvS).astype(np.float32)
    cu = np.cumsum(lengths).astype(np.int32)
    p = B.problem(NvS, H, I, G, 1, "mxfp4")
    Wd, Sd = [t.to(DEV) for t in W], [t.to(DEV) for t in S]
    packed = B.mx_pack_weights(p, *Wd, *Sd)
    args = (x.to(DEV), torch.from_numpy(cu).to(DEV), torch.from_numpy(rw).to(DEV), *Wd)
    a = B.experts_forward_grouped(*args, scales=Sd)
    b = B.experts_forward_grouped(*args, scales=Sd, mx_packed=packed)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
