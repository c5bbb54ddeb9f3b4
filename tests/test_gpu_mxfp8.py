"""MXFP8 activations with MXFP4 weights on the GPU (one e4m3 part per value
into the block-scaled MFMA) against the oracle's MXFP8 mode: the quantized
token rows bit for bit, the activation rows (quantized in GEMM1's epilogue
from fp32) against the oracle's exact activation, the output within the
tolerance (the margin printed per case), and the decode workload at full
size."""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL, rel_err, sampled_token_oracle, to_np, wl_act_kw
from mixture_experts_expert_02_amd import binding as B
from test_gpu_forward import ACT_PARAMS, make_problem, oracle_out, run_gpu

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def e4m3_bytes_to_f64(b: torch.Tensor) -> np.ndarray:
    return b.view(torch.float8_e4m3fn).to(torch.float64).cpu().numpy()


def edge_rows(x: torch.Tensor) -> torch.Tensor:
    """Blocks that exercise the quantizer's corners: all zero, one large value
    among small ones, a maximum whose scaled value saturates (1.9375 * 2^8 =
    496 > 448), tiny magnitudes, exact powers of two."""
    x = x.clone()
    H = x.shape[1]
    x[0, 0:32] = 0
    x[0, 32:64] = 1e-3
    x[0, 40] = 3.0e4
    x[1, 0:32] = torch.linspace(-1.0, 1.0, 32)
    x[1, 5] = -1.9375
    x[2, 0:32] = 1e-30
    x[2, 32:64] = torch.tensor([2.0 ** (i % 8 - 4) for i in range(32)])
    if H >= 128:
        x[3, 64:96] = 448.0
        x[3, 96:128] = -7.5e-3
    return x


def check_split(ws, off, R, K, rows_f64, nrows):
    """GPU split rows (hi codes and scale codes) against the oracle quantizer."""
    sc_stride = (K // 32 + 15) // 16 * 16
    hi = ws[off: off + R * K].view(R, K)[:nrows]
    sc = ws[off + 2 * R * K: off + 2 * R * K + R * sc_stride].view(R, sc_stride)[:nrows, : K // 32]
    _, elem, codes = oracle.mxfp8_quantize(rows_f64[:nrows])
    got_elem = e4m3_bytes_to_f64(hi)
    assert np.array_equal(sc.cpu().numpy(), codes), "scale codes differ"
    assert np.array_equal(got_elem, elem), f"e4m3 codes differ at {np.argwhere(got_elem != elem)[:5].tolist()}"


@pytest.mark.parametrize("shape", [(9, 256, 320, 6, 3), (6, 2880, 192, 4, 2), (40, 128, 256, 5, 2)])
def test_mxfp8_split_rows_bit_exact(shape):
    T, H, I, E, k = shape
    print(f"[mxfp8] split rows T={T} H={H} I={I} E={E} k={k}", flush=True)
    x, ids, w, W, S = make_problem(17 + T, T, H, I, E, k, "mxfp4")
    x = edge_rows(x)
    act_kw = dict(act="swiglu_oai", **ACT_PARAMS["swiglu_oai"], act_fmt="mxfp8")
    p = B.problem(T, H, I, E, k, "mxfp4", act_fmt="mxfp8", **{kk: v for kk, v in act_kw.items() if kk != "act_fmt"})
    ws = B.alloc_workspace(B.moe_experts_workspace_bytes(p), DEV)
    B.experts_forward(x.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                      *[t.to(DEV) for t in W], scales=[t.to(DEV) for t in S], workspace=ws, **act_kw)
    torch.cuda.synchronize()
    lay = B.moe_experts_workspace_layout(p)
    assert lay.xq_rows == T  # small problems split the token rows in token order
    check_split(ws, lay.xq, T, H, to_np(x), T)
    M = T * k
    n_valid = int(ws[lay.status + 4: lay.status + 8].view(torch.int32).item())
    check_epilogue_quant(ws, lay.aq, M, I, oracle_activation(x, ids, w, W, S, act_kw), n_valid)


def oracle_activation(x, ids, w, W, S, act_kw):
    """The oracle's down-projection input before quantization, in sorted row
    order: the activation of the MXFP8-quantized token rows times the route
    weight (float64)."""
    E, k = W[0].shape[0], ids.shape[1]
    al = oracle.align(ids, E)
    xr = oracle.mxfp8_quantize(to_np(x)[al["perm"] // k])[0]
    Wn = [(c.numpy(), s.numpy()) for c, s in zip(W, S)]
    g = oracle.grouped_mm(xr, lambda e: oracle.expert_matrix(Wn[0], e), al["cu_seqlens"])
    u = oracle.grouped_mm(xr, lambda e: oracle.expert_matrix(Wn[1], e), al["cu_seqlens"])
    kw = {kk: v for kk, v in act_kw.items() if kk in ("alpha", "beta", "limit")}
    a = oracle.activation(act_kw["act"], g, u, **kw)
    return a * w.reshape(-1)[al["perm"]][:, None]


def e4m3_spacing(v):
    a = np.abs(v)
    _, ex = np.frexp(a)
    return np.ldexp(1.0, (np.maximum(ex - 1, -6) - 3).astype(np.int32))


def check_epilogue_quant(ws, off, R, K, a64, nrows):
    """GEMM1's epilogue quantizes the activation rows from their fp32 value;
    the oracle from the float64 value. Scale codes must agree (except where
    a block's largest magnitude lies within fp32 noise of a power of two),
    and every e4m3 element must be one of the two grid neighbours of the
    exact scaled value, the oracle's own rounding except within fp32 noise of
    a rounding midpoint."""
    sc_stride = (K // 32 + 15) // 16 * 16
    hi = ws[off: off + R * K].view(R, K)[:nrows]
    sc = ws[off + 2 * R * K: off + 2 * R * K + R * sc_stride].view(R, sc_stride)[:nrows]
    codes = sc[:, : K // 32].cpu().numpy().astype(np.int64)
    assert np.all(sc[:, K // 32:].cpu().numpy() == 0), "scale padding bytes not zero"
    _, elem, want = oracle.mxfp8_quantize(a64[:nrows])
    amax = np.abs(a64[:nrows]).reshape(nrows, K // 32, 32).max(axis=-1)
    frac = amax / np.ldexp(1.0, np.frexp(amax)[1] - 1)          # in [1, 2)
    near_pow2 = (np.abs(frac - 1) < 1e-4) | (np.abs(frac - 2) < 1e-4)
    bad_codes = (codes != want) & ~near_pow2
    assert not bad_codes.any(), f"{int(bad_codes.sum())} scale codes differ"
    got = e4m3_bytes_to_f64(hi).reshape(nrows, K // 32, 32)
    X = np.ldexp(1.0, (codes - 127).astype(np.int32))[..., None]
    v = np.clip(a64[:nrows].reshape(nrows, K // 32, 32) / X, -448, 448)
    sp = e4m3_spacing(v)
    assert np.all(np.abs(got - v) <= sp * (1 + 1e-9)), "an element is not a neighbour of its exact value"
    same_code = (codes == want)[..., None] & np.ones((1, 1, 32), dtype=bool)
    diff = (got != elem.reshape(nrows, K // 32, 32)) & same_code
    mid = np.abs(np.abs(v - got) - sp / 2) <= 1e-2 * sp
    assert np.all(mid[diff]), f"{int((diff & ~mid).sum())} elements rounded differently away from a midpoint"
    print(f"[mxfp8] epilogue quantization: {int(diff.sum())} of {diff.size} elements on the other side of a "
          f"midpoint, {int(((codes != want) & near_pow2).sum())} scale codes at a power-of-two boundary", flush=True)


CASES = [
    ("decode_swiglu", (9, 256, 320, 6, 3), "swiglu_oai", {}),
    ("decode_silu_masked", (13, 192, 128, 5, 2), "silu", {"masked": 0.2}),
    ("decode_ktail", (6, 2880, 192, 4, 2), "swiglu_oai", {}),
    ("many_rows", (150, 128, 256, 3, 2), "silu", {}),
    ("weight_on_input", (13, 192, 128, 5, 1), "silu", {"on_input": True}),
    ("sorted_split_chunked", (2100, 128, 256, 4, 2), "swiglu_oai", {"masked": 0.05}),
    ("k8192", (4, 8192, 256, 3, 2), "swiglu_oai", {}),
    ("one_token", (1, 256, 320, 6, 3), "silu", {}),
    ("k16384_down", (3, 256, 16384, 2, 1), "silu", {}),   # GEMM2's K at the 16384 limit
    ("masked_bad", (20, 128, 192, 4, 2), "silu", {"masked": 0.5, "bad": 0.1}),
    ("situ", (9, 256, 320, 6, 3), "situ", {}),
]


@pytest.mark.parametrize("name,shape,act,extra", CASES, ids=[c[0] for c in CASES])
def test_mxfp8_forward_matches_oracle(name, shape, act, extra):
    T, H, I, E, k = shape
    print(f"[mxfp8] forward {name} T={T} H={H} I={I} E={E} k={k} {act}", flush=True)
    extra = dict(extra)
    on_input = extra.pop("on_input", False)
    x, ids, w, W, S = make_problem(zlib.crc32(name.encode()) % 1000, T, H, I, E, k, "mxfp4", **extra)
    act_kw = dict(act=act, **ACT_PARAMS[act], act_fmt="mxfp8")
    if on_input:
        act_kw["weight_on_input"] = True
    out = run_gpu(x, ids, w, W, S, act_kw)
    ref = oracle_out(x, ids, w, W, S, act_kw)
    got = to_np(out)
    assert np.all(np.isfinite(got))
    err = rel_err(got, ref)
    exact = oracle_out(x, ids, w, W, S, {kk: v for kk, v in act_kw.items() if kk != "act_fmt"})
    gap = rel_err(ref, exact)
    print(f"[mxfp8] {name} rel err {err:.2e} (MXFP8 vs exact activations in the oracle: {gap:.2e})", flush=True)
    assert err <= TOL
    again = run_gpu(x, ids, w, W, S, act_kw)
    assert torch.equal(out, again)
    dead = np.all((ids < 0) | (ids >= E), axis=1)
    assert np.all(got[dead] == 0)


def test_mxfp8_pregrouped_matches_oracle():
    lengths = [33, 0, 70, 2]
    cu = np.cumsum(lengths).astype(np.int32)
    NvS, H, I = int(cu[-1]) + 5, 128, 192
    print(f"[mxfp8] pregrouped NvS={NvS} segments={len(lengths)}", flush=True)
    x, _, _, W, S = make_problem(44, NvS, H, I, len(lengths), 1, "mxfp4")
    rw = np.random.default_rng(2).random(NvS).astype(np.float32)
    out = B.experts_forward_grouped(x.to(DEV), torch.from_numpy(cu).to(DEV), torch.from_numpy(rw).to(DEV),
                                    *[t.to(DEV) for t in W], scales=[t.to(DEV) for t in S], act_fmt="mxfp8")
    torch.cuda.synchronize()
    Wn = [(c.numpy(), s.numpy()) for c, s in zip(W, S)]
    ref = oracle.pregrouped_forward(to_np(x), cu, rw, *Wn, act_fmt="mxfp8")
    got = to_np(out)
    assert rel_err(got, ref) <= TOL
    assert np.all(got[cu[-1]:] == 0)


def test_mxfp8_decode_workload_full_size():
    wl = synth.workload("mxfp4_decode")
    print(f"[mxfp8] decode workload T={wl.T} H={wl.H} I={wl.I} E={wl.E} k={wl.k}", flush=True)
    ids, w = synth.make_routing(wl)
    x = synth.make_x(wl, device=DEV)
    (cg, sg), (cu_, su), (cd, sd) = synth.make_mxfp4_weights(wl, device=DEV)
    ids_d, w_d = torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    kw = dict(wl_act_kw(wl), act_fmt="mxfp8")
    out = B.experts_forward(x, ids_d, w_d, cg, cu_, cd, scales=(sg, su, sd), **kw)
    out2 = B.experts_forward(x, ids_d, w_d, cg, cu_, cd, scales=(sg, su, sd), **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    tokens = np.arange(wl.T)
    ref = sampled_token_oracle(x, ids_d, w_d, (cg, sg), (cu_, su), (cd, sd), tokens=tokens, act_kw=kw, mx=True)
    err = rel_err(to_np(out), ref)
    print(f"[mxfp8] decode workload rel err {err:.2e}", flush=True)
    assert err <= TOL
