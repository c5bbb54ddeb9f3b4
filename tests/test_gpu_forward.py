"""Experts step on the GPU against the CPU oracle, at sizes the oracle runs
in seconds: both GEMM paths (LDS-tiled prefill and weight-streaming decode),
bf16 and MXFP4 weights, SiLU and SwiGLU-OAI, ragged and empty segments,
column tails, masked and bad ids, the pre-grouped entry, determinism."""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL, rel_err, to_np
from mixture_experts_expert_02_amd import binding as B

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def make_problem(seed, T, H, I, E, k, wfmt="bf16", masked=0.0, bad=0.0, skew=None):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    if skew is None:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    else:  # Zipf-like: lower ids far more likely, some experts never picked
        p = (np.arange(E) + 1.0) ** -skew
        p /= p.sum()
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)])
    if masked:
        ids = np.where(rng.random((T, k)) < masked, -1, ids)
    if bad:
        ids = np.where(rng.random((T, k)) < bad, E + 1, ids)
    w = rng.random((T, k)).astype(np.float32)
    if wfmt == "bf16":
        W = [torch.from_numpy((rng.standard_normal((E, N, K)) / math.sqrt(K)).astype(np.float32)).to(torch.bfloat16)
             for N, K in ((I, H), (I, H), (H, I))]
        S = None
    else:
        W, S = [], []
        for N, K in ((I, H), (I, H), (H, I)):
            W.append(torch.from_numpy(rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)))
            S.append(torch.from_numpy((127 - rng.integers(0, 9, size=(E, N, K // 32))).astype(np.uint8)))
    return x, ids.astype(np.int32), w, W, S


def run_gpu(x, ids, w, W, S, act_kw):
    Wd = [t.to(DEV) for t in W]
    Sd = None if S is None else [t.to(DEV) for t in S]
    out = B.experts_forward(x.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), *Wd,
                            scales=Sd, **act_kw)
    torch.cuda.synchronize()
    return out


def oracle_out(x, ids, w, W, S, act_kw):
    if S is None:
        Wn = [to_np(t) for t in W]
    else:
        Wn = [(c.numpy(), s.numpy()) for c, s in zip(W, S)]
    return oracle.experts_forward(to_np(x), ids, w, *Wn, **act_kw)


CASES = [
    # name, (T, H, I, E, k), wfmt, act, extras
    ("prefill_ragged", (700, 256, 384, 5, 2), "bf16", "silu", {}),
    ("prefill_col_tails", (400, 320, 192, 3, 2), "bf16", "silu", {}),
    ("prefill_swiglu", (520, 128, 256, 4, 2), "bf16", "swiglu_oai", {}),
    ("prefill_skew_empty", (900, 192, 128, 12, 3), "bf16", "silu", {"skew": 2.0}),
    ("prefill_masked_bad", (600, 128, 256, 4, 2), "bf16", "silu", {"masked": 0.1, "bad": 0.05}),
    ("decode_bf16", (20, 256, 192, 16, 2), "bf16", "silu", {}),
    ("decode_bf16_swiglu_masked", (9, 128, 320, 12, 4), "bf16", "swiglu_oai", {"masked": 0.2}),
    ("decode_mxfp4_swiglu", (9, 256, 320, 6, 3), "mxfp4", "swiglu_oai", {}),
    ("decode_mxfp4_silu", (13, 192, 128, 5, 2), "mxfp4", "silu", {}),
    ("decode_mxfp4_ktail", (6, 2880, 192, 4, 2), "mxfp4", "swiglu_oai", {}),   # 90 scale blocks: ragged K steps
    ("mxfp4_many_rows", (150, 128, 256, 3, 2), "mxfp4", "silu", {}),          # several 16-row tiles per expert
    ("single_token", (1, 128, 256, 8, 2), "bf16", "silu", {}),
    ("prefill_situ", (520, 128, 256, 4, 2), "bf16", "situ", {}),
    ("decode_bf16_situ", (9, 128, 320, 12, 4), "bf16", "situ", {}),
    ("decode_mxfp4_situ", (9, 256, 320, 6, 3), "mxfp4", "situ", {}),
    ("prefill_weight_on_input_top1", (700, 256, 384, 5, 1), "bf16", "silu", {"on_input": True}),
    ("prefill_weight_on_input_k2_masked", (600, 128, 256, 4, 2), "bf16", "swiglu_oai",
     {"on_input": True, "masked": 0.1}),
    ("decode_mxfp4_weight_on_input", (13, 192, 128, 5, 1), "mxfp4", "silu", {"on_input": True}),
    ("decode_bf16_weight_on_input", (20, 256, 192, 16, 1), "bf16", "situ", {"on_input": True}),
    # MXFP4 scale staging with 8 and 16 pieces per thread (K above 4096 and 8192, up to the 16384 limit)
    ("decode_mxfp4_k8192", (4, 8192, 256, 3, 2), "mxfp4", "swiglu_oai", {}),
    ("decode_mxfp4_k16384", (3, 256, 16384, 2, 1), "mxfp4", "silu", {}),
    ("decode_mxfp4_k6144_ragged", (5, 6144, 320, 3, 2), "mxfp4", "silu", {}),
    # more than 4096 routed rows: the chunked align and the sorted-order x split
    ("mxfp4_chunked_align", (2100, 128, 256, 4, 2), "mxfp4", "swiglu_oai", {"masked": 0.05}),
    # MXFP4 decode with masked and bad ids: tokens whose slots are all dead get zero rows
    ("decode_mxfp4_masked_bad", (40, 256, 320, 6, 3), "mxfp4", "swiglu_oai", {"masked": 0.3, "bad": 0.1}),
]
ACT_PARAMS = {"silu": {}, "swiglu_oai": dict(alpha=1.702, beta=1.0, limit=7.0), "situ": dict(alpha=1.5, beta=0.8)}


@pytest.mark.parametrize("name,shape,wfmt,act,extra", CASES, ids=[c[0] for c in CASES])
def test_forward_matches_oracle(name, shape, wfmt, act, extra):
    T, H, I, E, k = shape
    print(f"[forward] {name} T={T} H={H} I={I} E={E} k={k} {wfmt} {act}", flush=True)
    extra = dict(extra)
    on_input = extra.pop("on_input", False)
    x, ids, w, W, S = make_problem(zlib.crc32(name.encode()) % 1000, T, H, I, E, k, wfmt, **extra)
    act_kw = dict(act=act, **ACT_PARAMS[act])
    if on_input:
        act_kw["weight_on_input"] = True
    out = run_gpu(x, ids, w, W, S, act_kw)
    ref = oracle_out(x, ids, w, W, S, act_kw)
    got = to_np(out)
    assert np.all(np.isfinite(got))
    err = rel_err(got, ref)
    print(f"[forward] {name} rel err {err:.2e}", flush=True)
    assert err <= TOL
    # rows whose slots are all masked or bad are exactly zero
    dead = np.all((ids < 0) | (ids >= E), axis=1)
    assert np.all(got[dead] == 0)


def test_tiny_workload_and_intermediates():
    wl = synth.workload("tiny")
    ids, w = synth.make_routing(wl)
    x = synth.make_x(wl)
    W = synth.make_bf16_weights(wl)
    p = B.problem(wl.T, wl.H, wl.I, wl.E, wl.k)
    ws = B.alloc_workspace(B.moe_experts_workspace_bytes(p), DEV)
    out = B.experts_forward(x.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                            *[t.to(DEV) for t in W], workspace=ws)
    torch.cuda.synchronize()
    Wn = [to_np(t) for t in W]
    ref = oracle.experts_forward(to_np(x), ids, w, *Wn)
    assert rel_err(to_np(out), ref) <= TOL
    # the activation rows in the workspace against the oracle's grouped intermediates
    lay = B.moe_experts_workspace_layout(p)
    M = wl.T * wl.k
    act = ws[lay.act: lay.act + M * wl.I * 2].view(torch.bfloat16).view(M, wl.I)
    al = oracle.align(ids, wl.E)
    xr = to_np(x)[al["perm"] // wl.k]
    g = oracle.grouped_mm(xr, lambda e: Wn[0][e].astype(np.float64), al["cu_seqlens"])
    u = oracle.grouped_mm(xr, lambda e: Wn[1][e].astype(np.float64), al["cu_seqlens"])
    a_ref = oracle.silu(g) * u * w.reshape(-1)[al["perm"]][:, None]
    assert rel_err(to_np(act), a_ref) <= TOL


@pytest.mark.parametrize("max_split", [1, 2, 3, 4])
def test_split_down_projection_matches_oracle(max_split, monkeypatch):
    # A problem with few tiles splits the down projection's K (6 stages of 64)
    # into as many ranges as allowed: 1, 2, 3 (2+2+2) or 4 (1+1+2+2 stages);
    # the combine adds the partial outputs.
    monkeypatch.setenv("MOE_EXPERTS_MAX_SPLIT_K", str(max_split))
    T, H, I, E, k = 700, 320, 384, 5, 2
    print(f"[forward] split<={max_split} T={T} H={H} I={I} E={E} k={k}", flush=True)
    x, ids, w, W, S = make_problem(11, T, H, I, E, k, "bf16")
    out = run_gpu(x, ids, w, W, S, dict(act="silu"))
    ref = oracle_out(x, ids, w, W, S, dict(act="silu"))
    err = rel_err(to_np(out), ref)
    print(f"[forward] split<={max_split} rel err {err:.2e}", flush=True)
    assert err <= TOL
    again = run_gpu(x, ids, w, W, S, dict(act="silu"))
    assert torch.equal(out, again)


@pytest.mark.parametrize("shape,wfmt", [((700, 256, 384, 5, 2), "bf16"), ((9, 256, 320, 6, 3), "mxfp4")])
def test_forward_is_bitwise_deterministic(shape, wfmt):
    T, H, I, E, k = shape
    x, ids, w, W, S = make_problem(5, T, H, I, E, k, wfmt)
    a = run_gpu(x, ids, w, W, S, dict(act="silu"))
    b = run_gpu(x, ids, w, W, S, dict(act="silu"))
    assert torch.equal(a, b)


def test_token_permutation_gives_permuted_output_bitwise():
    x, ids, w, W, S = make_problem(6, 300, 128, 256, 4, 2)
    pi = np.random.default_rng(1).permutation(300)
    a = run_gpu(x, ids, w, W, S, dict(act="silu"))
    b = run_gpu(x[torch.from_numpy(pi)], ids[pi].copy(), w[pi].copy(), W, S, dict(act="silu"))
    # the GEMM rows of a token move between tiles, but each output element is
    # the same fp32 dot product with the same K order, so the result is identical
    assert torch.equal(a[torch.from_numpy(pi).to(DEV)], b)


def test_bad_ids_counted_in_status_word():
    x, ids, w, W, S = make_problem(7, 64, 128, 256, 8, 2)
    ids[3, 1] = 8
    ids[10, 0] = 1000
    ids[11, 0] = -1
    p = B.problem(64, 128, 256, 8, 2)
    ws = B.alloc_workspace(B.moe_experts_workspace_bytes(p), DEV)
    B.experts_forward(x.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                      *[t.to(DEV) for t in W], workspace=ws)
    torch.cuda.synchronize()
    assert B.moe_device_error(ws) == 2


def test_workspace_reuse_with_smaller_T():
    x, ids, w, W, S = make_problem(8, 600, 128, 256, 4, 2)
    p = B.problem(600, 128, 256, 4, 2)
    ws = B.alloc_workspace(B.moe_experts_workspace_bytes(p), DEV)
    Wd = [t.to(DEV) for t in W]
    for T in (600, 37):
        out = B.experts_forward(x[:T].to(DEV), torch.from_numpy(ids[:T].copy()).to(DEV),
                                torch.from_numpy(w[:T].copy()).to(DEV), *Wd, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.experts_forward(to_np(x[:T]), ids[:T], w[:T], *[to_np(t) for t in W])
        assert rel_err(to_np(out), ref) <= TOL


# ------------------------------------------------------------------ cold segments
# Segments of 1..32 rows run in the cold-segment kernels beside the 256-row
# tiles (MOE_EXPERTS_COLD=0 keeps them in the tiles): both against the oracle,
# with the down projection's K split into partial outputs or not.
@pytest.mark.parametrize("cold", ["1", "0"])
@pytest.mark.parametrize("max_split", ["1", "4"])
def test_cold_segments_match_oracle(cold, max_split, monkeypatch):
    monkeypatch.setenv("MOE_EXPERTS_COLD", cold)
    monkeypatch.setenv("MOE_EXPERTS_MAX_SPLIT_K", max_split)
    T, H, I, E, k = 600, 192, 320, 24, 2
    print(f"[forward] cold={cold} split<={max_split} T={T} H={H} I={I} E={E} k={k}", flush=True)
    x, ids, w, W, S = make_problem(21, T, H, I, E, k, "bf16", skew=1.3)
    n = np.bincount(ids.ravel(), minlength=E)
    assert np.any((n > 0) & (n <= 16)) and np.any((n > 16) & (n <= 32)) and np.any(n > 256)
    for act in ("silu", "swiglu_oai"):
        act_kw = dict(act=act, **ACT_PARAMS[act])
        out = run_gpu(x, ids, w, W, S, act_kw)
        err = rel_err(to_np(out), oracle_out(x, ids, w, W, S, act_kw))
        print(f"[forward] cold={cold} split<={max_split} {act} rel err {err:.2e}", flush=True)
        assert err <= TOL
        assert torch.equal(out, run_gpu(x, ids, w, W, S, act_kw))


# ------------------------------------------------------------------ pre-grouped entry
def grouped_case(seed, lengths, tail, H=256, I=384, wfmt="bf16"):
    rng = np.random.default_rng(seed)
    G = len(lengths)
    NvS = int(sum(lengths)) + tail
    cu = np.cumsum(lengths).astype(np.int32)
    x = torch.from_numpy(rng.standard_normal((NvS, H)).astype(np.float32)).to(torch.bfloat16)
    rw = rng.random(NvS).astype(np.float32)
    if wfmt == "bf16":
        W = [torch.from_numpy((rng.standard_normal((G, N, K)) / math.sqrt(K)).astype(np.float32)).to(torch.bfloat16)
             for N, K in ((I, H), (I, H), (H, I))]
        S = None
    else:
        W = [torch.from_numpy(rng.integers(0, 256, size=(G, N, K // 2), dtype=np.uint8)) for N, K in ((I, H), (I, H), (H, I))]
        S = [torch.from_numpy((127 - rng.integers(0, 9, size=(G, N, K // 32))).astype(np.uint8)) for N, K in ((I, H), (I, H), (H, I))]
    return x, cu, rw, W, S


@pytest.mark.parametrize("lengths,tail,wfmt,on_input", [
    ([300, 0, 257, 1, 0, 512, 40], 13, "bf16", False),     # empty segments, ragged, padding rows
    ([400, 3, 32, 0, 17, 33, 290, 16], 6, "bf16", False),  # cold segments (1..32 rows) beside tiled ones
    ([0, 0, 5, 0], 7, "bf16", False),                      # decode-sized (weight-streaming path)
    ([33, 0, 70, 2], 5, "mxfp4", False),
    ([600, 600], 0, "bf16", False),
    ([300, 0, 257, 1, 0, 512, 40], 13, "bf16", True),      # route weight on the input rows
    ([33, 0, 70, 2], 5, "mxfp4", True),
])
def test_grouped_matches_oracle(lengths, tail, wfmt, on_input):
    x, cu, rw, W, S = grouped_case(len(lengths) * 10 + tail, lengths, tail, wfmt=wfmt)
    print(f"[grouped] lengths={lengths} tail={tail} {wfmt} on_input={on_input}", flush=True)
    Wd = [t.to(DEV) for t in W]
    Sd = None if S is None else [t.to(DEV) for t in S]
    out = B.experts_forward_grouped(x.to(DEV), torch.from_numpy(cu).to(DEV), torch.from_numpy(rw).to(DEV), *Wd,
                                    scales=Sd, weight_on_input=on_input)
    torch.cuda.synchronize()
    Wn = [to_np(t) for t in W] if S is None else [(c.numpy(), s.numpy()) for c, s in zip(W, S)]
    ref = oracle.pregrouped_forward(to_np(x), cu, rw, *Wn, weight_on_input=on_input)
    got = to_np(out)
    assert rel_err(got, ref) <= TOL
    assert np.all(got[int(cu[-1]):] == 0)


def test_grouped_malformed_offsets_flagged_and_zero():
    x, cu, rw, W, S = grouped_case(3, [10, 20, 30], 4)
    bad = np.array([10, 5, 60], dtype=np.int32)        # decreasing
    G, H, I = 3, 256, 384
    p = B.problem(x.shape[0], H, I, G, 1)
    ws = B.alloc_workspace(B.moe_experts_grouped_workspace_bytes(p), DEV)
    out = torch.full((x.shape[0], H), 7.0, dtype=torch.bfloat16, device=DEV)
    B.experts_forward_grouped(x.to(DEV), torch.from_numpy(bad).to(DEV), torch.from_numpy(rw).to(DEV),
                              *[t.to(DEV) for t in W], out=out, workspace=ws)
    torch.cuda.synchronize()
    assert B.moe_device_error(ws) == 1
    assert torch.all(out == 0)


def test_grouped_timed_matches_untimed_bitwise():
    """moe_experts_forward_grouped_timed only adds event records."""
    import ctypes
    x, cu, rw, W, S = grouped_case(11, [300, 0, 257, 1], 9)
    G, H, I = 4, 256, 384
    p = B.problem(x.shape[0], H, I, G, 1)
    ws = B.alloc_workspace(B.moe_experts_grouped_workspace_bytes(p), DEV)
    args = [x.to(DEV), torch.from_numpy(cu).to(DEV), torch.from_numpy(rw).to(DEV), *[t.to(DEV) for t in W]]
    ref = B.experts_forward_grouped(*args, workspace=ws)
    hip = ctypes.CDLL("libamdhip64.so")
    evs = []
    for _ in range(5):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    out = torch.empty_like(ref)
    rc = B.moe_experts_forward_grouped_timed(p, *args, None, None, None, out, ws, evs)
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(out, ref)
    for e in evs:
        hip.hipEventDestroy(ctypes.c_void_p(e))
