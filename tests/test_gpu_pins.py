"""Direct checks of properties the parity tests rely on:

* the exact split of bf16 activations into two e4m3 parts for the
  block-scaled MFMA, over every finite bf16 bit pattern;
* segments with no rows never read their expert's weights (moonep_experts
  page, module docstring: empty segments are skipped by the grouped GEMM):
  poisoning those weights with NaN leaves the output bitwise unchanged;
* no kernel writes outside the output or the workspace (canary bands), on
  small problems of every path, including a pre-grouped MXFP4 problem whose
  split activation rows end exactly at the end of the workspace."""
import numpy as np
import pytest
import torch

import oracle
from helpers import TOL, Guarded, rel_err, to_np
from mixture_experts_expert_02_amd import binding as B
from test_gpu_forward import ACT_PARAMS, grouped_case, make_problem

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def all_finite_bf16_bits(order: str, seed: int = 0) -> np.ndarray:
    """Every bf16 bit pattern with the NaN / inf exponent replaced by +0, in
    a seeded random order ("random": blocks mix magnitudes far apart) or
    sorted by magnitude ("sorted": blocks of neighbouring values)."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    bits[((bits >> 7) & 0xFF) == 0xFF] = 0
    if order == "random":
        bits = np.random.default_rng(seed).permutation(bits)
    else:
        bits = bits[np.argsort(bits & 0x7FFF, kind="stable")]
    return bits.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("order", ["random", "sorted"])
def test_hi_lo_split_reproduces_every_bf16_value(order):
    """x is split by the MXFP4 decode prologue (token order, bf16
    activations); every value must come back as hi + lo times its block
    scale to within 2^-17 of the block's largest magnitude, and exactly once
    its scaled magnitude is at least 2 (where lo is a normal e4m3)."""
    T, H, I, E, k = 32, 2048, 64, 2, 1
    print(f"[pins] hi/lo split, all finite bf16 values, {order} order", flush=True)
    bits = all_finite_bf16_bits(order)
    x = torch.from_numpy(bits.view(np.int16).reshape(T, H).copy()).view(torch.bfloat16)
    _, ids, w, W, S = make_problem(3, T, H, I, E, k, "mxfp4")
    ids[:] = 0
    p = B.problem(T, H, I, E, k, "mxfp4")
    ws = B.alloc_workspace(B.moe_experts_workspace_bytes(p), DEV)
    B.experts_forward(x.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                      *[t.to(DEV) for t in W], scales=[t.to(DEV) for t in S], workspace=ws)
    torch.cuda.synchronize()
    lay = B.moe_experts_workspace_layout(p)
    assert lay.xq_rows == T
    R = T
    sc_stride = (H // 32 + 15) // 16 * 16
    hi = ws[lay.xq: lay.xq + R * H].view(torch.float8_e4m3fn).to(torch.float64).cpu().numpy().reshape(T, H)
    lo = ws[lay.xq + R * H: lay.xq + 2 * R * H].view(torch.float8_e4m3fn).to(torch.float64).cpu().numpy()
    lo = lo.reshape(T, H)
    code = ws[lay.xq + 2 * R * H: lay.xq + 2 * R * H + R * sc_stride].view(R, sc_stride)[:, : H // 32]
    code = code.cpu().numpy().astype(np.int64)
    xv = bf16_bits_to_f64(bits).reshape(T, H)
    blocks = np.abs(xv).reshape(T, H // 32, 32)
    amax = blocks.max(axis=-1)
    # scale exponent: floor(log2 amax) - 7, clamped at the e8m0 minimum
    _, ex = np.frexp(amax)
    want_code = np.where(amax > 0, np.clip(ex - 1 - 7 + 127, 0, 254), 0)
    assert np.array_equal(code, want_code), "scale codes differ"
    scale = np.repeat(np.ldexp(1.0, (code - 127).astype(np.int32)), 32, axis=-1)
    recon = (hi + lo) * scale
    err = np.abs(recon - xv)
    bound = np.repeat(amax, 32, axis=-1) * 2.0 ** -17
    assert np.all(np.isfinite(hi)) and np.all(np.isfinite(lo))
    assert np.all(err <= bound), f"{int(np.sum(err > bound))} values off by more than 2^-17 of their block max"
    big = np.abs(xv) >= 2.0 * scale
    assert np.array_equal(recon[big], xv[big]), "a value with scaled magnitude >= 2 is not exact"
    print(f"[pins] {order}: {xv.size} values, {int(big.sum())} exact by the normal-lo rule, "
          f"max err / block max {float(np.max(err / np.maximum(bound * 2 ** 17, 1e-300))):.2e}", flush=True)


def poison_experts(W, S, empty, wfmt):
    """Copies of the weights with the empty experts' entries made NaN (bf16
    0x7fc0) or, for MXFP4, their scale bytes 255 (e8m0 NaN)."""
    Wp = [t.clone() for t in W]
    Sp = None if S is None else [t.clone() for t in S]
    for e in empty:
        for i in range(3):
            if wfmt == "bf16":
                Wp[i][e] = float("nan")
            else:
                Sp[i][e] = 255
    return Wp, Sp


@pytest.mark.parametrize("shape,wfmt", [((600, 256, 384, 12, 2), "bf16"),   # LDS-tiled prefill GEMMs
                                        ((20, 256, 192, 16, 2), "bf16"),    # weight-streaming GEMMs
                                        ((9, 256, 320, 12, 3), "mxfp4")])   # block-scaled MFMA
def test_empty_experts_weights_never_read(shape, wfmt):
    T, H, I, E, k = shape
    print(f"[pins] poisoned empty experts T={T} H={H} I={I} E={E} k={k} {wfmt}", flush=True)
    x, _, w, W, S = make_problem(21, T, H, I, E, k, wfmt)
    rng = np.random.default_rng(5)
    live = np.array([e for e in range(E) if e % 3 != 1])      # experts 1, 4, 7, ... stay empty
    ids = np.stack([rng.choice(live, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    empty = sorted(set(range(E)) - set(ids.ravel().tolist()))
    assert len(empty) >= E // 3
    Wp, Sp = poison_experts(W, S, empty, wfmt)
    args = (x.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV))
    clean = B.experts_forward(*args, *[t.to(DEV) for t in W], scales=None if S is None else [t.to(DEV) for t in S])
    pois = B.experts_forward(*args, *[t.to(DEV) for t in Wp], scales=None if Sp is None else [t.to(DEV) for t in Sp])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(pois.float()).all())
    assert torch.equal(clean, pois), "an empty expert's weights reached the output"


@pytest.mark.parametrize("wfmt", ["bf16", "mxfp4"])
def test_grouped_empty_segments_weights_never_read(wfmt):
    lengths = [33, 0, 70, 0, 2, 0]
    x, cu, rw, W, S = grouped_case(9, lengths, 5, wfmt=wfmt)
    empty = [g for g, n in enumerate(lengths) if n == 0]
    Wp, Sp = poison_experts(W, S, empty, wfmt)
    a = (x.to(DEV), torch.from_numpy(cu).to(DEV), torch.from_numpy(rw).to(DEV))
    clean = B.experts_forward_grouped(*a, *[t.to(DEV) for t in W], scales=None if S is None else [t.to(DEV) for t in S])
    pois = B.experts_forward_grouped(*a, *[t.to(DEV) for t in Wp],
                                     scales=None if Sp is None else [t.to(DEV) for t in Sp])
    torch.cuda.synchronize()
    assert torch.equal(clean, pois)


CANARY_CASES = [
    ("prefill_bf16", (700, 256, 384, 5, 2), "bf16", "silu", "bf16"),
    ("decode_bf16", (20, 256, 192, 16, 2), "bf16", "swiglu_oai", "bf16"),
    ("decode_mxfp4", (9, 256, 320, 6, 3), "mxfp4", "swiglu_oai", "bf16"),
    ("decode_mxfp4_mxfp8", (9, 256, 320, 6, 3), "mxfp4", "silu", "mxfp8"),
    ("chunked_align_mxfp4", (2100, 128, 256, 4, 2), "mxfp4", "silu", "bf16"),
]


@pytest.mark.parametrize("name,shape,wfmt,act,afmt", CANARY_CASES, ids=[c[0] for c in CANARY_CASES])
def test_no_writes_outside_out_and_workspace(name, shape, wfmt, act, afmt):
    T, H, I, E, k = shape
    print(f"[pins] canary bands {name}", flush=True)
    x, ids, w, W, S = make_problem(31, T, H, I, E, k, wfmt)
    kw = dict(act=act, **ACT_PARAMS[act])
    p = B.problem(T, H, I, E, k, wfmt, act_fmt=afmt, **kw)
    ws = Guarded(B.moe_experts_workspace_bytes(p), DEV)
    out = Guarded(T * H * 2, DEV)
    B.experts_forward(x.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                      *[t.to(DEV) for t in W], scales=None if S is None else [t.to(DEV) for t in S],
                      out=out.view_bf16(T, H), workspace=ws.body, act_fmt=afmt, **kw)
    torch.cuda.synchronize()
    ws.check_bands()
    out.check_bands()
    Wn = [to_np(t) for t in W] if S is None else [(c.numpy(), s.numpy()) for c, s in zip(W, S)]
    ref = oracle.experts_forward(to_np(x), ids, w, *Wn, act_fmt=afmt, **kw)
    assert rel_err(to_np(out.view_bf16(T, H)), ref) <= TOL


@pytest.mark.parametrize("afmt", ["bf16", "mxfp8"])
def test_grouped_mxfp4_split_rows_at_workspace_end(afmt):
    """NvS = 16 rows, all live, I = 512: the split activation rows of GEMM2
    are the workspace's last region and fill it to its last byte."""
    lengths = [9, 0, 7]
    H, I = 256, 512
    x, cu, rw, W, S = grouped_case(4, lengths, 0, H=H, I=I, wfmt="mxfp4")
    NvS = int(sum(lengths))
    p = B.problem(NvS, H, I, len(lengths), 1, "mxfp4", act_fmt=afmt)
    nbytes = B.moe_experts_grouped_workspace_bytes(p)
    ws = Guarded(nbytes, DEV)
    out = Guarded(NvS * H * 2, DEV)
    B.experts_forward_grouped(x.to(DEV), torch.from_numpy(cu).to(DEV), torch.from_numpy(rw).to(DEV),
                              *[t.to(DEV) for t in W], scales=[t.to(DEV) for t in S], out=out.view_bf16(NvS, H),
                              workspace=ws.body, act_fmt=afmt)
    torch.cuda.synchronize()
    ws.check_bands()
    out.check_bands()
    Wn = [(c.numpy(), s.numpy()) for c, s in zip(W, S)]
    ref = oracle.pregrouped_forward(to_np(x), cu, rw, *Wn, act_fmt=afmt)
    assert rel_err(to_np(out.view_bf16(NvS, H)), ref) <= TOL
