"""bf16 weights in the operand-block layout (moe_bf16_pack_weights,
moe_problem.bf16_packed): the packed bytes against the layout the header
describes, and the tiled and cold-segment prefill kernels reading them give
outputs bit for bit equal to the row layout's (same products, same order),
on both entries, with the oracle beside them on one case."""
import numpy as np
import pytest
import torch

import oracle
from helpers import TOL, rel_err, to_np
from test_gpu_forward import make_problem
from mixture_experts_expert_02_amd import binding as B

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def host_pack(Wt):
    """[E, N, K] bf16 -> the operand-block layout written out on the host
    from the header's description (test infrastructure, not the oracle):
    block (e, nb, kb), piece l = 16 q + r holds row 16 nb + r, values
    32 kb + 8 q..+7."""
    E, N, K = Wt.shape
    v = Wt.view(torch.int16).reshape(E, N // 16, 16, K // 32, 4, 8)   # e, nb, r, kb, q, v
    return v.permute(0, 1, 3, 4, 2, 5).contiguous().reshape(-1)       # e, nb, kb, q, r, v


def test_bf16_pack_layout_matches_host_packer():
    """Two experts, N not a multiple of the tile (I = 192, H = 320)."""
    T, H, I, E, k = 64, 320, 192, 2, 2
    _, _, _, W, _ = make_problem(5, T, H, I, E, k)
    p = B.problem(T, H, I, E, k)
    print(f"[bf16_packed] layout H={H} I={I} E={E}", flush=True)
    packed = B.bf16_pack_weights(p, *[t.to(DEV) for t in W])
    torch.cuda.synchronize()
    want = torch.cat([host_pack(t) for t in W]).numpy()
    got = packed.cpu().view(torch.int16).numpy()
    assert packed.numel() == B.moe_bf16_packed_bytes(p) == 2 * want.size
    assert np.array_equal(got, want), f"{int((got != want).sum())} elements differ"


CASES = [
    # name, (T, H, I, E, k), act, extras
    ("ragged", (700, 256, 384, 5, 2), "silu", {}),
    ("col_tails", (400, 320, 192, 3, 2), "silu", {}),                # partial column tiles in both GEMMs
    ("skew_cold", (900, 192, 128, 12, 3), "silu", {"skew": 2.0}),    # cold segments beside tiled ones, empty experts
    ("skew_cold_swiglu", (1100, 320, 192, 16, 2), "swiglu_oai", {"skew": 1.5}),
    ("cold_situ", (600, 256, 256, 24, 2), "situ", {"skew": 1.3}),
    ("decode_size", (20, 256, 192, 16, 2), "silu", {}),              # weight-streaming kernels: canonical weights
]
ACT = {"silu": {}, "swiglu_oai": dict(alpha=1.702, beta=1.0, limit=7.0), "situ": dict(alpha=1.0, beta=0.5)}


@pytest.mark.parametrize("name,shape,act,extra", CASES, ids=[c[0] for c in CASES])
def test_bf16_packed_forward_bitwise(name, shape, act, extra):
    T, H, I, E, k = shape
    print(f"[bf16_packed] forward {name} T={T} H={H} I={I} E={E} k={k} {act}", flush=True)
    x, ids, w, W, _ = make_problem(11, T, H, I, E, k, **extra)
    kw = dict(act=act, **ACT[act])
    p = B.problem(T, H, I, E, k, "bf16", **kw)
    Wd = [t.to(DEV) for t in W]
    packed = B.bf16_pack_weights(p, *Wd)
    xd, idd, wd = x.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    a = B.experts_forward(xd, idd, wd, *Wd, **kw)
    b = B.experts_forward(xd, idd, wd, *Wd, bf16_packed=packed, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    if name == "skew_cold_swiglu":
        ref = oracle.experts_forward(to_np(x), ids, w, *[to_np(t) for t in W], **kw)
        err = rel_err(to_np(b), ref)
        print(f"[bf16_packed] {name}: max|err|/max|ref| {err:.2e}", flush=True)
        assert err <= TOL


def test_bf16_packed_grouped_bitwise():
    """Pre-grouped entry: segments of 0, 3, 17, 40, 300 and 700 rows (cold and
    tiled), the packed weights against the row layout and the oracle."""
    H, I = 256, 192
    lengths = np.array([3, 0, 17, 300, 40, 700, 1, 33], dtype=np.int64)
    G, NvS = len(lengths), int(lengths.sum())
    print(f"[bf16_packed] grouped NvS={NvS} H={H} I={I} G={G}", flush=True)
    rng = np.random.default_rng(3)
    x = torch.from_numpy(rng.standard_normal((NvS, H)).astype(np.float32)).to(torch.bfloat16)
    W = [torch.from_numpy((rng.standard_normal((G, N, K)) / np.sqrt(K)).astype(np.float32)).to(torch.bfloat16)
         for N, K in ((I, H), (I, H), (H, I))]
    rw = rng.random(NvS).astype(np.float32)
    cu = np.cumsum(lengths).astype(np.int32)
    p = B.problem(NvS, H, I, G, 1)
    Wd = [t.to(DEV) for t in W]
    packed = B.bf16_pack_weights(p, *Wd)
    args = (x.to(DEV), torch.from_numpy(cu).to(DEV), torch.from_numpy(rw).to(DEV), *Wd)
    a = B.experts_forward_grouped(*args)
    b = B.experts_forward_grouped(*args, bf16_packed=packed)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = oracle.pregrouped_forward(to_np(x), cu, rw, *[to_np(t) for t in W])
    err = rel_err(to_np(b), ref)
    print(f"[bf16_packed] grouped: max|err|/max|ref| {err:.2e}", flush=True)
    assert err <= TOL
