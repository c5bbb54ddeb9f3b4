"""Per-expert activation parameters (alpha, beta, clamp limit) and fc1 / fc2
scales on the GPU against the oracle, on every GEMM path: the LDS-tiled
prefill GEMMs (with the down projection's K split), the weight-streaming
GEMMs with bf16 and MXFP4 weights, MXFP8 activations, and the pre-grouped
entry. Every expert gets its own values (trtllm_mxfp4_moe page,
TrtLlmMxfp4ExpertsBase constructor: per-expert activation tensors;
flashinfer_moe_ep page, epilogue_from_quant_config: one fc1 / fc2 alpha per
expert)."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from helpers import TOL, rel_err, to_np
from mixture_experts_expert_02_amd import binding as B
from test_gpu_forward import ACT_PARAMS, grouped_case, make_problem

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def expert_values(seed, E, act):
    rng = np.random.default_rng(seed)
    v = {"fc1_alpha": rng.uniform(0.25, 4.0, E), "fc2_alpha": rng.uniform(0.25, 4.0, E)}
    if act == "swiglu_oai":
        v["alpha_e"] = rng.uniform(0.8, 2.5, E)
        v["beta_e"] = rng.uniform(-0.5, 1.5, E)
        v["limit_e"] = rng.choice([np.inf, 7.0, 3.0, 0.8], E)
    elif act == "situ":
        v["alpha_e"] = rng.uniform(0.5, 3.0, E)
        v["beta_e"] = rng.uniform(0.3, 2.0, E)
    return {k: a.astype(np.float32) for k, a in v.items()}


def oracle_kw(vals):
    names = {"alpha_e": "alpha", "beta_e": "beta", "limit_e": "limit"}
    return {names.get(k, k): v.astype(np.float64) for k, v in vals.items()}


CASES = [
    ("prefill_swiglu", (700, 256, 384, 5, 2), "bf16", "swiglu_oai", "bf16"),
    ("prefill_situ_skew", (900, 192, 128, 12, 3), "bf16", "situ", "bf16"),
    ("decode_bf16_swiglu", (20, 256, 192, 16, 2), "bf16", "swiglu_oai", "bf16"),
    ("decode_mxfp4_swiglu", (9, 256, 320, 6, 3), "mxfp4", "swiglu_oai", "bf16"),
    ("decode_mxfp4_mxfp8", (13, 192, 128, 5, 2), "mxfp4", "swiglu_oai", "mxfp8"),
    ("decode_mxfp4_situ", (9, 256, 320, 6, 3), "mxfp4", "situ", "bf16"),
]


@pytest.mark.parametrize("name,shape,wfmt,act,afmt", CASES, ids=[c[0] for c in CASES])
def test_per_expert_params_match_oracle(name, shape, wfmt, act, afmt):
    T, H, I, E, k = shape
    print(f"[expert-params] {name} T={T} H={H} I={I} E={E} k={k} {wfmt} {act} {afmt}", flush=True)
    seed = zlib.crc32(name.encode()) % 1000
    x, ids, w, W, S = make_problem(seed, T, H, I, E, k, wfmt, skew=1.5 if "skew" in name else None)
    vals = expert_values(seed, E, act)
    p = B.problem(T, H, I, E, k, wfmt, act, **ACT_PARAMS[act])
    assert B.moe_check_expert_params(p, **vals) == B.MOE_OK
    ep = {kk: torch.from_numpy(v).to(DEV) for kk, v in vals.items()}
    out = B.experts_forward(x.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                            *[t.to(DEV) for t in W], scales=None if S is None else [t.to(DEV) for t in S],
                            act=act, act_fmt=afmt, expert_params=ep, **ACT_PARAMS[act])
    torch.cuda.synchronize()
    Wn = [to_np(t) for t in W] if S is None else [(c.numpy(), s.numpy()) for c, s in zip(W, S)]
    kw = dict(ACT_PARAMS[act])
    kw.update(oracle_kw(vals))
    ref = oracle.experts_forward(to_np(x), ids, w, *Wn, act=act, act_fmt=afmt, **kw)
    got = to_np(out)
    err = rel_err(got, ref)
    # the same problem with the scalar parameters differs clearly, so the
    # per-expert values are used
    plain = oracle.experts_forward(to_np(x), ids, w, *Wn, act=act, act_fmt=afmt, **ACT_PARAMS[act])
    print(f"[expert-params] {name} rel err {err:.2e} (scalar parameters would differ by "
          f"{rel_err(plain, ref):.2e})", flush=True)
    assert np.all(np.isfinite(got))
    assert err <= TOL
    assert rel_err(plain, ref) > 10 * TOL


@pytest.mark.parametrize("wfmt", ["bf16", "mxfp4"])
def test_per_expert_params_pregrouped(wfmt):
    lengths = [300, 0, 257, 1, 40] if wfmt == "bf16" else [33, 0, 70, 2]
    x, cu, rw, W, S = grouped_case(17, lengths, 6, wfmt=wfmt)
    G = len(lengths)
    vals = expert_values(5, G, "swiglu_oai")
    ep = {kk: torch.from_numpy(v).to(DEV) for kk, v in vals.items()}
    out = B.experts_forward_grouped(x.to(DEV), torch.from_numpy(cu).to(DEV), torch.from_numpy(rw).to(DEV),
                                    *[t.to(DEV) for t in W], scales=None if S is None else [t.to(DEV) for t in S],
                                    act="swiglu_oai", expert_params=ep, **ACT_PARAMS["swiglu_oai"])
    torch.cuda.synchronize()
    Wn = [to_np(t) for t in W] if S is None else [(c.numpy(), s.numpy()) for c, s in zip(W, S)]
    kw = dict(ACT_PARAMS["swiglu_oai"])
    kw.update(oracle_kw(vals))
    ref = oracle.pregrouped_forward(to_np(x), cu, rw, *Wn, act="swiglu_oai", **kw)
    got = to_np(out)
    assert rel_err(got, ref) <= TOL
    assert np.all(got[int(cu[-1]):] == 0)
