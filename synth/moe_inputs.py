"""Seeded synthetic workloads for the MoE experts path.

Every tensor is drawn from its own seed, derived from (workload id, tensor
tag, expert) through numpy's SeedSequence, so any single expert's weights can
be regenerated alone and on any device.

Recipes (the pages publish no workload data; these stand in for it):

* activations x ~ N(0, 1), rounded to bf16 (round-to-nearest-even);
* bf16 weights ~ N(0, 1/sqrt(fan_in)): fan_in = H for gate/up, I for down;
* router: logits ~ N(0, 1) [T, E] (plus a per-expert bias for Zipf-skewed
  load), softmax, top-k by descending probability with ties to the lower
  expert id, weights renormalised over the k picks; ids int32, weights fp32;
* Zipf skew with exponent s: bias_e = -s * ln(r_e) where r is a seeded
  permutation of 1..E, so an expert's softmax mass scales as r_e^-s;
* MXFP4 weights: e2m1 codes uniform over all 16 values (uniform random bytes,
  two codes per byte), e8m0 scale bytes 127 + U{-8..0};
* pre-grouped layout: E experts + B redundant slots, given empties, Zipf
  segment lengths rounded by largest remainder, route weights ~ U(0, 1).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np
import torch

__all__ = [
    "Workload", "WORKLOADS", "workload", "seed_for", "make_routing",
    "make_x", "make_bf16_weights", "make_mxfp4_weights", "make_pregrouped_layout",
    "make_route_weights_nvs", "expert_weight", "bf16_to_f32", "make_logits", "make_router_bias",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens (NvS rows for the pre-grouped layout)
    H: int
    I: int
    E: int            # experts (segments, incl. redundant slots, for pre-grouped)
    k: int            # top-k (1 for the pre-grouped layout)
    wfmt: str = "bf16"          # "bf16" | "mxfp4"
    act: str = "silu"           # "silu" | "swiglu_oai"
    alpha: float = 1.0
    beta: float = 0.0
    limit: float = float("inf")
    zipf_s: Optional[float] = None   # routing skew (None = uniform logits)
    pregrouped: bool = False
    n_real: int = 0                  # pre-grouped: real experts (E = n_real + B)
    n_empty_real: int = 0            # pre-grouped: real experts left empty
    n_used_slots: int = 0            # pre-grouped: redundant slots that hold rows
    wid: int = 0                     # workload id mixed into every seed
    act_fmt: str = "bf16"            # "bf16" | "mxfp8" (GEMM inputs as MXFP8, MXFP4 weights only)

    @property
    def M(self) -> int:
        return self.T * self.k

    @property
    def flops(self) -> float:
        """Multiply-add FLOPs of the routed rows: 2*M*H*I per GEMM, 3 GEMMs."""
        return 6.0 * self.M * self.H * self.I


WORKLOADS = {
    # T=64 H=128 I=256 E=8 top-2, SiLU, uniform routing.
    "tiny": Workload("tiny", T=64, H=128, I=256, E=8, k=2, wid=1),
    # Mixtral-shaped prefill layer.
    "mixtral_prefill": Workload("mixtral_prefill", T=4096, H=4096, I=14336, E=8, k=2, wid=2),
    # Fine-grained prefill, 256 resident experts, Zipf(1.0) skewed load.
    "fine_grained_prefill": Workload("fine_grained_prefill", T=8192, H=7168, I=2048, E=256, k=8,
                                     zipf_s=1.0, wid=3),
    # Decode with MXFP4 weights and clamped SwiGLU-OAI (alpha 1.702, limit 7, beta 1).
    "mxfp4_decode": Workload("mxfp4_decode", T=32, H=2880, I=2880, E=128, k=4, wfmt="mxfp4",
                             act="swiglu_oai", alpha=1.702, beta=1.0, limit=7.0, wid=4),
    # Prefill with MXFP4 weights and MXFP8 activations: the decode layer's
    # shapes (H=I=2880, E=128, top-4, clamped SwiGLU-OAI) at 8192 tokens,
    # 256 routed rows per expert on average.
    "mxfp4_prefill": Workload("mxfp4_prefill", T=8192, H=2880, I=2880, E=128, k=4, wfmt="mxfp4",
                              act="swiglu_oai", alpha=1.702, beta=1.0, limit=7.0, act_fmt="mxfp8", wid=6),
    # Pre-grouped redundant-slot layout: 32 experts + 8 slots, NvS=16384.
    "pregrouped": Workload("pregrouped", T=16384, H=7168, I=2048, E=40, k=1, pregrouped=True,
                           n_real=32, n_empty_real=2, n_used_slots=3, zipf_s=1.2, wid=5),
}


def workload(name: str, **overrides) -> Workload:
    return dataclasses.replace(WORKLOADS[name], **overrides)


_TAGS = {"x": 1, "logits": 2, "zipf": 3, "w_gate": 4, "w_up": 5, "w_down": 6,
         "s_gate": 7, "s_up": 8, "s_down": 9, "segments": 10, "route_w": 11,
         "slots": 12, "router_bias": 13}


def seed_for(wl: Workload, tag: str, expert: int = 0, seed: int = 0) -> int:
    """A 63-bit seed for one tensor (or one expert's slice of it)."""
    ss = np.random.SeedSequence([seed, wl.wid, _TAGS[tag], expert])
    return int(ss.generate_state(2, dtype=np.uint32).astype(np.uint64) @ np.array([1, 1 << 31], dtype=np.uint64)) & ((1 << 63) - 1)


def _gen(device, s: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def bf16_to_f32(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16 tensor to a float32 numpy array on the host."""
    return t.detach().to("cpu").to(torch.float32).numpy()


# ----------------------------------------------------------------- routing
def make_routing(wl: Workload, seed: int = 0, T: Optional[int] = None):
    """Router output for `wl`: (ids int32 [T,k], weights float32 [T,k]).

    Drawn on the host with numpy so every consumer sees identical ids."""
    T = wl.T if T is None else T
    rng = np.random.Generator(np.random.PCG64(seed_for(wl, "logits", 0, seed)))
    logits = rng.standard_normal((T, wl.E))
    if wl.zipf_s is not None:
        prng = np.random.Generator(np.random.PCG64(seed_for(wl, "zipf", 0, seed)))
        ranks = prng.permutation(wl.E) + 1
        logits = logits - wl.zipf_s * np.log(ranks.astype(np.float64))[None, :]
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    # top-k by descending probability; a stable sort keeps the lower id first on ties
    order = np.argsort(-p, axis=1, kind="stable")[:, : wl.k]
    psel = np.take_along_axis(p, order, axis=1)
    w = psel / psel.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def make_logits(wl: Workload, seed: int = 0, T: Optional[int] = None) -> np.ndarray:
    """Router logits float32 [T, E]: the same seeded N(0,1) draw as make_routing
    (plus its Zipf expert bias on skewed workloads), rounded to float32."""
    T = wl.T if T is None else T
    rng = np.random.Generator(np.random.PCG64(seed_for(wl, "logits", 0, seed)))
    logits = rng.standard_normal((T, wl.E))
    if wl.zipf_s is not None:
        prng = np.random.Generator(np.random.PCG64(seed_for(wl, "zipf", 0, seed)))
        ranks = prng.permutation(wl.E) + 1
        logits = logits - wl.zipf_s * np.log(ranks.astype(np.float64))[None, :]
    return logits.astype(np.float32)


def make_router_bias(wl: Workload, seed: int = 0, scale: float = 0.1) -> np.ndarray:
    """Score-correction bias float32 [E] ~ N(0, scale^2) for grouped routing."""
    rng = np.random.Generator(np.random.PCG64(seed_for(wl, "router_bias", 0, seed)))
    return (scale * rng.standard_normal(wl.E)).astype(np.float32)


# ----------------------------------------------------------------- activations
def make_x(wl: Workload, device="cpu", seed: int = 0, rows: Optional[int] = None) -> torch.Tensor:
    rows = wl.T if rows is None else rows
    g = _gen(device, seed_for(wl, "x", 0, seed))
    return torch.randn(rows, wl.H, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


# ----------------------------------------------------------------- weights
def _bf16_expert(wl, tag, e, N, K, std, device, seed):
    g = _gen(device, seed_for(wl, tag, e, seed))
    return (torch.randn(N, K, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def expert_weight(wl: Workload, tag: str, e: int, device="cpu", seed: int = 0) -> torch.Tensor:
    """One expert's bf16 weight matrix, [N, K] with K contiguous."""
    if tag in ("w_gate", "w_up"):
        return _bf16_expert(wl, tag, e, wl.I, wl.H, wl.H ** -0.5, device, seed)
    return _bf16_expert(wl, tag, e, wl.H, wl.I, wl.I ** -0.5, device, seed)


def make_bf16_weights(wl: Workload, device="cpu", seed: int = 0, source=None):
    """(w_gate [E,I,H], w_up [E,I,H], w_down [E,H,I]) in bf16.

    `source[e]` (optional) names the expert whose weights row e copies; the
    pre-grouped layout uses it for its redundant slots."""
    src = list(range(wl.E)) if source is None else list(source)
    out = []
    for tag, (N, K) in (("w_gate", (wl.I, wl.H)), ("w_up", (wl.I, wl.H)), ("w_down", (wl.H, wl.I))):
        w = torch.empty(wl.E, N, K, dtype=torch.bfloat16, device=device)
        for e in range(wl.E):
            w[e] = expert_weight(wl, tag, src[e], device, seed)
        out.append(w)
    return tuple(out)


def make_mxfp4_weights(wl: Workload, device="cpu", seed: int = 0):
    """Packed MXFP4 weights: for gate, up, down a (codes, scales) pair.

    codes: uint8 [E, N, K/2], two e2m1 codes per byte; scales: uint8
    [E, N, K/32], e8m0 bytes 127 + U{-8..0}. Codes are uniform bytes, so both
    nibbles are uniform over the 16 e2m1 codes."""
    res = []
    for wtag, stag, (N, K) in (("w_gate", "s_gate", (wl.I, wl.H)), ("w_up", "s_up", (wl.I, wl.H)),
                               ("w_down", "s_down", (wl.H, wl.I))):
        codes = torch.empty(wl.E, N, K // 2, dtype=torch.uint8, device=device)
        scales = torch.empty(wl.E, N, K // 32, dtype=torch.uint8, device=device)
        for e in range(wl.E):
            gc = _gen(device, seed_for(wl, wtag, e, seed))
            codes[e] = torch.randint(0, 256, (N, K // 2), generator=gc, device=device, dtype=torch.int32).to(torch.uint8)
            gs = _gen(device, seed_for(wl, stag, e, seed))
            scales[e] = (127 - torch.randint(0, 9, (N, K // 32), generator=gs, device=device, dtype=torch.int32)).to(torch.uint8)
        res.append((codes, scales))
    return tuple(res)


# ----------------------------------------------------------------- pre-grouped layout
def make_pregrouped_layout(wl: Workload, seed: int = 0):
    """Segment lengths and redundant-slot sources for the pre-grouped layout.

    Returns (lengths int64 [E], source int64 [E]): rows [0, n_real) are real
    experts, rows [n_real, E) redundant prefetch slots. `n_empty_real` real
    experts and all but `n_used_slots` slots are empty. Non-empty segments get
    lengths proportional to r^-s over a seeded permutation of ranks r, rounded
    by largest remainder so they sum to T (= NvS), each at least 1 row."""
    rng = np.random.Generator(np.random.PCG64(seed_for(wl, "segments", 0, seed)))
    E, R = wl.E, wl.n_real
    empty_real = rng.choice(R, size=wl.n_empty_real, replace=False)
    used_slots = R + np.arange(wl.n_used_slots)            # the first slots hold rows
    nonempty = np.array(sorted(set(range(R)) - set(empty_real.tolist())) + used_slots.tolist())
    ranks = rng.permutation(len(nonempty)) + 1
    share = ranks.astype(np.float64) ** -float(wl.zipf_s)
    share /= share.sum()
    extra = wl.T - len(nonempty)                           # one row guaranteed to each
    raw = share * extra
    base = np.floor(raw).astype(np.int64)
    rem = extra - int(base.sum())
    order = np.argsort(-(raw - base), kind="stable")
    base[order[:rem]] += 1
    lengths = np.zeros(E, dtype=np.int64)
    lengths[nonempty] = base + 1
    # every redundant slot copies a seeded real expert that is not empty
    real_nonempty = np.array(sorted(set(range(R)) - set(empty_real.tolist())))
    srng = np.random.Generator(np.random.PCG64(seed_for(wl, "slots", 0, seed)))
    source = np.arange(E, dtype=np.int64)
    source[R:] = srng.choice(real_nonempty, size=E - R, replace=True)
    return lengths, source


def make_route_weights_nvs(wl: Workload, seed: int = 0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed_for(wl, "route_w", 0, seed)))
    return rng.random(wl.T).astype(np.float32)
