"""Float64 CPU oracle of the MoE experts path (test infrastructure only).

Sources (the vLLM API pages this follows):
  * "vllm.model_executor.layers.fused_moe.experts.moonep_experts", module
    docstring: with rows contiguous per weight row, the experts step is a
    grouped GEMM for the gate projection and one for the up projection, the
    SiLU-gated product scaled per row by its route weight, and a grouped GEMM
    for the down projection; segments with no rows are skipped.
  * same page, MoonEPExperts.apply: cu_seqlens = cumsum of per-row token
    counts (int32 end offsets, one per weight row); route weights applied to
    the activation before the down GEMM; rows past the last end are zero.
  * same page, moonep_grouped_gemm: each segment's rows are multiplied by the
    transpose of that segment's [N, K] weight (weights stored [G, N, K]).
  * "vllm.model_executor.layers.fused_moe.experts.flashinfer_moe_ep", module
    docstring and FlashInferMoeEpExperts.apply: route on the top-k output, then
    compute and combine back to token order (the finalize is a no-op because
    the kernel already reduced); ids are int32.
  * "vllm.model_executor.layers.fused_moe.experts.trtllm_mxfp4_moe",
    TrtLlmMxfp4ExpertsBase: MXFP4 weights (kMxfp4Static with unquantized
    activations) and the SwiGLU-OAI activation parameterised by alpha, beta
    and a clamp limit; the SiTu closed form in the constructor's comment.

Readings where the pages are silent:
  * SwiGLU-OAI: g' = min(g, limit), u' = clamp(u, -limit, limit),
    f = g' * sigmoid(alpha * g') * (u' + beta)  (the gpt-oss definition).
  * MXFP4 = OCP Microscaling v1.0: e2m1 codes (sign, 2-bit exponent with bias
    1, 1-bit mantissa), two per byte, element 2i in the low nibble; one e8m0
    scale byte per 32 consecutive K elements, value 2^(v-127), v=255 is NaN.
  * Order inside a segment: ascending flat slot index t*k + j.
  * Expert id -1 marks a masked slot (contributes nothing, no error); any other
    id outside [0, E) is skipped and counted as bad.
  * Combine sums the k slot results of a token in ascending j.

  * MXFP8 activations (act_fmt="mxfp8"): the trtllm_mxfp4_moe page lists
    MXFP4 weights with dynamically quantized MXFP8 activations as a supported
    scheme but gives no formula. Reading: OCP Microscaling v1.0 with e4m3
    elements: per 32 consecutive values of a row along K, the scale is
    X = 2^(floor(log2(amax)) - 8) (8 = the e4m3 largest exponent), its e8m0
    code clamped to [0, 254] (code 0 when amax = 0); each value becomes
    rne_e4m3(v / X), saturated at +-448, times X. Both GEMM inputs are
    quantized this way: the token rows before the gate and up GEMMs, the
    activation rows (after the route weight) before the down GEMM. The token
    rows are the bf16 tensor handed to the experts step, quantized as they
    are (with the route weight on the input, the weighted rows are first
    rounded to bf16, the form in which the prepare step hands activations
    over: moonep_experts page, MoonEPExperts.apply). The activation rows are
    quantized from their exact value: the flashinfer_moe_ep page
    (epilogue_from_quant_config) quantizes activations dynamically inside the
    kernel, so no bf16 tensor of them exists in between.

Parity unpinned (the pages give a name and parameters but no formula, so the
pins check this code against the reading, not against the pages): the
SwiGLU-OAI formula, and the choice of the OCP MX scale and rounding rule for
MXFP8 activations. The e2m1 and e4m3 encodings themselves are pinned
exhaustively.

Everything is computed in float64 from exactly widened inputs.
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence, Tuple, Union

import numpy as np

__all__ = [
    "align", "grouped_mm", "silu", "swiglu_oai", "situ", "activation",
    "mxfp4_decode", "e4m3_round", "mxfp8_quantize", "bf16_round", "expert_matrix", "experts_grouped", "experts_forward",
    "experts_forward_literal", "pregrouped_forward",
]

# A weight argument is either a float array [E, N, K] or, for MXFP4, a pair
# (codes uint8 [E, N, K/2], scales uint8 [E, N, K/32]).
Weight = Union[np.ndarray, Tuple[np.ndarray, np.ndarray]]


# ----------------------------------------------------------------------------
# Grouping: histogram, prefix sum, stable permutation.
# moonep_experts page, MoonEPExperts.apply (cu_seqlens as a cumulative sum of
# per-row counts) and module docstring (rows contiguous per weight row).
# ----------------------------------------------------------------------------
def align(topk_ids: np.ndarray, E: int):
    """Group the T*k routed slots by expert.

    Returns a dict with
      counts   int64 [E]   slots routed to each expert (valid ids only)
      cu_seqlens int64 [E] cumulative end offsets (cumsum of counts)
      offsets  int64 [E+1] segment starts, offsets[E] = number of valid slots
      perm     int64 [M]   perm[p] = flat slot index i = t*k + j at sorted row p,
                           ascending in i inside each segment
      inv_perm int64 [T*k] inv_perm[i] = p, or -1 for masked / bad slots
      n_bad    int         ids outside [0, E) other than -1
    """
    flat = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    n_bad = int(np.sum((flat != -1) & ~valid))
    counts = np.bincount(flat[valid], minlength=E).astype(np.int64)
    cu = np.cumsum(counts)
    offsets = np.concatenate([[0], cu]).astype(np.int64)
    # stable sort by expert; masked and bad slots get key E and fall off the end
    key = np.where(valid, flat, E)
    order = np.argsort(key, kind="stable")
    M = int(offsets[E])
    perm = order[:M].astype(np.int64)
    inv_perm = np.full(flat.size, -1, dtype=np.int64)
    inv_perm[perm] = np.arange(M, dtype=np.int64)
    return dict(counts=counts, cu_seqlens=cu, offsets=offsets, perm=perm,
                inv_perm=inv_perm, n_bad=n_bad)


# ----------------------------------------------------------------------------
# Grouped GEMM. moonep_experts page, moonep_grouped_gemm.
# ----------------------------------------------------------------------------
def grouped_mm(a: np.ndarray, w_of: Callable[[int], np.ndarray], cu_seqlens: Sequence[int]) -> np.ndarray:
    """Segment g's rows of `a` times the transpose of segment g's weight, for
    segments given by end offsets.

    `w_of(g)` returns segment g's [N, K] weight in float64. Rows past the last
    end offset are zero; empty segments never ask for their weight."""
    a = np.asarray(a, dtype=np.float64)
    out = None
    start = 0
    for g, end in enumerate(cu_seqlens):
        end = int(end)
        if end > start:
            wg = w_of(g)
            if out is None:
                out = np.zeros((a.shape[0], wg.shape[0]), dtype=np.float64)
            out[start:end] = a[start:end] @ wg.T
        start = end
    return out


# ----------------------------------------------------------------------------
# Activations.
# ----------------------------------------------------------------------------
def silu(g):
    """silu(g) = g * sigmoid(g) (moonep_experts page, module docstring)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):  # exp(-g) = inf for very negative g gives the limit 0
        return g / (1.0 + np.exp(-g))


def swiglu_oai(g, u, alpha: float, beta: float, limit: float):
    """Clamped SwiGLU-OAI with the gemm1_alpha / gemm1_beta / clamp-limit
    parameters named on the trtllm_mxfp4_moe page (TrtLlmMxfp4ExpertsBase).
    The page gives no formula; this is the gpt-oss reading: the gate is capped
    at `limit` from above, the up projection clamped to [-limit, limit], and
    f = g' * sigmoid(alpha * g') * (u' + beta)."""
    g = np.minimum(np.asarray(g, dtype=np.float64), limit)
    u = np.clip(np.asarray(u, dtype=np.float64), -limit, limit)
    with np.errstate(over="ignore"):  # exp overflow to inf gives the limit 0
        return g / (1.0 + np.exp(-alpha * g)) * (u + beta)


def situ(g, u, alpha: float, beta: float):
    """SiTu gated activation (trtllm_mxfp4_moe page, TrtLlmMxfp4ExpertsBase
    constructor comment): left = alpha*tanh(g/alpha)*sigmoid(g) on the gate,
    right = beta*tanh(u/beta) on the up projection, product of the two."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    with np.errstate(over="ignore"):  # exp overflow to inf gives the limit 0
        return alpha * np.tanh(g / alpha) / (1.0 + np.exp(-g)) * (beta * np.tanh(u / beta))


def activation(name: str, g, u, alpha=1.0, beta=0.0, limit=math.inf):
    if name == "silu":
        return silu(g) * np.asarray(u, dtype=np.float64)
    if name == "swiglu_oai":
        return swiglu_oai(g, u, alpha, beta, limit)
    if name == "situ":
        return situ(g, u, alpha, beta)
    raise ValueError(f"unknown activation {name!r}")


# ----------------------------------------------------------------------------
# MXFP4 decoding (OCP Microscaling v1.0 reading; the pages only name the format).
# ----------------------------------------------------------------------------
def mxfp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact float64 value of MXFP4 weights.

    codes [..., K/2] uint8: element 2i in the low nibble of byte i, 2i+1 high.
    Each e2m1 code is s|e1 e0|m: for e > 0 the value is (-1)^s 2^(e-1) (1+m/2),
    for e = 0 it is (-1)^s m/2. scales [..., K/32] uint8: one e8m0 byte per 32
    consecutive elements, value 2^(v-127), and v = 255 is NaN."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = codes & 0x0F
    hi = codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2).astype(np.int64)
    sign = np.where(nib & 0x8, -1.0, 1.0)
    e = (nib >> 1) & 0x3
    m = (nib & 0x1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int32)))
    val = sign * mag
    s = np.asarray(scales, dtype=np.uint8).astype(np.int64)
    sc = np.where(s == 255, np.nan, np.ldexp(1.0, (s - 127).astype(np.int32)))
    sc = np.repeat(sc, 32, axis=-1)
    return val * sc


# ----------------------------------------------------------------------------
# MXFP8 activations (OCP Microscaling v1.0 reading with e4m3 elements; the
# trtllm_mxfp4_moe page, TrtLlmMxfp4ExpertsBase, names the scheme only).
# ----------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_round(v) -> np.ndarray:
    """Nearest e4m3 value, ties to even, magnitudes above 448 saturated to 448.

    e4m3 (the OCP "fn" variant): sign, 4 exponent bits with bias 7, 3 mantissa
    bits; normal values 2^(e-7) (1 + m/8) for e = 1..15 (e = 15, m = 7 is NaN,
    so 448 is the largest), subnormal values 2^-6 m/8. Inside the binade
    [2^b, 2^(b+1)) the spacing is 2^(b-3); below 2^-6 it is 2^-9."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)                      # a = f 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1
    b = np.maximum(ex - 1, -6)
    q = np.ldexp(1.0, (b - 3).astype(np.int32))
    r = np.round(a / q) * q                  # a / q is exact; np.round ties to even
    return np.sign(v) * np.minimum(r, E4M3_MAX)


def mxfp8_quantize(a: np.ndarray):
    """MXFP8 (e4m3 elements) quantization of the last axis in blocks of 32.

    Returns (values, elements, codes): values = elements * 2^(codes - 127) in
    float64; elements are the e4m3 values; codes the e8m0 scale bytes, one per
    block: floor(log2(amax)) + 127 - 8 clamped to [0, 254], and 0 for an
    all-zero block."""
    a = np.asarray(a, dtype=np.float64)
    K = a.shape[-1]
    if K % 32:
        raise ValueError("MXFP8 needs the last axis to be a multiple of 32")
    blk = a.reshape(*a.shape[:-1], K // 32, 32)
    amax = np.max(np.abs(blk), axis=-1)
    _, ex = np.frexp(amax)
    code = np.where(amax > 0, np.clip(ex - 1 + 127 - 8, 0, 254), 0).astype(np.int64)
    X = np.ldexp(1.0, (code - 127).astype(np.int32))[..., None]
    elem = e4m3_round(blk / X)
    vals = (elem * X).reshape(a.shape)
    return vals, elem.reshape(a.shape), code.astype(np.uint8)


def bf16_round(v) -> np.ndarray:
    """Nearest bf16 value (8 significant bits), ties to even, for finite
    values in the normal range: inside [2^b, 2^(b+1)) the spacing is 2^(b-7)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    q = np.ldexp(1.0, (ex - 1 - 7).astype(np.int32))
    return np.sign(v) * np.round(a / q) * q


def _act_in(rows: np.ndarray, act_fmt: str, bf16_first: bool) -> np.ndarray:
    """A GEMM's input rows as the GEMM sees them. With MXFP8 activations the
    rows are quantized; bf16_first: they are a bf16 tensor (the token rows, or
    the weighted token rows rounded to bf16), else their exact value (the
    activation rows, quantized inside the experts step)."""
    if act_fmt == "bf16":
        return rows
    if act_fmt == "mxfp8":
        return mxfp8_quantize(bf16_round(rows) if bf16_first else rows)[0]
    raise ValueError(f"unknown activation format {act_fmt!r}")


def expert_matrix(w: Weight, e: int) -> np.ndarray:
    """Expert e's [N, K] weight in float64 (decoded when MXFP4)."""
    if isinstance(w, tuple):
        codes, scales = w
        return mxfp4_decode(codes[e], scales[e])
    return np.asarray(w[e], dtype=np.float64)


# ----------------------------------------------------------------------------
# The experts computation in grouped form.
# moonep_experts page, module docstring + MoonEPExperts.apply.
# ----------------------------------------------------------------------------
def _per_expert(v, e):
    """Parameter v for expert (segment) e: v itself when it is a scalar, else
    its entry e (one value per expert)."""
    return v if np.ndim(v) == 0 else float(np.asarray(v, dtype=np.float64)[e])


def _per_row(v, cu_seqlens: Sequence[int], n_rows: int):
    """A per-expert parameter spread over the rows of a grouped problem: the
    scalar itself, or a float64 column [n_rows, 1] holding each row's segment's
    value (rows past the last end take the last segment's; they are zeroed)."""
    if v is None or np.ndim(v) == 0:
        return v
    seg = np.searchsorted(np.asarray(cu_seqlens), np.arange(n_rows), side="right")
    seg = np.minimum(seg, len(cu_seqlens) - 1)
    return np.asarray(v, dtype=np.float64)[seg][:, None]


def experts_grouped(x_rows: np.ndarray, cu_seqlens: Sequence[int], route_w: np.ndarray,
                    w_gate: Weight, w_up: Weight, w_down: Weight,
                    act: str = "silu", alpha=1.0, beta=0.0, limit=math.inf,
                    weight_on_input: bool = False, act_fmt: str = "bf16",
                    fc1_alpha=None, fc2_alpha=None) -> np.ndarray:
    """Rows already contiguous per weight row: gate and up grouped GEMMs, the
    activation times the per-row route weight, the down grouped GEMM. Rows past
    the last end offset come out zero.

    alpha, beta, limit: scalars, or one value per segment (the
    trtllm_mxfp4_moe page, TrtLlmMxfp4ExpertsBase constructor, keeps the
    activation's alpha, beta and clamp limit as per-expert tensors).
    fc1_alpha, fc2_alpha: None, or one scale per segment that multiplies the
    gate and up products (fc1) and the down product (fc2) of that segment's
    rows (the flashinfer_moe_ep page, epilogue_from_quant_config: one weight
    global scale per expert becomes the fc1 / fc2 epilogue alpha).

    weight_on_input: the route weight multiplies the input row before the gate
    and up GEMMs instead of the activation (moonep_experts page,
    MoonEPExperts.apply: input-weighted routing is applied to the activations
    before dispatch, and the experts step then skips its own multiply).

    act_fmt "mxfp8": both GEMMs' input rows are MXFP8-quantized first (the
    reading in the module docstring)."""
    x_rows = np.asarray(x_rows, dtype=np.float64)
    NvS = x_rows.shape[0]
    H = x_rows.shape[1]
    rw = np.asarray(route_w, dtype=np.float64)[:, None]
    if weight_on_input:
        x_rows = x_rows * rw
    x_rows = _act_in(x_rows, act_fmt, bf16_first=True)
    gate = grouped_mm(x_rows, lambda g: expert_matrix(w_gate, g), cu_seqlens)
    if gate is None:                                    # every segment empty
        return np.zeros((NvS, H), dtype=np.float64)
    up = grouped_mm(x_rows, lambda g: expert_matrix(w_up, g), cu_seqlens)
    if fc1_alpha is not None:
        s1 = _per_row(fc1_alpha, cu_seqlens, NvS)
        gate, up = gate * s1, up * s1
    a = activation(act, gate, up, _per_row(alpha, cu_seqlens, NvS), _per_row(beta, cu_seqlens, NvS),
                   _per_row(limit, cu_seqlens, NvS))
    if not weight_on_input:
        a = a * rw
    a = _act_in(a, act_fmt, bf16_first=False)
    out = grouped_mm(a, lambda g: expert_matrix(w_down, g), cu_seqlens)
    if fc2_alpha is not None:
        out = out * _per_row(fc2_alpha, cu_seqlens, NvS)
    end = int(cu_seqlens[-1]) if len(cu_seqlens) else 0
    out[end:] = 0.0
    return out


def experts_forward(x: np.ndarray, topk_ids: np.ndarray, topk_weights: np.ndarray,
                    w_gate: Weight, w_up: Weight, w_down: Weight,
                    act: str = "silu", alpha=1.0, beta=0.0, limit=math.inf,
                    weight_on_input: bool = False, act_fmt: str = "bf16",
                    fc1_alpha=None, fc2_alpha=None) -> np.ndarray:
    """Token-major MoE experts layer: group the routed slots by expert, run
    the grouped computation, then combine each token's k slot results in
    ascending j (flashinfer_moe_ep page: route, compute, combine)."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(topk_ids)
    T, k = ids.shape
    E = _num_experts(w_gate)
    al = align(ids, E)
    perm, inv = al["perm"], al["inv_perm"]
    x_rows = x[perm // k]
    rw = np.asarray(topk_weights, dtype=np.float64).reshape(-1)[perm]
    y = experts_grouped(x_rows, al["cu_seqlens"], rw, w_gate, w_up, w_down, act, alpha, beta, limit,
                        weight_on_input, act_fmt, fc1_alpha, fc2_alpha)
    out = np.zeros((T, x.shape[1]), dtype=np.float64)
    for t in range(T):
        acc = np.zeros(x.shape[1], dtype=np.float64)
        for j in range(k):
            p = inv[t * k + j]
            if p >= 0:
                acc = acc + y[p]
        out[t] = acc
    return out


def experts_forward_literal(x, topk_ids, topk_weights, w_gate, w_up, w_down,
                            act="silu", alpha=1.0, beta=0.0, limit=math.inf,
                            weight_on_input=False, act_fmt="bf16", fc1_alpha=None, fc2_alpha=None) -> np.ndarray:
    """The per-token definition: for each token and each of its k slots, run
    the selected expert's MLP on the token, scale by the route weight, and sum
    over the slots in ascending j. Masked (-1) and out-of-range ids add
    nothing. Slow; for small problems and as a check of `experts_forward`."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(topk_ids)
    wts = np.asarray(topk_weights, dtype=np.float64)
    T, k = ids.shape
    E = _num_experts(w_gate)
    out = np.zeros((T, x.shape[1]), dtype=np.float64)
    for t in range(T):
        acc = np.zeros(x.shape[1], dtype=np.float64)
        for j in range(k):
            e = int(ids[t, j])
            if e < 0 or e >= E:
                continue
            xin = x[t] * wts[t, j] if weight_on_input else x[t]
            xin = _act_in(xin, act_fmt, bf16_first=True)
            g = expert_matrix(w_gate, e) @ xin
            u = expert_matrix(w_up, e) @ xin
            if fc1_alpha is not None:
                g, u = g * _per_expert(fc1_alpha, e), u * _per_expert(fc1_alpha, e)
            a = activation(act, g, u, _per_expert(alpha, e), _per_expert(beta, e), _per_expert(limit, e))
            if not weight_on_input:
                a = a * wts[t, j]
            a = _act_in(a, act_fmt, bf16_first=False)
            yd = expert_matrix(w_down, e) @ a
            if fc2_alpha is not None:
                yd = yd * _per_expert(fc2_alpha, e)
            acc = acc + yd
        out[t] = acc
    return out


def pregrouped_forward(x_nvs, cu_seqlens, route_w, w_gate, w_up, w_down,
                       act="silu", alpha=1.0, beta=0.0, limit=math.inf, weight_on_input=False,
                       act_fmt="bf16", fc1_alpha=None, fc2_alpha=None) -> np.ndarray:
    """The pre-grouped entry: rows given in segment order with end offsets and
    per-row route weights (moonep_experts page, MoonEPExperts.apply). Same as
    `experts_grouped`; named for the entry point it checks."""
    return experts_grouped(x_nvs, cu_seqlens, route_w, w_gate, w_up, w_down, act, alpha, beta, limit,
                           weight_on_input, act_fmt, fc1_alpha, fc2_alpha)


def _num_experts(w: Weight) -> int:
    return (w[0] if isinstance(w, tuple) else w).shape[0]
