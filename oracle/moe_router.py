"""Float64 CPU oracle of the router step (test infrastructure only).

The router turns per-token expert logits into the top-k expert ids and route
weights that the experts step consumes.

Sources (the vLLM API pages this follows):
  * "vllm.model_executor.layers.fused_moe.experts.trtllm_mxfp4_moe",
    TrtLlmMxfp4ExpertsMonolithic (router + experts in one call):
    _supports_routing_method names the methods Renormalize, RenormalizeNaive
    and DeepSeekV3, and apply passes the DeepSeekV3 parameters: a score
    correction bias, the number of expert groups, the number of groups kept
    (topk_group) and a routed scaling factor.

The pages name these methods and parameters but print no formula, so parity
is unpinned for the formulas themselves: the pins check this code against the
readings below (and against scipy's softmax and expit), not against the
pages. Readings:
  * Renormalize / RenormalizeNaive: probabilities p = softmax(logits) over all
    experts, the k largest kept, divided by their sum. The two names differ
    only in evaluation order (top-k of the logits then a softmax over the k
    picks, or the full softmax first); in exact arithmetic both give
    w_j = exp(l_j) / sum over the picks of exp(l_i).
  * DeepSeekV3 (the DeepSeek-V3 technical report's gating): scores
    s = sigmoid(logits); selection scores s' = s + bias; experts split into
    n_group equal contiguous groups, each group scored by the sum of its two
    largest s'; the topk_group best groups kept; the k largest s' among their
    experts picked; weights w_j = s_j / sum of the picked s, times the routed
    scaling factor. n_group 0 or 1 means no group limit.
  * Ties go to the lower index (expert or group). Output slots are in
    selection order: descending selection score.
  * Logits are first clamped to the finite float32 range (NaN counts as the
    most negative value), so every score is finite.
  * Where a float decides an integer (DeepSeekV3 selection), the decision is
    taken on float32 values: s is sigmoid evaluated in float64 and rounded to
    float32, s' = float32(s + bias) and group sums are float32 adds. The
    weights are then computed in float64.
  * If the picked scores of a token sum to 0 (DeepSeekV3, every pick scored
    0), its weights are 0.
"""
from __future__ import annotations

import numpy as np

__all__ = ["clamp_logits", "topk_order", "route_renormalize", "route_deepseek_v3", "route"]

F32_MAX = float(np.finfo(np.float32).max)


def clamp_logits(logits: np.ndarray) -> np.ndarray:
    """float32 logits -> float64, clamped to the finite float32 range; NaN -> -FLT_MAX."""
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    l = np.where(np.isnan(l), -F32_MAX, l)
    return np.clip(l, -F32_MAX, F32_MAX)


def topk_order(score: np.ndarray, k: int, allowed: np.ndarray | None = None) -> np.ndarray:
    """Indices of the k largest entries of each row, largest first; ties to the
    lower index. `allowed` (bool, same shape) excludes entries from the pick."""
    s = np.asarray(score, dtype=np.float64)
    if allowed is not None:
        s = np.where(allowed, s, -np.inf)
    # stable sort on the negated score keeps ascending index among equal scores
    return np.argsort(-s, axis=-1, kind="stable")[..., :k]


def route_renormalize(logits: np.ndarray, k: int):
    """(ids int32 [T,k], weights float64 [T,k]): softmax over all experts, the
    k largest kept, renormalised over the picks."""
    l = clamp_logits(logits)
    ids = topk_order(l, k)
    z = l - l.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    pk = np.take_along_axis(p, ids, axis=1)
    return ids.astype(np.int32), pk / pk.sum(axis=1, keepdims=True)


def _sigmoid_f32(l: np.ndarray) -> np.ndarray:
    """sigmoid in float64, rounded to float32 (the scores decisions are taken on)."""
    with np.errstate(over="ignore"):  # exp overflow to inf gives the limit 0
        return (1.0 / (1.0 + np.exp(-l))).astype(np.float32)


def route_deepseek_v3(logits: np.ndarray, k: int, bias: np.ndarray | None = None, n_group: int = 0,
                      topk_group: int = 0, routed_scaling_factor: float = 1.0):
    """(ids int32 [T,k], weights float64 [T,k]) of the DeepSeekV3 reading above."""
    l = clamp_logits(logits)
    T, E = l.shape
    s = _sigmoid_f32(l)                                        # float32 [T,E]
    b = np.zeros(E, np.float32) if bias is None else np.asarray(bias, np.float32)
    sb = (s + b[None, :]).astype(np.float32)                   # float32 add
    allowed = None
    if n_group > 1:
        G = E // n_group
        grp = sb.reshape(T, n_group, G)
        top2 = np.sort(grp, axis=2)[:, :, ::-1][:, :, :2]
        gscore = (top2[:, :, 0] + top2[:, :, 1]).astype(np.float32)  # float32 add
        keep = topk_order(gscore, topk_group)                  # [T, topk_group]
        gmask = np.zeros((T, n_group), bool)
        np.put_along_axis(gmask, keep, True, axis=1)
        allowed = np.repeat(gmask, G, axis=1)
    ids = topk_order(sb, k, allowed)
    sk = np.take_along_axis(s, ids, axis=1).astype(np.float64)
    tot = sk.sum(axis=1, keepdims=True)
    w = np.where(tot > 0, sk / np.where(tot > 0, tot, 1.0), 0.0) * float(routed_scaling_factor)
    return ids.astype(np.int32), w


def route(logits, k, method="renormalize", **kw):
    if method == "renormalize":
        return route_renormalize(logits, k)
    if method == "deepseek_v3":
        return route_deepseek_v3(logits, k, **kw)
    raise ValueError(method)
