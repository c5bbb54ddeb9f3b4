"""Shared test plumbing: device inputs, relative error, and sub-problems that
let the CPU oracle check sampled tokens of full-size workloads.

A token's output depends only on its own row, its ids and weights, and the
selected experts, so the oracle run on a sub-problem made of sampled tokens
(experts renumbered to the touched ones) gives exactly those tokens' rows of
the full output."""
import numpy as np
import torch

import oracle
import synth

TOL = 1e-2  # max|err| / max|ref| bound for outputs


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.abs(ref).max()
    if denom == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / denom)


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return synth.bf16_to_f32(t)
    return t.detach().cpu().numpy()


class LazyExperts:
    """Indexable like an [E', N, K] array: item e copies expert src[e] of a
    device tensor to the host as float32 on demand (bf16 widening is exact)."""

    def __init__(self, w: torch.Tensor, src):
        self.w = w
        self.src = list(src)
        self.shape = (len(self.src),) + tuple(w.shape[1:])

    def __getitem__(self, e):
        return to_np(self.w[self.src[e]])


class LazyMx:
    """MXFP4 pair (codes, scales) restricted to experts src, copied on demand."""

    def __init__(self, codes, scales, src):
        self.codes = LazyExperts(codes, src)
        self.scales = LazyExperts(scales, src)


def sampled_token_oracle(x, ids, w, wg, wu, wd, tokens, act_kw=None, mx=False):
    """Oracle rows for `tokens` of a token-major problem held on the device."""
    act_kw = act_kw or {}
    ids_np = ids.cpu().numpy()[tokens]
    w_np = w.cpu().numpy()[tokens]
    x_np = to_np(x[torch.as_tensor(tokens, device=x.device)])
    E = (wg[0] if mx else wg).shape[0]
    touched = sorted({int(e) for e in ids_np.ravel() if 0 <= e < E})
    remap = {e: i for i, e in enumerate(touched)}
    ids_c = np.vectorize(lambda e: remap.get(int(e), -1))(ids_np).astype(np.int32)
    if mx:
        W = [(LazyExperts(c, touched), LazyExperts(s, touched)) for c, s in (wg, wu, wd)]
    else:
        W = [LazyExperts(t, touched) for t in (wg, wu, wd)]
    return oracle.experts_forward(x_np, ids_c, w_np, W[0], W[1], W[2], **act_kw)


def wl_act_kw(wl):
    kw = dict(act=wl.act, alpha=wl.alpha, beta=wl.beta, limit=wl.limit)
    if wl.act_fmt != "bf16":
        kw["act_fmt"] = wl.act_fmt
    return kw


class Guarded:
    """A device byte buffer between two canary bands. `body` is the usable
    part (256-byte aligned, `nbytes` long); `poison()` fills it with 0xff
    bytes (bf16 NaN, int32 -1, float32 NaN) and the bands with a fixed
    pattern; `check_bands()` asserts that the bands still hold it."""

    BAND = 4096

    def __init__(self, nbytes: int, device):
        self.nbytes = max(int(nbytes), 256)
        self.full = torch.empty(self.nbytes + 2 * self.BAND, dtype=torch.uint8, device=device)
        self.body = self.full[self.BAND: self.BAND + self.nbytes]
        self.pattern = (torch.arange(self.BAND, device=device, dtype=torch.int32) * 37 + 11).to(torch.uint8)
        self.poison()

    def poison(self):
        self.body.fill_(0xFF)
        self.full[: self.BAND].copy_(self.pattern)
        self.full[self.BAND + self.nbytes:].copy_(self.pattern)

    def check_bands(self):
        assert torch.equal(self.full[: self.BAND], self.pattern), "write below the buffer"
        assert torch.equal(self.full[self.BAND + self.nbytes:], self.pattern), "write past the buffer"

    def view_bf16(self, *shape):
        n = int(np.prod(shape))
        return self.body[: 2 * n].view(torch.bfloat16).view(*shape)


def _quantize_with_codes(a, codes):
    """MXFP8 values of rows `a` with the given e8m0 scale code per 32-block."""
    R, K = a.shape
    X = np.ldexp(1.0, codes.astype(np.int64) - 127)[..., None]
    return (oracle.e4m3_round(a.reshape(R, K // 32, 32) / X) * X).reshape(R, K)


def mxfp8_activation_bounds(x, ids, w, W, S, act_kw, kernel_err_factor=1.0):
    """The down projection's input rows of the MXFP8 path in sorted row
    order, as the oracle computes them (float64, before quantization), and a
    bound d on how far the kernels' fp32 value of each element may lie from
    it: GEMM1's products are exact in fp32, so each dot product over K terms
    is off by at most K * 2^-24 * sum |x_i w_i| (the standard bound of fp32
    summation in any order; times kernel_err_factor), and d is the largest
    change of f(g, u) * route weight over the corners of that box, plus
    eight fp32 roundings of the result.

    Returns (al, a, d, D_of): the oracle's align, a and d [valid rows, I],
    and D_of(e) the expert's down matrix."""
    T, k = ids.shape
    Wn = [(c.numpy(), s.numpy()) for c, s in zip(W, S)]
    E = Wn[0][0].shape[0]
    par = {kk: v for kk, v in act_kw.items() if kk in ("alpha", "beta", "limit")}
    act = act_kw.get("act", "silu")
    al = oracle.align(ids, E)
    cu = al["cu_seqlens"]
    nv = int(cu[-1])
    I = Wn[0][0].shape[1]
    xq = oracle.mxfp8_quantize(to_np(x).astype(np.float64))[0]
    a_all = np.zeros((nv, I))
    d_all = np.zeros((nv, I))
    u_ = 2.0 ** -24
    start = 0
    for e in range(E):
        end = int(cu[e])
        if end == start:
            continue
        rows = al["perm"][start:end]
        wr = w.reshape(-1)[rows][:, None].astype(np.float64)
        if act_kw.get("weight_on_input"):
            # route weight on the input: weighted token rows, rounded to bf16,
            # quantized; the activation carries no weight
            xr = oracle.mxfp8_quantize(oracle.bf16_round(to_np(x).astype(np.float64)[rows // k] * wr))[0]
            wr = np.ones_like(wr)
        else:
            xr = xq[rows // k]
        G, U = (oracle.expert_matrix(Wn[i], e) for i in range(2))
        g, u = xr @ G.T, xr @ U.T
        Kg = xr.shape[1]
        dg = kernel_err_factor * Kg * u_ * (np.abs(xr) @ np.abs(G).T)
        du = kernel_err_factor * Kg * u_ * (np.abs(xr) @ np.abs(U).T)
        a = oracle.activation(act, g, u, **par) * wr
        da = np.zeros_like(a)
        for sg in (-1.0, 1.0):
            for su in (-1.0, 1.0):
                da = np.maximum(da, np.abs(oracle.activation(act, g + sg * dg, u + su * du, **par) * wr - a))
        a_all[start:end] = a
        d_all[start:end] = da + 8 * u_ * np.abs(a)
        start = end
    return al, a_all, d_all, lambda e: oracle.expert_matrix(Wn[2], e)


def mxfp8_code_range(a, d):
    """Smallest and largest e8m0 scale code per 32-block that values within d
    of a can give (the code grows with the block's largest magnitude)."""
    return (oracle.mxfp8_quantize(np.maximum(np.abs(a) - d, 0.0))[2].astype(np.int64),
            oracle.mxfp8_quantize(np.abs(a) + d)[2].astype(np.int64))


def mxfp8_reference_with_envelope(x, ids, w, W, S, act_kw, kernel_err_factor=1.0):
    """Oracle output of the MXFP8 path and an elementwise envelope for the
    quantization decisions the kernels may take the other way.

    The MXFP8 rounding of an activation element (e4m3 rounds to nearest, one
    step is 1/16 to 1/8 of the value) and its block's scale code (from the
    block's largest magnitude) are both fixed by values in [a - d, a + d]
    (mxfp8_activation_bounds); where that interval holds a rounding midpoint
    or a power of two the kernels may take either decision, and both are
    correct to the kernels' precision. The envelope is the largest change of
    the down projection's output those elements can make (their largest
    change of quantized value times |W_down|), summed over a token's slots;
    it is 0 wherever every decision is fixed.

    Returns (ref, envelope, n_ambiguous_elements)."""
    T, k = ids.shape
    H = x.shape[1]
    al, a, d, D_of = mxfp8_activation_bounds(x, ids, w, W, S, act_kw, kernel_err_factor)
    cu = al["cu_seqlens"]
    q, _, codes = oracle.mxfp8_quantize(a)
    c_lo, c_hi = mxfp8_code_range(a, d)
    dev = np.zeros_like(a)
    for c in (codes, c_lo, c_hi):
        for v in (a - d, a + d):  # rounding is monotone: the interval's ends bound its results
            dev = np.maximum(dev, np.abs(_quantize_with_codes(v, c) - q))
    M = T * k
    y = np.zeros((M, H))
    env = np.zeros((M, H))
    start = 0
    for e in range(len(cu)):
        end = int(cu[e])
        if end == start:
            continue
        D = D_of(e)
        y[start:end] = q[start:end] @ D.T
        env[start:end] = dev[start:end] @ np.abs(D).T
        start = end
    inv = al["inv_perm"].reshape(T, k)
    out = np.zeros((T, H))
    out_env = np.zeros((T, H))
    for j in range(k):
        r = inv[:, j]
        ok = r >= 0
        out[ok] += y[r[ok]]
        out_env[ok] += env[r[ok]]
    return out, out_env, int(np.count_nonzero(dev))


def check_mxfp8_output(got, ref, env, tol=TOL):
    """|got - ref| <= tol * max|ref| + env elementwise; returns (plain rel
    error, rel error beyond the envelope, outputs that needed the envelope)."""
    got = np.asarray(got, dtype=np.float64)
    scale = np.abs(ref).max()
    d = np.abs(got - ref)
    beyond = np.maximum(d - env, 0.0)
    used = int(np.count_nonzero((d > tol * scale) & (d <= tol * scale + env)))
    return float(d.max() / scale), float(beyond.max() / scale), used
