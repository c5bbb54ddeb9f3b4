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
    return dict(act=wl.act, alpha=wl.alpha, beta=wl.beta, limit=wl.limit)


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
