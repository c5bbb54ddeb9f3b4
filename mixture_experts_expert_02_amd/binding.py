"""ctypes binding of libmoe_experts.so (include/moe_experts.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t. Every step of the computation runs in the HIP
library; if the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_experts.so")

MOE_OK, MOE_EINVAL, MOE_ENOTSUP, MOE_ENOSPC, MOE_EHIP, MOE_ETIMEDOUT = 0, -1, -2, -3, -4, -5
MOE_W_BF16, MOE_W_MXFP4 = 0, 1
MOE_ACT_SILU, MOE_ACT_SWIGLU_OAI, MOE_ACT_SITU = 0, 1, 2

_ACT = {"silu": MOE_ACT_SILU, "swiglu_oai": MOE_ACT_SWIGLU_OAI, "situ": MOE_ACT_SITU}
_WFMT = {"bf16": MOE_W_BF16, "mxfp4": MOE_W_MXFP4}
MOE_A_BF16, MOE_A_MXFP8 = 0, 1
_AFMT = {"bf16": MOE_A_BF16, "mxfp8": MOE_A_MXFP8}

EXPORTED = (
    "moe_experts_workspace_bytes", "moe_experts_workspace_layout", "moe_experts_forward",
    "moe_experts_forward_timed", "moe_align_workspace_bytes", "moe_align",
    "moe_experts_grouped_workspace_bytes", "moe_experts_forward_grouped", "moe_device_error",
    "moe_strerror", "moe_route", "moe_experts_forward_grouped_timed", "moe_experts_forward_noalloc",
    "moe_check_expert_params", "moe_mx_packed_bytes", "moe_mx_pack_weights", "moe_bf16_packed_bytes",
    "moe_bf16_pack_weights",
)
MOE_ROUTE_RENORMALIZE, MOE_ROUTE_DEEPSEEK_V3 = 0, 1
_ROUTE = {"renormalize": MOE_ROUTE_RENORMALIZE, "deepseek_v3": MOE_ROUTE_DEEPSEEK_V3}


class MoeProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("wfmt", ctypes.c_int32),
                ("act", ctypes.c_int32), ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
                ("limit", ctypes.c_float), ("weight_on_input", ctypes.c_int32), ("a_fmt", ctypes.c_int32),
                ("alpha_e", ctypes.c_void_p), ("beta_e", ctypes.c_void_p), ("limit_e", ctypes.c_void_p),
                ("fc1_alpha", ctypes.c_void_p), ("fc2_alpha", ctypes.c_void_p), ("mx_packed", ctypes.c_void_p),
                ("bf16_packed", ctypes.c_void_p)]


class MoeRouteProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("method", ctypes.c_int32), ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float)]


class MoeWsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("status", "counts", "cu_seqlens", "perm", "inv_perm", "w_sorted", "act", "y", "total",
                 "xq", "xq_rows", "aq", "single_launch", "mx_tiled", "aq_sc")]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        P = ctypes.POINTER(MoeProblem)
        L.moe_experts_workspace_bytes.argtypes = [P]
        L.moe_experts_workspace_bytes.restype = sz
        L.moe_experts_workspace_layout.argtypes = [P, ctypes.POINTER(MoeWsLayout)]
        L.moe_experts_workspace_layout.restype = ctypes.c_int
        fwd = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_experts_forward.argtypes = fwd
        L.moe_experts_forward.restype = ctypes.c_int
        L.moe_experts_forward_timed.argtypes = fwd + [ctypes.POINTER(vp), ctypes.c_int]
        L.moe_experts_forward_timed.restype = ctypes.c_int
        L.moe_experts_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_experts_forward_noalloc.restype = ctypes.c_int
        L.moe_align_workspace_bytes.argtypes = [i32, i32, i32]
        L.moe_align_workspace_bytes.restype = sz
        L.moe_align.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_align.restype = ctypes.c_int
        L.moe_experts_grouped_workspace_bytes.argtypes = [P]
        L.moe_experts_grouped_workspace_bytes.restype = sz
        L.moe_experts_forward_grouped.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_experts_forward_grouped.restype = ctypes.c_int
        L.moe_experts_forward_grouped_timed.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                                        ctypes.POINTER(vp), ctypes.c_int]
        L.moe_experts_forward_grouped_timed.restype = ctypes.c_int
        L.moe_device_error.argtypes = [vp, ctypes.POINTER(i32)]
        L.moe_device_error.restype = ctypes.c_int
        L.moe_route.argtypes = [ctypes.POINTER(MoeRouteProblem), vp, vp, vp, vp, vp]
        L.moe_route.restype = ctypes.c_int
        fp = ctypes.POINTER(ctypes.c_float)
        L.moe_check_expert_params.argtypes = [P, fp, fp, fp, fp, fp]
        L.moe_check_expert_params.restype = ctypes.c_int
        L.moe_mx_packed_bytes.argtypes = [P]
        L.moe_mx_packed_bytes.restype = sz
        L.moe_mx_pack_weights.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_mx_pack_weights.restype = ctypes.c_int
        L.moe_bf16_packed_bytes.argtypes = [P]
        L.moe_bf16_packed_bytes.restype = sz
        L.moe_bf16_pack_weights.argtypes = [P, vp, vp, vp, vp, sz, vp]
        L.moe_bf16_pack_weights.restype = ctypes.c_int
        L.moe_strerror.argtypes = [ctypes.c_int]
        L.moe_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().moe_strerror(status).decode()


EXPERT_PARAMS = ("alpha_e", "beta_e", "limit_e", "fc1_alpha", "fc2_alpha")


def problem(T, H, I, E, k=1, wfmt="bf16", act="silu", alpha=1.0, beta=0.0, limit=math.inf,
            weight_on_input=False, act_fmt="bf16", expert_params=None) -> MoeProblem:
    """expert_params: optional dict from EXPERT_PARAMS names to device float32
    tensors of E values (their pointers go into the problem)."""
    p = MoeProblem(int(T), int(H), int(I), int(E), int(k), _WFMT[wfmt] if isinstance(wfmt, str) else int(wfmt),
                   _ACT[act] if isinstance(act, str) else int(act), float(alpha), float(beta), float(limit),
                   int(weight_on_input), _AFMT[act_fmt] if isinstance(act_fmt, str) else int(act_fmt))
    for name, t in (expert_params or {}).items():
        if name not in EXPERT_PARAMS:
            raise KeyError(name)
        setattr(p, name, None if t is None else t.data_ptr())
    return p


def moe_check_expert_params(p: MoeProblem, alpha_e=None, beta_e=None, limit_e=None, fc1_alpha=None,
                            fc2_alpha=None) -> int:
    """Host-side check; each argument None or a sequence / CPU tensor of p.E floats."""
    keep = []

    def arr(v):
        if v is None:
            return None
        a = (ctypes.c_float * p.E)(*[float(x) for x in (v.tolist() if hasattr(v, "tolist") else v)])
        keep.append(a)
        return ctypes.cast(a, ctypes.POINTER(ctypes.c_float))

    return lib().moe_check_expert_params(ctypes.byref(p), arr(alpha_e), arr(beta_e), arr(limit_e), arr(fc1_alpha),
                                         arr(fc2_alpha))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int, where: str):
    if rc != MOE_OK:
        raise MoeError(rc, where)


# ---------------------------------------------------------------- C ABI, same names
def moe_experts_workspace_bytes(p: MoeProblem) -> int:
    return lib().moe_experts_workspace_bytes(ctypes.byref(p))


def moe_experts_workspace_layout(p: MoeProblem) -> MoeWsLayout:
    lay = MoeWsLayout()
    _check(lib().moe_experts_workspace_layout(ctypes.byref(p), ctypes.byref(lay)), "moe_experts_workspace_layout")
    return lay


def moe_mx_packed_bytes(p: MoeProblem) -> int:
    return lib().moe_mx_packed_bytes(ctypes.byref(p))


def moe_mx_pack_weights(p: MoeProblem, w_gate, w_up, w_down, s_gate, s_up, s_down, packed, stream=None) -> int:
    return lib().moe_mx_pack_weights(ctypes.byref(p), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate),
                                     _ptr(s_up), _ptr(s_down), _ptr(packed), packed.numel() * packed.element_size(),
                                     _stream(stream))


def mx_pack_weights(p: MoeProblem, w_gate, w_up, w_down, s_gate, s_up, s_down, stream=None) -> torch.Tensor:
    """Packed weights of problem p (a new uint8 device tensor); set p.mx_packed to its pointer."""
    n = moe_mx_packed_bytes(p)
    if n == 0:
        raise MoeError(MOE_EINVAL, "moe_mx_packed_bytes")
    packed = torch.empty(n, dtype=torch.uint8, device=w_gate.device)
    _check(moe_mx_pack_weights(p, w_gate, w_up, w_down, s_gate, s_up, s_down, packed, stream=stream),
           "moe_mx_pack_weights")
    return packed


def moe_bf16_packed_bytes(p: MoeProblem) -> int:
    return lib().moe_bf16_packed_bytes(ctypes.byref(p))


def moe_bf16_pack_weights(p: MoeProblem, w_gate, w_up, w_down, packed, stream=None) -> int:
    return lib().moe_bf16_pack_weights(ctypes.byref(p), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(packed),
                                       packed.numel() * packed.element_size(), _stream(stream))


def bf16_pack_weights(p: MoeProblem, w_gate, w_up, w_down, stream=None) -> torch.Tensor:
    """Operand-block weights of problem p (a new uint8 device tensor); set p.bf16_packed to its pointer."""
    n = moe_bf16_packed_bytes(p)
    if n == 0:
        raise MoeError(MOE_EINVAL, "moe_bf16_packed_bytes")
    packed = torch.empty(n, dtype=torch.uint8, device=w_gate.device)
    _check(moe_bf16_pack_weights(p, w_gate, w_up, w_down, packed, stream=stream), "moe_bf16_pack_weights")
    return packed


def moe_experts_forward(p: MoeProblem, x, topk_ids, topk_weights, w_gate, w_up, w_down, s_gate, s_up, s_down,
                        out, workspace, stream=None) -> int:
    return lib().moe_experts_forward(ctypes.byref(p), _ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(w_gate),
                                     _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(out),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream))


def moe_experts_forward_timed(p: MoeProblem, x, topk_ids, topk_weights, w_gate, w_up, w_down, s_gate, s_up,
                              s_down, out, workspace, events: Sequence[int], stream=None) -> int:
    arr = (ctypes.c_void_p * len(events))(*events)
    return lib().moe_experts_forward_timed(ctypes.byref(p), _ptr(x), _ptr(topk_ids), _ptr(topk_weights),
                                           _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up),
                                           _ptr(s_down), _ptr(out), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(stream), arr,
                                           len(events))


def moe_experts_forward_noalloc(p: MoeProblem, x, topk_ids, topk_weights, w_gate, w_up, w_down, s_gate, s_up,
                                s_down, out, stream=None) -> int:
    return lib().moe_experts_forward_noalloc(ctypes.byref(p), _ptr(x), _ptr(topk_ids), _ptr(topk_weights),
                                             _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up),
                                             _ptr(s_down), _ptr(out), _stream(stream))


def moe_align_workspace_bytes(T: int, k: int, E: int) -> int:
    return lib().moe_align_workspace_bytes(T, k, E)


def moe_align(topk_ids, T, k, E, counts, cu_seqlens, perm, inv_perm, workspace, stream=None) -> int:
    return lib().moe_align(_ptr(topk_ids), T, k, E, _ptr(counts), _ptr(cu_seqlens), _ptr(perm), _ptr(inv_perm),
                           _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))


def moe_experts_grouped_workspace_bytes(p: MoeProblem) -> int:
    return lib().moe_experts_grouped_workspace_bytes(ctypes.byref(p))


def moe_experts_forward_grouped(p: MoeProblem, x_nvs, cu_seqlens, route_w, w_gate, w_up, w_down, s_gate, s_up,
                                s_down, out_nvs, workspace, stream=None) -> int:
    return lib().moe_experts_forward_grouped(ctypes.byref(p), _ptr(x_nvs), _ptr(cu_seqlens), _ptr(route_w),
                                             _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up),
                                             _ptr(s_down), _ptr(out_nvs), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(stream))


def moe_experts_forward_grouped_timed(p: MoeProblem, x_nvs, cu_seqlens, route_w, w_gate, w_up, w_down, s_gate,
                                      s_up, s_down, out_nvs, workspace, events: Sequence[int], stream=None) -> int:
    arr = (ctypes.c_void_p * len(events))(*events)
    return lib().moe_experts_forward_grouped_timed(ctypes.byref(p), _ptr(x_nvs), _ptr(cu_seqlens), _ptr(route_w),
                                                   _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate),
                                                   _ptr(s_up), _ptr(s_down), _ptr(out_nvs), _ptr(workspace),
                                                   workspace.numel() * workspace.element_size(), _stream(stream),
                                                   arr, len(events))


def moe_device_error(workspace) -> int:
    n = ctypes.c_int32(0)
    _check(lib().moe_device_error(_ptr(workspace), ctypes.byref(n)), "moe_device_error")
    return n.value


def moe_strerror(status: int) -> str:
    return strerror(status)


def moe_route(p: MoeRouteProblem, logits, bias, topk_ids, topk_weights, stream=None) -> int:
    return lib().moe_route(ctypes.byref(p), _ptr(logits), _ptr(bias), _ptr(topk_ids), _ptr(topk_weights),
                           _stream(stream))


# ---------------------------------------------------------------- torch conveniences
def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """A caller-owned workspace (torch allocations are 256-byte aligned)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def experts_forward(x, topk_ids, topk_weights, w_gate, w_up, w_down, scales=None, act="silu", alpha=1.0, beta=0.0,
                    limit=math.inf, out=None, workspace=None, weight_on_input=False,
                    act_fmt="bf16", expert_params=None, mx_packed=None, bf16_packed=None) -> torch.Tensor:
    """Token-major experts step on torch tensors; allocates out/workspace if not given.
    mx_packed: the weights packed by mx_pack_weights (MXFP4 x MXFP8 only), or None.
    bf16_packed: the weights packed by bf16_pack_weights (bf16 only), or None."""
    T, H = x.shape
    k = topk_ids.shape[1]
    E = w_gate.shape[0]
    wfmt = "mxfp4" if w_gate.dtype == torch.uint8 else "bf16"
    I = w_gate.shape[1]
    p = problem(T, H, I, E, k, wfmt, act, alpha, beta, limit, weight_on_input, act_fmt, expert_params)
    if mx_packed is not None:
        p.mx_packed = mx_packed.data_ptr()
    if bf16_packed is not None:
        p.bf16_packed = bf16_packed.data_ptr()
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(moe_experts_workspace_bytes(p), x.device)
    sg, su, sd = scales if scales is not None else (None, None, None)
    _check(moe_experts_forward(p, x, topk_ids, topk_weights, w_gate, w_up, w_down, sg, su, sd, out, workspace),
           "moe_experts_forward")
    return out


def experts_forward_grouped(x_nvs, cu_seqlens, route_w, w_gate, w_up, w_down, scales=None, act="silu", alpha=1.0,
                            beta=0.0, limit=math.inf, out=None, workspace=None, weight_on_input=False,
                            act_fmt="bf16", expert_params=None, bf16_packed=None, mx_packed=None) -> torch.Tensor:
    """Pre-grouped experts step; bf16_packed / mx_packed: the weights packed by bf16_pack_weights /
    mx_pack_weights (for bf16 / MXFP4 weights), or None."""
    NvS, H = x_nvs.shape
    G = w_gate.shape[0]
    I = w_gate.shape[1]
    wfmt = "mxfp4" if w_gate.dtype == torch.uint8 else "bf16"
    p = problem(NvS, H, I, G, 1, wfmt, act, alpha, beta, limit, weight_on_input, act_fmt, expert_params)
    if bf16_packed is not None:
        p.bf16_packed = bf16_packed.data_ptr()
    if mx_packed is not None:
        p.mx_packed = mx_packed.data_ptr()
    if out is None:
        out = torch.empty(NvS, H, dtype=torch.bfloat16, device=x_nvs.device)
    if workspace is None:
        workspace = alloc_workspace(moe_experts_grouped_workspace_bytes(p), x_nvs.device)
    sg, su, sd = scales if scales is not None else (None, None, None)
    _check(moe_experts_forward_grouped(p, x_nvs, cu_seqlens, route_w, w_gate, w_up, w_down, sg, su, sd, out,
                                       workspace), "moe_experts_forward_grouped")
    return out


def route_problem(T, E, k, method="renormalize", n_group=0, topk_group=0,
                  routed_scaling_factor=1.0) -> MoeRouteProblem:
    return MoeRouteProblem(int(T), int(E), int(k), _ROUTE[method] if isinstance(method, str) else int(method),
                           int(n_group), int(topk_group), float(routed_scaling_factor))


def route(logits, k: int, method="renormalize", bias=None, n_group=0, topk_group=0, routed_scaling_factor=1.0,
          ids=None, weights=None):
    """moe_route on a float32 [T, E] tensor; returns (ids int32 [T, k], weights float32 [T, k])."""
    T, E = logits.shape
    dev = logits.device
    if ids is None:
        ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty(T, k, dtype=torch.float32, device=dev)
    p = route_problem(T, E, k, method, n_group, topk_group, routed_scaling_factor)
    _check(moe_route(p, logits, bias, ids, weights), "moe_route")
    return ids, weights


def align(topk_ids, E: int, workspace=None):
    """moe_align on a torch int32 [T, k] tensor; returns (counts, cu_seqlens, perm, inv_perm)."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    cu = torch.empty(E, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(moe_align_workspace_bytes(T, k, E), dev)
    _check(moe_align(topk_ids, T, k, E, counts, cu, perm, inv, workspace), "moe_align")
    return counts, cu, perm, inv, workspace
